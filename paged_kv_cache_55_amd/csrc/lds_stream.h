// Streaming tiles from HBM into LDS with loads that carry an LDS destination
// (gfx950 buffer_load_dwordx4 ... lds and global_load_lds_dwordx4): lane l
// of a wave load writes 16 bytes at M0 + 16 l. The buffer form reads any
// byte offset of a descriptor (offsets past its range load zeros); the
// global form reads one address per lane. Shared by the kernels whose
// workgroups share each tile among their waves.
#pragma once

#include "device_common.h"

namespace pagedkv {
namespace lds_stream {

typedef __attribute__((address_space(3))) char lds_char;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPastRange = 0x7ffffff0;  // buffer offset past any range: the load gives zeros

// A raw buffer descriptor of `bytes` bytes at `base` (32-bit data format,
// unswizzled; reads past the range give zero).
__device__ __forceinline__ u32x4_t raw_rsrc(const void* base, int bytes) {
  const uint64_t p = (uint64_t)base;
  return (u32x4_t){(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, (uint32_t)bytes, 0x00020000u};
}

// 16 bytes per lane from the buffer at byte offset `off` into LDS at
// `dst` + 16 * lane (buffer_load_dwordx4 with the LDS destination in M0),
// with the non-temporal cache policy: for data read once. Written as
// assembly so that the compiler does not track these LDS writes: it cannot
// tell the stages apart and would otherwise make every later LDS read wait
// for all of them, the prefetch included. Completion is awaited explicitly
// (tile_barrier).
//
// Both load forms leave M0 holding `dst`. The compiler keeps M0 reserved
// and would not honour it as an asm clobber, so they are only for kernels
// in which nothing else reads M0 (no relative moves, messages or other
// M0-addressed instructions): the chunked-prefill and latent-decode
// kernels, whose generated code a test checks for exactly that. Dropping
// the save and restore measured 1.2% on prefill (its loader waves share
// the scalar unit with the waves beside them) and 2.1% on latent decode
// (one wave per SIMD: the refill's scalar instructions sit on its path).
__device__ __forceinline__ void load_to_lds(u32x4_t rsrc, lds_char* dst, int off) {
  const uint32_t m0 = (uint32_t)(uintptr_t)dst;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
      :
      : "s"(m0), "v"(off), "s"(rsrc)
      : "memory");
}

// 16 bytes per lane from the global address `src` (one per lane) into LDS
// at `dst` + 16 * lane (global_load_lds_dwordx4), default cache policy: the
// lines stay in L2 for other workgroups that read the same tile. Untracked
// by the compiler like load_to_lds, awaited with wait_loads, and leaving
// M0 holding `dst` as load_to_lds does.
__device__ __forceinline__ void global_load_to_lds(const void* src, lds_char* dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)dst;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(m0), "v"(src)
      : "memory");
}

// Waits until at most kYounger of this wave's vector memory operations are
// outstanding (they complete in order: everything older has landed), and
// for this wave's LDS operations.
template <int kYounger>
__device__ __forceinline__ void wait_loads() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kYounger) : "memory");
}

// Every wave of the workgroup gets here; no memory operation is awaited.
__device__ __forceinline__ void workgroup_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// wait_loads<kYounger>, then a workgroup barrier. With kYounger no larger
// than the loads each wave issued after a tile's, the tile is complete in
// LDS for every wave, and every wave is done with the stages read before.
template <int kYounger>
__device__ __forceinline__ void tile_barrier() {
  wait_loads<kYounger>();
  workgroup_barrier();
}

// A workgroup barrier for LDS traffic only; outstanding loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace lds_stream
}  // namespace pagedkv
