// MFMA tile helpers shared by the matrix-core attention kernels of
// libpagedkv (gfx950): operand types, buffer resources and the loader of a
// 16-token K/V tile (K token-major [16, D], V^T dim-major [D, 16]) in the
// layout the 16x16 MFMA operands want.
#pragma once

#include "device_common.h"

namespace pagedkv {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;  // MFMA tile edge = padded head group

__device__ __forceinline__ uint32_t pack_bf16x2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

template <int D>
struct Tile {
  static constexpr int kQkSteps = D / 32;   // 16x16x32 products per score tile
  static constexpr int kDimTiles = D / 16;  // 16-dim output tiles
  bf16x8_t k[kQkSteps];                     // this lane's 8-element K pieces
  short4_t v[kDimTiles];                    // this lane's 4-token V pieces
};

// Buffer resource of one wave-uniform memory range: the base sits in
// scalar registers and every lane addresses it through a fixed 32-bit byte
// offset, so a new tile costs a few scalar instructions and no per-lane
// 64-bit address arithmetic. Reads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int bytes) {
  constexpr int kRsrcWord3 = 0x00020000;  // 32-bit data format, raw (unswizzled) access
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// Per-lane byte offsets of the tile operands, fixed for a kernel.
template <int D>
struct LaneOffsets {
  int k;  // K tile: token row, 8 dims at kg * 8 (+ 64 bytes per 32-dim step)
  int v;  // V^T tile: dim row, 4 tokens at kg * 4 (+ 512 bytes per 16-dim tile)
  __device__ __forceinline__ LaneOffsets(int row, int kg)
      : k((row * D + kg * 8) * 2), v((row * kBlockTokens + kg * 4) * 2) {}
};

// K/V tiles are read exactly once per call: their loads carry the
// nontemporal hint (cache policy bit `nt`), so they stream through the
// caches instead of displacing Q, the tables and each other. On MI355X this
// lifts a pure tile gather from about 5.9 to about 6.7 TB/s.
constexpr int kStreamLoad = 2;  // buffer-load cache policy: nt

// kPolicy: buffer-load cache policy, kStreamLoad for tiles read once;
// 0 (default) where several waves read the same tiles.
template <int D, int kPolicy = kStreamLoad>
__device__ __forceinline__ void load_tile(Tile<D>& tl, const bf16_t* kt, const bf16_t* vt,
                                          const LaneOffsets<D>& lo) {
  constexpr int kTileBytes = kBlockTokens * D * 2;
  const __amdgpu_buffer_rsrc_t kr = range_rsrc(kt, kTileBytes);
  const __amdgpu_buffer_rsrc_t vr = range_rsrc(vt, kTileBytes);
#pragma unroll
  for (int c = 0; c < Tile<D>::kQkSteps; ++c)
    tl.k[c] = __builtin_bit_cast(
        bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(kr, lo.k + c * 64, 0, kPolicy));
#pragma unroll
  for (int n = 0; n < Tile<D>::kDimTiles; ++n)
    tl.v[n] = __builtin_bit_cast(
        short4_t, __builtin_amdgcn_raw_buffer_load_b64(vr, lo.v + n * kTile * kBlockTokens * 2, 0,
                                                       kPolicy));
}

}  // namespace mfma
}  // namespace pagedkv
