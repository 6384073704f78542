// Device helpers shared by the gfx950 kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pagedkv {

constexpr int kBlockTokens = 16;  // tokens per KV block (fixed)

// bf16 is carried as its raw 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

// ---- element conversion ---------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct ElemTraits;

template <> struct ElemTraits<float> {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
  __device__ static __forceinline__ void store1(float* p, float v) { *p = v; }
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  }
  // zero the elements whose index (0..3) is >= nvalid
  __device__ static __forceinline__ float zero() { return 0.f; }
};

template <> struct ElemTraits<bf16_t> {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ float load1(const bf16_t* p) {
    return __uint_as_float((uint32_t)p->bits << 16);
  }
  __device__ static __forceinline__ void store1(bf16_t* p, float v) { p->bits = f32_to_bf16_bits(v); }
  __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
    f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
    f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
  }
};

// ---- math ----------------------------------------------------------------

// 2^x on the hardware exponential unit; 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- wave-level exchange -------------------------------------------------

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// The value of lane l and of lane l ^ 16 (xor16) or l ^ 32 (xor32), lower
// lane first, in every lane, through the gfx950 permlane swaps: VALU
// instructions, so unlike LDS-based shuffles they never wait behind
// outstanding scalar loads.
__device__ __forceinline__ float2 pair_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 pair_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max / sum over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 (same in all four)
__device__ __forceinline__ float max_over_kg(float v) {
  float2 p = pair_xor16(v);
  v = fmaxf(p.x, p.y);
  p = pair_xor32(v);
  return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float sum_over_kg(float v) {
  float2 p = pair_xor16(v);
  v = p.x + p.y;
  p = pair_xor32(v);
  return p.x + p.y;
}

// Orders this wave's LDS writes before its later LDS reads (and vice versa)
// without a workgroup barrier: waves of one workgroup run loops of
// different trip counts, so only the issuing wave may be synchronised.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- streaming reads -------------------------------------------------------

// 16 bytes of data that is read once per call (K/V tiles, blocks being
// copied), with the nontemporal hint so it streams through the caches.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 stream_load16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- uniform reads ---------------------------------------------------------

// Read-only int32 inputs indexed by wave-uniform values (block tables,
// lengths) are read through the constant address space, which makes them
// scalar loads: they are counted apart from the vector loads of K/V tiles,
// so waiting for a table entry never drains the tile prefetch.
typedef __attribute__((address_space(4))) const int32_t const_i32_t;

__device__ __forceinline__ int32_t uniform_load(const int32_t* base, size_t idx) {
  return ((const const_i32_t*)base)[idx];
}

// The same for a non-negative index below 2^30: the byte offset stays a
// 32-bit register operand of the scalar load, with no 64-bit address math.
__device__ __forceinline__ int32_t uniform_load_u32(const int32_t* base, uint32_t idx) {
  typedef __attribute__((address_space(4))) const char const_char_t;
  return *(const const_i32_t*)((const const_char_t*)base + (idx << 2));
}

// ---- decode arguments ------------------------------------------------------

// Everything a decode kernel needs; passed by value.
struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  // fp32 partials (log2-domain max m, sum of 2^(s - m), unnormalised output):
  //   fixed split     ws_m, ws_l [rows], ws_o [rows, D] with
  //                   row (b * Hq + h) * NPmax + partition
  //   balanced split  ws_o holds one record per piece slot (2 * wave + k):
  //                   O^T in accumulator order, then m[G], then l[G]
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int* ws_cnt;   // pieces (balanced) or partitions (fixed, matrix-core kernel) finished
                 // per (b, kvh); zero between calls
  float scale_log2;  // scale * log2(e)
  int num_seqs, num_q_heads, num_kv_heads, group, max_blocks, part_tokens, num_parts;
  int split_waves;     // balanced split: waves of the decode grid (4 per workgroup)
  int min_seg_blocks;  // balanced split: least blocks per wave range
  int stage_slots;     // balanced split: complete outputs a wave stages in LDS (0 = none)
  int slot_grid;       // fixed split (matrix-core kernel): 1 when the grid has one workgroup
                       // per (row, partition, KV head) slot, in that order, empty ones included
  int block_shift;     // log2 of the tokens per KV block (4 = 16 tokens)
  // fused KV append (balanced split): row b's new token k_new/v_new[b] is
  // stored at slot_mapping[b] (skipped when negative) before it is read;
  // null when the call appends nothing
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
};

// Everything the chunked-prefill kernel needs; passed by value.
struct PrefillArgs {
  const void* q;             // [T, Hq, D]
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;     // [S], the chunk included
  const int32_t* query_start;  // [S + 1]: rows of q owned by each sequence
  void* out;                   // [T, Hq, D]
  float scale_log2;
  int num_seqs, num_q_heads, num_kv_heads, group, max_blocks, block_shift;
};

// Everything the latent (MLA-style) decode kernel needs; passed by value.
struct LatentArgs {
  const void* q;               // [B, H, 576] absorbed queries
  const void* kv_pool;         // [NB, 64, 576] latent blocks
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;                   // [B, H, 512]
  // cut rows: records of two piece slots per workgroup (fp16 O[h][d]
  // normalised by the piece's sum and scaled per head by a power of two,
  // then fp32 m[H], l[H] and the inverse scales s[H]) and per row a
  // description of its pieces (first slot, count), written by every call
  // for the rows with tokens
  void* ws_rec;
  int* ws_cnt;   // [B][2]
  float scale_log2;
  int num_seqs, max_blocks;
  int grid;       // workgroups of the launch
  int min_tiles;  // least 32-token tiles per workgroup range
};

}  // namespace pagedkv
