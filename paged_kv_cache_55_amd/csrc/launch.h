// Host-side launchers of the libpagedkv kernels (internal; the public
// interface is include/pagedkv.h). Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace pagedkv {

// dtype: 0 = f32, 1 = bf16 (pa_dtype).
// Persistent decode kernels: `grid` workgroups of 256 threads, dynamic LDS
// of (num_seqs + 1) ints for the work list.
hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_dim, int grid,
                              hipStream_t s);
// contiguous: the balanced kernel over unpaged caches (tile j of (b, kvh)
// at ((b * Hkv + kvh) * max_blocks + j) * 16 * D; no table)
hipError_t launch_decode_mfma(const DecodeArgs& a, int head_dim, bool balanced, int grid,
                              hipStream_t s, bool contiguous = false);
const void* decode_valu_fn(int dtype, int head_dim, int group);
const void* decode_mfma_fn(int head_dim, bool balanced, int block_shift, bool contiguous = false);
// dynamic LDS bytes of a decode_mfma launch (stage_slots: balanced split only)
size_t decode_mfma_smem(int num_seqs, int group, int head_dim, bool balanced, int stage_slots);
// Balanced split: fp32 record of one piece of a (sequence, KV head) pair,
// O[g][d] (head-major), then m[G], then l[G], padded to 16 bytes.
__host__ __device__ inline int piece_floats(int group, int head_dim) {
  return group * head_dim + ((2 * group + 3) & ~3);
}
// LDS area of one wave of the balanced kernel, in floats: two parked
// pieces, then `slots` staged bf16 outputs of G x D, then their destination
// pair indices (int32, padded to 16 bytes).
__host__ __device__ inline int staged_output_floats(int group, int head_dim) {
  return group * head_dim / 2;
}
__host__ __device__ inline int balanced_wave_floats(int group, int head_dim, int slots) {
  return 2 * piece_floats(group, head_dim) + slots * staged_output_floats(group, head_dim) +
         ((slots + 3) & ~3);
}
// Largest number of staged outputs per wave (bounded by kMaxStageSlots) for
// which a balanced-split workgroup fits `lds_bytes` of LDS.
constexpr int kMaxStageSlots = 16;
inline int balanced_stage_slots(int num_seqs, int group, int head_dim, size_t lds_bytes) {
  for (int slots = kMaxStageSlots; slots > 0; --slots) {
    const size_t need = (size_t)((num_seqs + 4) & ~3) * sizeof(int) +
                        (size_t)4 * balanced_wave_floats(group, head_dim, slots) * sizeof(float);
    if (need <= lds_bytes) return slots;
  }
  return 0;
}
hipError_t launch_decode_reduce(const DecodeArgs& a, int dtype, int head_dim, hipStream_t s);

// Chunked-prefill attention (bf16, blocks of 16 or more tokens): persistent
// grid of `grid` workgroups; dynamic LDS: the tile stages and (num_seqs + 1)
// ints.
constexpr int kPrefillThreads = 512;  // workgroup size of the prefill kernel
const void* prefill_mfma_fn(int head_dim);
size_t prefill_mfma_smem(int num_seqs, int head_dim);  // dynamic LDS bytes of a launch
hipError_t launch_prefill_mfma(const PrefillArgs& a, int head_dim, int grid, hipStream_t s);

// Latent (MLA-style) decode, fixed shape: 128 heads over one 576-element
// latent per token (512 value elements), 64-token blocks, 32-token tiles in
// three LDS stages of 39 KiB, one workgroup of 256 threads per compute unit.
constexpr int kLatentHeads = 128;
constexpr int kLatentDim = 576;
constexpr int kLatentValueDim = 512;
constexpr int kLatentBlockTokens = 64;
constexpr int kLatentTileTokens = 32;
constexpr int kLatentStageBytes = 39 * 1024;
constexpr int kLatentStages = 3;
// record of one piece of a cut row: its output normalised by its own sum
// and scaled per head by a power of two, fp16 [H][512], then fp32 max m[H],
// sum l[H] and inverse scale s[H] (129.5 KiB)
constexpr int kLatentRecordBytes = kLatentHeads * kLatentValueDim * 2 + 3 * kLatentHeads * 4;
const void* latent_decode_fn();
size_t latent_decode_smem(int num_seqs);
hipError_t launch_latent_decode(const LatentArgs& a, hipStream_t s);
// Latent append: kv_pool row slot_mapping[t] <- kv_new[t] (576 elements).
hipError_t launch_latent_write(const void* kv_new, const int32_t* slots, int num_tokens,
                               void* kv_pool, hipStream_t s);

hipError_t launch_write_kv(const void* k_new, const void* v_new, const int32_t* slots,
                           int num_tokens, void* k_pool, void* v_pool, int num_kv_heads,
                           int head_dim, int block_shift, int elem_bytes, hipStream_t s);
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int num_pairs,
                              size_t block_bytes, hipStream_t s);
// Zero-fills `bytes` (a multiple of 16) at the 16-byte aligned device
// address `p` with a kernel.
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s);

}  // namespace pagedkv
