// KV append (pa_write_kv) and copy-on-write block copy (pa_copy_blocks).
//
// Both are bit copies. A new token's K row is contiguous in the token-major
// K tile; its V column is strided by 16 elements in the dim-major V tile.
// A block of one pool is a contiguous run of Hkv * 16 * D elements, so a
// block copy is a flat 16-byte-vector copy.
#include "launch.h"

namespace pagedkv {

namespace {

// One workgroup per new token; threads stride over (kv head, dim).
template <typename W>
__global__ __launch_bounds__(256) void write_kv_kernel(const W* __restrict__ k_new,
                                                       const W* __restrict__ v_new,
                                                       const int32_t* __restrict__ slots,
                                                       W* __restrict__ k_pool,
                                                       W* __restrict__ v_pool, int hkv, int d) {
  const int t = blockIdx.x;
  const int s = slots[t];
  if (s < 0) return;
  const int blk = s / kBlockTokens;
  const int off = s % kBlockTokens;
  const int n = hkv * d;
  const W* kn = k_new + (size_t)t * n;
  const W* vn = v_new + (size_t)t * n;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int h = i / d;
    const int c = i - h * d;
    const size_t tile = ((size_t)blk * hkv + h) * (size_t)(kBlockTokens * d);
    k_pool[tile + (size_t)off * d + c] = kn[i];
    v_pool[tile + (size_t)c * kBlockTokens + off] = vn[i];
  }
}

// grid (pairs, 2): y = 0 copies the K block, y = 1 the V block.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_pool,
                                                          uint4* __restrict__ v_pool,
                                                          const int32_t* __restrict__ pairs,
                                                          size_t vecs_per_block) {
  const int i = blockIdx.x;
  const int src = pairs[2 * i];
  const int dst = pairs[2 * i + 1];
  uint4* pool = blockIdx.y ? v_pool : k_pool;
  const uint4* from = pool + (size_t)src * vecs_per_block;
  uint4* to = pool + (size_t)dst * vecs_per_block;
  for (size_t j = threadIdx.x; j < vecs_per_block; j += blockDim.x) to[j] = stream_load16(from + j);
}

}  // namespace

hipError_t launch_write_kv(const void* k_new, const void* v_new, const int32_t* slots,
                           int num_tokens, void* k_pool, void* v_pool, int num_kv_heads,
                           int head_dim, int elem_bytes, hipStream_t s) {
  dim3 grid(num_tokens), block(256);
  if (elem_bytes == 2) {
    const uint16_t* kn = (const uint16_t*)k_new;
    const uint16_t* vn = (const uint16_t*)v_new;
    uint16_t* kp = (uint16_t*)k_pool;
    uint16_t* vp = (uint16_t*)v_pool;
    void* args[] = {&kn, &vn, &slots, &kp, &vp, &num_kv_heads, &head_dim};
    return hipLaunchKernel((const void*)&write_kv_kernel<uint16_t>, grid, block, args, 0, s);
  }
  const uint32_t* kn = (const uint32_t*)k_new;
  const uint32_t* vn = (const uint32_t*)v_new;
  uint32_t* kp = (uint32_t*)k_pool;
  uint32_t* vp = (uint32_t*)v_pool;
  void* args[] = {&kn, &vn, &slots, &kp, &vp, &num_kv_heads, &head_dim};
  return hipLaunchKernel((const void*)&write_kv_kernel<uint32_t>, grid, block, args, 0, s);
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int num_pairs,
                              size_t block_bytes, hipStream_t s) {
  uint4* kp = (uint4*)k_pool;
  uint4* vp = (uint4*)v_pool;
  size_t vecs = block_bytes / sizeof(uint4);
  void* args[] = {&kp, &vp, &pairs, &vecs};
  return hipLaunchKernel((const void*)&copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), args,
                         0, s);
}

}  // namespace pagedkv
