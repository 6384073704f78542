// KV append (pa_write_kv, pa_latent_write), copy-on-write block copy
// (pa_copy_blocks) and a zero fill of device memory.
//
// Both are bit copies. A new token's K row is contiguous in the token-major
// K region of its block; its V column is strided in the dim-major V tile
// that holds it (the whole block up to 16 tokens, else the 16-token tile).
// A block of one pool is a contiguous run of Hkv * block_size * D elements,
// so a block copy is a flat 16-byte-vector copy.
#include "launch.h"

namespace pagedkv {

namespace {

// One wave per (new token, KV head), four per workgroup. The K row (D
// contiguous elements) moves as 16-byte vectors on the first
// D * sizeof(W) / 16 lanes; the V column (one element per dim, 16 elements
// apart) on all lanes, D / 64 elements each. All loads are issued before
// the slot is known, so the copy costs one memory round trip.
template <typename W>
__global__ __launch_bounds__(256) void write_kv_kernel(const W* __restrict__ k_new,
                                                       const W* __restrict__ v_new,
                                                       const int32_t* __restrict__ slots,
                                                       W* __restrict__ k_pool,
                                                       W* __restrict__ v_pool, int num_tokens,
                                                       int hkv, int d, int block_shift) {
  constexpr int kPerVec = 16 / sizeof(W);
  const int lane = threadIdx.x & 63;
  const int kvec = d / kPerVec;  // <= 32
  const long long npairs = (long long)num_tokens * hkv;
  const long long stride = (long long)gridDim.x * 4;
  for (long long p = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); p < npairs; p += stride) {
    const int t = (int)(p / hkv);
    const int h = (int)(p - (long long)t * hkv);
    const size_t src = (size_t)p * d;  // k_new / v_new [t, h, :]
    uint4 kv = make_uint4(0, 0, 0, 0);
    if (lane < kvec) kv = *(const uint4*)(k_new + src + lane * kPerVec);
    W vv[2];
    vv[0] = v_new[src + lane];
    if (d > 64) vv[1] = v_new[src + 64 + lane];
    const int s = uniform_load(slots, t);
    if (s < 0) continue;
    const int bs = 1 << block_shift;
    const int inner = bs < kBlockTokens ? bs : kBlockTokens;  // V: dim-major tiles
    const int blk = s >> block_shift;
    const int off = s & (bs - 1);
    const size_t region = (((size_t)blk * hkv + h) << block_shift) * d;
    if (lane < kvec) *(uint4*)(k_pool + region + (size_t)off * d + lane * kPerVec) = kv;
    W* vp = v_pool + region + (size_t)(off & ~(inner - 1)) * d + (off & (inner - 1));
    vp[(size_t)lane * inner] = vv[0];
    if (d > 64) vp[(size_t)(64 + lane) * inner] = vv[1];
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

// One wave per new latent, four per workgroup: 72 16-byte vectors of the
// 1,152-byte latent row, loaded before the slot is known.
__global__ __launch_bounds__(256) void latent_write_kernel(const uint4* __restrict__ kv_new,
                                                           const int32_t* __restrict__ slots,
                                                           uint4* __restrict__ kv_pool,
                                                           int num_tokens) {
  constexpr int kVecs = kLatentDim * 2 / 16;  // 72
  const int lane = threadIdx.x & 63;
  const long long stride = (long long)gridDim.x * 4;
  for (long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); t < num_tokens; t += stride) {
    const uint4* src = kv_new + (size_t)t * kVecs;
    const uint4 a = src[lane];
    uint4 b = make_uint4(0, 0, 0, 0);
    if (lane < kVecs - 64) b = src[64 + lane];
    const int s = uniform_load(slots, t);
    if (s < 0) continue;
    uint4* dst = kv_pool + (size_t)s * kVecs;
    dst[lane] = a;
    if (lane < kVecs - 64) dst[64 + lane] = b;
  }
}

}  // namespace

hipError_t launch_latent_write(const void* kv_new, const int32_t* slots, int num_tokens,
                               void* kv_pool, hipStream_t s) {
  const long long wgs = ((long long)num_tokens + 3) / 4;
  dim3 grid((unsigned)(wgs < (1 << 16) ? wgs : (1 << 16))), block(256);
  const uint4* kn = (const uint4*)kv_new;
  uint4* kp = (uint4*)kv_pool;
  void* args[] = {&kn, &slots, &kp, &num_tokens};
  return hipLaunchKernel((const void*)&latent_write_kernel, grid, block, args, 0, s);
}

hipError_t launch_write_kv(const void* k_new, const void* v_new, const int32_t* slots,
                           int num_tokens, void* k_pool, void* v_pool, int num_kv_heads,
                           int head_dim, int block_shift, int elem_bytes, hipStream_t s) {
  // four (token, head) pairs per workgroup; a grid-stride loop covers the rest
  const long long pairs = (long long)num_tokens * num_kv_heads;
  const long long wgs = (pairs + 3) / 4;
  dim3 grid((unsigned)(wgs < (1 << 16) ? wgs : (1 << 16))), block(256);
  if (elem_bytes == 2) {
    const uint16_t* kn = (const uint16_t*)k_new;
    const uint16_t* vn = (const uint16_t*)v_new;
    uint16_t* kp = (uint16_t*)k_pool;
    uint16_t* vp = (uint16_t*)v_pool;
    void* args[] = {&kn, &vn, &slots, &kp, &vp, &num_tokens, &num_kv_heads, &head_dim,
                    &block_shift};
    return hipLaunchKernel((const void*)&write_kv_kernel<uint16_t>, grid, block, args, 0, s);
  }
  const uint32_t* kn = (const uint32_t*)k_new;
  const uint32_t* vn = (const uint32_t*)v_new;
  uint32_t* kp = (uint32_t*)k_pool;
  uint32_t* vp = (uint32_t*)v_pool;
  void* args[] = {&kn, &vn, &slots, &kp, &vp, &num_tokens, &num_kv_heads, &head_dim,
                  &block_shift};
  return hipLaunchKernel((const void*)&write_kv_kernel<uint32_t>, grid, block, args, 0, s);
}

// Zero-fill of n 16-byte vectors: a kernel rather than a memset, so that a
// captured graph replays it like any other launch.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  uint4* v = (uint4*)p;
  size_t n = bytes / sizeof(uint4);
  const size_t blocks = (n + 255) / 256;
  void* args[] = {&v, &n};
  return hipLaunchKernel((const void*)&zero_fill_kernel,
                         dim3((unsigned)(blocks < 1024 ? (blocks > 0 ? blocks : 1) : 1024)),
                         dim3(256), args, 0, s);
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
