// Cross-partition merge of split-K paged decode.
//
// Partition p of (sequence b, query head h) left (m_p, l_p, o_p): the max
// of its base-2 scaled scores, the sum of 2^(s - m_p) and the unnormalised
// sum of 2^(s - m_p) V. With M = max_p m_p the merged result is
//   out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// taken in partition order, so reruns are bit-identical. Sequences with at
// most one partition were finished by the partition kernel and are skipped.
// The vector-ALU kernel's fixed split uses this pass; the matrix-core
// kernel merges its partitions in place.
#include "launch.h"

namespace pagedkv {

namespace {

// One workgroup per (KV head, sequence): its G query heads x D outputs.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const int L = a.seq_lens[b];
  const int np = (L + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;
  const int G = a.group;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int g = idx / D;
    const int d = idx - g * D;
    const int h = kvh * G + g;
    const size_t r0 = ((size_t)b * a.num_q_heads + h) * a.num_parts;
    float M = -INFINITY;
    for (int p = 0; p < np; ++p) M = fmaxf(M, a.ws_m[r0 + p]);
    float lsum = 0.f, o = 0.f;
    for (int p = 0; p < np; ++p) {
      const float f = fast_exp2(a.ws_m[r0 + p] - M);
      lsum = fmaf(a.ws_l[r0 + p], f, lsum);
      o = fmaf(a.ws_o[(r0 + p) * D + d], f, o);
    }
    ElemTraits<T>::store1((T*)a.out + ((size_t)b * a.num_q_heads + h) * D + d, o / lsum);
  }
}

template <typename T, int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  DecodeArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel((const void*)&decode_reduce_kernel<T, D>,
                         dim3(a.num_kv_heads, a.num_seqs), dim3(256), args, 0, s);
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeArgs& a, int dtype, int head_dim, hipStream_t s) {
  if (dtype == 0) return head_dim == 64 ? launch_t<float, 64>(a, s) : launch_t<float, 128>(a, s);
  return head_dim == 64 ? launch_t<bf16_t, 64>(a, s) : launch_t<bf16_t, 128>(a, s);
}

}  // namespace pagedkv
