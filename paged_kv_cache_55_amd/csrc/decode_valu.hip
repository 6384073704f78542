// Paged decode attention on the vector ALUs (f32 and bf16, D = 64 or 128).
//
// A persistent grid of 4-wave workgroups walks the work list of
// (sequence, partition, KV head) items (worklist.h). A partition is
// `part_tokens` consecutive tokens (a multiple of 16); the waves of a
// workgroup take the partition's 16-token blocks round robin. For each
// block the wave
//   1. reads the block's physical id from the table (wave-uniform load),
//   2. loads the 16 x D K tile (16-byte loads, 4 lanes per token row),
//   3. forms the G scores of each token (q held in LDS, fp32 FMA), reduces
//      them over the 4 lanes of a row and masks tokens >= L to -inf by
//      select (tail slots may hold anything, NaN included),
//   4. updates the per-head running max m and sum l (online softmax, in
//      the base-2 domain with scale * log2(e) folded into q),
//   5. loads the D x 16 V tile (each lane owns D / 64 dims, all 16 tokens)
//      and accumulates p * V into fp32, masking V of invalid tokens to 0.
// The 4 waves' (m, l, acc) are merged through LDS. A sequence with one
// partition writes its output directly; otherwise the partition writes its
// fp32 partial (m, l, acc) to the workspace for decode_reduce.
//
// The gather and the attention follow cs2680 Lecture 10, §10.3 ("Step
// three": per block, a table read then a gather) and llm-serving.xyz
// "KV-cache systems" (the table read sits in front of the gather).
#include "launch.h"
#include "worklist.h"

namespace pagedkv {

namespace {

constexpr int kWaves = 4;

template <typename T, int D, int GP>
struct ValuSmem {
  float qs[GP][D];
  float pbuf[kWaves][kBlockTokens][GP];
  float red_m[kWaves][GP];
  float red_l[kWaves][GP];
  float red_o[kWaves][GP][D];
};

// One work item: partition `part` of sequence b against KV head kvh.
template <typename T, int D, int GP>
__device__ __forceinline__ void valu_item(const DecodeArgs& a, int b, int kvh, int part, int L,
                                          ValuSmem<T, D, GP>& sm) {
  using Tr = ElemTraits<T>;
  constexpr int E = Tr::kPerVec;           // elements per 16-byte load
  constexpr int NCH = D / (4 * E);         // 16-byte chunks per lane per K row
  constexpr int DPL = D / 64;              // V dims owned by each lane
  static_assert(NCH >= 1 && DPL >= 1, "unsupported head dim");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int h0 = kvh * G;
  T* out = (T*)a.out;

  const int tok0 = part * a.part_tokens;
  const int tok_end = min(L, tok0 + a.part_tokens);
  const int nblk = (tok_end - tok0 + kBlockTokens - 1) / kBlockTokens;
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  auto& qs = sm.qs;
  auto& pbuf = sm.pbuf;
  auto& red_m = sm.red_m;
  auto& red_l = sm.red_l;
  auto& red_o = sm.red_o;

  const T* qp = (const T*)a.q + ((size_t)b * Hq + h0) * D;
  for (int i = tid; i < GP * D; i += blockDim.x) {
    const int g = i / D;
    qs[g][i - g * D] = g < G ? Tr::load1(qp + i) * a.scale_log2 : 0.f;
  }
  __syncthreads();

  float m_run[GP], l_lane[GP], acc[GP][DPL];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    m_run[g] = -INFINITY;
    l_lane[g] = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[g][k] = 0.f;
  }

  const int t = lane >> 2;  // token row this lane scores
  const int c = lane & 3;   // quarter of the row
  const T* kbase = (const T*)a.k_pool;
  const T* vbase = (const T*)a.v_pool;
  const size_t bt_row = (size_t)b * a.max_blocks + tok0 / kBlockTokens;
  const size_t tile_elems = (size_t)kBlockTokens * D;

  for (int i = w; i < nblk; i += kWaves) {
    const int phys = uniform_load(a.block_tables, bt_row + i);
    const size_t tile = ((size_t)phys * a.num_kv_heads + kvh) * tile_elems;
    const T* kt = kbase + tile;
    const T* vt = vbase + tile;
    const int nvalid = min(kBlockTokens, tok_end - (tok0 + i * kBlockTokens));

    // ---- scores ----
    float s[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) s[g] = 0.f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int d0 = ch * 4 * E + c * E;
      const uint4 raw = stream_load16(kt + (size_t)t * D + d0);
      float kf[E];
      Tr::unpack(raw, kf);
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < E; ++e) s[g] = fmaf(qs[g][d0 + e], kf[e], s[g]);
    }
    const bool valid = t < nvalid;
    float alpha[GP], p[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      s[g] += shfl_xor(s[g], 1);
      s[g] += shfl_xor(s[g], 2);
      s[g] = valid ? s[g] : -INFINITY;
      float mb = s[g];
      mb = fmaxf(mb, shfl_xor(mb, 4));
      mb = fmaxf(mb, shfl_xor(mb, 8));
      mb = fmaxf(mb, shfl_xor(mb, 16));
      mb = fmaxf(mb, shfl_xor(mb, 32));
      const float m_new = fmaxf(m_run[g], mb);
      alpha[g] = fast_exp2(m_run[g] - m_new);
      p[g] = fast_exp2(s[g] - m_new);
      m_run[g] = m_new;
      l_lane[g] = l_lane[g] * alpha[g] + (c == 0 ? p[g] : 0.f);
    }
    if (c == 0) {
#pragma unroll
      for (int g = 0; g < GP; ++g) pbuf[w][t][g] = p[g];
    }
    wave_lds_sync();

    // ---- values ----
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int d = lane + 64 * k;
      const T* vrow = vt + (size_t)d * kBlockTokens;
      float vf[kBlockTokens];
#pragma unroll
      for (int j = 0; j < kBlockTokens / E; ++j) {
        const uint4 raw = stream_load16(vrow + j * E);
        Tr::unpack(raw, vf + j * E);
      }
      if (nvalid < kBlockTokens) {
#pragma unroll
        for (int j = 0; j < kBlockTokens; ++j) vf[j] = j < nvalid ? vf[j] : 0.f;
      }
#pragma unroll
      for (int g = 0; g < GP; ++g) acc[g][k] *= alpha[g];
#pragma unroll
      for (int j = 0; j < kBlockTokens; ++j) {
#pragma unroll
        for (int g = 0; g < GP; ++g) acc[g][k] = fmaf(pbuf[w][j][g], vf[j], acc[g][k]);
      }
    }
    wave_lds_sync();
  }

  // ---- merge the waves ----
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    float l = l_lane[g];
    l += shfl_xor(l, 1);
    l += shfl_xor(l, 2);
    l += shfl_xor(l, 4);
    l += shfl_xor(l, 8);
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (lane == 0) {
      red_m[w][g] = m_run[g];
      red_l[w][g] = l;
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) red_o[w][g][lane + 64 * k] = acc[g][k];
  }
  __syncthreads();

  for (int i = tid; i < G * D; i += blockDim.x) {
    const int g = i / D;
    const int d = i - g * D;
    float M = red_m[0][g];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) M = fmaxf(M, red_m[v][g]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float f = fast_exp2(red_m[v][g] - M);  // a wave with no block has m = -inf
      lsum = fmaf(red_l[v][g], f, lsum);
      o = fmaf(red_o[v][g][d], f, o);
    }
    if (nparts == 1) {
      Tr::store1(out + ((size_t)b * Hq + h0 + g) * D + d, o / lsum);
    } else {
      const size_t r = ((size_t)b * Hq + h0 + g) * a.num_parts + part;
      a.ws_o[r * D + d] = o;
      if (d == 0) {
        a.ws_m[r] = M;
        a.ws_l[r] = lsum;
      }
    }
  }
  __syncthreads();  // q and the merge buffers are reused by the next item
}

template <typename T, int D, int GP>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  extern __shared__ int prefix[];  // [B + 1]
  __shared__ int scan_scratch[kWaves];
  __shared__ ValuSmem<T, D, GP> sm;

  const int B = a.num_seqs;
  build_partition_prefix(a.seq_lens, B, a.part_tokens, prefix, scan_scratch);

  // padded rows (L <= 0): exact zeros, no K/V or table reads
  const int row_elems = a.num_q_heads * D;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    if (prefix[b + 1] != prefix[b]) continue;
    T* o = (T*)a.out + (size_t)b * row_elems;
    for (int i = threadIdx.x; i < row_elems; i += blockDim.x) ElemTraits<T>::store1(o + i, 0.f);
  }

  const int Hkv = a.num_kv_heads;
  const int nitems = prefix[B] * Hkv;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int j = item / Hkv;
    const int kvh = item - j * Hkv;
    const int b = find_sequence(prefix, B, j);
    const int bu = __builtin_amdgcn_readfirstlane(b);
    valu_item<T, D, GP>(a, bu, kvh, j - prefix[bu], uniform_load(a.seq_lens, bu), sm);
  }
}

template <typename T, int D>
const void* pick_fn(int G) {
  if (G <= 1) return (const void*)&decode_valu_kernel<T, D, 1>;
  if (G <= 2) return (const void*)&decode_valu_kernel<T, D, 2>;
  if (G <= 4) return (const void*)&decode_valu_kernel<T, D, 4>;
  if (G <= 8) return (const void*)&decode_valu_kernel<T, D, 8>;
  return (const void*)&decode_valu_kernel<T, D, 16>;
}

}  // namespace

const void* decode_valu_fn(int dtype, int head_dim, int group) {
  if (dtype == 0) return head_dim == 64 ? pick_fn<float, 64>(group) : pick_fn<float, 128>(group);
  return head_dim == 64 ? pick_fn<bf16_t, 64>(group) : pick_fn<bf16_t, 128>(group);
}

hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_dim, int grid,
                              hipStream_t s) {
  DecodeArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(decode_valu_fn(dtype, head_dim, a.group), dim3(grid), dim3(256), args,
                         (size_t)(a.num_seqs + 1) * sizeof(int), s);
}

}  // namespace pagedkv
