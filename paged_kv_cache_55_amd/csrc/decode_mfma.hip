// Paged decode attention on the CDNA4 matrix cores (bf16, D = 64 or 128,
// up to 16 query heads per KV head).
//
// Same decomposition as the vector-ALU kernel: one workgroup (4 waves) per
// (partition, KV head, sequence), waves taking the partition's 16-token
// blocks round robin, an online softmax per wave and a merge of the waves
// through LDS. The G query heads that share a KV head are padded to the
// 16 columns of a 16x16 MFMA tile, so each 16-token block is two small
// dense products:
//
//   scores  S^T[t][g] = sum_d K[t][d] Q[g][d]       v_mfma_f32_16x16x32_bf16,
//           A = K tile (row t = lane % 16), B = Q^T (column g = lane % 16);
//   values  O^T[d][g] += sum_t V^T[d][t] P^T[t][g]   v_mfma_f32_16x16x16_bf16,
//           A = V^T tile (row d), B = P^T.
//
// The 16x16 accumulator layout gives lane l the rows 4 * (l / 16) + r,
// r = 0..3, of column l % 16. After the score product a lane therefore
// holds the scores of head l % 16 for tokens 4 * (l / 16) .. + 3, which is
// exactly the B operand the value product needs (k = token), and the value
// accumulator keeps head l % 16 in the same lane, so the softmax rescale is
// lane-local. The dim-major V tile makes the A operand of the value product
// a contiguous 8-byte load (4 tokens of one dim).
//
// Precision: scores and the output accumulate in fp32; the probabilities
// are fed to the bf16 value product as the sum of two bf16 numbers
// (p = hi + lo), so the product sees p to about 2^-17 relative.
//
// Tokens at or past the sequence length are masked by select: scores to
// -inf and V elements to 0, so stale or NaN tail slots never reach the
// result.
#include "launch.h"

namespace pagedkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
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
  static constexpr int kQkSteps = D / 32;  // 16x16x32 products per score tile
  static constexpr int kDimTiles = D / 16; // 16-dim output tiles
  bf16x8_t k[kQkSteps];                    // this lane's 8-element K pieces
  short4_t v[kDimTiles];                   // this lane's 4-token V pieces
};

template <int D>
__device__ __forceinline__ void load_tile(Tile<D>& tl, const bf16_t* kt, const bf16_t* vt,
                                          int row, int kg) {
#pragma unroll
  for (int c = 0; c < Tile<D>::kQkSteps; ++c)
    tl.k[c] = *(const bf16x8_t*)(kt + row * D + c * 32 + kg * 8);
#pragma unroll
  for (int n = 0; n < Tile<D>::kDimTiles; ++n)
    tl.v[n] = *(const short4_t*)(vt + (n * kTile + row) * kBlockTokens + kg * 4);
}

template <int D>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NQK = Tile<D>::kQkSteps;
  constexpr int NDT = Tile<D>::kDimTiles;

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 15;  // tile row/column index of this lane
  const int kg = lane >> 4;   // k group (0..3)
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int h0 = kvh * G;
  bf16_t* out = (bf16_t*)a.out;

  const int L = a.seq_lens[b];
  if (L <= 0) {
    if (part == 0)
      for (int i = tid; i < G * D; i += blockDim.x)
        out[((size_t)b * Hq + h0) * D + i].bits = 0;
    return;
  }
  const int tok0 = part * a.part_tokens;
  if (tok0 >= L) return;
  const int tok_end = min(L, tok0 + a.part_tokens);
  const int nblk = (tok_end - tok0 + kBlockTokens - 1) / kBlockTokens;
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;

  __shared__ float red_m[kWaves][kTile];
  __shared__ float red_l[kWaves][kTile];
  __shared__ float red_o[kWaves][kTile][D + 1];

  // Q^T operand: column g = row (zero for padded heads), k = dims.
  bf16x8_t qb[NQK];
  {
    const bf16_t* qp = (const bf16_t*)a.q + ((size_t)b * Hq + h0 + row) * D;
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      if (row < G) {
        qb[c] = *(const bf16x8_t*)(qp + c * 32 + kg * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[c][e] = (__bf16)0.f;
      }
    }
  }

  float4_t acc[NDT];
#pragma unroll
  for (int n = 0; n < NDT; ++n) acc[n] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // head `row`, base-2 scaled scores
  float l_lane = 0.f;       // this lane's share of the softmax denominator

  const bf16_t* kbase = (const bf16_t*)a.k_pool;
  const bf16_t* vbase = (const bf16_t*)a.v_pool;
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks + tok0 / kBlockTokens;
  const size_t tile_elems = (size_t)kBlockTokens * D;
  const size_t head_stride = tile_elems;
  const size_t block_stride = (size_t)a.num_kv_heads * tile_elems;

  Tile<D> cur, nxt;
  int i = w;
  if (i < nblk) {
    const size_t base = (size_t)bt[i] * block_stride + kvh * head_stride;
    load_tile<D>(cur, kbase + base, vbase + base, row, kg);
  }
  for (; i < nblk; i += kWaves) {
    const int inext = i + kWaves;
    if (inext < nblk) {
      const size_t base = (size_t)bt[inext] * block_stride + kvh * head_stride;
      load_tile<D>(nxt, kbase + base, vbase + base, row, kg);
    }
    const int nvalid = min(kBlockTokens, tok_end - (tok0 + i * kBlockTokens));

    // ---- scores: S^T[t = 4 kg + r][g = row] ----
    float4_t s = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQK; ++c)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[c], qb[c], s, 0, 0, 0);
    float sv[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool valid = kg * 4 + r < nvalid;
      sv[r] = valid ? s[r] * a.scale_log2 : -INFINITY;
      mloc = fmaxf(mloc, sv[r]);
    }
    mloc = fmaxf(mloc, shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    uint16_t ph[4], pl[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(sv[r] - m_new);
      psum += p;
      ph[r] = bf16_rne(p);
      pl[r] = bf16_rne(p - __uint_as_float((uint32_t)ph[r] << 16));
    }
    l_lane = l_lane * alpha + psum;
    const uint32_t h01 = pack_bf16x2(ph[0], ph[1]), h23 = pack_bf16x2(ph[2], ph[3]);
    const uint32_t l01 = pack_bf16x2(pl[0], pl[1]), l23 = pack_bf16x2(pl[2], pl[3]);
    short4_t bhi, blo;
    {
      uint2 th = make_uint2(h01, h23), tl = make_uint2(l01, l23);
      bhi = __builtin_bit_cast(short4_t, th);
      blo = __builtin_bit_cast(short4_t, tl);
    }

    // ---- values: O^T[d][g] += V^T[d][t] P^T[t][g] ----
    if (nvalid < kBlockTokens) {
      uint32_t m0 = (kg * 4 + 0 < nvalid ? 0x0000ffffu : 0u) | (kg * 4 + 1 < nvalid ? 0xffff0000u : 0u);
      uint32_t m1 = (kg * 4 + 2 < nvalid ? 0x0000ffffu : 0u) | (kg * 4 + 3 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        uint2 raw = __builtin_bit_cast(uint2, cur.v[n]);
        raw.x &= m0;
        raw.y &= m1;
        cur.v[n] = __builtin_bit_cast(short4_t, raw);
      }
    }
#pragma unroll
    for (int n = 0; n < NDT; ++n) {
      float4_t o = acc[n] * alpha;
      o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cur.v[n], bhi, o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cur.v[n], blo, o, 0, 0, 0);
      acc[n] = o;
    }
    cur = nxt;
  }

  // ---- merge the waves ----
  float l = l_lane;
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (kg == 0) {
    red_m[w][row] = m_run;
    red_l[w][row] = l;
  }
#pragma unroll
  for (int n = 0; n < NDT; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[w][row][n * kTile + kg * 4 + r] = acc[n][r];
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += blockDim.x) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = red_m[0][g];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) M = fmaxf(M, red_m[v][g]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float f = fast_exp2(red_m[v][g] - M);
      lsum = fmaf(red_l[v][g], f, lsum);
      o = fmaf(red_o[v][g][d], f, o);
    }
    if (nparts == 1) {
      out[((size_t)b * Hq + h0 + g) * D + d].bits = f32_to_bf16_bits(o / lsum);
    } else {
      const size_t r = ((size_t)b * Hq + h0 + g) * a.num_parts + part;
      a.ws_o[r * D + d] = o;
      if (d == 0) {
        a.ws_m[r] = M;
        a.ws_l[r] = lsum;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int head_dim, hipStream_t s) {
  dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs), block(256);
  DecodeArgs arg = a;
  void* args[] = {&arg};
  const void* fn = head_dim == 64 ? (const void*)&decode_mfma_kernel<64>
                                  : (const void*)&decode_mfma_kernel<128>;
  return hipLaunchKernel(fn, grid, block, args, 0, s);
}

}  // namespace pagedkv
