// Paged decode attention on the CDNA4 matrix cores (bf16, D = 64 or 128,
// up to 16 query heads per KV head).
//
// The G query heads that share a KV head are padded to the 16 columns of a
// 16x16 MFMA tile, so each 16-token block is two small dense products:
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
// accumulator keeps head l % 16 in the same lane, so the online-softmax
// rescale is lane-local. The dim-major V tile makes the A operand of the
// value product a contiguous 8-byte load (4 tokens of one dim).
//
// Precision: scores and the output accumulate in fp32; the probabilities
// are fed to the bf16 value product as the sum of two bf16 numbers
// (p = hi + lo), so the product sees p to about 2^-17 relative.
//
// Tokens at or past the sequence length are masked by select: scores to
// -inf and V elements to 0, so stale or NaN tail slots never reach the
// result.
//
// Two ways to split the work over a persistent grid (sized to what the GPU
// holds at once):
//   fixed     (partition_tokens > 0): items are (sequence, partition,
//             KV head); a workgroup's 4 waves share an item, take its blocks
//             round robin and merge through LDS (worklist.h);
//   balanced  (partition_tokens == 0): the blocks of all (sequence, KV head)
//             pairs are laid end to end and every wave streams an equal
//             contiguous range of them, prefetching across pair boundaries.
//             A pair whose blocks lie inside one wave's range is finished
//             in place; a pair cut by range boundaries leaves one fp32
//             partial per piece, and the wave that completes the last piece
//             (an atomic count per pair) merges them: one kernel, no reduce
//             pass.
#include "launch.h"
#include "worklist.h"

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
  static constexpr int kQkSteps = D / 32;   // 16x16x32 products per score tile
  static constexpr int kDimTiles = D / 16;  // 16-dim output tiles
  bf16x8_t k[kQkSteps];                     // this lane's 8-element K pieces
  short4_t v[kDimTiles];                    // this lane's 4-token V pieces
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

// Q^T operand of one (sequence, KV head): column g = row, zero for g >= G.
template <int D>
__device__ __forceinline__ void load_q(bf16x8_t (&qb)[Tile<D>::kQkSteps], const DecodeArgs& a,
                                       int b, int kvh, int row, int kg) {
  const bf16_t* qp =
      (const bf16_t*)a.q + ((size_t)b * a.num_q_heads + (size_t)kvh * a.group + row) * D;
#pragma unroll
  for (int c = 0; c < Tile<D>::kQkSteps; ++c) {
    if (row < a.group) {
      qb[c] = *(const bf16x8_t*)(qp + c * 32 + kg * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[c][e] = (__bf16)0.f;
    }
  }
}

// Online-softmax state of one wave for one (sequence, KV head): head `row`,
// this lane's 4-token share of the denominator, and O^T[d][row].
template <int D>
struct WaveState {
  float4_t acc[Tile<D>::kDimTiles];
  float m;
  float l;
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int n = 0; n < Tile<D>::kDimTiles; ++n) acc[n] = (float4_t){0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }
  // Folds one 16-token block (nvalid of its tokens are real) into the state.
  __device__ __forceinline__ void block(Tile<D>& t, const bf16x8_t (&qb)[Tile<D>::kQkSteps],
                                        int nvalid, float scale_log2, int kg) {
    constexpr int NQK = Tile<D>::kQkSteps;
    constexpr int NDT = Tile<D>::kDimTiles;
    float4_t s = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQK; ++c)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[c], qb[c], s, 0, 0, 0);
    float sv[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = kg * 4 + r < nvalid ? s[r] * scale_log2 : -INFINITY;
      mloc = fmaxf(mloc, sv[r]);
    }
    mloc = fmaxf(mloc, shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, shfl_xor(mloc, 32));
    const float m_new = fmaxf(m, mloc);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    uint16_t ph[4], pl[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(sv[r] - m_new);
      psum += p;
      ph[r] = bf16_rne(p);
      pl[r] = bf16_rne(p - __uint_as_float((uint32_t)ph[r] << 16));
    }
    l = l * alpha + psum;
    const short4_t bhi = __builtin_bit_cast(
        short4_t, make_uint2(pack_bf16x2(ph[0], ph[1]), pack_bf16x2(ph[2], ph[3])));
    const short4_t blo = __builtin_bit_cast(
        short4_t, make_uint2(pack_bf16x2(pl[0], pl[1]), pack_bf16x2(pl[2], pl[3])));
    if (nvalid < kBlockTokens) {
      const uint32_t m0 = (kg * 4 + 0 < nvalid ? 0x0000ffffu : 0u) |
                          (kg * 4 + 1 < nvalid ? 0xffff0000u : 0u);
      const uint32_t m1 = (kg * 4 + 2 < nvalid ? 0x0000ffffu : 0u) |
                          (kg * 4 + 3 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        uint2 raw = __builtin_bit_cast(uint2, t.v[n]);
        raw.x &= m0;
        raw.y &= m1;
        t.v[n] = __builtin_bit_cast(short4_t, raw);
      }
    }
#pragma unroll
    for (int n = 0; n < NDT; ++n) {
      float4_t o = acc[n] * alpha;
      o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[n], bhi, o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[n], blo, o, 0, 0, 0);
      acc[n] = o;
    }
  }
  // Sum of the denominator over the 4 lanes that share head `row`.
  __device__ __forceinline__ float total_l() const {
    float t = l;
    t += shfl_xor(t, 16);
    t += shfl_xor(t, 32);
    return t;
  }
};

template <typename T>
__device__ __forceinline__ void zero_padded_rows(const DecodeArgs& a, const int* prefix,
                                                 int row_elems) {
  for (int b = blockIdx.x; b < a.num_seqs; b += gridDim.x) {
    if (prefix[b + 1] != prefix[b]) continue;
    T* o = (T*)a.out + (size_t)b * row_elems;
    for (int i = threadIdx.x; i < row_elems; i += blockDim.x) ElemTraits<T>::store1(o + i, 0.f);
  }
}

// ===========================================================================
// fixed partitions
// ===========================================================================

template <int D>
__device__ __forceinline__ void fixed_item(const DecodeArgs& a, int b, int kvh, int part, int L,
                                           float (*red_m)[kTile], float (*red_l)[kTile],
                                           float (*red_o)[kTile][D + 1]) {
  constexpr int NDT = Tile<D>::kDimTiles;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 15;
  const int kg = lane >> 4;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int h0 = kvh * G;
  bf16_t* out = (bf16_t*)a.out;

  const int tok0 = part * a.part_tokens;
  const int tok_end = min(L, tok0 + a.part_tokens);
  const int nblk = (tok_end - tok0 + kBlockTokens - 1) / kBlockTokens;
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;

  bf16x8_t qb[Tile<D>::kQkSteps];
  load_q<D>(qb, a, b, kvh, row, kg);
  WaveState<D> st;
  st.reset();

  const bf16_t* kbase = (const bf16_t*)a.k_pool;
  const bf16_t* vbase = (const bf16_t*)a.v_pool;
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks + tok0 / kBlockTokens;
  const size_t tile_elems = (size_t)kBlockTokens * D;
  const size_t block_stride = (size_t)a.num_kv_heads * tile_elems;
  const size_t head_off = (size_t)kvh * tile_elems;

  Tile<D> cur, nxt;
  int i = w;
  if (i < nblk) {
    const size_t base = (size_t)bt[i] * block_stride + head_off;
    load_tile<D>(cur, kbase + base, vbase + base, row, kg);
  }
  for (; i < nblk; i += kWaves) {
    const int inext = i + kWaves;
    if (inext < nblk) {
      const size_t base = (size_t)bt[inext] * block_stride + head_off;
      load_tile<D>(nxt, kbase + base, vbase + base, row, kg);
    }
    st.block(cur, qb, min(kBlockTokens, tok_end - (tok0 + i * kBlockTokens)), a.scale_log2, kg);
    cur = nxt;
  }

  // merge the 4 waves through LDS
  const float l = st.total_l();
  if (kg == 0) {
    red_m[w][row] = st.m;
    red_l[w][row] = l;
  }
#pragma unroll
  for (int n = 0; n < NDT; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[w][row][n * kTile + kg * 4 + r] = st.acc[n][r];
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
      const float f = fast_exp2(red_m[v][g] - M);  // a wave with no block has m = -inf
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
  __syncthreads();  // the LDS merge buffers are reused by the next item
}

template <int D>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  extern __shared__ int prefix[];  // [B + 1]
  __shared__ int scan_scratch[kWaves];
  __shared__ float red_m[kWaves][kTile];
  __shared__ float red_l[kWaves][kTile];
  __shared__ float red_o[kWaves][kTile][D + 1];

  const int B = a.num_seqs;
  build_partition_prefix(a.seq_lens, B, a.part_tokens, prefix, scan_scratch);
  zero_padded_rows<bf16_t>(a, prefix, a.num_q_heads * D);

  const int Hkv = a.num_kv_heads;
  const int nitems = prefix[B] * Hkv;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int j = item / Hkv;
    const int kvh = item - j * Hkv;
    const int b = find_sequence(prefix, B, j);
    fixed_item<D>(a, b, kvh, j - prefix[b], a.seq_lens[b], red_m, red_l, red_o);
  }
}

// ===========================================================================
// balanced split
// ===========================================================================

// A wave's view of one (sequence, KV head) pair inside its block range.
struct Segment {
  int b, kvh;
  int nb;        // blocks of the sequence
  int L;         // tokens of the sequence
  int j;         // current block of the sequence
  long long fs;  // flat index of the segment's first block
  long long fe;  // flat index one past the segment's last block
  long long ps;  // flat index of the pair's block 0
};

// Pair layout: sequence b's pairs start at Hkv * prefix[b]; pair (b, kvh)
// covers nb_b consecutive flat indices.
__device__ __forceinline__ Segment locate(const int* prefix, const int32_t* seq_lens, int B,
                                          int Hkv, long long f, long long f1) {
  Segment s;
  s.b = __builtin_amdgcn_readfirstlane(find_sequence(prefix, B, (int)(f / Hkv)));
  const long long base = (long long)Hkv * prefix[s.b];
  s.nb = __builtin_amdgcn_readfirstlane(prefix[s.b + 1] - prefix[s.b]);
  s.L = seq_lens[s.b];
  const long long r = f - base;
  s.kvh = __builtin_amdgcn_readfirstlane((int)(r / s.nb));
  s.j = __builtin_amdgcn_readfirstlane((int)(r - (long long)s.kvh * s.nb));
  s.ps = base + (long long)s.kvh * s.nb;
  s.fs = f;
  s.fe = min(f1, s.ps + s.nb);
  return s;
}

// The segment that follows `c` (which ends at c.fe < f1): the next KV head
// of the same sequence, else the first KV head of the next non-empty one.
__device__ __forceinline__ Segment next_segment(const Segment& c, const int* prefix,
                                                const int32_t* seq_lens, int Hkv, long long f1) {
  Segment s = c;
  if (c.kvh + 1 < Hkv) {
    s.kvh = c.kvh + 1;
  } else {
    int b = c.b + 1;
    while (prefix[b + 1] == prefix[b]) ++b;  // skip padded rows; a later pair exists
    s.b = __builtin_amdgcn_readfirstlane(b);
    s.kvh = 0;
    s.nb = __builtin_amdgcn_readfirstlane(prefix[s.b + 1] - prefix[s.b]);
    s.L = seq_lens[b];
  }
  s.j = 0;
  s.ps = c.fe;
  s.fs = c.fe;
  s.fe = min(f1, s.ps + s.nb);
  return s;
}

__device__ __forceinline__ long long balanced_chunk(long long total, int waves, int min_blocks) {
  const long long even = (total + waves - 1) / waves;
  return even > min_blocks ? even : (long long)min_blocks;
}

// Pieces of the pair starting at flat index s with nb blocks: waves
// v0 = s / chunk .. v1 = (s + nb - 1) / chunk. The first piece is wave v0's
// slot 1 when that wave's range began before s, else its slot 0; every later
// piece is the first segment (slot 0) of its wave.
struct Pieces {
  int v0, v1, first_slot;
  __device__ __forceinline__ Pieces(long long s, int nb, long long chunk) {
    v0 = (int)(s / chunk);
    v1 = (int)((s + nb - 1) / chunk);
    first_slot = 2 * v0 + ((long long)v0 * chunk < s ? 1 : 0);
  }
  __device__ __forceinline__ int slot(int v) const { return v == v0 ? first_slot : 2 * v; }
};

// Partials cross workgroups on different XCDs, whose L2 caches are not
// coherent with each other. They are written and read with agent-scope
// relaxed atomic accesses (coherent at the device level without flushing or
// invalidating the whole L2), and the writer waits for its stores to
// complete before it counts its piece.
__device__ __forceinline__ void put_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_complete() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// One wave merges every piece of pair (b, kvh), in piece order, and writes
// the bf16 output. Lane work unit: 4 consecutive dims of one head. The loads
// of up to kBatch pieces are issued together so a merge costs one or two
// memory round trips instead of one per piece.
template <int D>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int b, int kvh,
                                             const Pieces& pc, int lane) {
  constexpr int kBatch = 8;
  const int G = a.group;
  const int n = pc.v1 - pc.v0 + 1;
  bf16_t* out = (bf16_t*)a.out + ((size_t)b * a.num_q_heads + (size_t)kvh * G) * D;
  for (int c = lane; c < G * D / 4; c += 64) {
    const int g = c * 4 / D;
    const int d0 = c * 4 - g * D;
    float M = -INFINITY;
    if (n > kBatch) {  // long pairs: find the max first
      for (int p0 = 0; p0 < n; p0 += kBatch) {
        float mb[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          mb[i] = p0 + i < n ? get_coherent(a.ws_m + (size_t)pc.slot(pc.v0 + p0 + i) * G + g)
                             : -INFINITY;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) M = fmaxf(M, mb[i]);
      }
    }
    float lsum = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < n; p0 += kBatch) {
      float mb[kBatch], lb[kBatch], ob[kBatch][4];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (p0 + i < n) {
          const size_t r = (size_t)pc.slot(pc.v0 + p0 + i) * G + g;
          mb[i] = get_coherent(a.ws_m + r);
          lb[i] = get_coherent(a.ws_l + r);
#pragma unroll
          for (int e = 0; e < 4; ++e) ob[i][e] = get_coherent(a.ws_o + r * D + d0 + e);
        } else {
          mb[i] = -INFINITY;
          lb[i] = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) ob[i][e] = 0.f;
        }
      }
      if (n <= kBatch) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) M = fmaxf(M, mb[i]);
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const float f = fast_exp2(mb[i] - M);  // absent pieces: 2^-inf = 0
        lsum = fmaf(lb[i], f, lsum);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(ob[i][e], f, o[e]);
      }
    }
    const float inv = 1.f / lsum;
    *(uint2*)(out + (size_t)g * D + d0) =
        make_uint2(pack_bf16x2(f32_to_bf16_bits(o[0] * inv), f32_to_bf16_bits(o[1] * inv)),
                   pack_bf16x2(f32_to_bf16_bits(o[2] * inv), f32_to_bf16_bits(o[3] * inv)));
  }
}

template <int D>
__device__ __forceinline__ void finish_segment(const DecodeArgs& a, const Segment& s,
                                               WaveState<D>& st, long long f0, long long chunk,
                                               int wave_id, int lane, int row, int kg) {
  constexpr int NDT = Tile<D>::kDimTiles;
  const float l = st.total_l();
  const bool complete = s.fs == s.ps && s.fe == s.ps + s.nb;
  if (complete) {
    if (row < a.group) {
      const float inv = 1.f / l;
      bf16_t* o = (bf16_t*)a.out +
                  ((size_t)s.b * a.num_q_heads + (size_t)s.kvh * a.group + row) * D + kg * 4;
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        const uint2 v = make_uint2(pack_bf16x2(f32_to_bf16_bits(st.acc[n][0] * inv),
                                               f32_to_bf16_bits(st.acc[n][1] * inv)),
                                   pack_bf16x2(f32_to_bf16_bits(st.acc[n][2] * inv),
                                               f32_to_bf16_bits(st.acc[n][3] * inv)));
        *(uint2*)(o + n * kTile) = v;
      }
    }
    return;
  }
  const int slot = 2 * wave_id + (s.fs == f0 ? 0 : 1);
  if (row < a.group) {
    const size_t r = (size_t)slot * a.group + row;
    float* o = a.ws_o + r * D + kg * 4;
#pragma unroll
    for (int n = 0; n < NDT; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) put_coherent(o + n * kTile + e, st.acc[n][e]);
    if (kg == 0) {
      put_coherent(a.ws_m + r, st.m);
      put_coherent(a.ws_l + r, l);
    }
  }
  // Publish the piece, then count it; the wave that brings the count to the
  // number of pieces merges them all and rearms the counter for the next
  // call. No wave ever waits for another.
  wait_stores_complete();
  const Pieces pc(s.ps, s.nb, chunk);
  int* cnt = a.ws_cnt + (size_t)s.b * a.num_kv_heads + s.kvh;
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, 64);
  if (old == pc.v1 - pc.v0) {
    merge_pieces<D>(a, s.b, s.kvh, pc, lane);
    if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_mfma_balanced_kernel(DecodeArgs a) {
  extern __shared__ int prefix[];  // [B + 1]: exclusive prefix of blocks per sequence
  __shared__ int scan_scratch[kWaves];

  const int B = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  build_partition_prefix(a.seq_lens, B, kBlockTokens, prefix, scan_scratch);
  zero_padded_rows<bf16_t>(a, prefix, a.num_q_heads * D);

  const int lane = threadIdx.x & 63;
  const int row = lane & 15;
  const int kg = lane >> 4;
  const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
  const long long total = (long long)Hkv * prefix[B];
  const long long chunk = balanced_chunk(total, a.split_waves, a.min_seg_blocks);
  const long long f0 = (long long)wave_id * chunk;
  const long long f1 = min(total, f0 + chunk);
  if (f0 >= f1) return;  // no barrier follows: waves run independently from here

  const bf16_t* kbase = (const bf16_t*)a.k_pool;
  const bf16_t* vbase = (const bf16_t*)a.v_pool;
  const size_t tile_elems = (size_t)kBlockTokens * D;
  const size_t block_stride = (size_t)Hkv * tile_elems;

  Segment cur = locate(prefix, a.seq_lens, B, Hkv, f0, f1);
  bf16x8_t qb[Tile<D>::kQkSteps], qn[Tile<D>::kQkSteps];
  load_q<D>(qb, a, cur.b, cur.kvh, row, kg);
  Tile<D> tc, tn;
  {
    const int32_t phys = a.block_tables[(size_t)cur.b * a.max_blocks + cur.j];
    const size_t base = (size_t)phys * block_stride + (size_t)cur.kvh * tile_elems;
    load_tile<D>(tc, kbase + base, vbase + base, row, kg);
  }
  WaveState<D> st;
  st.reset();

  for (long long f = f0;; ++f) {
    const bool more = f + 1 < f1;
    const bool seg_end = f + 1 == cur.fe;
    Segment nx = cur;
    if (more) {
      if (seg_end) {
        nx = next_segment(cur, prefix, a.seq_lens, Hkv, f1);
        load_q<D>(qn, a, nx.b, nx.kvh, row, kg);
      } else {
        nx.j = cur.j + 1;
      }
      const int32_t phys = a.block_tables[(size_t)nx.b * a.max_blocks + nx.j];
      const size_t base = (size_t)phys * block_stride + (size_t)nx.kvh * tile_elems;
      load_tile<D>(tn, kbase + base, vbase + base, row, kg);
    }
    st.block(tc, qb, min(kBlockTokens, cur.L - cur.j * kBlockTokens), a.scale_log2, kg);
    if (seg_end) {
      finish_segment<D>(a, cur, st, f0, chunk, wave_id, lane, row, kg);
      st.reset();
#pragma unroll
      for (int c = 0; c < Tile<D>::kQkSteps; ++c) qb[c] = qn[c];
    }
    if (!more) break;
    cur = nx;
    tc = tn;
  }
}

}  // namespace

const void* decode_mfma_fn(int head_dim, bool balanced) {
  if (balanced)
    return head_dim == 64 ? (const void*)&decode_mfma_balanced_kernel<64>
                          : (const void*)&decode_mfma_balanced_kernel<128>;
  return head_dim == 64 ? (const void*)&decode_mfma_kernel<64>
                        : (const void*)&decode_mfma_kernel<128>;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int head_dim, bool balanced, int grid,
                              hipStream_t s) {
  DecodeArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(decode_mfma_fn(head_dim, balanced), dim3(grid), dim3(256), args,
                         (size_t)(a.num_seqs + 1) * sizeof(int), s);
}

}  // namespace pagedkv
