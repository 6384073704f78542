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
//             round robin and merge through LDS. Items come from a work
//             list (worklist.h), or, when every (sequence, partition, KV
//             head) slot fits on a compute unit of its own, each slot gets a
//             workgroup and no list is built. A sequence over several
//             partitions leaves one fp32 partial per partition, and the
//             item that completes a pair's count (an atomic per pair) merges
//             them: one kernel, no reduce pass;
//   balanced  (partition_tokens == 0): the blocks of all (sequence, KV head)
//             pairs are laid end to end and every wave streams an equal
//             contiguous range of them, prefetching across pair boundaries.
//             A pair whose blocks lie inside one wave's range is finished
//             in place; a pair cut by range boundaries leaves one fp32
//             partial per piece. After its stream a wave counts its (at most
//             two) pieces, and the wave that completes a pair's count (an
//             atomic per pair) merges its pieces: one kernel, no reduce
//             pass.
#include "launch.h"
#include "mfma_tile.h"
#include "worklist.h"

namespace pagedkv {

namespace {

using namespace mfma;

constexpr int kWaves = 4;

// A 16-token tile made of two 8-token blocks: tokens 0-7 from block A
// (`region_a`), 8-15 from block B. Every lane issues each load against both
// blocks' descriptors with an offset that is out of range for the block it
// does not read; a range-checked buffer load returns zero there without
// touching memory, so OR-ing the two results gives the lane's data with no
// divergent branch and no extra traffic.
template <int D>
__device__ __forceinline__ void load_tile_two_blocks(Tile<D>& tl, const bf16_t* kpool,
                                                     const bf16_t* vpool, size_t region_a,
                                                     size_t region_b, int row, int kg) {
  constexpr int kHalf = 8;
  constexpr int kBytes = kHalf * D * 2;
  constexpr int kOut = 0x40000000;  // beyond any 8-token block
  const __amdgpu_buffer_rsrc_t ka = range_rsrc(kpool + region_a, kBytes);
  const __amdgpu_buffer_rsrc_t kb = range_rsrc(kpool + region_b, kBytes);
  const __amdgpu_buffer_rsrc_t va = range_rsrc(vpool + region_a, kBytes);
  const __amdgpu_buffer_rsrc_t vb = range_rsrc(vpool + region_b, kBytes);
  const int k_off = ((row & 7) * D + kg * 8) * 2;
  const int k_a = row < kHalf ? k_off : kOut;
  const int k_b = row < kHalf ? kOut : k_off;
  const int v_off = (row * kHalf + (kg & 1) * 4) * 2;
  const int v_a = kg < 2 ? v_off : kOut;
  const int v_b = kg < 2 ? kOut : v_off;
#pragma unroll
  for (int c = 0; c < Tile<D>::kQkSteps; ++c) {
    const u32x4_t x = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ka, k_a + c * 64, 0, kStreamLoad));
    const u32x4_t y = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(kb, k_b + c * 64, 0, kStreamLoad));
    tl.k[c] = __builtin_bit_cast(bf16x8_t, x | y);
  }
#pragma unroll
  for (int n = 0; n < Tile<D>::kDimTiles; ++n) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    // the step goes into the vector offset: out-of-range masking must see it
    const u32x2_t x = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(va, v_a + n * kTile * kHalf * 2, 0,
                                                      kStreamLoad));
    const u32x2_t y = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(vb, v_b + n * kTile * kHalf * 2, 0,
                                                      kStreamLoad));
    tl.v[n] = __builtin_bit_cast(short4_t, x | y);
  }
}

// Q^T operand of one (sequence, KV head), branch-free: column g = row for
// g < G; the padded columns g >= G repeat head G - 1. Their scores and
// outputs land in MFMA columns that are never written out, so they only
// need to be finite.
template <int D>
__device__ __forceinline__ void load_q_clamped(bf16x8_t (&qb)[Tile<D>::kQkSteps],
                                               const DecodeArgs& a, int b, int kvh, int qoff) {
  const bf16_t* qp =
      (const bf16_t*)a.q + ((size_t)b * a.num_q_heads + (size_t)kvh * a.group) * D;
  const __amdgpu_buffer_rsrc_t qr = range_rsrc(qp, a.group * D * 2);
#pragma unroll
  for (int c = 0; c < Tile<D>::kQkSteps; ++c)
    qb[c] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + c * 64, 0, 0));
}

// Byte offset of this lane's Q^T elements within its pair's G heads.
template <int D>
__device__ __forceinline__ int q_lane_offset(int group, int row, int kg) {
  const int g = row < group ? row : group - 1;
  return (g * D + kg * 8) * 2;
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
    const float m_new = fmaxf(m, max_over_kg(mloc));
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
  __device__ __forceinline__ float total_l() const { return sum_over_kg(l); }
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

// Partials of the fixed split cross workgroups on different XCDs, whose L2
// caches are not coherent with each other: they are stored and loaded as
// agent-scope relaxed atomics, which the L2 keeps coherent at the device
// level (sc1) without flushing or invalidating it.
__device__ __forceinline__ void store_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_partial(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Four consecutive partial outputs, as two 8-byte loads with the same
// coherence as load_partial.
__device__ __forceinline__ float4_t load_partial4(const float* p) {
  typedef uint64_t u64x2_t __attribute__((ext_vector_type(2)));
  const u64x2_t v = {
      __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
      __hip_atomic_load((uint64_t*)(p + 2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
  return __builtin_bit_cast(float4_t, v);
}

// Merges the nparts partitions of (sequence b, the G heads from h0) into
// the bf16 output. Work unit: 4 consecutive dims of one head. The T threads
// of a unit split its partitions (thread s takes p = s, s + T, ...), load up
// to kB of them in one memory round trip and fold them into a running max,
// sum and output rescaled as in the online softmax; the T results are then
// combined through LDS (`lds`: 6 floats per thread) in thread order. Every
// partition's loads go out at once for nparts <= kB T, and the result does
// not depend on timing.
template <int D, int kB>
__device__ __forceinline__ void merge_partitions(const DecodeArgs& a, int b, int h0, int nparts,
                                                 int tid, float* lds) {
  constexpr int kQuads = D / 4;
  const int G = a.group;
  const int units = G * kQuads;
  const int nt = blockDim.x;
  const int T = units >= nt ? 1 : nt / units;  // threads per unit
  const int per_pass = nt / T;                 // units per pass
  const int s = tid % T;
  bf16_t* out = (bf16_t*)a.out + ((size_t)b * a.num_q_heads + h0) * D;
  for (int u0 = 0; u0 < units; u0 += per_pass) {
    const int u = u0 + tid / T;
    const bool on = u < units && tid < per_pass * T;
    const int uc = min(u, units - 1);
    const int g = uc / kQuads;
    const int q = uc - g * kQuads;
    const size_t r0 = ((size_t)b * a.num_q_heads + h0 + g) * a.num_parts;
    float M = -INFINITY, lsum = 0.f;
    float4_t o = (float4_t){0.f, 0.f, 0.f, 0.f};
    for (int p0 = s; p0 < nparts; p0 += kB * T) {
      float mv[kB], lv[kB];
      float4_t ov[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const int p = p0 + k * T;
        const size_t r = r0 + min(p, nparts - 1);
        const float m = load_partial(a.ws_m + r);
        const float l = load_partial(a.ws_l + r);
        const float4_t v = load_partial4(a.ws_o + r * D + 4 * q);
        mv[k] = p < nparts ? m : -INFINITY;
        lv[k] = p < nparts ? l : 0.f;
        ov[k] = p < nparts ? v : (float4_t){0.f, 0.f, 0.f, 0.f};
      }
      float Mb = M;
#pragma unroll
      for (int k = 0; k < kB; ++k) Mb = fmaxf(Mb, mv[k]);
      const float f = fast_exp2(M - Mb);  // 0 before the first batch
      lsum *= f;
      o *= f;
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const float e = fast_exp2(mv[k] - Mb);  // 0 past the last partition
        lsum = fmaf(lv[k], e, lsum);
        o += ov[k] * e;
      }
      M = Mb;
    }
    float* mine = lds + 6 * tid;
    mine[0] = M;
    mine[1] = lsum;
    mine[2] = o[0];
    mine[3] = o[1];
    mine[4] = o[2];
    mine[5] = o[3];
    __syncthreads();
    if (on && s == 0) {
      float Mt = M;
      for (int t = 1; t < T; ++t) Mt = fmaxf(Mt, mine[6 * t]);
      float lt = 0.f;
      float4_t ot = (float4_t){0.f, 0.f, 0.f, 0.f};
      for (int t = 0; t < T; ++t) {
        const float* th = mine + 6 * t;
        const float e = fast_exp2(th[0] - Mt);  // a thread with no partition has M = -inf
        lt = fmaf(th[1], e, lt);
        ot += (float4_t){th[2], th[3], th[4], th[5]} * e;
      }
      const float inv = 1.f / lt;
      *(uint2*)(out + (size_t)uc * 4) =
          make_uint2(pack_bf16x2(f32_to_bf16_bits(ot[0] * inv), f32_to_bf16_bits(ot[1] * inv)),
                     pack_bf16x2(f32_to_bf16_bits(ot[2] * inv), f32_to_bf16_bits(ot[3] * inv)));
    }
    __syncthreads();
  }
}

// Table entry of the first block wave w folds in partition `part` of row b.
// It is read before the row's length is known, so the index is kept inside
// the row's table (a partition past the row's end reads an entry it never
// uses).
__device__ __forceinline__ int32_t first_entry(const DecodeArgs& a, int b, int part, int w) {
  const int blk = part * (a.part_tokens / kBlockTokens) + w;
  return uniform_load(a.block_tables,
                      (size_t)b * a.max_blocks + max(0, min(blk, a.max_blocks - 1)));
}

// Partition `part` of (row b, KV head kvh), L tokens in the row; qb holds
// the G queries (load_q) and e_first the table entry of this wave's first
// block (first_entry), both read by the caller so that their loads overlap
// the row length's.
template <int D>
__device__ __forceinline__ void fixed_item(const DecodeArgs& a, int b, int kvh, int part, int L,
                                           const bf16x8_t (&qb)[Tile<D>::kQkSteps],
                                           int32_t e_first, float (*red_m)[kTile],
                                           float (*red_l)[kTile], float (*red_o)[kTile][D + 1],
                                           int* last) {
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

  WaveState<D> st;
  st.reset();

  const bf16_t* kbase = (const bf16_t*)a.k_pool;
  const bf16_t* vbase = (const bf16_t*)a.v_pool;
  const size_t bt_row = (size_t)b * a.max_blocks + tok0 / kBlockTokens;
  const size_t tile_elems = (size_t)kBlockTokens * D;
  const size_t block_stride = (size_t)a.num_kv_heads * tile_elems;
  const size_t head_off = (size_t)kvh * tile_elems;

  // ping-pong over two register tiles: the loads of block i + 4 are in
  // flight while block i is computed; each block's table entry is read a
  // step before its loads
  const LaneOffsets<D> lo(row, kg);
  Tile<D> ta, tb;
  int i = w;
  int32_t e_next = 0;
  if (i < nblk) {
    const size_t base = (size_t)e_first * block_stride + head_off;
    load_tile<D>(ta, kbase + base, vbase + base, lo);
    if (i + kWaves < nblk) e_next = uniform_load(a.block_tables, bt_row + i + kWaves);
  }
  auto step = [&](Tile<D>& cur, Tile<D>& nxt) {
    const int inext = i + kWaves;
    if (inext < nblk) {
      const size_t base = (size_t)e_next * block_stride + head_off;
      load_tile<D>(nxt, kbase + base, vbase + base, lo);
      if (inext + kWaves < nblk) e_next = uniform_load(a.block_tables, bt_row + inext + kWaves);
    }
    st.block(cur, qb, min(kBlockTokens, tok_end - (tok0 + i * kBlockTokens)), a.scale_log2, kg);
    i = inext;
  };
  while (i < nblk) {
    step(ta, tb);
    if (i >= nblk) break;
    step(tb, ta);
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
      store_partial(a.ws_o + r * D + d, o);
      if (d == 0) {
        store_partial(a.ws_m + r, M);
        store_partial(a.ws_l + r, lsum);
      }
    }
  }
  if (nparts == 1) {
    __syncthreads();  // the LDS merge buffers are reused by the next item
    return;
  }
  // Count this partition once every thread's partials are stored; the item
  // that completes the count merges the pair's partitions (merge_partitions:
  // one load round for up to 16 per thread) and rearms the counter for the next
  // call. No workgroup waits for another.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    int* cnt = a.ws_cnt + (size_t)b * a.num_kv_heads + kvh;
    *last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            nparts - 1;
  }
  __syncthreads();
  if (*last) {
    // partitions per thread of a work unit (4 dims of one head)
    const int units = G * (D / 4);
    const int T = units >= (int)blockDim.x ? 1 : blockDim.x / units;
    const int per_thread = (nparts + T - 1) / T;
    float* lds = &red_o[0][0][0];
    if (per_thread <= 4)
      merge_partitions<D, 4>(a, b, h0, nparts, tid, lds);
    else if (per_thread <= 8)
      merge_partitions<D, 8>(a, b, h0, nparts, tid, lds);
    else
      merge_partitions<D, 16>(a, b, h0, nparts, tid, lds);
    if (tid == 0)
      __hip_atomic_store(a.ws_cnt + (size_t)b * a.num_kv_heads + kvh, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // the LDS merge buffers and `last` are reused by the next item
}

template <int D>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  extern __shared__ int prefix[];  // [B + 1]
  __shared__ int scan_scratch[kWaves];
  __shared__ float red_m[kWaves][kTile];
  __shared__ float red_l[kWaves][kTile];
  __shared__ float red_o[kWaves][kTile][D + 1];
  __shared__ int last;

  const int B = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  bf16x8_t qb[Tile<D>::kQkSteps];

  if (a.slot_grid) {
    // A workgroup for every (row, partition, KV head) slot, empty ones
    // included: no work list, and the row's length, the queries and the
    // first table entries load together.
    const int kvh = blockIdx.x % Hkv;
    const int j = blockIdx.x / Hkv;
    const int part = j % a.num_parts;
    const int b = j / a.num_parts;
    const int32_t e_first = first_entry(a, b, part, w);
    load_q<D>(qb, a, b, kvh, lane & 15, lane >> 4);
    const int L = uniform_load(a.seq_lens, b);
    if (part * a.part_tokens >= L) {
      if (part == 0) {  // a padded row (L = 0): its outputs are zero
        bf16_t* o = (bf16_t*)a.out + ((size_t)b * a.num_q_heads + (size_t)kvh * a.group) * D;
        for (int i = threadIdx.x; i < a.group * D; i += blockDim.x) o[i].bits = 0;
      }
      return;
    }
    fixed_item<D>(a, b, kvh, part, L, qb, e_first, red_m, red_l, red_o, &last);
    return;
  }

  build_partition_prefix(a.seq_lens, B, a.part_tokens, prefix, scan_scratch);
  zero_padded_rows<bf16_t>(a, prefix, a.num_q_heads * D);

  const int nitems = prefix[B] * Hkv;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int j = item / Hkv;
    const int kvh = item - j * Hkv;
    const int b = __builtin_amdgcn_readfirstlane(find_sequence(prefix, B, j));
    const int part = __builtin_amdgcn_readfirstlane(j - prefix[b]);
    const int32_t e_first = first_entry(a, b, part, w);
    load_q<D>(qb, a, b, kvh, lane & 15, lane >> 4);
    fixed_item<D>(a, b, kvh, part, uniform_load(a.seq_lens, b), qb, e_first, red_m, red_l, red_o,
                  &last);
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
  s.L = uniform_load(seq_lens, s.b);
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
    s.L = uniform_load(seq_lens, s.b);
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
// coherent with each other. Records of cut pieces are written and read 16
// bytes at a time with the cache policy that agent-scope relaxed atomics
// use (sc1: coherent at the device level without flushing or invalidating
// the whole L2), and the writer waits for its stores to complete before it
// counts its piece. Every access of a record goes through this descriptor.
constexpr int kCoherent = 16;  // buffer cache policy: sc1

__device__ __forceinline__ void wait_stores_complete() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t records_rsrc(const DecodeArgs& a, int pf) {
  return range_rsrc(a.ws_o, 2 * a.split_waves * pf * (int)sizeof(float));
}

// Byte offset of the record of piece slot `slot` (2 * wave + k).
__device__ __forceinline__ int record_bytes(int slot, int pf) {
  return slot * pf * (int)sizeof(float);
}

__device__ __forceinline__ float load_coherent_f32(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoherent));
}

// One wave merges every piece of pair (b, kvh), in piece order, and writes
// the bf16 output; it runs after the wave's own stream, when the tile
// registers are free. Work unit: 4 consecutive dims of one head (one
// 16-byte piece of a record). For kUnits units per lane and kBatch pieces at
// a time, the pieces' (m, l) and outputs are loaded in one round and folded
// into a running (M, L, O) with the same rescaling as the online softmax,
// so a merge of up to kBatch pieces costs one memory round trip.
template <int D, int kBatch>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, __amdgpu_buffer_rsrc_t rec,
                                             int pf, int b, int kvh, const Pieces& pc,
                                             int lane) {
  constexpr int kUnits = 2;
  const int G = a.group;
  const int n = pc.v1 - pc.v0 + 1;
  bf16_t* out = (bf16_t*)a.out + ((size_t)b * a.num_q_heads + (size_t)kvh * G) * D;
  const int units = G * D / 4;
  for (int u0 = lane; u0 < units; u0 += 64 * kUnits) {
    int u[kUnits], g[kUnits];
    float M[kUnits], L[kUnits];
    float4_t O[kUnits];
#pragma unroll
    for (int h = 0; h < kUnits; ++h) {
      u[h] = min(u0 + 64 * h, units - 1);
      g[h] = u[h] / (D / 4);
      M[h] = -INFINITY;
      L[h] = 0.f;
      O[h] = (float4_t){0.f, 0.f, 0.f, 0.f};
    }
    for (int p0 = 0; p0 < n; p0 += kBatch) {
      float mb[kUnits][kBatch], lb[kUnits][kBatch];
      float4_t ob[kUnits][kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int base = record_bytes(pc.slot(pc.v0 + min(p0 + i, n - 1)), pf);
#pragma unroll
        for (int h = 0; h < kUnits; ++h) {
          const float m = load_coherent_f32(rec, base + (G * D + g[h]) * 4);
          mb[h][i] = p0 + i < n ? m : -INFINITY;
          lb[h][i] = load_coherent_f32(rec, base + (G * D + G + g[h]) * 4);
          ob[h][i] = __builtin_bit_cast(
              float4_t, __builtin_amdgcn_raw_buffer_load_b128(rec, base + u[h] * 16, 0, kCoherent));
        }
      }
#pragma unroll
      for (int h = 0; h < kUnits; ++h) {
        float Mn = M[h];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) Mn = fmaxf(Mn, mb[h][i]);
        const float alpha = fast_exp2(M[h] - Mn);  // 0 before the first batch
        L[h] *= alpha;
        O[h] *= alpha;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const float f = fast_exp2(mb[h][i] - Mn);  // absent pieces: 2^-inf = 0
          L[h] = fmaf(lb[h][i], f, L[h]);
          O[h] += ob[h][i] * f;
        }
        M[h] = Mn;
      }
    }
#pragma unroll
    for (int h = 0; h < kUnits; ++h) {
      if (u0 + 64 * h >= units) continue;
      const float inv = 1.f / L[h];
      *(uint2*)(out + (size_t)u[h] * 4) =
          make_uint2(pack_bf16x2(f32_to_bf16_bits(O[h][0] * inv), f32_to_bf16_bits(O[h][1] * inv)),
                     pack_bf16x2(f32_to_bf16_bits(O[h][2] * inv), f32_to_bf16_bits(O[h][3] * inv)));
    }
  }
}

// Partial of one piece, in record layout: O[g][d] (this lane's 4 dims
// 16 n + 4 kg .. + 3 of head `row` are contiguous), then m[G], then l[G].
// During the stream pieces are parked in the wave's LDS area and copied to
// the workspace only after it: vector memory operations retire in order, so
// a store issued mid-stream would hold up the wait for the next prefetched
// tile until the store had reached memory.
template <int D>
__device__ __forceinline__ void park_piece(float* dst, const WaveState<D>& st, float l, int G,
                                           int row, int kg) {
  constexpr int NDT = Tile<D>::kDimTiles;
  if (row >= G) return;
#pragma unroll
  for (int n = 0; n < NDT; ++n) *(float4_t*)(dst + row * D + n * kTile + kg * 4) = st.acc[n];
  if (kg == 0) {
    dst[G * D + row] = st.m;
    dst[G * D + G + row] = l;
  }
}

// Complete outputs staged in the wave's LDS area: `n` bf16 G x D blocks and
// the pair index (b * Hkv + kvh) of each. Like parked pieces they are
// written to memory after the stream (a store mid-stream holds up the next
// tile's wait); outputs beyond the stage's capacity are stored directly.
struct OutStage {
  bf16_t* data;
  int* dest;
  int n;
};

// Copies the staged outputs to `out`, 16 bytes per lane and store.
template <int D>
__device__ __forceinline__ void flush_outputs(const DecodeArgs& a, OutStage& os, int lane) {
  wave_lds_sync();
  const int vecs = a.group * D / 8;
  for (int k = 0; k < os.n; ++k) {
    const int pair = __builtin_amdgcn_readfirstlane(os.dest[k]);
    uint4* dst = (uint4*)((bf16_t*)a.out + (size_t)pair * a.group * D);
    const uint4* src = (const uint4*)(os.data + (size_t)k * a.group * D);
    for (int i = lane; i < vecs; i += 64) dst[i] = src[i];
  }
  os.n = 0;
  wave_lds_sync();
}

// This lane's 4-dim pieces of its head's output, normalised by the
// denominator `l`, as bf16 at o[16 n], n = 0 .. D / 16 - 1.
template <int D>
__device__ __forceinline__ void store_normalised(bf16_t* o, const WaveState<D>& st, float l) {
  const float inv = 1.f / l;
#pragma unroll
  for (int n = 0; n < Tile<D>::kDimTiles; ++n) {
    const uint2 v = make_uint2(pack_bf16x2(f32_to_bf16_bits(st.acc[n][0] * inv),
                                           f32_to_bf16_bits(st.acc[n][1] * inv)),
                               pack_bf16x2(f32_to_bf16_bits(st.acc[n][2] * inv),
                                           f32_to_bf16_bits(st.acc[n][3] * inv)));
    *(uint2*)(o + n * kTile) = v;
  }
}

// A finished segment: a pair that lies wholly in the wave's range is
// normalised and staged (or written, once the stage is full); a piece
// of a cut pair is parked in LDS as an fp32 partial and reported for
// publishing after the stream.
template <int D>
__device__ __forceinline__ bool finish_segment(const DecodeArgs& a, const Segment& s,
                                               WaveState<D>& st, long long f0, float* park,
                                               OutStage& os, int row, int kg) {
  const float l = st.total_l();
  const bool complete = s.fs == s.ps && s.fe == s.ps + s.nb;
  if (complete) {
    // two separate store paths keep each pointer's address space known
    // (LDS or global); a pointer that may be either makes flat stores,
    // which the compiler can only wait for by draining all memory traffic
    if (os.n < a.stage_slots) {
      if (kg == 0 && row == 0) os.dest[os.n] = s.b * a.num_kv_heads + s.kvh;
      if (row < a.group)
        store_normalised<D>(os.data + (size_t)os.n * a.group * D + row * D + kg * 4, st, l);
      ++os.n;
    } else if (row < a.group) {
      store_normalised<D>((bf16_t*)a.out +
                              ((size_t)s.b * a.num_q_heads + (size_t)s.kvh * a.group + row) * D +
                              kg * 4,
                          st, l);
    }
    return false;
  }
  // park slot 0: the wave's first segment; slot 1: its last
  park_piece<D>(park + (s.fs == f0 ? 0 : piece_floats(a.group, D)), st, l, a.group, row, kg);
  return true;
}

// A piece written during the stream, published after it.
struct PendingPiece {
  int b, kvh, nb;
  long long ps;
};

// After the stream: copy the parked pieces to their workspace records
// (slot 2 wave + k for the wave's k-th park slot), wait for the stores to
// complete, then count the wave's pieces (both counters in one round trip,
// during which the staged complete outputs are written);
// the wave that brings a pair's count to its number of pieces merges it and
// rearms the counter for the next call. No wave ever waits for another.
template <int D>
__device__ __forceinline__ void publish_pieces(const DecodeArgs& a, const PendingPiece& p0,
                                               const PendingPiece& p1, int npend,
                                               unsigned parked, long long chunk, int wave_id,
                                               int lane, const float* lds, OutStage& os) {
  const int pf = piece_floats(a.group, D);
  const __amdgpu_buffer_rsrc_t rec = records_rsrc(a, pf);
  for (int k = 0; k < 2; ++k) {
    if (!(parked & (1u << k))) continue;
    const int base = record_bytes(2 * wave_id + k, pf);
    const float4_t* src = (const float4_t*)(lds + k * pf);
    for (int i = lane; i < pf / 4; i += 64)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, src[i]), rec,
                                             base + i * 16, 0, kCoherent);
  }
  wait_stores_complete();
  int* cnt0 = a.ws_cnt + (size_t)p0.b * a.num_kv_heads + p0.kvh;
  int* cnt1 = a.ws_cnt + (size_t)p1.b * a.num_kv_heads + p1.kvh;
  int old0 = 0, old1 = 0;
  if (lane == 0) {
    if (npend > 0) old0 = __hip_atomic_fetch_add(cnt0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (npend > 1) old1 = __hip_atomic_fetch_add(cnt1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // staged outputs go out while the counters' round trip is in flight
  flush_outputs<D>(a, os, lane);
  old0 = __shfl(old0, 0, 64);
  old1 = __shfl(old1, 0, 64);
  for (int k = 0; k < npend; ++k) {
    const PendingPiece& pp = k == 0 ? p0 : p1;
    const Pieces pc(pp.ps, pp.nb, chunk);
    if ((k == 0 ? old0 : old1) == pc.v1 - pc.v0) {
      const int n = pc.v1 - pc.v0 + 1;  // pieces; the batch follows their number
      if (n <= 4)
        merge_pieces<D, 4>(a, rec, pf, pp.b, pp.kvh, pc, lane);
      else if (n <= 8)
        merge_pieces<D, 8>(a, rec, pf, pp.b, pp.kvh, pc, lane);
      else
        merge_pieces<D, 16>(a, rec, pf, pp.b, pp.kvh, pc, lane);
      if (lane == 0)
        __hip_atomic_store(k == 0 ? cnt0 : cnt1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Fused KV append. Row b's new token is the last token of each of its pairs,
// so the wave whose range holds a pair's last block stores that pair's K row
// and V column of the new token (16-byte K vectors on the first D / 8
// lanes, 2-byte V elements on all lanes) before issuing any tile load. Its
// own later tile loads are issued after these stores and, vector memory
// operations completing in order, are waited for only after them; a block
// among the first two of the range, whose loads would be in flight before
// that first wait, is covered by waiting for the stores here. Returns
// whether that wait is needed.
template <int D>
__device__ __forceinline__ bool append_new_tokens(const DecodeArgs& a, const int* prefix,
                                                  Segment s, long long f0, long long f1,
                                                  int lane) {
  const int Hkv = a.num_kv_heads;
  bool early = false;
  while (true) {
    if (s.fe == s.ps + s.nb) {  // the pair's last block lies in this range
      const int slot = uniform_load(a.slot_mapping, s.b);
      if (slot >= 0) {
        const size_t src = ((size_t)s.b * Hkv + s.kvh) * D;
        const int bs = 1 << a.block_shift;
        const int inner = bs < kTile ? bs : kTile;  // V: dim-major tiles of `inner` slots
        const int blk = slot >> a.block_shift;
        const int off = slot & (bs - 1);
        const size_t region = (((size_t)blk * Hkv + s.kvh) << a.block_shift) * D;
        const bf16_t* kn = (const bf16_t*)a.k_new + src;
        const bf16_t* vn = (const bf16_t*)a.v_new + src;
        bf16_t* kp = (bf16_t*)a.k_pool + region + (size_t)off * D;
        bf16_t* vp = (bf16_t*)a.v_pool + region + (size_t)(off & ~(inner - 1)) * D +
                     (off & (inner - 1));
        if (lane < D / 8) *(uint4*)(kp + lane * 8) = *(const uint4*)(kn + lane * 8);
#pragma unroll
        for (int d = lane; d < D; d += 64) vp[(size_t)d * inner] = vn[d];
        early |= s.fe - 1 <= f0 + 1;
      }
    }
    if (s.fe >= f1) break;
    s = next_segment(s, prefix, a.seq_lens, Hkv, f1);
  }
  return early;
}

// Block shapes of the balanced kernel: 8-token blocks (two per 16-token
// tile) or blocks of 16 << k tokens (1 << k tiles each). In the latter every
// tile is contiguous in both pools: K rows [16, D] and a dim-major V tile
// [D, 16] (longer blocks store V as one such tile per 16 tokens), both at
// ((block * Hkv + head) * bs + 16 * sub) * D. The third shape is no paging
// at all: each (sequence, KV head) owns one contiguous run of
// max_blocks 16-token tiles, tile j at ((b * Hkv + head) * max_blocks + j)
// * 16 * D in both caches, and no table is read.
enum BlockShape { kHalfTileBlocks = 0, kTileBlocks = 1, kContiguous = 2 };

template <int D, int kShape>
__global__ __launch_bounds__(256) void decode_mfma_balanced_kernel(DecodeArgs a) {
  // dynamic LDS: prefix [B + 1] ints, then per wave an area of
  // balanced_wave_floats(G, D, stage_slots) floats: two parked pieces, the
  // staged outputs and their destinations
  extern __shared__ int prefix[];
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
  // flat positions count 16-token tiles, whatever the block size
  const int sub_shift = kShape == kTileBlocks ? a.block_shift - 4 : 0;
  const int sub_mask = (1 << sub_shift) - 1;
  const LaneOffsets<D> lo(row, kg);

  Segment cur = locate(prefix, a.seq_lens, B, Hkv, f0, f1);
  if (a.k_new != nullptr && append_new_tokens<D>(a, prefix, cur, f0, f1, lane))
    wait_stores_complete();
  // physical block(s) of a tile: one, or two for 8-token blocks (the second
  // read only when the sequence reaches into it)
  struct Phys {
    int32_t a, b;
  };
  auto table_entry = [&](const Segment& sg) {
    const size_t rowb = (size_t)sg.b * a.max_blocks;
    Phys p;
    if (kShape == kContiguous) {
      p.a = p.b = 0;  // the address is a formula of (b, kvh, j)
    } else if (kShape == kHalfTileBlocks) {
      const int j0 = 2 * sg.j;
      p.a = uniform_load(a.block_tables, rowb + j0);
      p.b = j0 + 1 < ((sg.L + 7) >> 3) ? uniform_load(a.block_tables, rowb + j0 + 1) : p.a;
    } else {
      p.a = uniform_load(a.block_tables, rowb + (sg.j >> sub_shift));
      p.b = p.a;
    }
    return p;
  };
  auto load_tile_at = [&](Tile<D>& dst, const Segment& sg, const Phys& p) {
    if (kShape == kContiguous) {
      const size_t base =
          (((size_t)sg.b * Hkv + sg.kvh) * (size_t)a.max_blocks + (size_t)sg.j) * kTile * D;
      load_tile<D>(dst, kbase + base, vbase + base, lo);
    } else if (kShape == kHalfTileBlocks) {
      load_tile_two_blocks<D>(dst, kbase, vbase, ((size_t)p.a * Hkv + sg.kvh) * (8 * D),
                              ((size_t)p.b * Hkv + sg.kvh) * (8 * D), row, kg);
    } else {
      const size_t base =
          ((((size_t)p.a * Hkv + sg.kvh) << a.block_shift) + (size_t)(sg.j & sub_mask) * kTile) *
          D;
      load_tile<D>(dst, kbase + base, vbase + base, lo);
    }
  };
  // The position after segment position `sg` (flat index `fpos`), which must
  // lie before f1: the next block of the pair, else the next pair.
  auto advance = [&](const Segment& sg, long long fpos) {
    if (fpos + 1 == sg.fe) return next_segment(sg, prefix, a.seq_lens, Hkv, f1);
    Segment r = sg;
    r.j = sg.j + 1;
    return r;
  };
  // A step's loads: the K and V tiles of a block and, when the block starts
  // a new (sequence, KV head) pair, that pair's Q^T operand. Table entries
  // are read one block further ahead, so a tile's address never waits for
  // its table read.
  const int qoff = q_lane_offset<D>(a.group, row, kg);
  Tile<D> ta, tb;
  bf16x8_t qa[Tile<D>::kQkSteps], qz[Tile<D>::kQkSteps];
  Phys phys_cur = table_entry(cur);
  Segment nx = f0 + 1 < f1 ? advance(cur, f0) : cur;
  Phys phys_nx = table_entry(nx);
  load_tile_at(ta, cur, phys_cur);
  load_q_clamped<D>(qa, a, cur.b, cur.kvh, qoff);
  WaveState<D> st;
  st.reset();
  PendingPiece pend0{0, 0, 1, 0}, pend1{0, 0, 1, 0};  // at most two cut pieces per wave
  int npend = 0;
  unsigned parked = 0;
  float* park = (float*)(prefix + ((B + 4) & ~3)) +
                (size_t)(threadIdx.x >> 6) * balanced_wave_floats(a.group, D, a.stage_slots);
  OutStage os;
  os.data = (bf16_t*)(park + 2 * piece_floats(a.group, D));
  os.dest = (int*)(park + 2 * piece_floats(a.group, D) +
                   a.stage_slots * staged_output_floats(a.group, D));
  os.n = 0;

  // Two register tiles alternate: the loads of block f + 1 are issued before
  // block f is folded in. After the last block the current block is
  // requested again (a cache hit that is never used), which keeps the tile
  // loads unconditional.
  long long f = f0;
  Segment nn = nx;
  Phys phys_nn = phys_nx;
  auto prefetch = [&](Tile<D>& dst, bf16x8_t (&qdst)[Tile<D>::kQkSteps],
                      const bf16x8_t (&qsrc)[Tile<D>::kQkSteps], bool more) {
    const Segment sg = more ? nx : cur;
    load_tile_at(dst, sg, more ? phys_nx : phys_cur);
    if (sg.b == cur.b && sg.kvh == cur.kvh) {
#pragma unroll
      for (int c = 0; c < Tile<D>::kQkSteps; ++c) qdst[c] = qsrc[c];
    } else {
      load_q_clamped<D>(qdst, a, sg.b, sg.kvh, qoff);
    }
    // keep the scheduler from sinking these loads below the math on the
    // current block (it would then reuse the current block's registers)
    __builtin_amdgcn_sched_barrier(0);
    nn = f + 2 < f1 ? advance(nx, f + 1) : nx;
    phys_nn = table_entry(nn);
  };
  auto fold = [&](Tile<D>& t, const bf16x8_t (&q)[Tile<D>::kQkSteps]) {
    st.block(t, q, min(kBlockTokens, cur.L - cur.j * kBlockTokens), a.scale_log2, kg);
    if (f + 1 == cur.fe) {
      if (finish_segment<D>(a, cur, st, f0, park, os, row, kg)) {
        parked |= cur.fs == f0 ? 1u : 2u;
        const PendingPiece pp{cur.b, cur.kvh, cur.nb, cur.ps};
        if (npend == 0) pend0 = pp; else pend1 = pp;
        ++npend;
      }
      st.reset();
    }
    cur = nx;
    phys_cur = phys_nx;
    nx = nn;
    phys_nx = phys_nn;
    ++f;
  };
  while (true) {
    bool more = f + 1 < f1;
    prefetch(tb, qz, qa, more);
    fold(ta, qa);
    if (!more) break;
    more = f + 1 < f1;
    prefetch(ta, qa, qz, more);
    fold(tb, qz);
    if (!more) break;
  }
  publish_pieces<D>(a, pend0, pend1, npend, parked, chunk, wave_id, lane, park, os);
}

}  // namespace

const void* decode_mfma_fn(int head_dim, bool balanced, int block_shift, bool contiguous) {
  if (contiguous)
    return head_dim == 64 ? (const void*)&decode_mfma_balanced_kernel<64, kContiguous>
                          : (const void*)&decode_mfma_balanced_kernel<128, kContiguous>;
  if (balanced) {
    const bool half = block_shift == 3;
    if (head_dim == 64)
      return half ? (const void*)&decode_mfma_balanced_kernel<64, kHalfTileBlocks>
                  : (const void*)&decode_mfma_balanced_kernel<64, kTileBlocks>;
    return half ? (const void*)&decode_mfma_balanced_kernel<128, kHalfTileBlocks>
                : (const void*)&decode_mfma_balanced_kernel<128, kTileBlocks>;
  }
  return head_dim == 64 ? (const void*)&decode_mfma_kernel<64>
                        : (const void*)&decode_mfma_kernel<128>;
}

size_t decode_mfma_smem(int num_seqs, int group, int head_dim, bool balanced, int stage_slots) {
  if (!balanced) return (size_t)(num_seqs + 1) * sizeof(int);
  return (size_t)((num_seqs + 4) & ~3) * sizeof(int) +
         (size_t)4 * balanced_wave_floats(group, head_dim, stage_slots) * sizeof(float);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int head_dim, bool balanced, int grid,
                              hipStream_t s, bool contiguous) {
  DecodeArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(decode_mfma_fn(head_dim, balanced, a.block_shift, contiguous), dim3(grid),
                         dim3(256), args,
                         decode_mfma_smem(a.num_seqs, a.group, head_dim, balanced,
                                          a.stage_slots), s);
}

}  // namespace pagedkv
