// Chunked-prefill paged attention on the CDNA4 matrix cores (bf16, D = 64
// or 128, blocks of 16 << k tokens).
//
// Sequence s brings n_s query tokens, its newest, at positions
// L_s - n_s .. L_s - 1; their K/V are already in the pool. Query token i at
// position p_i attends to the sequence's tokens 0 .. p_i, so a chunk of a
// long prompt sees the earlier chunks and, causally, itself; a one-token
// chunk is a decode row. For one (sequence, KV head) the G query heads of
// every query token form the columns c = i G + g of the decode kernel's two
// products:
//   scores  S^T[t][c] = K[t] . q[c]             v_mfma_f32_16x16x32_bf16
//   values  O^T[d][c] += V^T[d][t] P^T[t][c]   v_mfma_f32_16x16x16_bf16
// with the causal test t <= p(c) applied to the scores by select. The
// accumulator layout gives every lane one column and 4 tokens, so the
// causal test and the online softmax are lane-local, with two cross-lane
// steps per tile for the column's max and sum.
//
// A wave owns kColTiles column tiles of 16 (64 columns): each K/V tile it
// loads feeds all of them, and it streams the tiles 0 .. up to the last
// position any of its columns sees. The probabilities enter the value
// product as single bf16 numbers: their 2^-9 relative rounding averages out
// over the weighted sum (the measured 8 x 512 step uses 78% of the parity
// bar), and a hi/lo pair would double the value product's matrix work.
//
// Work items are (sequence, KV head, 64-column block); every workgroup
// counts the items per sequence into an LDS prefix, and the waves of a
// persistent grid take items in serpentine order (w, 2W - 1 - w, 2W + w,
// ...), which pairs long items with short ones when their cost grows with
// the item index. The four waves of a workgroup get neighbouring column
// blocks of one (sequence, KV head) and read the same K/V tiles at about the
// same time, so the tiles are loaded with the default cache policy (they
// are shared through the caches, unlike decode's read-once tiles).
#include "launch.h"
#include "mfma_tile.h"
#include "worklist.h"

namespace pagedkv {

namespace {

using namespace mfma;

constexpr int kWaves = 4;
constexpr int kColTiles = 4;
constexpr int kCols = kColTiles * kTile;  // columns per work item
constexpr float kLazyLog2 = 8.f;          // reference-max slack, log2 units
constexpr bool kSplitP = false;           // true: probabilities as bf16 hi + lo

template <int D>
struct ColState {
  float4_t acc[D / 16];  // O^T[d][c]: dims 16 n + 4 kg + r of this lane's column
  float m;               // running max (log2 domain) of the column
  float l;               // this lane's 4-token share of the column's sum
};

// Folds one 16-token tile (tokens tok0 .. tok0 + 15, the first nvalid of
// them inside the sequence) into the kColTiles column states.
template <int D>
__device__ __forceinline__ void fold_tile(Tile<D>& t, const bf16x8_t (&qb)[kColTiles][D / 32],
                                          ColState<D> (&st)[kColTiles],
                                          const int (&pos)[kColTiles], int tok0, int nvalid,
                                          float scale_log2, int kg) {
  constexpr int NQK = D / 32;
  constexpr int NDT = D / 16;
  if (nvalid < kTile) {
    // slots past the sequence may hold anything (NaN included): zero their
    // V so that p = 0 there contributes nothing
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
  for (int ct = 0; ct < kColTiles; ++ct) {
    float4_t s = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQK; ++c)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[c], qb[ct][c], s, 0, 0, 0);
    float sv[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = tok0 + kg * 4 + r <= pos[ct] ? s[r] * scale_log2 : -INFINITY;
      mloc = fmaxf(mloc, sv[r]);
    }
    // lazy reference max: the column keeps its reference m until a score
    // exceeds it by 2^kLazyLog2 (its first tile always does: m starts at
    // -inf, and token 0 is seen by every column); p = 2^(s - m) then stays
    // <= 2^kLazyLog2, and the rescale of O and l runs only when some column
    // of the wave moves its reference
    const float mcol = max_over_kg(mloc);
    const bool grow = mcol > st[ct].m + kLazyLog2;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mcol : st[ct].m;
      const float alpha = fast_exp2(st[ct].m - m_new);  // 1 for columns that keep m
      st[ct].m = m_new;
      st[ct].l *= alpha;
#pragma unroll
      for (int n = 0; n < NDT; ++n) st[ct].acc[n] *= alpha;
    }
    float psum = 0.f;
    uint16_t ph[4], pl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(sv[r] - st[ct].m);
      psum += p;
      ph[r] = bf16_rne(p);
      pl[r] = bf16_rne(p - __uint_as_float((uint32_t)ph[r] << 16));
    }
    st[ct].l += psum;
    const short4_t bhi = __builtin_bit_cast(
        short4_t, make_uint2(pack_bf16x2(ph[0], ph[1]), pack_bf16x2(ph[2], ph[3])));
    const short4_t blo = __builtin_bit_cast(
        short4_t, make_uint2(pack_bf16x2(pl[0], pl[1]), pack_bf16x2(pl[2], pl[3])));
#pragma unroll
    for (int n = 0; n < NDT; ++n) {
      float4_t o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[n], bhi, st[ct].acc[n], 0, 0, 0);
      if (kSplitP) o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[n], blo, o, 0, 0, 0);
      st[ct].acc[n] = o;
    }
  }
}

// One work item: columns cb * 64 .. cb * 64 + 63 of (sequence s, KV head).
template <int D>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, int s, int kvh, int cb,
                                             int row, int kg) {
  constexpr int NQK = D / 32;
  constexpr int NDT = D / 16;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int r0 = uniform_load(a.query_start, s);
  const int n = uniform_load(a.query_start, s + 1) - r0;
  const int L = uniform_load(a.seq_lens, s);
  const int p0 = L - n;          // position of query token 0
  const int ncols = n * G;

  // this lane's column in each column tile; padded columns repeat the
  // block's last real column (computed, never written)
  int pos[kColTiles];
  bf16x8_t qb[kColTiles][NQK];
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    const int c = min(cb * kCols + ct * kTile + row, ncols - 1);
    const int i = c / G;
    const int g = c - i * G;
    pos[ct] = p0 + i;
    const bf16_t* qp = (const bf16_t*)a.q + ((size_t)(r0 + i) * Hq + (size_t)kvh * G + g) * D;
#pragma unroll
    for (int k = 0; k < NQK; ++k) qb[ct][k] = *(const bf16x8_t*)(qp + k * 32 + kg * 8);
  }
  const int clast = min(cb * kCols + kCols - 1, ncols - 1);
  const int ntiles = (p0 + clast / G) / kTile + 1;

  ColState<D> st[kColTiles];
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
#pragma unroll
    for (int k = 0; k < NDT; ++k) st[ct].acc[k] = (float4_t){0.f, 0.f, 0.f, 0.f};
    st[ct].m = -INFINITY;
    st[ct].l = 0.f;
  }

  const bf16_t* kbase = (const bf16_t*)a.k_pool;
  const bf16_t* vbase = (const bf16_t*)a.v_pool;
  const int sub_shift = a.block_shift - 4;
  const int sub_mask = (1 << sub_shift) - 1;
  const size_t trow = (size_t)s * a.max_blocks;
  const LaneOffsets<D> lo(row, kg);
  auto table = [&](int j) { return uniform_load(a.block_tables, trow + (j >> sub_shift)); };
  auto load = [&](Tile<D>& dst, int j, int32_t phys) {
    const size_t base =
        ((((size_t)phys * Hkv + kvh) << a.block_shift) + (size_t)(j & sub_mask) * kTile) * D;
    load_tile<D, 0>(dst, kbase + base, vbase + base, lo);
  };

  // two register tiles alternate; the table entry of tile j + 2 is read
  // while tile j is folded in, so no tile address waits for its table read
  Tile<D> ta, tb;
  int32_t ph_cur = table(0);
  int32_t ph_nx = table(ntiles > 1 ? 1 : 0);
  load(ta, 0, ph_cur);
  int j = 0;
  auto prefetch = [&](Tile<D>& dst, bool more) {
    load(dst, more ? j + 1 : j, more ? ph_nx : ph_cur);
    __builtin_amdgcn_sched_barrier(0);
    const int32_t ph_nn = table(j + 2 < ntiles ? j + 2 : (more ? j + 1 : j));
    if (more) {
      ph_cur = ph_nx;
      ph_nx = ph_nn;
    }
  };
  while (true) {
    bool more = j + 1 < ntiles;
    prefetch(tb, more);
    fold_tile<D>(ta, qb, st, pos, j * kTile, min(kTile, L - j * kTile), a.scale_log2, kg);
    if (!more) break;
    ++j;
    more = j + 1 < ntiles;
    prefetch(ta, more);
    fold_tile<D>(tb, qb, st, pos, j * kTile, min(kTile, L - j * kTile), a.scale_log2, kg);
    if (!more) break;
    ++j;
  }

#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    const float l = sum_over_kg(st[ct].l);  // every lane takes part
    const int c = cb * kCols + ct * kTile + row;
    if (c >= ncols) continue;
    const int i = c / G;
    const int g = c - i * G;
    bf16_t* o = (bf16_t*)a.out + ((size_t)(r0 + i) * Hq + (size_t)kvh * G + g) * D + kg * 4;
    const float inv = 1.f / l;
#pragma unroll
    for (int k = 0; k < NDT; ++k) {
      const float4_t v = st[ct].acc[k] * inv;
      *(uint2*)(o + k * kTile) =
          make_uint2(pack_bf16x2(f32_to_bf16_bits(v[0]), f32_to_bf16_bits(v[1])),
                     pack_bf16x2(f32_to_bf16_bits(v[2]), f32_to_bf16_bits(v[3])));
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillArgs a) {
  extern __shared__ int prefix[];  // [S + 1]: work items before each sequence
  __shared__ int scan_scratch[kWaves];
  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  for (int i = threadIdx.x; i < S; i += blockDim.x) {
    const int n = a.query_start[i + 1] - a.query_start[i];
    prefix[i] = n > 0 ? (n * a.group + kCols - 1) / kCols * Hkv : 0;
  }
  __syncthreads();
  scan_counts_in_place(S, prefix, scan_scratch);

  const int total = prefix[S];
  const int lane = threadIdx.x & 63;
  const int row = lane & 15;
  const int kg = lane >> 4;
  const int W = gridDim.x * kWaves;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
  for (int k = 0; k * W < total; ++k) {
    const int item = (k & 1) ? (k + 1) * W - 1 - w : k * W + w;
    if (item >= total) continue;
    // items of one sequence: KV head major, column block minor, so the waves
    // of a workgroup take neighbouring column blocks of one (sequence, KV
    // head) and stream the same K/V tiles at the same time
    const int s = __builtin_amdgcn_readfirstlane(find_sequence(prefix, S, item));
    const int r = item - prefix[s];
    const int n = uniform_load(a.query_start, s + 1) - uniform_load(a.query_start, s);
    const int ncb = (n * a.group + kCols - 1) / kCols;
    const int kvh = r / ncb;
    prefill_item<D>(a, s, kvh, r - kvh * ncb, row, kg);
  }
}

}  // namespace

const void* prefill_mfma_fn(int head_dim) {
  return head_dim == 64 ? (const void*)&prefill_mfma_kernel<64>
                        : (const void*)&prefill_mfma_kernel<128>;
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, int head_dim, int grid, hipStream_t s) {
  PrefillArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(prefill_mfma_fn(head_dim), dim3(grid), dim3(256), args,
                         (size_t)(a.num_seqs + 1) * sizeof(int), s);
}

}  // namespace pagedkv
