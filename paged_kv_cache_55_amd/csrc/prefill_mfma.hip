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
//   values  O^T[d][c] += V^T[d][t] P^T[t][c]   v_mfma_f32_16x16x32_bf16
// with the causal test t <= p(c) applied to the scores by select. The
// accumulator layout gives every lane one column and 4 tokens, so the
// causal test and the online softmax are lane-local, with two cross-lane
// steps per tile for the column's max and sum.
//
// A work item is 256 columns of one (sequence, KV head): its workgroup's
// eight waves (two per SIMD, so that one wave's softmax overlaps the other's
// matrix work) own 32 columns each, and all of them read the same K/V
// tiles. The 16-token tiles are staged once per workgroup in LDS by global
// loads with an LDS destination (no staging registers; each lane holds its
// own address, so a tile's issue is one uniform offset added per load),
// eight stages deep: the pair being scored, the pair whose value product is
// pending, and four tiles in flight (measured faster than two or six). K
// token rows are padded to 2 D + 16 bytes and V^T dim rows left at 32: each
// operand read then steps through rows an odd multiple of 32 bytes apart,
// which the LDS serves without bank conflicts (even multiples, and 48- or
// 80-byte steps, conflict two ways). Tiles are folded in pairs: the value
// product's
// k = 32 is the pair's 32 tokens. The two score products take the pair's
// even and odd tokens as their rows, so that each lane's eight scores are
// eight consecutive tokens: the probabilities' k slots, and one 16-byte
// read of a V^T row for the value operand. The probabilities
// enter it as single bf16 numbers: their 2^-9 relative rounding averages
// out over the weighted sum, and a hi/lo pair would double the value
// product's matrix work. A lazy reference max keeps the rescale of the
// accumulators off the common path, where each score is only compared with
// its column's threshold. Pairs wholly at or before a wave's first query
// position, all but the last one or two, skip the causal and length masks.
//
// Every workgroup counts the items per sequence into an LDS prefix, and the
// workgroups of a persistent grid take items in serpentine order (w,
// 2W - 1 - w, 2W + w, ...), which pairs long items with short ones when
// their cost grows with the item index.
#include <type_traits>

#include "launch.h"
#include "lds_stream.h"
#include "mfma_tile.h"
#include "worklist.h"

namespace pagedkv {

namespace {

using namespace mfma;
using lds_stream::lds_barrier;
using lds_stream::lds_char;
using lds_stream::u32x4_t;

typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = kPrefillThreads / 64;
constexpr int kColTiles = 2;
constexpr int kCols = kColTiles * kTile;     // columns per wave
constexpr int kItemCols = kWaves * kCols;    // columns per work item
constexpr float kLazySum = 256.f;            // a lane's probability sum that moves m
constexpr float kFarBelow = 1e30f;           // -m before a column's first pair
constexpr int kStages = 8;                  // LDS tile stages
constexpr int kXcds = 8;                     // L2 domains of the chip
constexpr int kAhead = 4;                    // tiles in flight beyond the pair being folded
constexpr int kTileLoaders = 2;              // waves that load one tile
constexpr int kLoadWaves = 2 * kTileLoaders; // loaders of a pair's even and of its odd tile
static_assert(kAhead % 2 == 0, "each loader refills one tile of every pair");
static_assert(kAhead + 4 == kStages,
              "the pair being scored and the pair whose value product is pending stay in LDS");

// LDS stage of one 16-token tile: K rows [16][2 D + 16 bytes], then V^T
// rows [D][32 bytes], each region whole wave loads of 1 KiB (lane l of
// load k fills bytes 1024 k + 16 l).
template <int D>
struct Stage {
  static constexpr int kKRow = 2 * D + 16;
  static constexpr int kKRowChunks = kKRow / 16;
  static constexpr int kKDataChunks = 2 * D / 16;
  static constexpr int kKLoads = (kTile * kKRowChunks + 63) / 64;
  static constexpr int kVRow = 2 * kTile;
  static constexpr int kVRowChunks = kVRow / 16;
  static constexpr int kVLoads = (D * kVRowChunks + 63) / 64;
  static constexpr int kVBase = kKLoads * 1024;
  static constexpr int kLoads = kKLoads + kVLoads;
  static constexpr int kBytes = kLoads * 1024;
  static constexpr int kFewest = kLoads / kTileLoaders;  // loads of one tile a loader issues, at least
  static constexpr int kMore = kLoads % kTileLoaders;    // loaders below this issue one more
};

template <int D>
struct ColState {
  float4_t acc[D / 16];  // O^T[d][c]: dims 16 n + 4 kg + r of this lane's column
  float m;               // running reference max (log2 domain) of the column
  float l;               // this lane's share of the column's sum
};

// A loading wave's share of its tiles' loads, fixed for the kernel: load
// k = wave % kTileLoaders + kTileLoaders i (i < n; n = 0 for the waves that
// load nothing) fills bytes 1024 k .. + 1023 of a stage, lane
// l the 16 bytes at 1024 k + 16 l, taken from the tile's K rows (16 x D,
// contiguous) for k < kKLoads, else from its V^T rows (D x 16, contiguous),
// at byte offset off[i]. Lanes whose 16 bytes are stage padding (the pad of
// a K row, the gap after the K rows), which nothing reads, load the tile's
// first 16 bytes. Worked out once so that a tile's issue is a few
// instructions: the scalar unit serves both waves of a SIMD, and per-tile
// address arithmetic there measurably slowed the whole kernel.
template <int D>
struct TileLoads {
  using S = Stage<D>;
  static constexpr int kPerWave = (S::kLoads + kTileLoaders - 1) / kTileLoaders;
  int n;                // loads per tile (uniform)
  bool v[kPerWave];     // from the V^T rows (uniform)
  int off[kPerWave];    // this lane's byte offset within the tile's K or V^T rows
  __device__ __forceinline__ TileLoads(int wave, int lane) {
    n = 0;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int k = wave % kTileLoaders + kTileLoaders * i;
      v[i] = k >= S::kKLoads;
      off[i] = 0;
      if (wave >= kLoadWaves || k >= S::kLoads) continue;
      n = i + 1;
      if (k < S::kKLoads) {
        const int slot = 64 * k + lane;
        const int t = slot / S::kKRowChunks;
        const int ch = slot - t * S::kKRowChunks;
        off[i] = t < kTile && ch < S::kKDataChunks ? t * 2 * D + ch * 16 : 0;
      } else {
        const int slot = 64 * (k - S::kKLoads) + lane;
        const int d = slot / S::kVRowChunks;
        const int ch = slot - d * S::kVRowChunks;
        off[i] = d < D && ch < 2 ? d * 2 * kTile + ch * 16 : 0;
      }
    }
  }
};

// Issues this wave's loads of one tile into `stage`: lane src[i] + toff
// for load i, src[i] being this lane's address in the tile at offset 0 of
// its pool. The default cache policy: the other column blocks of the
// (sequence, KV head), on the same XCD, read the same tiles through its L2.
template <int D>
__device__ __forceinline__ void load_tile(const TileLoads<D>& tl, lds_char* stage,
                                          const char* const (&src)[TileLoads<D>::kPerWave],
                                          uint64_t toff, int wave) {
#pragma unroll
  for (int i = 0; i < TileLoads<D>::kPerWave; ++i) {
    if (i >= tl.n) break;
    lds_stream::global_load_to_lds(src[i] + toff,
                                   stage + 1024 * (wave % kTileLoaders + kTileLoaders * i));
  }
}

// Scores of the pair of tiles (tok0 .. tok0 + 15) in stage a and
// (tok0 + 16 .. tok0 + 31) in stage b for every column tile. kMasked: the
// scores of tokens past a column's position (hence of every token past L)
// become -inf; a pair wholly at or before every column's position needs no
// mask.
template <int D, bool kMasked>
__device__ __forceinline__ void pair_scores(const lds_char* sa, const lds_char* sb,
                                            const bf16x8_t (&qb)[kColTiles][D / 32],
                                            const int (&pos)[kColTiles], int tok0, int row,
                                            int kg, float4_t (&s0)[kColTiles],
                                            float4_t (&s1)[kColTiles]) {
  using S = Stage<D>;
  constexpr int NQK = D / 32;
  // score operands: row i of the first product is the pair's token 2 i, of
  // the second token 2 i + 1 (elements 32 c + 8 kg .. + 7), so that lane
  // (column, kg) ends up with the pair's tokens 8 kg .. 8 kg + 7: even ones
  // in the first accumulator, odd ones in the second
  const lds_char* kt = (row < 8 ? sa : sb) + 2 * (row & 7) * S::kKRow + kg * 16;
  bf16x8_t ka[NQK], kb[NQK];
#pragma unroll
  for (int c = 0; c < NQK; ++c) {
    ka[c] = *(lds_bf16x8*)(kt + c * 64);
    kb[c] = *(lds_bf16x8*)(kt + S::kKRow + c * 64);
  }
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    s0[ct] = (float4_t){0.f, 0.f, 0.f, 0.f};
    s1[ct] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      s0[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c], qb[ct][c], s0[ct], 0, 0, 0);
      s1[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[c], qb[ct][c], s1[ct], 0, 0, 0);
    }
  }
  if (kMasked) {
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[ct][r] = tok0 + 8 * kg + 2 * r <= pos[ct] ? s0[ct][r] : -INFINITY;
        s1[ct][r] = tok0 + 8 * kg + 2 * r + 1 <= pos[ct] ? s1[ct][r] : -INFINITY;
      }
    }
  }
}

// The pair's probabilities pf from its scores, folded into l (and, when the
// reference moves, into the rescale of O and l).
//
// Lazy reference max: the probabilities p = 2^(s scale - m) are taken
// against each column's reference m, and m moves only when a lane's eight
// of them sum past kLazySum (so every p stays below it; an overflow to inf
// counts too). Then, rarely, the wave takes the columns' maxima, rescales
// O and l, and takes the probabilities again. m starts at a finite
// -kFarBelow, so the first pair, which holds token 0 for every column,
// always moves it, and a masked score still gives p = 0. The sums add the
// bf16 probabilities themselves, the weights the value product applies.
template <int D>
__device__ __forceinline__ void pair_softmax(const float4_t (&s0)[kColTiles],
                                             const float4_t (&s1)[kColTiles],
                                             ColState<D> (&st)[kColTiles], float scale_log2,
                                             bf16x8_t (&pf)[kColTiles]) {
  constexpr int NDT = D / 16;
  float psum[kColTiles];
  auto probabilities = [&]() {
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // k slots 8 kg + 2 r and 8 kg + 2 r + 1: the pair's tokens of those numbers
        pf[ct][2 * r] = (__bf16)fast_exp2(fmaf(s0[ct][r], scale_log2, -st[ct].m));
        pf[ct][2 * r + 1] = (__bf16)fast_exp2(fmaf(s1[ct][r], scale_log2, -st[ct].m));
      }
      const bf16x2_t* pp = (const bf16x2_t*)&pf[ct];
      const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
      float sum = __builtin_amdgcn_fdot2_f32_bf16(pp[0], ones, 0.f, false);
#pragma unroll
      for (int q = 1; q < 4; ++q) sum = __builtin_amdgcn_fdot2_f32_bf16(pp[q], ones, sum, false);
      psum[ct] = sum;
    }
  };
  probabilities();
  bool grow = false;
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) grow |= !(psum[ct] <= kLazySum);
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) {
      float mloc = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, fmaxf(s0[ct][r], s1[ct][r]));
      // the scale is positive, so it commutes with the max
      const float m_new = fmaxf(st[ct].m, max_over_kg(mloc) * scale_log2);
      const float alpha = fast_exp2(st[ct].m - m_new);
      st[ct].m = m_new;
      st[ct].l *= alpha;
#pragma unroll
      for (int n = 0; n < NDT; ++n) st[ct].acc[n] *= alpha;
    }
    probabilities();
  }
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) st[ct].l += psum[ct];
}

// The value product of the pair in stages a, b (first token tok0) with its
// probabilities pf. kMasked: V^T slots of tokens at or past `limit` (the
// first token no column of the wave sees: past L, or past the wave's last
// position), which may hold anything (NaN included, and a stage's older
// data), are zeroed; their weights are 0, and 0 * NaN would not be.
template <int D, bool kMasked>
__device__ __forceinline__ void pair_values(const lds_char* sa, const lds_char* sb,
                                            const bf16x8_t (&pf)[kColTiles],
                                            ColState<D> (&st)[kColTiles], int tok0, int limit,
                                            int row, int kg) {
  using S = Stage<D>;
  constexpr int NDT = D / 16;
  // value operand: dim 16 n + row, the pair's tokens 8 kg .. 8 kg + 7 (of
  // tile a for kg < 2, else of tile b): 16 contiguous bytes of a V^T row
  const lds_char* vt = (kg < 2 ? sa : sb) + S::kVBase + row * S::kVRow + (kg & 1) * 16;
  const int t8 = tok0 + 8 * kg;
  uint32_t vm[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    vm[q] = (t8 + 2 * q < limit ? 0x0000ffffu : 0u) | (t8 + 2 * q + 1 < limit ? 0xffff0000u : 0u);
#pragma unroll
  for (int n = 0; n < NDT; ++n) {
    u32x4_t v = *(lds_u32x4*)(vt + 16 * n * S::kVRow);
    if (kMasked) v &= (u32x4_t){vm[0], vm[1], vm[2], vm[3]};
    const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, v);
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct)
      st[ct].acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ct], st[ct].acc[n], 0, 0, 0);
  }
}

// One work item: columns grp * 256 .. + 255 of (sequence s, KV head); wave
// w owns columns grp * 256 + 64 w .. + 63.
template <int D>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, const TileLoads<D>& tl,
                                             lds_char* stages, int s, int kvh, int grp, int wave,
                                             int lane) {
  using S = Stage<D>;
  constexpr int NQK = D / 32;
  constexpr int NDT = D / 16;
  const int row = lane & 15;
  const int kg = lane >> 4;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int r0 = uniform_load(a.query_start, s);
  const int n = uniform_load(a.query_start, s + 1) - r0;
  const int L = uniform_load(a.seq_lens, s);
  const int p0 = L - n;  // position of query token 0
  const int ncols = n * G;
  const int c0 = grp * kItemCols + wave * kCols;  // this wave's first column
  const bool active = c0 < ncols;
  const int pos_min = p0 + c0 / G;  // no column of this wave sits before it

  // this lane's column in each column tile; padded columns repeat the
  // wave's last real column (computed, never written)
  int pos[kColTiles];
  bf16x8_t qb[kColTiles][NQK];
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    const int c = max(0, min(c0 + ct * kTile + row, ncols - 1));
    const int i = c / G;
    const int g = c - i * G;
    pos[ct] = p0 + i;
    const bf16_t* qp = (const bf16_t*)a.q + ((size_t)(r0 + i) * Hq + (size_t)kvh * G + g) * D;
#pragma unroll
    for (int k = 0; k < NQK; ++k) qb[ct][k] = *(const bf16x8_t*)(qp + k * 32 + kg * 8);
  }
  // tiles this wave folds, and the item's (the last active wave's)
  const int pos_max = p0 + min(c0 + kCols - 1, ncols - 1) / G;  // no column sits after it
  const int wave_tiles = pos_max / kTile + 1;
  const int vlimit = min(L, pos_max + 1);  // tokens from here on have weight 0 in every column
  const int item_tiles = (p0 + min(grp * kItemCols + kItemCols - 1, ncols - 1) / G) / kTile + 1;
  const int pairs = (item_tiles + 1) / 2;

  ColState<D> st[kColTiles];
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
#pragma unroll
    for (int k = 0; k < NDT; ++k) st[ct].acc[k] = (float4_t){0.f, 0.f, 0.f, 0.f};
    st[ct].m = -kFarBelow;
    st[ct].l = 0.f;
  }
  // the queries are in registers before any tile load is issued: the
  // compiler's wait for them stays out of the tile loop
  __builtin_amdgcn_s_waitcnt(0);

  // tile j's rows start phys * blk + kvh_off + (j & sub_mask) * kTile D
  // elements into either pool (phys: the sequence's block holding the tile)
  const size_t kvh_off = ((size_t)kvh << a.block_shift) * D * sizeof(bf16_t);
  const uint32_t blk_bytes = ((uint32_t)Hkv << a.block_shift) * D * sizeof(bf16_t);
  constexpr uint32_t kTileBytes = kTile * D * sizeof(bf16_t);
  const int sub_shift = a.block_shift - 4;
  const int sub_mask = (1 << sub_shift) - 1;
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks;
  const char* src[TileLoads<D>::kPerWave];
#pragma unroll
  for (int i = 0; i < TileLoads<D>::kPerWave; ++i)
    src[i] = (const char*)(tl.v[i] ? a.v_pool : a.k_pool) + kvh_off + tl.off[i];
  // block-table entry of tile j (clamped to the item's last block for the
  // lookahead past the item's end)
  const int last_block = (item_tiles - 1) >> sub_shift;
  auto entry = [&](int j) {
    return uniform_load_u32(trow, (uint32_t)min(j >> sub_shift, last_block));
  };
  auto issue = [&](lds_char* stage, int j, int32_t phys) {  // tile j (< item_tiles)
    const uint64_t toff =
        (uint64_t)(uint32_t)phys * blk_bytes + (uint32_t)(j & sub_mask) * kTileBytes;
    load_tile<D>(tl, stage, src, toff, wave);
  };
  // the entries of the two tiles a refill issues are read one step before
  // it: waiting for a scalar load right after the barrier held up both the
  // refill and the fold
  // waves 0, 1 load the even tiles, waves 2, 3 the odd ones (one per SIMD
  // and pair); the others issue no tile loads
  const bool loader = wave < kLoadWaves;
  const int parity = wave / kTileLoaders;
  int32_t next = 0;
  if (loader) next = entry(kAhead + parity);
  // The padding tile that rounds an odd item up to whole pairs is never
  // loaded: its stage keeps older data (or none). Its tokens lie past every
  // column's position, so the masks, which select, turn their scores into
  // -inf and their values into 0 (values by the wave's limit, not by L: an
  // item that ends before its sequence has such tokens below L).
  auto advance = [&](int p) {  // pair p is in LDS for every wave; refill
    // tiles 2p, 2p + 1 landed: the loads of the kAhead - 2 tiles issued
    // after them may still be in flight while all of them are real tiles
    // (a loader's own count of them: half those tiles, its parity's);
    // else nothing may. The loader with one more load per tile waits as
    // the other does, for part of the next tile too: safe, and measured
    // faster than branching on the wave.
    if (2 * p + kAhead > item_tiles)
      lds_stream::wait_loads<0>();
    else if (S::kFewest == 0 && wave < S::kMore)
      lds_stream::wait_loads<(S::kFewest + 1) * (kAhead - 2) / 2>();
    else
      lds_stream::wait_loads<S::kFewest * (kAhead - 2) / 2>();
    lds_stream::workgroup_barrier();
    // refill the stage of this loader's tile of pair p + kAhead / 2 (every
    // wave is past the value product of pair p - 2, which held it)
    if (!loader) return;
    const int j = 2 * p + kAhead + parity;
    const int32_t pj = next;
    next = entry(j + 2);
    if (j < item_tiles) issue(stages + (j % kStages) * S::kBytes, j, pj);
  };
  if (loader)
    for (int j = parity; j < kAhead && j < item_tiles; j += 2)
      issue(stages + j * S::kBytes, j, entry(j));
  auto stage = [&](int j) -> const lds_char* { return stages + (j % kStages) * S::kBytes; };
  // Software pipeline: iteration p takes the scores of pair p, then the
  // value product of pair p - 1, whose probabilities are ready, then the
  // softmax of pair p: the value product's matrix instructions do not wait
  // on the softmax's vector instructions, so the two interleave. Pairs
  // wholly at or before this wave's first position need no masks; they run
  // in a loop of their own, so that it keeps its accumulators in place (one
  // loop that branches between the forms copies them).
  // The two waves of a SIMD (w and w + 4) run half an iteration apart: the
  // second half of the waves opens iteration p with the softmax of pair
  // p - 1 (its scores held across the barrier), then the scores of pair p
  // and the value product of pair p - 1. Its vector work then meets the
  // first half's score product instead of its own, and the barrier no
  // longer lines the two waves up on the same phase. Both orders fold the
  // pairs in the same order, so the result is the same bit for bit.
  const int clear = active ? (pos_min + 1) / (2 * kTile) : 0;
  if (wave < kWaves / 2) {
    bf16x8_t pf[kColTiles];  // probabilities of the pair whose value product is pending
    int pending = -1;        // that pair, or -1
    int p = 0;
    if (clear > 0) {
      advance(0);
      float4_t s0[kColTiles], s1[kColTiles];
      pair_scores<D, false>(stage(0), stage(1), qb, pos, 0, row, kg, s0, s1);
      pair_softmax<D>(s0, s1, st, a.scale_log2, pf);
      for (p = 1; p < clear; ++p) {
        advance(p);
        pair_scores<D, false>(stage(2 * p), stage(2 * p + 1), qb, pos, 2 * p * kTile, row, kg, s0,
                              s1);
        pair_values<D, false>(stage(2 * p - 2), stage(2 * p - 1), pf, st, (2 * p - 2) * kTile, vlimit,
                              row, kg);
        pair_softmax<D>(s0, s1, st, a.scale_log2, pf);
      }
      pending = clear - 1;
    }
    for (; p < pairs; ++p) {
      advance(p);
      const bool fold = active && 2 * p < wave_tiles;
      float4_t s0[kColTiles], s1[kColTiles];
      if (fold)
        pair_scores<D, true>(stage(2 * p), stage(2 * p + 1), qb, pos, 2 * p * kTile, row, kg, s0,
                             s1);
      if (pending >= 0)
        pair_values<D, true>(stage(2 * pending), stage(2 * pending + 1), pf, st,
                             2 * pending * kTile, vlimit, row, kg);
      pending = -1;
      if (fold) {
        pair_softmax<D>(s0, s1, st, a.scale_log2, pf);
        pending = p;
      }
    }
    if (pending >= 0)
      pair_values<D, true>(stage(2 * pending), stage(2 * pending + 1), pf, st, 2 * pending * kTile,
                           vlimit, row, kg);
  } else {
    float4_t s0[kColTiles], s1[kColTiles];
    int held = -1;  // the pair whose scores are held for its softmax, or -1
    int p = 0;
    if (clear > 0) {
      advance(0);
      pair_scores<D, false>(stage(0), stage(1), qb, pos, 0, row, kg, s0, s1);
      for (p = 1; p < clear; ++p) {
        advance(p);
        bf16x8_t pf[kColTiles];
        pair_softmax<D>(s0, s1, st, a.scale_log2, pf);
        pair_scores<D, false>(stage(2 * p), stage(2 * p + 1), qb, pos, 2 * p * kTile, row, kg,
                              s0, s1);
        pair_values<D, false>(stage(2 * p - 2), stage(2 * p - 1), pf, st, (2 * p - 2) * kTile,
                              vlimit, row, kg);
      }
      held = clear - 1;
    }
    for (; p < pairs; ++p) {
      advance(p);
      const bool fold = active && 2 * p < wave_tiles;
      if (held >= 0) {
        bf16x8_t pf[kColTiles];
        pair_softmax<D>(s0, s1, st, a.scale_log2, pf);
        pair_values<D, true>(stage(2 * held), stage(2 * held + 1), pf, st, 2 * held * kTile,
                             vlimit, row, kg);
      }
      held = -1;
      if (fold) {
        pair_scores<D, true>(stage(2 * p), stage(2 * p + 1), qb, pos, 2 * p * kTile, row, kg, s0,
                             s1);
        held = p;
      }
    }
    if (held >= 0) {
      bf16x8_t pf[kColTiles];
      pair_softmax<D>(s0, s1, st, a.scale_log2, pf);
      pair_values<D, true>(stage(2 * held), stage(2 * held + 1), pf, st, 2 * held * kTile, vlimit,
                           row, kg);
    }
  }
  lds_barrier();  // every wave is done with the stages before the next item

  if (!active) return;
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    const float l = sum_over_kg(st[ct].l);  // every lane takes part
    const int c = c0 + ct * kTile + row;
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
__global__ __launch_bounds__(kPrefillThreads) void prefill_mfma_kernel(PrefillArgs a) {
  // dynamic LDS: kStages tile stages, then the work-list prefix [S + 1]
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int scan_scratch[kWaves];
  lds_char* stages = (lds_char*)smem;
  int* prefix = (int*)(smem + kStages * Stage<D>::kBytes);
  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  for (int i = threadIdx.x; i < S; i += blockDim.x) {
    const int n = a.query_start[i + 1] - a.query_start[i];
    prefix[i] = n > 0 ? (n * a.group + kItemCols - 1) / kItemCols * Hkv : 0;
  }
  __syncthreads();
  scan_counts_in_place<kPrefillThreads>(S, prefix, scan_scratch);

  const int total = prefix[S];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const TileLoads<D> tl(wave, lane);
  const int W = gridDim.x;
  // workgroups are dispatched to the XCDs in turn (w on XCD w % kXcds), and
  // each XCD has its own L2: slot numbers run across one XCD's workgroups
  // first, so consecutive items (the column groups of one sequence and KV
  // head, which stream the same tiles) run side by side on one L2
  const int wg = W % kXcds == 0 ? (blockIdx.x % kXcds) * (W / kXcds) + blockIdx.x / kXcds
                                : (int)blockIdx.x;
  for (int k = 0; k * W < total; ++k) {
    const int item = (k & 1) ? (k + 1) * W - 1 - wg : k * W + wg;
    if (item >= total) continue;
    const int s = __builtin_amdgcn_readfirstlane(find_sequence(prefix, S, item));
    const int r = item - prefix[s];
    const int n = uniform_load(a.query_start, s + 1) - uniform_load(a.query_start, s);
    const int ngrp = (n * a.group + kItemCols - 1) / kItemCols;
    const int kvh = r / ngrp;
    prefill_item<D>(a, tl, stages, s, kvh, r - kvh * ngrp, wave, lane);
  }
}

}  // namespace

const void* prefill_mfma_fn(int head_dim) {
  return head_dim == 64 ? (const void*)&prefill_mfma_kernel<64>
                        : (const void*)&prefill_mfma_kernel<128>;
}

size_t prefill_mfma_smem(int num_seqs, int head_dim) {
  const size_t stage = head_dim == 64 ? Stage<64>::kBytes : Stage<128>::kBytes;
  return kStages * stage + (size_t)(num_seqs + 1) * sizeof(int);
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, int head_dim, int grid, hipStream_t s) {
  PrefillArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(prefill_mfma_fn(head_dim), dim3(grid), dim3(kPrefillThreads), args,
                         prefill_mfma_smem(a.num_seqs, head_dim), s);
}

}  // namespace pagedkv
