// Latent (MLA-style) paged decode on the CDNA4 matrix cores (bf16).
//
// Every cached token holds one latent of 576 elements (a 512-element
// compressed KV and a 64-element positional key); each of the 128 query
// heads of a row scores its absorbed 576-element query against every
// latent of the row, and its output is the softmax-weighted sum of the
// latents' first 512 elements [llm-serving.xyz "KV-cache systems", MLA
// section: the cached latent with its decoupled positional key, the absorbed
// (MQA) computation mode, the 64-token page]. This is multi-query attention
// with head dim 576: a token costs 4 x 128 x 576 flops against 1,152 bytes,
// so on MI355X the two rooflines nearly meet (the bf16 matrix cores must
// run at about 77% of peak to keep pace with HBM).
//
// A workgroup of four waves owns all 128 heads, 32 per wave: a wave's
// output accumulator O^T (32 heads x 512 dims, fp32) is 256 registers, the
// accumulation registers of one wave per SIMD. A 32-token latent tile is
// brought from HBM once per workgroup, straight into LDS (buffer loads with
// an LDS destination: no staging registers; three tiles in flight), token
// rows padded to 1,248 bytes, a stride at which both operand reads below
// run without bank conflicts:
//   scores  S^T[t][h] = C[t] . q[h]             v_mfma_f32_16x16x32_bf16;
//           A = 16 tokens x 32 elements, one ds_read_b128 of a token row
//   values  O^T[d][h] += C^T[d][t] P^T[t][h]    v_mfma_f32_16x16x32_bf16;
//           A = 16 dims x 32 tokens, two ds_read_b64_tr_b16 (the LDS read
//           that transposes 16-bit elements across lanes)
// The probabilities enter the value product as single bf16 numbers (their
// 2^-9 relative rounding averages out over the weighted sum; a hi/lo pair
// as in the grouped-query kernels would double the value product's matrix
// work, which here is the other bound). The softmax keeps a lazy reference
// max, as the prefill kernel does.
//
// Work split: the flat list of (row, 32-token tile) is cut into contiguous
// ranges, one per workgroup of a persistent grid (one workgroup per compute
// unit), equal in cost: a row's tiles plus kFinishSlots tiles' worth for
// writing it, so that workgroups with many short rows take fewer tiles. A
// row cut by range boundaries leaves one record per piece (its output
// normalised by the piece's sum, scaled per head by a power of two and
// stored as fp16, then its max, sum and scale in fp32: 129.5 KiB, as
// much as 115 tokens of latent cache) and a description of its pieces; a
// second kernel merges each cut row in parallel over its heads. No
// workgroup waits for another, and no merge sits at the end of a range.
#include <type_traits>

#include "launch.h"
#include "lds_stream.h"
#include "mfma_tile.h"
#include "worklist.h"

namespace pagedkv {

namespace {

using namespace mfma;

using lds_stream::lds_char;
using lds_stream::kPastRange;
using lds_stream::load_to_lds;
using lds_stream::raw_rsrc;
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kHeads = kLatentHeads;
constexpr int kHeadsPerWave = kHeads / kWaves;  // 32: two 16-head tiles
constexpr int kLatent = kLatentDim;
constexpr int kValue = kLatentValueDim;
constexpr int kPageTokens = kLatentBlockTokens;
constexpr int kTileTokens = kLatentTileTokens;
constexpr int kTokenBytes = kLatent * 2;             // 1,152
constexpr int kRowBytes = 1248;                       // padded LDS row of one token
constexpr int kRowChunks = kRowBytes / 16;            // 78 16-byte chunks, 72 of data
constexpr int kDataChunks = kTokenBytes / 16;         // 72
constexpr int kTileLoads = kTileTokens * kRowChunks / 64;  // 39 wave loads of 1 KiB
static_assert(kTileTokens * kRowChunks % 64 == 0, "a tile is whole wave loads");
static_assert(kTileLoads * 1024 == kLatentStageBytes, "stage size");
constexpr int kStageBytes = kLatentStageBytes;
constexpr int kStages = kLatentStages;
constexpr int kAhead = kStages - 1;  // tiles in flight while one is folded
static_assert(kAhead <= 3, "tile_barrier counts at most two younger tiles");
constexpr int kWaveLoads = (kTileLoads + kWaves - 1) / kWaves;  // 10
constexpr int kFewestLoads = kTileLoads / kWaves;               // 9
static_assert(kWaveLoads <= kLatent / 32, "a wave's loads of a tile fit one per score step");
constexpr int kQkSteps = kLatent / 32;  // 18 score steps
constexpr int kDimTiles = kValue / 16;  // 32 output dim tiles
constexpr int kOverflowLog2 = 32;  // weights up to 2^32 over the reference
constexpr float kOverflowWeight = (float)(1ull << kOverflowLog2);
constexpr int kRecordBytes = kLatentRecordBytes;
constexpr int kFinishSlots = 8;         // a row's finish, in tile-equivalents of work
constexpr int kMergePieces = 2;         // pieces whose record loads a merge round issues together
constexpr int kFewPieces = 8;           // rows of at most this many pieces: (m, l) in registers
#ifndef LATENT_K_AHEAD
#define LATENT_K_AHEAD 2
#endif
#ifndef LATENT_V_AHEAD
#define LATENT_V_AHEAD 8
#endif
constexpr int kKAhead = LATENT_K_AHEAD;  // score steps of LDS reads in flight
constexpr int kVAhead = LATENT_V_AHEAD;  // value steps of LDS reads in flight

static_assert(kPageTokens % kTileTokens == 0, "tiles never straddle a page");
static_assert(kTileTokens == 32, "one value step of 32 tokens per tile");

// ---- tile stream ----------------------------------------------------------

// Position of flat tile f: row b, tile j of the row's n tiles.
struct Cursor {
  int b, j, n;
};

__device__ __forceinline__ Cursor locate_tile(const int* prefix, int B, int f) {
  Cursor c;
  c.b = __builtin_amdgcn_readfirstlane(find_sequence(prefix, B, f));
  c.n = __builtin_amdgcn_readfirstlane(prefix[c.b + 1] - prefix[c.b]);
  c.j = __builtin_amdgcn_readfirstlane(f - prefix[c.b]);
  return c;
}

// Moves to the next flat tile; called only when one exists.
__device__ __forceinline__ void next_tile(Cursor& c, const int* prefix) {
  if (++c.j < c.n) return;
  int b = c.b + 1;
  while (prefix[b + 1] == prefix[b]) ++b;  // rows of length 0 have no tiles
  c.b = __builtin_amdgcn_readfirstlane(b);
  c.j = 0;
  c.n = __builtin_amdgcn_readfirstlane(prefix[b + 1] - prefix[b]);
}

// This wave's share of the loads of tile c into `stage`: wave load k
// (k = wave, wave + 4, ...) fills LDS bytes 1024 k .. 1024 k + 1023, lane l
// the 16 bytes at 1024 k + 16 l, i.e. chunk ch of token t with
// 78 t + ch = 64 k + l. Pad chunks (ch >= 72) and tokens past the row get
// an offset past the descriptor's range, which loads zeros. Prepared once
// per tile; load(i) issues the wave's load i (nothing past kTileLoads).
struct TileIssue {
  u32x4_t r;
  lds_char* stage;
  int wave, lane;
  __device__ __forceinline__ void load(int i) const {
    const int k = wave + kWaves * i;
    if (k < kTileLoads) {
      const int slot = 64 * k + lane;
      const int t = slot / kRowChunks;
      const int ch = slot - t * kRowChunks;
      const int off = ch < kDataChunks ? t * kTokenBytes + ch * 16 : kPastRange;
      load_to_lds(r, stage + 1024 * k, off);
    }
  }
};

__device__ __forceinline__ TileIssue prepare_tile(const LatentArgs& a, const Cursor& c,
                                                  lds_char* stage, int wave, int lane) {
  const int L = uniform_load(a.seq_lens, c.b);
  const int valid = min(kTileTokens, L - c.j * kTileTokens);
  const int page = uniform_load(a.block_tables, (size_t)c.b * a.max_blocks +
                                                    (c.j / (kPageTokens / kTileTokens)));
  const char* base =
      (const char*)a.kv_pool +
      ((size_t)page * kPageTokens + (size_t)(c.j % (kPageTokens / kTileTokens)) * kTileTokens) *
          kTokenBytes;
  TileIssue t;
  t.r = raw_rsrc(base, valid * kTokenBytes);
  t.stage = stage;
  t.wave = wave;
  t.lane = lane;
  return t;
}

// All of this wave's loads of tile c at once.
__device__ __forceinline__ void load_tile(const LatentArgs& a, const Cursor& c, lds_char* stage,
                                          int wave, int lane) {
  const TileIssue t = prepare_tile(a, c, stage, wave, lane);
#pragma unroll
  for (int i = 0; i < kWaveLoads; ++i) t.load(i);
}

// Waits until this wave's loads of the current tile have landed in LDS (at
// most kFewestLoads younger ones, those of the next tile, may remain; none
// when no tile follows), then for every wave of the workgroup.
template <int kYoungerTiles>
__device__ __forceinline__ void tile_barrier() {
  lds_stream::tile_barrier<kYoungerTiles * kFewestLoads>();
}

using lds_stream::lds_barrier;

// ---- one wave's 32 heads of one row -----------------------------------------
//
// The output accumulator fills the accumulation registers, and the compiler
// keeps it there only if nothing but the matrix instructions writes it:
// the fast path never rescales, resets or merges it in place. A segment's
// first tile starts the accumulator from zero (a zero C operand) and fixes
// the segment's reference max (its tile max); later weights are
// 2^(s - reference), which stays far from overflow unless a score exceeds
// the reference by more than kOverflowLog2 (then the segment is flagged and
// recomputed exactly by the slow path below).

struct RowState {
  float4_t o[2][kDimTiles];  // O^T[d][h]: dims 16 n + 4 kg + r of head h0 + 16 ht + col
  float m[2];                // reference max (log2 domain) of the lane's head
  float l[2];                // this lane's share of the head's sum of weights
  bool overflow;             // a lane's weights reached 2^kOverflowLog2 in a tile
};

// The B operand of the score product: head h0 + 16 ht + col, elements
// 32 s + 8 kg .. + 7.
__device__ __forceinline__ void load_queries(const LatentArgs& a, int b, int h0, int col, int kg,
                                             bf16x8_t (&qf)[2][kQkSteps]) {
  const bf16_t* q = (const bf16_t*)a.q + ((size_t)b * kHeads + h0 + col) * kLatent + kg * 8;
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int s = 0; s < kQkSteps; ++s)
      qf[ht][s] = *(const bf16x8_t*)(q + (size_t)ht * 16 * kLatent + s * 32);
}

// Raw scores of the tile: sc[tt][ht][r] = C[token 16 tt + 4 kg + r] .
// q[head h0 + 16 ht + col].
// on_step(s) runs after the products of score step s (the tile refill's
// loads go out there, one per step, among the matrix instructions).
template <typename OnStep>
__device__ __forceinline__ void score_products(const lds_char* tile,
                                               const bf16x8_t (&qf)[2][kQkSteps], int col,
                                               int kg, float4_t (&sc)[2][2], OnStep on_step) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) sc[tt][ht] = (float4_t){0.f, 0.f, 0.f, 0.f};
  // kKAhead steps of fragments in flight (LDS latency exceeds a step's
  // four products); the schedule barriers keep the compiler from hoisting
  // more, for which the accumulators and the queries leave no registers
  const lds_char* krow = tile + col * kRowBytes + kg * 16;
  bf16x8_t k0[kQkSteps], k1[kQkSteps];
#pragma unroll
  for (int s = 0; s < kKAhead; ++s) {
    k0[s] = *(lds_bf16x8*)(krow + s * 64);
    k1[s] = *(lds_bf16x8*)(krow + 16 * kRowBytes + s * 64);
  }
#pragma unroll
  for (int s = 0; s < kQkSteps; ++s) {
    if (s + kKAhead < kQkSteps) {
      k0[s + kKAhead] = *(lds_bf16x8*)(krow + (s + kKAhead) * 64);
      k1[s + kKAhead] = *(lds_bf16x8*)(krow + 16 * kRowBytes + (s + kKAhead) * 64);
    }
    sc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[s], qf[0][s], sc[0][0], 0, 0, 0);
    sc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[s], qf[1][s], sc[0][1], 0, 0, 0);
    sc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[s], qf[0][s], sc[1][0], 0, 0, 0);
    sc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[s], qf[1][s], sc[1][1], 0, 0, 0);
    on_step(s);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Scores of the tile, scaled to the log2 domain: x[ht][tt][r] for token
// 16 tt + 4 kg + r and head h0 + 16 ht + col; -inf past the row's end (the
// stage holds zeros there).
__device__ __forceinline__ void score_tile(const lds_char* tile,
                                           const bf16x8_t (&qf)[2][kQkSteps], int valid,
                                           float scale_log2, int col, int kg,
                                           float (&x)[2][2][4]) {
  float4_t sc[2][2];
  score_products(tile, qf, col, kg, sc, [](int) {});
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[ht][tt][r] = 16 * tt + 4 * kg + r < valid ? sc[tt][ht][r] * scale_log2 : -INFINITY;
}

// Max of the lane's head over the tile (same in the head's four lanes).
__device__ __forceinline__ float tile_max(const float (&xh)[2][4]) {
  float mx = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, xh[tt][r]);
  return max_over_kg(mx);
}

// Weights 2^e as bf16, the value product's B operand (k slot 8 kg + 4 tt + r
// is token 16 tt + 4 kg + r); returns their sum, taken over the rounded
// weights (bf16 dot products with ones) so that the normalisation matches
// the product.
__device__ __forceinline__ float weights(const float (&e)[2][4], bf16x8_t& pf) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) pf[4 * tt + r] = (__bf16)fast_exp2(e[tt][r]);
  const bf16x2_t* pp = (const bf16x2_t*)&pf;
  const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
  float ps = __builtin_amdgcn_fdot2_f32_bf16(pp[0], ones, 0.f, false);
#pragma unroll
  for (int q = 1; q < 4; ++q) ps = __builtin_amdgcn_fdot2_f32_bf16(pp[q], ones, ps, false);
  return ps;
}

// Weights 2^(x - m) of scaled scores x (see weights).
__device__ __forceinline__ float make_weights(const float (&xh)[2][4], float m, bf16x8_t& pf) {
  float e[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) e[tt][r] = xh[tt][r] - m;
  return weights(e, pf);
}

// O^T += C^T P^T over the tile (kFirst: O^T = C^T P^T). The transposing
// read gives lane (kg, col) dim 16 n + col of tokens 16 tt + 4 kg .. + 3
// when lane 16 kg + 4 e + c4 addresses token 16 tt + 4 kg + e at dims
// 16 n + 4 c4 .. + 3.
__device__ __forceinline__ const lds_char* value_row(const lds_char* tile, int col, int kg) {
  return tile + (4 * kg + (col >> 2)) * kRowBytes + (col & 3) * 8;
}

// The value operand's first kVAhead steps of fragments (kVAhead steps stay
// in flight: a step is only two products). Issued before the weights are
// taken, their LDS latency passes under that vector work.
__device__ __forceinline__ void value_prefetch(const lds_char* tile, int col, int kg,
                                               short4_t (&v0)[kDimTiles],
                                               short4_t (&v1)[kDimTiles]) {
  const lds_char* vrow = value_row(tile, col, kg);
#pragma unroll
  for (int n = 0; n < kVAhead; ++n) {
    v0[n] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(vrow + n * 32));
    v1[n] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(vrow + 16 * kRowBytes + n * 32));
  }
}

template <bool kFirst>
__device__ __forceinline__ void value_products(const lds_char* tile, const bf16x8_t (&pf)[2],
                                               float4_t (&o)[2][kDimTiles], int col, int kg,
                                               short4_t (&v0)[kDimTiles],
                                               short4_t (&v1)[kDimTiles]) {
  const float4_t zero = {0.f, 0.f, 0.f, 0.f};
  const lds_char* vrow = value_row(tile, col, kg);
#pragma unroll
  for (int n = 0; n < kDimTiles; ++n) {
    if (n + kVAhead < kDimTiles) {
      v0[n + kVAhead] =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(vrow + (n + kVAhead) * 32));
      v1[n + kVAhead] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4*)(vrow + 16 * kRowBytes + (n + kVAhead) * 32));
    }
    const bf16x8_t vf = __builtin_bit_cast(
        bf16x8_t, __builtin_shufflevector(v0[n], v1[n], 0, 1, 2, 3, 4, 5, 6, 7));
    o[0][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[0], kFirst ? zero : o[0][n], 0, 0, 0);
    o[1][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[1], kFirst ? zero : o[1][n], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool kFirst>
__device__ __forceinline__ void value_tile(const lds_char* tile, const bf16x8_t (&pf)[2],
                                           float4_t (&o)[2][kDimTiles], int col, int kg) {
  short4_t v0[kDimTiles], v1[kDimTiles];
  value_prefetch(tile, col, kg, v0, v1);
  value_products<kFirst>(tile, pf, o, col, kg, v0, v1);
}

// Folds a tile into the row state. kFirst: the segment's first tile, which
// sets the reference max. Otherwise a lane whose weights sum to 2^32 or more
// (inf and NaN included) marks the segment: every score above
// reference + kOverflowLog2 does, its weight alone rounding to at least
// 2^32. The test is lane-local, so later tiles take no tile max at all
// (its cross-lane steps sat between the two products); their exponents are
// one fused multiply-add each, masked only in a row's partial last tile.
template <bool kFirst, typename OnStep>
__device__ __forceinline__ void fold_tile(const lds_char* tile, const bf16x8_t (&qf)[2][kQkSteps],
                                          RowState& st, int valid, float scale_log2, int col,
                                          int kg, OnStep on_step) {
  float4_t sc[2][2];
  score_products(tile, qf, col, kg, sc, on_step);
  short4_t v0[kDimTiles], v1[kDimTiles];
  value_prefetch(tile, col, kg, v0, v1);
  bf16x8_t pf[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    float e[2][4];
    if (kFirst) {
      float x[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          x[tt][r] = 16 * tt + 4 * kg + r < valid ? sc[tt][ht][r] * scale_log2 : -INFINITY;
      st.m[ht] = tile_max(x);
      st.l[ht] = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) e[tt][r] = x[tt][r] - st.m[ht];
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) e[tt][r] = fmaf(sc[tt][ht][r], scale_log2, -st.m[ht]);
      if (valid < kTileTokens) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * tt + 4 * kg + r >= valid) e[tt][r] = -INFINITY;
      }
    }
    const float ps = weights(e, pf[ht]);
    if (!kFirst) st.overflow |= !(ps < kOverflowWeight);
    st.l[ht] += ps;
  }
  value_products<kFirst>(tile, pf, st.o, col, kg, v0, v1);
}

// ---- finishing a row ----------------------------------------------------------
//
// Every use of the accumulator here only reads it.

// Lane 16 kg + col holds dims 4 kg .. 4 kg + 3 of its head in every 16-dim
// tile, as two packed dwords per tile. Given those of tiles 2 p (a) and
// 2 p + 1 (b), a swap between the wave's halves and one between its 16-lane
// rows (two dwords each) leave lane kg with dims 32 p + 8 kg .. + 7, in
// order: one 16-byte store per lane and tile pair where two 8-byte stores
// would be needed. (Vector memory operations retire in order and stores
// count with the tile loads, so every store instruction a row finish saves
// is one fewer that the next tile waits behind.)
__device__ __forceinline__ uint4 dims8_of_pair(uint2 a, uint2 b) {
  // row r then holds a of rows r and r + 2 (r < 2), or b of rows r - 2 and r
  const auto x32 = __builtin_amdgcn_permlane32_swap(a.x, b.x, false, false);
  const auto y32 = __builtin_amdgcn_permlane32_swap(a.y, b.y, false, false);
  // row r: a (r < 2) or b (r >= 2) of rows 2 (r & 1) and 2 (r & 1) + 1
  const auto x16 = __builtin_amdgcn_permlane16_swap(x32[0], x32[1], false, false);
  const auto y16 = __builtin_amdgcn_permlane16_swap(y32[0], y32[1], false, false);
  return make_uint4(x16[0], y16[0], x16[1], y16[1]);
}

// Row b's outputs of this wave's heads: O^T scaled per head, as bf16.
__device__ __forceinline__ void store_scaled(const LatentArgs& a, const float4_t (&o)[2][kDimTiles],
                                             const float (&mul)[2], int b, int h0, int col,
                                             int kg) {
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    bf16_t* out = (bf16_t*)a.out + ((size_t)b * kHeads + h0 + 16 * ht + col) * kValue + 8 * kg;
#pragma unroll
    for (int p = 0; p < kDimTiles / 2; ++p) {
      const float4_t v = o[ht][2 * p] * mul[ht];
      const float4_t u = o[ht][2 * p + 1] * mul[ht];
      *(uint4*)(out + 32 * p) = dims8_of_pair(
          make_uint2(pack_bf16x2(bf16_rne(v[0]), bf16_rne(v[1])),
                     pack_bf16x2(bf16_rne(v[2]), bf16_rne(v[3]))),
          make_uint2(pack_bf16x2(bf16_rne(u[0]), bf16_rne(u[1])),
                     pack_bf16x2(bf16_rne(u[2]), bf16_rne(u[3]))));
    }
  }
}

// Record of a piece: y[h][d] = (O / l) 2^k_h as fp16, then m[H], l[H] and
// s[H] = 2^-k_h as fp32. k_h puts the head's largest |O / l| in
// [2^14, 2^15): the scaling is exact, no finite value overflows fp16, and
// each element keeps fp16's 2^-11 relative rounding, a quarter of bf16's
// (bf16 records added their rounding to the output's in rows merged from
// partly cancelling pieces).
__device__ __forceinline__ int record_base(int slot) { return slot * kRecordBytes; }
__device__ __forceinline__ int record_x(int slot, int h, int d) {
  return record_base(slot) + (h * kValue + d) * 2;
}
__device__ __forceinline__ int record_m(int slot, int h) {
  return record_base(slot) + kHeads * kValue * 2 + h * 4;
}
__device__ __forceinline__ int record_l(int slot, int h) {
  return record_base(slot) + kHeads * kValue * 2 + kHeads * 4 + h * 4;
}
__device__ __forceinline__ int record_s(int slot, int h) {
  return record_base(slot) + kHeads * kValue * 2 + 2 * kHeads * 4 + h * 4;
}

__device__ __forceinline__ void store_rec16(__amdgpu_buffer_rsrc_t rec, int off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rec, off, 0, 0);
}
__device__ __forceinline__ void store_rec(__amdgpu_buffer_rsrc_t rec, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rec, off, 0, 0);
}

// k with max_abs 2^k in [2^14, 2^15), as the fp32 power 2^k; 1 for a zero
// or non-finite max_abs. Clamped to fp32's normal powers.
__device__ __forceinline__ float record_scale(float max_abs) {
  const uint32_t e = (__builtin_bit_cast(uint32_t, max_abs) >> 23) & 0xffu;  // biased exponent
  if (!(max_abs > 0.f) || e == 0xffu) return 1.f;
  // max_abs in [2^(e - 127), 2^(e - 126)) for e >= 1 (below for subnormals)
  const int k = min(127, max(-126, 14 - ((int)e - 127)));
  return __builtin_bit_cast(float, (uint32_t)(k + 127) << 23);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

__device__ __forceinline__ float4_t zero4() { return (float4_t){0.f, 0.f, 0.f, 0.f}; }

// Four fp16 (two packed pairs, low half first) as fp32, exactly.
__device__ __forceinline__ float4_t f16x4_to_f32(uint32_t lo, uint32_t hi) {
  return (float4_t){(float)__builtin_bit_cast(_Float16, (uint16_t)(lo & 0xffffu)),
                    (float)__builtin_bit_cast(_Float16, (uint16_t)(lo >> 16)),
                    (float)__builtin_bit_cast(_Float16, (uint16_t)(hi & 0xffffu)),
                    (float)__builtin_bit_cast(_Float16, (uint16_t)(hi >> 16))};
}

// x * w + acc elementwise, one rounding each (the merge's only operation,
// so that its result depends on the pieces' order alone)
__device__ __forceinline__ float4_t fma4(float4_t x, float w, float4_t acc) {
  return (float4_t){__builtin_fmaf(x[0], w, acc[0]), __builtin_fmaf(x[1], w, acc[1]),
                    __builtin_fmaf(x[2], w, acc[2]), __builtin_fmaf(x[3], w, acc[3])};
}


__device__ __forceinline__ void write_record(__amdgpu_buffer_rsrc_t rec, int slot,
                                             const RowState& st, const float (&ltot)[2], int h0,
                                             int col, int kg) {
  float up[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int h = h0 + 16 * ht + col;
    // the head's largest |O|: this lane's 4 dims of every dim tile, then
    // the four lanes of the head's column
    float amax = 0.f;
#pragma unroll
    for (int n = 0; n < kDimTiles; ++n)
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(st.o[ht][n][0]), fabsf(st.o[ht][n][1])),
                               fmaxf(fabsf(st.o[ht][n][2]), fabsf(st.o[ht][n][3]))));
    const float inv = 1.f / ltot[ht];
    up[ht] = record_scale(max_over_kg(amax) * inv);
    const float mul = inv * up[ht];
#pragma unroll
    for (int p = 0; p < kDimTiles / 2; ++p) {
      const float4_t v = st.o[ht][2 * p] * mul;
      const float4_t u = st.o[ht][2 * p + 1] * mul;
      store_rec16(rec, record_x(slot, h, 32 * p + 8 * kg),
                  dims8_of_pair(make_uint2(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])),
                                make_uint2(pack_f16x2(u[0], u[1]), pack_f16x2(u[2], u[3]))));
    }
  }
  // m, l and s are the same in a head's four lanes: lane rows 0 and 1 store
  // m of head tiles 0 and 1 and rows 2 and 3 their l, in one instruction;
  // rows 0 and 1 then store s
  // (selects, not indexing: an index that varies by lane would move the
  // row state out of registers)
  const bool t1 = kg & 1;
  const int h = h0 + 16 * (kg & 1) + col;
  const float m = t1 ? st.m[1] : st.m[0];
  const float l = t1 ? ltot[1] : ltot[0];
  store_rec(rec, kg < 2 ? record_m(slot, h) : record_l(slot, h), kg < 2 ? m : l);
  if (kg < 2) store_rec(rec, record_s(slot, h), 1.f / (t1 ? up[1] : up[0]));
}

// Writes a finished segment (flat tiles seg0 .. seg1 - 1 of row c.b): a
// whole row to `out`, a piece of a cut row as a record, in slot 2 w of
// workgroup w for its range's first segment and 2 w + 1 for its last, for
// the merge kernel.
__device__ __forceinline__ void write_segment(const LatentArgs& a, int b, const RowState& st,
                                              int seg0, int seg1, int row0, int row1, int f0,
                                              __amdgpu_buffer_rsrc_t rec, int h0, int col,
                                              int kg) {
  const float ltot[2] = {sum_over_kg(st.l[0]), sum_over_kg(st.l[1])};
  if (seg0 == row0 && seg1 == row1) {
    const float inv[2] = {1.f / ltot[0], 1.f / ltot[1]};
    store_scaled(a, st.o, inv, b, h0, col, kg);
    return;
  }
  write_record(rec, 2 * (int)blockIdx.x + (seg0 == f0 ? 0 : 1), st, ltot, h0, col, kg);
}

// A finished segment of row c.b. The workgroup holding the row's first tile
// describes the row's pieces: its first slot and their number (workgroups
// floor(x / T) over the row's tiles' cost positions x). A segment in which
// some lane's weights outran the reference is not written: the workgroup
// marks its row in the LDS set `redo` and, after its stream, recomputes this
// same segment exactly and writes it then (the segment's only write). The
// protocol is workgroup-uniform.
//
// The per-wave overflow votes in bcast[1 + wave] carry the segment's tag
// (seg0 + 1, unique within the launch), so they need no reset: between two
// finishes every wave passes the barrier of at least one tile.
//
// The order here (the sums first, the writes last and each one guarded)
// keeps the streaming loop's registers as they are: other arrangements of
// the same steps made the compiler move the tile loads' lane offsets to
// scratch, and the reloads' waits drained the tile prefetch (twice the
// call time).
__device__ __forceinline__ void finish_segment(const LatentArgs& a, const Cursor& c,
                                               const RowState& st, int seg0, int seg1, int f0,
                                               int T, const int* prefix, const int* cprefix,
                                               __amdgpu_buffer_rsrc_t rec, int* bcast,
                                               unsigned* redo, int wave, int h0, int col,
                                               int kg) {
  const float ltot[2] = {sum_over_kg(st.l[0]), sum_over_kg(st.l[1])};
  const int tag = seg0 + 1;
  if (__builtin_amdgcn_ballot_w64(st.overflow) != 0 && (threadIdx.x & 63) == 0)
    bcast[1 + wave] = tag;
  lds_barrier();
  bool flagged = false;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) flagged |= bcast[1 + w] == tag;
  if (flagged && threadIdx.x == 0) redo[c.b >> 5] |= 1u << (c.b & 31);
  const int row0 = prefix[c.b];
  const int row1 = prefix[c.b + 1];
  if (seg0 == row0 && threadIdx.x == 0) {
    const int v1 = (cprefix[c.b] + (row1 - row0) - 1) / T;
    __hip_atomic_store(a.ws_cnt + 2 * c.b, 2 * (int)blockIdx.x + (row0 == f0 ? 0 : 1),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.ws_cnt + 2 * c.b + 1, v1 - (int)blockIdx.x + 1, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  if (seg0 == row0 && seg1 == row1) {
    if (!flagged) {
      const float inv[2] = {1.f / ltot[0], 1.f / ltot[1]};
      store_scaled(a, st.o, inv, c.b, h0, col, kg);
    }
    return;
  }
  if (!flagged)
    write_record(rec, 2 * (int)blockIdx.x + (seg0 == f0 ? 0 : 1), st, ltot, h0, col, kg);
}

// ---- slow path: segments whose scores outran their reference --------------
//
// The slow path's tile loader: tile j of row b into `stage` in the layout
// of the streaming loop (token rows of kRowBytes, pad chunks and tokens past
// the row zero), by plain loads through registers and LDS stores, followed
// by a workgroup barrier.
__device__ __forceinline__ void load_tile_plain(const LatentArgs& a, int b, int j, int L,
                                                lds_char* stage) {
  const int valid = min(kTileTokens, L - j * kTileTokens);
  const int page = a.block_tables[(size_t)b * a.max_blocks + j / (kPageTokens / kTileTokens)];
  const char* base =
      (const char*)a.kv_pool +
      ((size_t)page * kPageTokens + (size_t)(j % (kPageTokens / kTileTokens)) * kTileTokens) *
          kTokenBytes;
  for (int i = threadIdx.x; i < kTileTokens * kRowChunks; i += blockDim.x) {
    const int t = i / kRowChunks;
    const int ch = i - t * kRowChunks;
    typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (ch < kDataChunks && t < valid) v = *(const u32x4_t*)(base + t * kTokenBytes + ch * 16);
    *(lds_u32x4*)(stage + t * kRowBytes + ch * 16) = v;
  }
  __syncthreads();
}

// Exact two-pass recompute of row b's tiles j0 .. j1 - 1 (one segment) by
// its workgroup: the first pass finds every head's maximum score over the
// segment, the second folds the segment with it as the reference (all
// weights <= 1); the result is the segment's exact (O, m, l), written like a
// fast-path segment. Runs after the workgroup's streaming loop, when the
// accumulator registers and the tile stages are free, so its cost is bounded
// by the workgroup's own range.
__device__ __forceinline__ void recompute_segment(const LatentArgs& a, int b, int j0, int j1,
                                                  lds_char* stage, int h0, int col, int kg,
                                                  RowState& st) {
  const int L = a.seq_lens[b];
  bf16x8_t qf[2][kQkSteps];
  load_queries(a, b, h0, col, kg, qf);
  float mx[2] = {-INFINITY, -INFINITY};
  for (int j = j0; j < j1; ++j) {
    load_tile_plain(a, b, j, L, stage);
    float x[2][2][4];
    score_tile(stage, qf, min(kTileTokens, L - j * kTileTokens), a.scale_log2, col, kg, x);
    mx[0] = fmaxf(mx[0], tile_max(x[0]));
    mx[1] = fmaxf(mx[1], tile_max(x[1]));
    __syncthreads();  // everyone is done with the stage
  }
  st.m[0] = mx[0];
  st.m[1] = mx[1];
  for (int j = j0; j < j1; ++j) {
    load_tile_plain(a, b, j, L, stage);
    float x[2][2][4];
    score_tile(stage, qf, min(kTileTokens, L - j * kTileTokens), a.scale_log2, col, kg, x);
    bf16x8_t pf[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const float w = make_weights(x[ht], mx[ht], pf[ht]);
      st.l[ht] = j == j0 ? w : st.l[ht] + w;
    }
    if (j == j0)
      value_tile<true>(stage, pf, st.o, col, kg);
    else
      value_tile<false>(stage, pf, st.o, col, kg);
    __syncthreads();
  }
}

// Recomputes and writes every segment of this workgroup's range [f0, f1)
// whose row is marked in `redo`. Kept out of line: inlined, its second
// accumulator changed the register allocation of the streaming loop (twice
// the spills, and the call took twice as long).
__device__ __forceinline__ void recompute_flagged(const LatentArgs& a,
                                                            const int* prefix,
                                                            const unsigned* redo, int f0, int f1,
                                                            lds_char* stages, int wave, int col,
                                                            int kg) {
  const int B = a.num_seqs;
  const int h0 = wave * kHeadsPerWave;
  const __amdgpu_buffer_rsrc_t rec = range_rsrc(a.ws_rec, 2 * a.grid * kRecordBytes);
  const int b_first = find_sequence(prefix, B, f0);
  const int b_last = find_sequence(prefix, B, f1 - 1);
  for (int b = b_first; b <= b_last; ++b) {
    if (!(redo[b >> 5] & (1u << (b & 31)))) continue;
    const int row0 = prefix[b], row1 = prefix[b + 1];
    const int seg0 = max(f0, row0), seg1 = min(f1, row1);
    RowState st;
    recompute_segment(a, b, seg0 - row0, seg1 - row0, stages, h0, col, kg, st);
    write_segment(a, b, st, seg0, seg1, row0, row1, f0, rec, h0, col, kg);
  }
}

__global__ __launch_bounds__(256) void latent_decode_kernel(LatentArgs a) {
  // dynamic LDS: kStages tile stages, then the rows' tile prefix [B + 1]
  // and cost prefix [B + 1]; static: the bit set of rows whose segment in
  // this range is to be recomputed (a fixed address, so no register holds
  // it through the streaming loop)
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int scan_scratch[kWaves];
  __shared__ int bcast[1 + kWaves];
  __shared__ unsigned redo[kMaxSeqs / 32];
  lds_char* stages = (lds_char*)smem;
  int* prefix = (int*)(smem + kStages * kStageBytes);
  int* cprefix = prefix + a.num_seqs + 1;

  const int B = a.num_seqs;
  if (threadIdx.x < 1 + kWaves) bcast[threadIdx.x] = 0;
  for (int i = threadIdx.x; i < (B + 31) / 32; i += blockDim.x) redo[i] = 0u;
  // a row of L tokens is ceil(L / 32) tiles and costs kFinishSlots more for
  // its finish (L > 0)
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    const int L = a.seq_lens[i];
    const int t = L > 0 ? (L + kTileTokens - 1) / kTileTokens : 0;
    prefix[i] = t;
    cprefix[i] = t > 0 ? t + kFinishSlots : 0;
  }
  __syncthreads();
  scan_counts_in_place(B, prefix, scan_scratch);
  scan_counts_in_place(B, cprefix, scan_scratch);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int h0 = wave * kHeadsPerWave;

  // rows of length 0 are zeros: workgroup g writes rows g, g + grid, ...
  for (int b = blockIdx.x; b < B; b += a.grid) {
    if (prefix[b + 1] != prefix[b]) continue;
    uint4* o = (uint4*)((bf16_t*)a.out + (size_t)b * kHeads * kValue);
    for (int i = threadIdx.x; i < kHeads * kValue / 8; i += 256) o[i] = make_uint4(0, 0, 0, 0);
  }

  // Workgroup w takes the cost range [w T, (w + 1) T): its tiles, with a
  // boundary that falls among a row's finish slots moved to the row's end.
  // With T > kFinishSlots every full range holds a tile, so the pieces of a
  // cut row are consecutive workgroups, the tile at cost position x lies in
  // workgroup floor(x / T), and the finishes spread with the tiles.
  const int total = prefix[B];
  const int ctotal = cprefix[B];
  const int T = max((ctotal + a.grid - 1) / a.grid, a.min_tiles);
  auto boundary = [&](int w) {
    const int x = w * T;
    if (x >= ctotal) return total;
    const int b = find_sequence(cprefix, B, x);
    return prefix[b] + min(x - cprefix[b], prefix[b + 1] - prefix[b]);
  };
  const int f0 = boundary(blockIdx.x);
  const int f1 = boundary(blockIdx.x + 1);
  const __amdgpu_buffer_rsrc_t rec = range_rsrc(a.ws_rec, 2 * a.grid * kRecordBytes);

  if (f0 < f1) {
    Cursor cc = locate_tile(prefix, B, f0);
    Cursor lc = cc;
    load_tile(a, lc, stages, wave, lane);
    // written out: as a loop, the compiler loses track of the stage
    // addresses being uniform
    if (kAhead > 1 && f0 + 1 < f1) {
      next_tile(lc, prefix);
      load_tile(a, lc, stages + kStageBytes, wave, lane);
    }
    if (kAhead > 2 && f0 + 2 < f1) {
      next_tile(lc, prefix);
      load_tile(a, lc, stages + 2 * kStageBytes, wave, lane);
    }
    // tile f of the range sits in stage (f - f0) % kStages; segments: the
    // range's part of one row each, inside which the queries and the row
    // state live
    for (int f = f0; f < f1;) {
      const int seg0 = f;
      const int seg1 = min(f1, prefix[cc.b + 1]);
      const int L = uniform_load(a.seq_lens, cc.b);
      bf16x8_t qf[2][kQkSteps];
      load_queries(a, cc.b, h0, col, kg, qf);
      RowState st;
      st.overflow = false;
      // one tile: wait for it (the tiles issued after it may stay in
      // flight), start the tile kAhead ahead in the stage folded last, fold
      auto tile_step = [&](auto first) {
        const int younger = min(kAhead - 1, f1 - 1 - f);
        if (kAhead > 2 && younger >= 2)
          tile_barrier<kAhead - 1>();
        else if (younger >= 1)
          tile_barrier<1>();
        else
          tile_barrier<0>();
        // the refill's loads go out one per score step
        const bool refill = f + kAhead < f1;
        TileIssue next;
        if (refill) {
          next_tile(lc, prefix);
          next = prepare_tile(a, lc, stages + ((f + kAhead - f0) % kStages) * kStageBytes, wave,
                              lane);
        }
        const int valid = min(kTileTokens, L - (cc.j + f - seg0) * kTileTokens);
        const lds_char* tile = stages + ((f - f0) % kStages) * kStageBytes;
        fold_tile<decltype(first)::value>(tile, qf, st, valid, a.scale_log2, col, kg,
                                          [&](int s) {
                                            if (refill && s < kWaveLoads) next.load(s);
                                          });
        ++f;
      };
      // the first tile is peeled: it consumes the queries, so the
      // compiler's wait for their loads stays out of the tile loop (where
      // it would also drain the tile prefetch)
      tile_step(std::true_type{});
      while (f < seg1) tile_step(std::false_type{});
      finish_segment(a, cc, st, seg0, seg1, f0, T, prefix, cprefix, rec, bcast, redo, wave, h0,
                     col, kg);
      if (f < f1) {  // the next row with tiles
        int b = cc.b + 1;
        while (prefix[b + 1] == prefix[b]) ++b;
        cc.b = __builtin_amdgcn_readfirstlane(b);
        cc.j = 0;
        cc.n = __builtin_amdgcn_readfirstlane(prefix[b + 1] - prefix[b]);
      }
    }
  }

  // the segments this workgroup flagged, recomputed exactly one at a time
  // (every stage load has landed: the last tile waited for all of them)
  lds_barrier();
  if (f0 < f1) recompute_flagged(a, prefix, redo, f0, f1, stages, wave, col, kg);
}

// ---- merging cut rows -----------------------------------------------------------
//
// Workgroup (b, q) writes heads 32 q .. 32 q + 31 of cut row b: out = sum_i
// w_i y_i over the row's pieces in piece order, y_i a piece's scaled
// normalised output as its record holds it (fp16), w_i = s_i l_i
// 2^(m_i - M) / L (log-sum-exp merge, with the piece's inverse scale), one
// fused multiply-add per piece and element. Thread
// t takes head 32 q + t / 8 and 8 chunks of 8 dims (dims 64 j + 8 (t % 8)
// .. + 7, j = 0..7); the record loads of kMergePieces pieces go out
// together. Rows that are whole or empty are left as the decode kernel
// wrote them.
__global__ __launch_bounds__(256) void latent_merge_kernel(LatentArgs a) {
  const int b = blockIdx.x >> 2;
  const int q = blockIdx.x & 3;
  if (uniform_load(a.seq_lens, b) <= 0) return;
  const int n = uniform_load(a.ws_cnt, 2 * b + 1);
  if (n < 2) return;
  const int first_slot = uniform_load(a.ws_cnt, 2 * b);
  const int v0 = first_slot >> 1;
  const int h = 32 * q + (threadIdx.x >> 3);
  const int d0 = 8 * (threadIdx.x & 7);
  const __amdgpu_buffer_rsrc_t rec = range_rsrc(a.ws_rec, 2 * a.grid * kRecordBytes);
  auto slot_of = [&](int i) { return i == 0 ? first_slot : 2 * (v0 + i); };
  auto load_f = [&](int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rec, off, 0, 0));
  };
  // the first kMergePieces records' outputs go out with the (m, l, s) loads
  // below: they do not depend on the merged max
  u32x4_t x[kMergePieces][8];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int k = 0; k < kMergePieces; ++k) {
      if (i0 + k >= n) break;
      const int sl = slot_of(i0 + k);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        x[k][j] = __builtin_amdgcn_raw_buffer_load_b128(rec, record_x(sl, h, 64 * j + d0), 0, 0);
    }
  };
  load_batch(0);
  // merged max and sum of the head, in piece order: every (m, l) in one
  // round trip when the row has at most kFewPieces pieces
  float M = -INFINITY, Lsum = 0.f;
  float mv[kFewPieces], lv[kFewPieces], sv[kFewPieces];
  if (n <= kFewPieces) {
#pragma unroll
    for (int k = 0; k < kFewPieces; ++k) {
      const bool in = k < n;
      mv[k] = in ? load_f(record_m(slot_of(k), h)) : -INFINITY;
      lv[k] = in ? load_f(record_l(slot_of(k), h)) : 0.f;
      sv[k] = in ? load_f(record_s(slot_of(k), h)) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kFewPieces; ++k) M = fmaxf(M, mv[k]);
#pragma unroll
    for (int k = 0; k < kFewPieces; ++k)
      if (k < n) Lsum += lv[k] * fast_exp2(mv[k] - M);
  } else {
    for (int i = 0; i < n; ++i) M = fmaxf(M, load_f(record_m(slot_of(i), h)));
    for (int i = 0; i < n; ++i) {
      const int sl = slot_of(i);
      Lsum += load_f(record_l(sl, h)) * fast_exp2(load_f(record_m(sl, h)) - M);
    }
  }
  const float invL = 1.f / Lsum;
  float4_t acc[8][2];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j][0] = acc[j][1] = zero4();
  for (int i0 = 0; i0 < n; i0 += kMergePieces) {
    if (i0 > 0) load_batch(i0);
    float w[kMergePieces];
#pragma unroll
    for (int k = 0; k < kMergePieces; ++k) {
      if (i0 + k >= n) break;
      const int sl = slot_of(i0 + k);
      if (n <= kFewPieces) {  // weights from the registers (i0 + k < kFewPieces)
        float mk = mv[0], lk = lv[0], sk = sv[0];
#pragma unroll
        for (int u = 1; u < kFewPieces; ++u)
          if (u == i0 + k) mk = mv[u], lk = lv[u], sk = sv[u];
        w[k] = sk * (lk * fast_exp2(mk - M) * invL);
      } else {
        w[k] = load_f(record_s(sl, h)) *
               (load_f(record_l(sl, h)) * fast_exp2(load_f(record_m(sl, h)) - M) * invL);
      }
    }
#pragma unroll
    for (int k = 0; k < kMergePieces; ++k) {
      if (i0 + k >= n) break;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[j][0] = fma4(f16x4_to_f32(x[k][j][0], x[k][j][1]), w[k], acc[j][0]);
        acc[j][1] = fma4(f16x4_to_f32(x[k][j][2], x[k][j][3]), w[k], acc[j][1]);
      }
    }
  }
  bf16_t* out = (bf16_t*)a.out + ((size_t)b * kHeads + h) * kValue + d0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *(uint4*)(out + 64 * j) =
        make_uint4(pack_bf16x2(bf16_rne(acc[j][0][0]), bf16_rne(acc[j][0][1])),
                   pack_bf16x2(bf16_rne(acc[j][0][2]), bf16_rne(acc[j][0][3])),
                   pack_bf16x2(bf16_rne(acc[j][1][0]), bf16_rne(acc[j][1][1])),
                   pack_bf16x2(bf16_rne(acc[j][1][2]), bf16_rne(acc[j][1][3])));
}

}  // namespace

const void* latent_decode_fn() { return (const void*)latent_decode_kernel; }

size_t latent_decode_smem(int num_seqs) {
  return (size_t)kStages * kStageBytes + (size_t)2 * (num_seqs + 1) * sizeof(int);
}

hipError_t launch_latent_decode(const LatentArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(latent_decode_kernel, dim3(a.grid), dim3(256), latent_decode_smem(a.num_seqs),
                     s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(latent_merge_kernel, dim3(4 * a.num_seqs), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pagedkv
