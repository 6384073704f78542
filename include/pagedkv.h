/*
 * pagedkv.h — C ABI of libpagedkv.so: paged decode attention for MI355X
 * (gfx950), plus the two cache-maintenance calls it needs.
 *
 * What the calls compute
 *   The KV cache is one preallocated pool of fixed-size blocks of BS tokens
 *   (BS = block_size, 16 by default);
 *   every sequence has a block table mapping its logical block j to a
 *   physical block, and a length; blocks need not be adjacent
 *   [cs2680 Lecture 10, §10.3 "PagedAttention: the KV cache as virtual
 *   memory"]. The attention call takes a block-table pointer and a length
 *   per sequence, so its arguments keep a fixed shape while sequences grow
 *   ["The inference server" (srikanthmalla.com), the answer on fixed-shape
 *   kernel signatures and bucketed graph capture]. A paged kernel reads each
 *   block's table entry and then gathers the block; the FLOPs and bytes are
 *   those of contiguous attention [§10.3 "Step three"; llm-serving.xyz
 *   "KV-cache systems", paragraph on the price of paging].
 *
 * Layouts (row-major, contiguous; all device memory unless noted)
 *   q, out        [B, Hq, D]                        element type = dtype
 *   k_pool        [NB, Hkv, BS, D]   token-major K blocks
 *   v_pool        [NB, Hkv, D, BS]   dim-major (transposed) V blocks
 *   block_tables  int32 [B, MB]      row b, entry j = physical block of
 *                                    tokens BS*j .. BS*j+BS-1 of sequence b
 *   seq_lens      int32 [B]          tokens attended, newest included;
 *                                    0 = padded row (output is exact zeros)
 *   k_new, v_new  [T, Hkv, D]
 *   slot_mapping  int32 [T]          slot = block * BS + offset; < 0 = skip
 *   block_mapping int32 [n, 2]       (src, dst) physical block pairs
 *   Query head h reads KV head h / (Hq / Hkv).
 *
 * Ownership and execution
 *   The caller allocates and owns every buffer, including the workspace.
 *   The library allocates nothing and keeps no pointer after a call
 *   returns; its only state is a per-device cache of launch geometry (CU
 *   count and kernel occupancy), filled on first use under a lock, so calls
 *   are re-entrant. Each call only enqueues work on `stream` (a
 *   hipStream_t on the current device; NULL = the default stream) and
 *   returns without synchronising. Launch grids depend only on the pa_dims
 *   values and the device, never on device-resident lengths or table
 *   entries.
 *
 * Errors
 *   Arguments the host can see (pointers, dims, sizes) are checked before
 *   anything is launched; a bad one returns PA_ERR_INVALID_ARG or
 *   PA_ERR_UNSUPPORTED and nothing runs. A launch failure reported by the
 *   HIP runtime returns PA_ERR_LAUNCH. Device-resident values are NOT
 *   checked (that would need a synchronisation); the caller guarantees:
 *     0 <= seq_lens[b] <= MB * BS;
 *     0 <= block_tables[b][j] < NB for every j < ceil(seq_lens[b] / BS);
 *     write slots are distinct and < NB * BS;
 *     copy pairs name blocks < NB, destinations are distinct and no
 *     destination is also a source in the same call.
 *   Violations give undefined results (out-of-range reads or racing
 *   writes); the Python binding offers an opt-in host validator.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,  /* null pointer, bad dims, workspace too small */
  PA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (dtype, head dim, G) */
  PA_ERR_LAUNCH = 3        /* the HIP runtime rejected a kernel launch */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Decode kernel selection. AUTO picks the matrix-core kernel for bf16 and
 * the vector-ALU kernel for f32. */
typedef enum { PA_KERNEL_AUTO = 0, PA_KERNEL_VALU = 1, PA_KERNEL_MFMA = 2 } pa_kernel;

/* partition_tokens value for the library's choice, made from the dims alone
 * (so a captured launch stays valid for any lengths): with the matrix-core
 * kernel and 16-token blocks, batches of at most 8 rows take fixed
 * partitions (every (row, partition, KV head) its own workgroup, merged in
 * the same kernel by the last partition of a row and KV head to finish):
 * 256 tokens for one row, 192 for two, 320 for three or four and 384 for
 * five to eight; larger batches take the balanced split. The vector-ALU
 * kernel takes 512-token partitions. */
#define PA_PARTITION_AUTO (-1)

/* Host-side dimensions; all fields are fixed for a given captured shape. */
typedef struct {
  int32_t num_seqs;           /* B   (1 .. 4096) */
  int32_t num_q_heads;        /* Hq  (multiple of Hkv, Hq / Hkv <= 16) */
  int32_t num_kv_heads;       /* Hkv (>= 1) */
  int32_t head_dim;           /* D   (64 or 128) */
  int32_t block_size;         /* tokens per block: 16; 8, 32, 64, 128 or 256
                                 are taken by the balanced split only */
  int32_t max_blocks_per_seq; /* MB: row stride of block_tables (>= 1) */
  int32_t num_blocks;         /* NB: pool capacity in blocks (>= 1) */
  int32_t partition_tokens;   /* split-K partition length: a multiple of 16;
                                 0 for the balanced split (matrix-core kernel)
                                 or one partition per sequence (vector-ALU
                                 kernel); PA_PARTITION_AUTO for the library's
                                 choice by dims (below) */
  int32_t dtype;              /* pa_dtype of q, pools, k_new/v_new and out */
  int32_t kernel;             /* pa_kernel */
} pa_dims;

/* Bytes of device workspace pa_decode needs for these dims.
 *   Fixed split (partition_tokens > 0, or the vector-ALU kernel): 0 when
 *   every sequence fits one partition, else int32 partition counters for
 *   every (sequence, KV head), then fp32 partial results (max, sum,
 *   unnormalised output) of every (sequence, query head, partition).
 *   Balanced split (matrix-core kernel, partition_tokens == 0): int32 piece
 *   counters for every (sequence, KV head), then fp32 partials for two
 *   pieces per wave of the decode grid (at most 1024 waves).
 * The workspace must be zero-filled before its first use; every pa_decode
 * call leaves its counters at zero, so it can be reused without clearing by
 * calls with the same dims. A call with other dims (another batch size, KV
 * head count, partition size or split) may find its counters where the
 * previous layout kept partials: zero-fill the workspace again before it.
 * Calls that may overlap in time need separate workspaces. Returns 0 for
 * invalid dims as well; pa_decode reports those. */
size_t pa_decode_workspace_bytes(const pa_dims* dims);

/* Paged decode attention: for every sequence b and query head h,
 *   out[b,h,:] = sum_t softmax_t(scale * <q[b,h,:], K_b[t]>) V_b[t]
 * over t < seq_lens[b], with K_b/V_b gathered through block_tables[b]
 * (naive softmax over the whole row; computed with an online softmax per
 * piece of the sequence and a log-sum-exp merge across pieces, fp32
 * accumulation). Pieces are fixed partitions of partition_tokens tokens
 * (with the matrix-core kernel the last partition of a sequence to finish
 * merges them in the same kernel; the vector-ALU kernel merges in a second
 * kernel), or, with partition_tokens == 0 and the matrix-core kernel, the
 * balanced split: every wave of a persistent grid streams an equal share
 * of all blocks and the last wave to finish a cut sequence merges its
 * pieces.
 * Results do not depend on timing: pieces merge in a fixed order.
 * Rows with seq_lens[b] == 0 get zeros. Slots at or past seq_lens[b] never
 * reach the result (they are masked, so they may hold anything, NaN
 * included), and table entries at or past ceil(seq_lens[b] / BS) are never
 * read. bf16 output is rounded to nearest even.
 * `workspace` may be NULL when pa_decode_workspace_bytes() is 0. */
pa_status pa_decode(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    float scale, void* out, const pa_dims* dims,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Decode attention over an unpaged KV cache: the same computation as
 * pa_decode, but each (sequence, KV head) owns one contiguous run of
 * Lmax = 16 * max_blocks_per_seq token slots, so token t of sequence b sits
 * at base + stride * t and no table is read. This is the contiguous cache
 * that paging is priced against: a paged kernel reads each block's table
 * entry and then gathers the block, a contiguous one computes the address
 * [llm-serving.xyz "KV-cache systems", paragraph on the price of paging;
 * cs2680 Lecture 10, Exercise 3(a)].
 *   k_cache  [B, Hkv, Lmax, D]           token-major
 *   v_cache  [B, Hkv, Lmax / 16, D, 16]  a dim-major 16-token tile per 16
 *                                        slots (the paged V tile's layout)
 * Slots at or past seq_lens[b] are never used (they may hold anything). The
 * balanced split of the matrix-core kernel only: dims->dtype bf16,
 * block_size 16, partition_tokens 0 or PA_PARTITION_AUTO, kernel AUTO or MFMA (else
 * PA_ERR_UNSUPPORTED); num_blocks is not used. Workspace as pa_decode's for
 * the same dims (pa_decode_workspace_bytes). Results are bit-identical to
 * pa_decode's on the same values: the work split and the arithmetic are
 * those of the paged kernel. */
pa_status pa_decode_contiguous(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* seq_lens, float scale, void* out,
                               const pa_dims* dims, void* workspace, size_t workspace_bytes,
                               void* stream);

/* pa_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, serving loops and harnesses that
 * forbid allocation). Same arguments, kernels and results as pa_decode,
 * bit for bit; the workspace is instead a device array of
 * PA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends. The call allocates nothing. Dims whose
 * pa_decode_workspace_bytes() exceeds PA_NOALLOC_SCRATCH_BYTES return
 * PA_ERR_UNSUPPORTED before anything runs (the balanced split at the
 * supported head groups needs at most about 17 MiB; the fixed split's
 * partials grow with B * Hq * partitions). When the dims need a workspace,
 * a zero fill of its counters (the balanced split's piece counters or the
 * fixed split's partition counters) runs on `stream` before the decode.
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (other streams, other threads) race and give undefined
 * results. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pa_status pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            float scale, void* out, const pa_dims* dims, void* stream);

/* One decode step in one call: the KV append of every row's new token,
 * then paged decode attention over the updated cache. Equivalent to
 *   pa_write_kv(k_new, v_new, slot_mapping, num_seqs, ...);
 *   pa_decode(q, k_pool, v_pool, block_tables, seq_lens, ...);
 * for the usual decode step, where row b appends exactly one token, the
 * newest one it attends to: k_new and v_new are [B, Hkv, D] and
 * slot_mapping[b] is either negative (row b appends nothing) or the slot of
 * position seq_lens[b] - 1 of row b's table, i.e.
 *   block_tables[b][(seq_lens[b] - 1) / BS] * BS + (seq_lens[b] - 1) % BS.
 * A decode step writes the new token's K/V into its slot and then attends
 * over the sequence including it [cs2680 Lecture 10, §10.3 and its notes on
 * growing a sequence by one token]. With the balanced split (matrix-core
 * kernel, partition_tokens == 0) the append runs inside the decode kernel
 * (one launch); otherwise the append kernel runs first on the same stream.
 * Any other slot_mapping gives undefined results. Arguments, workspace and
 * errors as pa_decode. */
pa_status pa_decode_append(const void* q, const void* k_new, const void* v_new,
                           const int32_t* slot_mapping, void* k_pool, void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           float scale, void* out, const pa_dims* dims,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Chunked-prefill paged attention. Sequence s owns the query rows
 * query_start[s] .. query_start[s+1]-1 of q ([T, Hq, D], T =
 * num_query_tokens = query_start[num_seqs]): its newest
 * n_s = query_start[s+1] - query_start[s] tokens, at positions
 * seq_lens[s] - n_s .. seq_lens[s] - 1, whose K/V are already in the pools
 * (written by pa_write_kv). The query token at position p attends to the
 * sequence's tokens 0 .. p:
 *   out[r,h,:] = sum_{t<=p} softmax_t(scale * <q[r,h,:], K_s[t]>) V_s[t]
 * with K_s/V_s gathered through block_tables[s] and KV head h / (Hq / Hkv).
 * A long prompt is prefilled in pieces of a few hundred tokens that share a
 * step with decode rows; each piece sees the earlier pieces and itself
 * ["The inference server" (srikanthmalla.com), the answer on prefill and
 * decode competing for the device]. A sequence with n_s = 1 is a decode
 * row, n_s = 0 a row with nothing to do. Matrix-core kernel: bf16, D = 64
 * or 128, block_size >= 16 (PA_ERR_UNSUPPORTED otherwise); no workspace.
 * scale must be finite and positive (PA_ERR_INVALID_ARG otherwise). The
 * caller guarantees 0 = query_start[0] <= ... <= query_start[num_seqs]
 * = num_query_tokens and n_s <= seq_lens[s]; other values give undefined
 * results. out[r] is written for every query row r; bf16 rounding is to
 * nearest even. dims->partition_tokens and dims->kernel are ignored. */
pa_status pa_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     const int32_t* query_start, int32_t num_query_tokens, float scale,
                     void* out, const pa_dims* dims, void* stream);

/* KV append: for t < num_tokens with s = slot_mapping[t] >= 0,
 *   k_pool[s / BS, h, s % BS, :] = k_new[t, h, :]
 *   v_pool[s / BS, h, :, s % BS] = v_new[t, h, :]   for every KV head h.
 * A bit copy: no value is converted. Growth takes a new block only when a
 * sequence's last block is full [cs2680 Lecture 10, §10.3 and its notes on
 * growing a sequence by one token]. Uses num_kv_heads, head_dim,
 * block_size, num_blocks and dtype from `dims`. num_tokens == 0 is a no-op
 * (pointers may then be NULL). */
pa_status pa_write_kv(const void* k_new, const void* v_new,
                      const int32_t* slot_mapping, int32_t num_tokens,
                      void* k_pool, void* v_pool, const pa_dims* dims,
                      void* stream);

/* Copy-on-write block copy: for each pair (src, dst) in block_mapping,
 * the whole K block and the whole V block of dst (every KV head) become
 * bit-identical to those of src [cs2680 Lecture 10, §10.4; llm-serving.xyz
 * "KV-cache systems", copy-on-write paragraph]. Uses num_kv_heads,
 * head_dim, block_size, num_blocks and dtype from `dims`.
 * num_pairs == 0 is a no-op. */
pa_status pa_copy_blocks(void* k_pool, void* v_pool,
                         const int32_t* block_mapping, int32_t num_pairs,
                         const pa_dims* dims, void* stream);

/* ---- Latent (MLA-style) decode ------------------------------------------
 *
 * Multi-head latent attention caches, per token, one latent vector of
 * latent_dim = 576 elements: a 512-element compressed KV and a 64-element
 * positional key, shared by every query head; keys and values are never
 * materialised. With the up-projections absorbed into the queries and the
 * output projection, decode is multi-query attention with head dim 576
 * whose values are the first 512 latent elements [llm-serving.xyz
 * "KV-cache systems", MLA section: the cached latent and its decoupled
 * positional key, the two computation modes (the absorbed one here), the
 * 64-token page of the dedicated decode kernels].
 *
 * Layouts (row-major, contiguous, device memory)
 *   q             [B, H, 576]       absorbed queries (compressed part, then
 *                                   positional part), dtype
 *   kv_pool       [NB, BS, 576]     latent blocks, token-major
 *   block_tables  int32 [B, MB]     as for pa_decode, entry j = block of
 *                                   tokens BS*j .. BS*j+BS-1
 *   seq_lens      int32 [B]         tokens attended; 0 = padded row (zeros)
 *   out           [B, H, 512]
 *   kv_new        [T, 576], slot_mapping int32 [T] (slot = block*BS + offset)
 * Ownership, stream semantics and device-value guarantees as for the calls
 * above (table entries below NB for the blocks a row uses, lengths at most
 * MB * BS). */
typedef struct {
  int32_t num_seqs;           /* B   (1 .. 4096) */
  int32_t num_heads;          /* H   query heads sharing each latent: 128 */
  int32_t latent_dim;         /* elements per cached latent: 576 */
  int32_t value_dim;          /* leading latent elements that form the values: 512 */
  int32_t block_size;         /* BS  tokens per block: 64 */
  int32_t max_blocks_per_seq; /* MB: row stride of block_tables (1 .. 2^20) */
  int32_t num_blocks;         /* NB: pool capacity in blocks (>= 1) */
  int32_t dtype;              /* pa_dtype; PA_BF16 */
} pa_latent_dims;

/* Bytes of device workspace pa_latent_decode needs: per row a description
 * of its pieces, then partial
 * records (each piece's output normalised by its own sum and scaled per
 * head by a power of two, as fp16, then its max, sum and inverse scale as
 * fp32, for 128 heads) for two pieces per workgroup of a grid
 * of at most 256. Every call writes what it reads back (no zero-fill
 * needed). Calls that may overlap in time need separate workspaces.
 * Returns 0 for invalid dims (pa_latent_decode reports those). */
size_t pa_latent_workspace_bytes(const pa_latent_dims* dims);

/* Latent decode: for every row b and head h,
 *   out[b,h,:] = sum_t softmax_t(scale * <q[b,h,:], c_b[t]>) c_b[t][0:512]
 * over t < seq_lens[b], with the latents c_b gathered through
 * block_tables[b] (fp32 accumulation; weights enter the value product as
 * bf16). A persistent grid streams equal shares of all 32-token tiles
 * (each row's finish counted as a few tiles); the pieces of a row split
 * across workgroups are merged by a second kernel on the same stream
 * (log-sum-exp over the pieces' fp32 normalised outputs, in piece order),
 * so results do not depend on timing.
 * A piece of a row in which some weight 2^(s - m) reaches 2^32, m being the
 * piece's first-tile maximum of the log2-scaled scores s, is recomputed
 * exactly (two passes, with the piece's true maximum) by its workgroup after
 * that workgroup's share of the stream, and written then instead of the
 * overflowed result. Slots at or
 * past seq_lens[b] never reach the result; bf16 output is rounded to
 * nearest even. PA_ERR_UNSUPPORTED for any shape but H = 128, 576 / 512,
 * BS = 64, bf16. */
pa_status pa_latent_decode(const void* q, const void* kv_pool, const int32_t* block_tables,
                           const int32_t* seq_lens, float scale, void* out,
                           const pa_latent_dims* dims, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Latent append: kv_pool row slot_mapping[t] (block s / BS, offset s % BS)
 * becomes kv_new[t] for every t < num_tokens with slot_mapping[t] >= 0; a
 * bit copy. The cache grows by one latent per generated token [same MLA
 * section]. num_tokens == 0 is a no-op. */
pa_status pa_latent_write(const void* kv_new, const int32_t* slot_mapping, int32_t num_tokens,
                          void* kv_pool, const pa_latent_dims* dims, void* stream);

/* Static description of a status code. */
const char* pa_status_string(pa_status status);

/* Library version string, e.g. "pagedkv 0.1 gfx950". */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
