"""Oracle: paged decode attention, KV append and block copy, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages fix it
--------------------------------------------
* KV lives in fixed-size blocks of 16 tokens held in one preallocated pool;
  each sequence owns a block table that maps its logical block index to a
  physical block, and blocks need not be neighbours
  [cs2680 Lecture 10, §10.3 "PagedAttention: the KV cache as virtual memory";
  the 16-token default is in the same section's block-size table and in
  "The inference server" (srikanthmalla.com), PagedAttention answer].
* A paged kernel reads, for every block, the table entry and then gathers
  that block; the FLOPs and bytes are those of contiguous attention
  [§10.3 "Step three"; llm-serving.xyz "KV-cache systems", paging paragraph
  on block-table cost].
* The attention is GQA: several query heads share one KV head, n_kv = 8 for
  the shapes used here [llm-serving.xyz "KV-cache systems", bytes-per-token
  equation].
* The kernel takes a block-table pointer and a length per sequence
  ["The inference server", fixed-shape kernel signature answer].

Readings where the pages are silent (each also listed in the design notes):
* The attention formula is standard scaled dot-product softmax attention of
  one query token over the sequence's L cached tokens, scale given by the
  caller; query head h reads KV head floor(h / G) with G = Hq / Hkv.
* ``seq_lens[b]`` counts every cached token including the newest one; a
  row with length 0 is a padded row whose output is exactly zero.
* Pool layout (the library's interface; the pages leave it open):
      k_pool[block, kv_head, slot, d]     token-major K blocks
      v_pool[block, kv_head, d, slot]     dim-major V blocks (blocks of up
                                          to 16 tokens)
      v_pool[block, kv_head, slot // 16, d, slot % 16]
                                          blocks longer than 16 tokens: a
                                          dim-major V tile per 16 slots
  A token at position t of sequence b lives in block
  ``block_tables[b, t // block_size]`` at slot ``t % block_size``
  (block_size = 16 unless stated).
* Inputs are exact: bf16 values are widened to float64 without rounding.

The arithmetic is done in float64 with a naive (two-pass) softmax over the
whole row; nothing is blocked, fused or reordered.
"""

from __future__ import annotations

import math

import numpy as np

BLOCK_SIZE = 16


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to float64 exactly.

    ``dtype`` names the storage format: "f32" arrays are float32; "bf16"
    arrays hold the raw 16-bit patterns (uint16), which are the upper half of
    the float32 with the same value, so widening is a 16-bit left shift.
    """
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a).astype(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (round to nearest, ties to even).

    Written from the format's definition: bfloat16 keeps the sign, the
    8 exponent bits and the top 7 fraction bits of an IEEE binary32. The
    value is first rounded to binary32 (numpy, RNE), then the low 16 bits
    are rounded away with ties to even. NaN maps to a quiet NaN.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    rounded = np.where(nan, np.uint16(0x7FC0), rounded)
    return rounded.astype(np.uint16)


# --------------------------------------------------------------------------
# Table walk and attention
# --------------------------------------------------------------------------

def v_at(v_pool, phys, slot):
    """V values [.., Hkv, D] of slot(s) ``slot`` of block(s) ``phys``, in
    either V layout (4-D: [NB, Hkv, D, slot]; 5-D: [NB, Hkv, slot // 16, D,
    slot % 16])."""
    if v_pool.ndim == 5:
        return v_pool[phys, :, slot // 16, :, slot % 16]
    return v_pool[phys, :, :, slot]


def gather_sequence(k_pool, v_pool, table_row, seq_len, dtype,
                    block_size=BLOCK_SIZE):
    """Materialise one sequence's contiguous K and V by walking its table.

    Returns ``K, V`` of shape [Hkv, L, D] in float64, where token t comes
    from physical block ``table_row[t // block_size]`` at slot
    ``t % block_size`` [cs2680 Lecture 10, §10.3: logical block index ->
    physical block]. Table entries at or beyond ceil(L / block_size) and
    slots at or beyond L are never touched.
    """
    L = int(seq_len)
    Hkv = k_pool.shape[1]
    D = k_pool.shape[3]
    if L == 0:
        z = np.zeros((Hkv, 0, D))
        return z, z.copy()
    t = np.arange(L)
    phys = np.asarray(table_row)[t // block_size].astype(np.int64)
    slot = t % block_size
    # k_pool[phys, :, slot, :] -> [L, Hkv, D]; v_pool[phys, :, :, slot] -> [L, Hkv, D]
    k = k_pool[phys, :, slot, :]
    v = v_at(v_pool, phys, slot)
    K = as_f64(k, dtype).transpose(1, 0, 2)
    V = as_f64(v, dtype).transpose(1, 0, 2)
    return K, V


def decode_contiguous(q_b, K, V, scale):
    """Attention of one sequence's query heads over contiguous K/V.

    q_b: [Hq, D] float64; K, V: [Hkv, L, D] float64. Query head h uses KV
    head h // (Hq // Hkv). For each head: s = scale * K q, p = exp(s - max s),
    out = (p V) / sum p. L == 0 gives zeros. This is the contiguous
    (base + stride * t) attention that paging leaves unchanged
    [cs2680 Lecture 10, §10.3 "Step three"].
    """
    Hq, D = q_b.shape
    Hkv, L, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D))
    if L == 0:
        return out
    for kv in range(Hkv):
        qg = q_b[kv * G:(kv + 1) * G]              # [G, D]
        s = scale * (qg @ K[kv].T)                 # [G, L]
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        out[kv * G:(kv + 1) * G] = (p @ V[kv]) / p.sum(axis=1, keepdims=True)
    return out


def paged_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, dtype,
                 rows=None, block_size=BLOCK_SIZE):
    """Paged decode attention for a batch, in float64.

    q [B, Hq, D], k_pool [NB, Hkv, bs, D], v_pool in either V layout
    (storage format ``dtype``), block_tables int [B, MB], seq_lens int [B],
    bs = ``block_size``. For each
    selected row b the sequence is gathered through its table and attended
    contiguously; rows with length 0 are zero. ``rows`` selects a subset of
    sequences (for sampled checks at full size); the result then has one
    entry per selected row, in the given order.
    """
    B, Hq, D = q.shape
    rows = range(B) if rows is None else list(rows)
    out = np.zeros((len(rows), Hq, D))
    for i, b in enumerate(rows):
        L = int(seq_lens[b])
        if L == 0:
            continue
        K, V = gather_sequence(k_pool, v_pool, block_tables[b], L, dtype,
                               block_size)
        out[i] = decode_contiguous(as_f64(q[b], dtype), K, V, scale)
    return out


def contiguous_cache_decode(q, k_cache, v_cache, seq_lens, scale, dtype, rows=None):
    """Decode attention over an unpaged KV cache, in float64.

    Each (sequence, KV head) owns one contiguous run of capacity Lmax
    tokens: k_cache [B, Hkv, Lmax, D] holds token t at [b, h, t];
    v_cache [B, Hkv, Lmax // 16, D, 16] holds it at [b, h, t // 16, :, t % 16]
    (the V layout of a paged 16-token tile, tiles laid end to end). Token t's
    address is then base + stride * t with no table to read, the
    contiguous cache that paging is measured against [llm-serving.xyz
    "KV-cache systems", paragraph on the price of paging; cs2680 Lecture 10,
    Exercise 3(a)]. Attention is the same as ``paged_decode``'s over the first
    seq_lens[b] tokens; positions at or past seq_lens[b] are never read.
    """
    B, Hq, D = q.shape
    rows = range(B) if rows is None else list(rows)
    out = np.zeros((len(rows), Hq, D))
    for i, b in enumerate(rows):
        L = int(seq_lens[b])
        if L == 0:
            continue
        t = np.arange(L)
        K = as_f64(k_cache[b, :, :L, :], dtype)                        # [Hkv, L, D]
        V = as_f64(v_cache[b, :, t // 16, :, t % 16], dtype).transpose(1, 0, 2)
        out[i] = decode_contiguous(as_f64(q[b], dtype), K, V, scale)
    return out


def paged_prefill(q, k_pool, v_pool, block_tables, seq_lens, query_start, scale,
                  dtype, block_size=BLOCK_SIZE, seqs=None):
    """Chunked-prefill paged attention for a batch, in float64.

    q [T, Hq, D] holds the query tokens of every sequence back to back:
    sequence s owns rows query_start[s] .. query_start[s + 1] - 1, its
    newest n_s tokens, at positions L_s - n_s .. L_s - 1 (L_s = seq_lens[s]
    counts them, and their K/V are already in the pool). The query token at
    position p attends to the sequence's tokens 0 .. p: a chunk of a long
    prompt sees the earlier chunks and, causally, itself, and a sequence
    with one query token is a decode row ["The inference server"
    (srikanthmalla.com), the answer on prefill and decode competing for the
    device: chunked prefill runs pieces of a prompt in the same step as
    decode rows; cs2680 Lecture 10, §10.3 for the table walk]. ``seqs``
    restricts the work to some sequences (other rows stay zero).
    """
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D))
    seqs = range(len(seq_lens)) if seqs is None else seqs
    for s in seqs:
        r0, r1 = int(query_start[s]), int(query_start[s + 1])
        n, L = r1 - r0, int(seq_lens[s])
        if n == 0:
            continue
        if n > L:
            raise ValueError(f"sequence {s}: {n} query tokens but length {L}")
        K, V = gather_sequence(k_pool, v_pool, block_tables[s], L, dtype, block_size)
        for i in range(n):
            p = L - n + i
            out[r0 + i] = decode_contiguous(as_f64(q[r0 + i], dtype), K[:, :p + 1],
                                            V[:, :p + 1], scale)
    return out


def latent_decode(q, kv_pool, block_tables, seq_lens, scale, dtype, value_dim=512,
                  rows=None):
    """Latent (MLA-style) paged decode, in float64.

    Every cached token holds one latent vector of C elements (kv_pool
    [NB, block, C]: a 512-element compressed KV plus a 64-element positional
    key, C = 576); all H query heads of a row attend to that one latent, so
    this is multi-query attention with head dim C. Each head's (absorbed)
    query q[b, h] (C elements) scores against every cached latent,
    s_t = scale * <q[b, h], c_t>, and the head's output is the softmax-
    weighted sum of the first ``value_dim`` latent elements,
    out[b, h] = sum_t softmax(s)_t c_t[:value_dim]; the up-projection back
    to the model width is outside attention [llm-serving.xyz "KV-cache
    systems", the MLA section: cached latent and decoupled RoPE key (576
    elements per token), the absorbed computation mode, and its reading as
    MQA with head dim 576; block size from the kernel's page size].
    q [B, H, C]; returns [B or len(rows), H, value_dim]. Rows of length 0
    are zero; slots past a row's length are never read.
    """
    B, H, C = q.shape
    bs = kv_pool.shape[1]
    rows = range(B) if rows is None else list(rows)
    out = np.zeros((len(rows), H, value_dim))
    for i, b in enumerate(rows):
        L = int(seq_lens[b])
        if L == 0:
            continue
        t = np.arange(L)
        phys = np.asarray(block_tables[b])[t // bs].astype(np.int64)
        lat = as_f64(kv_pool[phys, t % bs, :], dtype)   # [L, C]
        qb = as_f64(q[b], dtype)                       # [H, C]
        sc = scale * (qb @ lat.T)                      # [H, L]
        m = sc.max(axis=1, keepdims=True)
        p = np.exp(sc - m)
        out[i] = (p @ lat[:, :value_dim]) / p.sum(axis=1, keepdims=True)
    return out


def brute_force_decode(q, k_pool, v_pool, block_tables, seq_lens, scale,
                       dtype, block_size=BLOCK_SIZE):
    """Same quantity as ``paged_decode`` with scalar Python loops.

    For tiny inputs only. Uses its own element-wise table walk and
    ``math.exp``; shares nothing with ``paged_decode`` except the exact
    widening of stored values.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    qf = as_f64(q, dtype)
    kf = as_f64(k_pool, dtype)
    vf = as_f64(v_pool, dtype)
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hq):
            kv = h // G
            scores = []
            for t in range(L):
                blk = int(block_tables[b][t // block_size])
                slot = t % block_size
                acc = 0.0
                for d in range(D):
                    acc += float(qf[b, h, d]) * float(kf[blk, kv, slot, d])
                scores.append(scale * acc)
            if L == 0:
                continue
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for d in range(D):
                num = 0.0
                for t in range(L):
                    blk = int(block_tables[b][t // block_size])
                    slot = t % block_size
                    if vf.ndim == 5:
                        num += w[t] * float(vf[blk, kv, slot // 16, d, slot % 16])
                    else:
                        num += w[t] * float(vf[blk, kv, d, slot])
                out[b][h][d] = num / tot
    return np.array(out, dtype=np.float64).reshape(B, Hq, D)


# --------------------------------------------------------------------------
# Cache maintenance
# --------------------------------------------------------------------------

def write_kv(k_pool, v_pool, k_new, v_new, slot_mapping,
             block_size=BLOCK_SIZE):
    """Append new tokens' K/V into their slots; returns updated copies.

    Token i goes to slot s = slot_mapping[i]: block s // 16, position
    s % 16, for every KV head; a negative slot means "skip". A sequence grows
    into the next position of its last block and takes a new block only when
    the last one is full [cs2680 Lecture 10, §10.3 and its instructor notes
    on growing a sequence by one token]. Pure data movement: the stored bits
    are copied unchanged.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        blk, pos = divmod(int(s), block_size)
        k_out[blk, :, pos, :] = k_new[i]
        if v_out.ndim == 5:
            v_out[blk, :, pos // 16, :, pos % 16] = v_new[i]
        else:
            v_out[blk, :, :, pos] = v_new[i]
    return k_out, v_out


def copy_blocks(k_pool, v_pool, block_mapping):
    """Copy-on-write block copy; returns updated copies.

    For each (src, dst) pair the whole K block and the whole V block of dst
    become bit-identical to src, for every KV head [cs2680 Lecture 10, §10.4
    (a divergent write gets a new block); llm-serving.xyz "KV-cache systems",
    copy-on-write paragraph].
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for src, dst in np.asarray(block_mapping).reshape(-1, 2).tolist():
        k_out[dst] = k_pool[src]
        v_out[dst] = v_pool[src]
    return k_out, v_out
