"""Seeded synthetic inputs for paged decode attention.

This module produces inputs and nothing else: lengths, physical block
placement, block tables, slot numbers, block-copy pairs and N(0, 1) values,
with poison (NaN) in every pool position that a correct kernel must never
read. It holds none of the attention arithmetic, and both the HIP path and
the oracle consume what it returns.

Seeds: lengths and placements come from ``numpy.random.default_rng``, values
from a CPU ``torch.Generator`` (the 32-layer step draws its per-layer values
on the device), all derived from 55_000 + configuration number.

Layouts (the library's interface):
  q, out            [B, Hq, D]
  k_pool            [NB, Hkv, 16, D]   token-major K tiles
  v_pool            [NB, Hkv, D, 16]   dim-major V tiles
  block_tables      int32 [B, MB]      unused entries name a poisoned block
  seq_lens          int32 [B]          0 marks a padded row
  k_new, v_new      [T, Hkv, D];  slot_mapping int32 [T] (negative = skip)
  block_mapping     int32 [n, 2]       (src, dst)

The five workloads follow the pages' shapes: an 8B-like layer (32 query /
8 KV heads, head dim 128) and a 70B-like layer (64 / 8), 16-token blocks,
lengths up to 8K, a 256-page pool with a 2,048-token shared prefix and a
257-token suffix per request [cs2680 Lecture 10, §10.3; llm-serving.xyz
"KV-cache systems"; inferenceinterviews.com "Reserve the page a request has
not written yet"].
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from paged_kv_cache_55_amd.block_manager import AdmissionLedger, BlockManager

SEED_BASE = 55_000
BLOCK = 16
BF16_NAN_BITS = 0x7FC0

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Case:
    """One batch of paged-decode inputs (CPU or device tensors)."""

    name: str
    dtype: str
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    scale: float
    partition_tokens: int = 512
    poison_block: int = -1
    k_new: Optional[torch.Tensor] = None
    v_new: Optional[torch.Tensor] = None
    slot_mapping: Optional[torch.Tensor] = None
    block_mapping: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)
    query_start: Optional[torch.Tensor] = None  # chunked prefill: int32 [S + 1]

    # shapes
    @property
    def num_seqs(self):
        return self.q.shape[0]

    @property
    def num_q_heads(self):
        return self.q.shape[1]

    @property
    def num_kv_heads(self):
        return self.k_pool.shape[1]

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def num_blocks(self):
        return self.k_pool.shape[0]

    @property
    def max_blocks_per_seq(self):
        return self.block_tables.shape[1]

    @property
    def block_size(self):
        return self.k_pool.shape[2]

    def kv_bytes(self) -> int:
        """Bytes of K and V the decode must read: valid tokens only."""
        elem = 4 if self.dtype == "f32" else 2
        total = int(self.seq_lens.to(torch.int64).sum())
        return total * self.num_kv_heads * self.head_dim * 2 * elem

    def to(self, device) -> "Case":
        def mv(t):
            return None if t is None else t.to(device)
        return Case(self.name, self.dtype, mv(self.q), mv(self.k_pool),
                    mv(self.v_pool), mv(self.block_tables), mv(self.seq_lens),
                    self.scale, self.partition_tokens, self.poison_block,
                    mv(self.k_new), mv(self.v_new), mv(self.slot_mapping),
                    mv(self.block_mapping), dict(self.meta), mv(self.query_start))


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host array of a tensor: bf16 as raw uint16 bits, others as they are."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------

def _randn(gen: torch.Generator, shape, dtype: str) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(TORCH_DTYPE[dtype])


def _poison_value(dtype: str):
    return float("nan")


def v_pool_shape(num_blocks, num_kv_heads, head_dim, block_size):
    """V pool layout: [NB, Hkv, D, bs] (dim-major blocks) up to 16 tokens per
    block; longer blocks are a run of 16-token dim-major tiles,
    [NB, Hkv, bs // 16, D, 16]."""
    if block_size <= BLOCK:
        return (num_blocks, num_kv_heads, head_dim, block_size)
    return (num_blocks, num_kv_heads, block_size // BLOCK, head_dim, BLOCK)


def set_v_slot(v_pool, blk, pos, value):
    """v_pool[blk, :, slot pos, :] = value in either V layout."""
    if v_pool.dim() == 5:
        v_pool[blk, :, pos // BLOCK, :, pos % BLOCK] = value
    else:
        v_pool[blk, :, :, pos] = value


def _poison_tails(k_pool, v_pool, tables, lens, block_size=BLOCK):
    """NaN in every slot at or past L inside a sequence's last block."""
    for b, L in enumerate(lens.tolist()):
        if L % block_size == 0:
            continue
        blk = int(tables[b, L // block_size])
        k_pool[blk, :, L % block_size:, :] = float("nan")
        for pos in range(L % block_size, block_size):
            set_v_slot(v_pool, blk, pos, float("nan"))


def place_blocks(lens, rng, pool_blocks=None, mb=None, consecutive=False, block_size=BLOCK):
    """Assign physical blocks to every logical block of every sequence.

    Returns (tables int32 [B, MB], num_blocks, poison_block). Physical ids
    come from a seeded permutation of the pool (``consecutive``: the
    identity, so every sequence's blocks are physically contiguous and the
    sequences lie back to back); logical blocks take consecutive entries of
    it in (sequence, block) order. One block outside all tables is the
    poison block that unused table entries name.
    """
    lens = np.asarray(lens, dtype=np.int64)
    nblk = [math.ceil(int(L) / block_size) for L in lens]
    total = int(sum(nblk))
    nb = pool_blocks if pool_blocks is not None else total + 1
    if nb < total + 1:
        raise ValueError("pool too small for the tables plus a poison block")
    perm = rng.permutation(nb)
    if consecutive:
        perm = np.arange(nb)
    width = mb if mb is not None else max(1, max(nblk) if nblk else 1)
    poison = int(perm[total])
    tables = np.full((len(lens), width), poison, dtype=np.int32)
    k = 0
    for b, n in enumerate(nblk):
        if n > width:
            raise ValueError("sequence longer than the table width")
        tables[b, :n] = perm[k:k + n]
        k += n
    return tables, nb, poison


def build_case(name, lens, num_q_heads, num_kv_heads, head_dim, dtype, seed,
               *, pool_blocks=None, mb=None, with_write=False,
               partition_tokens=512, scale=None, block_size=BLOCK,
               placement="random") -> Case:
    """A decode batch with the given lengths and random block placement.

    With ``with_write`` the newest token of each sequence (position L - 1)
    is not yet in the pool (its slot is poisoned) and is supplied as
    ``k_new``/``v_new`` with its slot in ``slot_mapping``; rows with L = 0
    get slot -1.
    """
    rng = np.random.default_rng(seed)
    gen = torch.Generator().manual_seed(seed)
    lens = np.asarray(lens, dtype=np.int64)
    if placement not in ("random", "contiguous"):
        raise ValueError("placement is 'random' or 'contiguous'")
    bs = int(block_size)
    tables, nb, poison = place_blocks(lens, rng, pool_blocks, mb,
                                      consecutive=placement == "contiguous", block_size=bs)
    B = len(lens)
    q = _randn(gen, (B, num_q_heads, head_dim), dtype)
    k_pool = _randn(gen, (nb, num_kv_heads, bs, head_dim), dtype)
    v_pool = _randn(gen, v_pool_shape(nb, num_kv_heads, head_dim, bs), dtype)
    used = np.zeros(nb, dtype=bool)
    for b, L in enumerate(lens.tolist()):
        used[tables[b, :math.ceil(L / bs)]] = True
    unused = torch.from_numpy(np.nonzero(~used)[0])
    k_pool[unused] = float("nan")
    v_pool[unused] = float("nan")
    _poison_tails(k_pool, v_pool, tables, lens, bs)
    case = Case(name, dtype, q, k_pool, v_pool,
                torch.from_numpy(tables), torch.from_numpy(lens.astype(np.int32)),
                scale if scale is not None else 1.0 / math.sqrt(head_dim),
                partition_tokens, poison)
    if with_write:
        k_new = _randn(gen, (B, num_kv_heads, head_dim), dtype)
        v_new = _randn(gen, (B, num_kv_heads, head_dim), dtype)
        slots = np.full(B, -1, dtype=np.int32)
        for b, L in enumerate(lens.tolist()):
            if L == 0:
                continue
            pos = L - 1
            blk = int(tables[b, pos // bs])
            slots[b] = blk * bs + pos % bs
            k_pool[blk, :, pos % bs, :] = float("nan")
            set_v_slot(v_pool, blk, pos % bs, float("nan"))
        case.k_new, case.v_new = k_new, v_new
        case.slot_mapping = torch.from_numpy(slots)
    return case


# --------------------------------------------------------------------------
# the five configurations
# --------------------------------------------------------------------------

def config1() -> Case:
    """Tiny fp32: B = 4, L = {1, 17, 33, 50}, 4/2 heads, D = 64, 32-block pool.

    10 of the 32 blocks are used, taken in logical order from a seeded
    permutation; the other 22 are poisoned. Scale 1/sqrt(64).
    """
    return build_case("config1_tiny_fp32", [1, 17, 33, 50], 4, 2, 64, "f32",
                      SEED_BASE + 1, pool_blocks=32, partition_tokens=512,
                      scale=1.0 / 8.0)


def config2_lens(seed=SEED_BASE + 2, batch=64):
    rng = np.random.default_rng([seed, 0])
    return rng.integers(128, 4096, size=batch, endpoint=True)


def config2(batch: int = 64, block_size: int = BLOCK, placement: str = "random") -> Case:
    """Llama-3-8B-shaped layer: bf16, 32/8 heads, D = 128, B = 64.

    Lengths uniform in [128, 4096]; the pool holds exactly the needed blocks
    plus one poison block, randomly permuted (or, for the contiguity sweep,
    in order); the newest token of every sequence is appended through
    ``slot_mapping`` before decoding. ``block_size`` other than 16 serves
    the block-size sweep.
    """
    lens = config2_lens(batch=batch)
    return build_case("config2_llama3_8b_layer", lens, 32, 8, 128, "bf16",
                      SEED_BASE + 2, with_write=True, block_size=block_size,
                      placement=placement)


def config4_lens(seed=SEED_BASE + 4, batch=256):
    rng = np.random.default_rng([seed, 0])
    z = rng.standard_normal(batch)
    return np.clip(np.rint(np.exp(math.log(1024.0) + 1.0 * z)), 16, 8192).astype(np.int64)


def config4(batch: int = 256, block_size: int = BLOCK, placement: str = "random") -> Case:
    """Llama-3.3-70B-shaped layer: bf16, 64/8 heads (GQA 8), D = 128, B = 256.

    Lengths lognormal with median 1024 and sigma 1, clipped to [16, 8192];
    randomly permuted physical blocks (``placement`` and ``block_size`` as
    for the 8B layer).
    """
    lens = config4_lens(batch=batch)
    return build_case("config4_llama3_70b_layer", lens, 64, 8, 128, "bf16",
                      SEED_BASE + 4, block_size=block_size, placement=placement)


def config3() -> Case:
    """Copy-on-write over a shared prefix, 8B layer shape, 256-page pool.

    Admission: 7 requests of one trust group (2,048-token shared prompt,
    257 output tokens) reserve 128 + 7 x 17 = 247 pages; an eighth is
    refused. Sequences 0..6 hold 2,305 tokens each, sharing the 128 prompt
    blocks. Sequence 0 is then forked into sequence 7, and one decode step
    appends a token to all eight: sequence 7's token lands in a block it
    shares with sequence 0, so that block is copied first. The case carries
    the copy pair, the eight slots and the resulting tables (L = 2,306).
    """
    seed = SEED_BASE + 3
    rng = np.random.default_rng([seed, 0])
    gen = torch.Generator().manual_seed(seed)
    prompt, output, pool = 2048, 257, 256
    ledger = AdmissionLedger(pool, BLOCK)
    admitted = [ledger.reserve(i, prompt, output, group="g", shared_prefix_tokens=prompt)
                for i in range(8)]
    bm = BlockManager(pool, BLOCK, free_order=rng.permutation(pool))
    L0 = prompt + output
    bm.add_sequence(0, L0)
    for s in range(1, 7):
        bm.add_sequence(s, L0, prefix_from=0, prefix_blocks=prompt // BLOCK)
    used_after_admission = pool - bm.num_free
    Hkv, D = 8, 128
    k_pool = _randn(gen, (pool, Hkv, BLOCK, D), "bf16")
    v_pool = _randn(gen, (pool, Hkv, D, BLOCK), "bf16")
    live = sorted({b for t in bm.tables.values() for b in t})
    dead = torch.tensor(sorted(set(range(pool)) - set(live)), dtype=torch.long)
    k_pool[dead] = float("nan")
    v_pool[dead] = float("nan")
    pre_tables = bm.table_array(range(7), math.ceil(L0 / BLOCK), pad=0)
    _poison_tails(k_pool, v_pool, pre_tables, np.full(7, L0))
    bm.fork(0, 7)
    refcount_prefix_after_fork = int(bm.refcount[bm.tables[0][0]])
    refcount_last_after_fork = int(bm.refcount[bm.tables[0][-1]])
    seqs = list(range(8))
    slots, pairs = [], []
    # the fork writes first: its token lands in the shared last block
    order = [7] + list(range(7))
    slot_of = {}
    for s in order:
        slot, cow = bm.append_token(s)
        slot_of[s] = slot
        if cow is not None:
            pairs.append(cow)
    slots = [slot_of[s] for s in seqs]
    L1 = L0 + 1
    mb = math.ceil(L1 / BLOCK)
    poison = int(dead[0]) if len(dead) else 0
    remaining_dead = sorted(set(range(pool)) - {b for t in bm.tables.values() for b in t})
    if remaining_dead:
        poison = remaining_dead[0]
    tables = bm.table_array(seqs, mb, pad=poison)
    q = _randn(gen, (8, 32, D), "bf16")
    k_new = _randn(gen, (8, Hkv, D), "bf16")
    v_new = _randn(gen, (8, Hkv, D), "bf16")
    case = Case("config3_cow_shared_prefix", "bf16", q, k_pool, v_pool,
                torch.from_numpy(tables), torch.from_numpy(bm.len_array(seqs)),
                1.0 / math.sqrt(D), 512, poison, k_new, v_new,
                torch.tensor(slots, dtype=torch.int32),
                torch.tensor(pairs, dtype=torch.int32).reshape(-1, 2),
                meta={
                    "admitted": admitted,
                    "used_after_admission": used_after_admission,
                    "free_after_admission": pool - used_after_admission,
                    "refcount_prefix_after_fork": refcount_prefix_after_fork,
                    "refcount_last_after_fork": refcount_last_after_fork,
                    "cow_pairs": pairs,
                    "refcount_after_cow": {"src": int(bm.refcount[pairs[0][0]]),
                                           "dst": int(bm.refcount[pairs[0][1]])} if pairs else {},
                    "free_after_step": bm.num_free,
                })
    return case


# --------------------------------------------------------------------------
# configuration 5: the bucketed 32-layer step
# --------------------------------------------------------------------------

C5_LAYERS = 32
C5_MB = 512
C5_BUCKETS = [1, 2, 4, 8, 16, 32, 64, 128, 256]


@dataclass
class StepSpec:
    """Integer inputs of one bucketed decode step (shared by all layers)."""

    bucket: int
    n_real: int
    seq_lens: np.ndarray          # int32 [bucket], zeros after n_real
    block_tables: np.ndarray      # int32 [bucket, 512]
    num_blocks: int               # per-layer pool blocks
    poison_block: int
    layers: int = C5_LAYERS
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 128
    partition_tokens: int = 512

    def kv_bytes_per_layer(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum()) * self.num_kv_heads \
            * self.head_dim * 2 * 2


def config5_spec(bucket: int) -> StepSpec:
    """Bucket ``bucket``: n_real ~ U[floor(bucket/2) + 1, bucket] real rows
    with L ~ U[1, 8192], padded with L = 0 rows at the end; one table of
    width 512 for every layer."""
    if bucket not in C5_BUCKETS:
        raise ValueError(f"bucket must be one of {C5_BUCKETS}")
    rng = np.random.default_rng([SEED_BASE + 5, bucket])
    n_real = int(rng.integers(bucket // 2 + 1, bucket, endpoint=True))
    lens = np.zeros(bucket, dtype=np.int64)
    lens[:n_real] = rng.integers(1, 8192, size=n_real, endpoint=True)
    tables, nb, poison = place_blocks(lens, rng, mb=C5_MB)
    return StepSpec(bucket, n_real, lens.astype(np.int32), tables, nb, poison)


def config5_layer(spec: StepSpec, layer: int, device) -> tuple:
    """(q, k_pool, v_pool) of one layer, drawn on ``device`` from the layer's
    own generator (seed 55_005 * 100 + layer), poisoned like the others."""
    gen = torch.Generator(device=device).manual_seed((SEED_BASE + 5) * 100 + layer)
    B, Hq, Hkv, D = spec.bucket, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    q = torch.randn((B, Hq, D), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    k_pool = torch.empty((spec.num_blocks, Hkv, BLOCK, D), device=device, dtype=torch.bfloat16)
    v_pool = torch.empty((spec.num_blocks, Hkv, D, BLOCK), device=device, dtype=torch.bfloat16)
    for t in (k_pool, v_pool):
        # draw in chunks to bound the fp32 staging buffer
        flat = t.view(spec.num_blocks, -1)
        step = 4096
        for i in range(0, spec.num_blocks, step):
            j = min(spec.num_blocks, i + step)
            flat[i:j] = torch.randn((j - i, flat.shape[1]), generator=gen,
                                    device=device, dtype=torch.float32).to(torch.bfloat16)
    k_pool[spec.poison_block] = float("nan")
    v_pool[spec.poison_block] = float("nan")
    lens = spec.seq_lens
    for b in range(spec.n_real):
        L = int(lens[b])
        if L % BLOCK:
            blk = int(spec.block_tables[b, L // BLOCK])
            k_pool[blk, :, L % BLOCK:, :] = float("nan")
            v_pool[blk, :, :, L % BLOCK:] = float("nan")
    return q, k_pool, v_pool


# --------------------------------------------------------------------------
# small random cases for parity sweeps
# --------------------------------------------------------------------------

def random_case(seed, batch, num_q_heads, num_kv_heads, head_dim, dtype,
                max_len=300, min_len=0, lens=None, with_write=False,
                partition_tokens=512, extra_table_cols=0, block_size=BLOCK,
                placement="random") -> Case:
    rng = np.random.default_rng([seed, 1])
    if lens is None:
        lens = rng.integers(min_len, max_len, size=batch, endpoint=True)
    lens = np.asarray(lens, dtype=np.int64)
    mb = max(1, max((math.ceil(int(L) / block_size) for L in lens), default=1)) \
        + extra_table_cols
    return build_case(f"random_{seed}", lens, num_q_heads, num_kv_heads,
                      head_dim, dtype, seed, mb=mb, with_write=with_write,
                      partition_tokens=partition_tokens, block_size=block_size,
                      placement=placement)


def prefill_case(seed, chunks, contexts, num_q_heads, num_kv_heads, head_dim, dtype="bf16",
                 block_size=BLOCK, name=None) -> Case:
    """A chunked-prefill batch: sequence s has ``contexts[s]`` tokens cached
    and appends a chunk of ``chunks[s]`` new tokens (length
    L_s = contexts[s] + chunks[s]). q is [T, Hq, D] with T = sum(chunks),
    sequence s owning rows query_start[s] .. query_start[s + 1] - 1. The
    chunk's K/V come as k_new / v_new [T, Hkv, D] with their slots in
    slot_mapping (positions L_s - n_s .. L_s - 1, in order); those slots are
    poisoned in the pool until the append writes them."""
    chunks = np.asarray(chunks, dtype=np.int64)
    contexts = np.asarray(contexts, dtype=np.int64)
    lens = contexts + chunks
    rng = np.random.default_rng([seed, 7])
    gen = torch.Generator().manual_seed(seed)
    bs = int(block_size)
    tables, nb, poison = place_blocks(lens, rng, block_size=bs)
    T = int(chunks.sum())
    S = len(lens)
    q = _randn(gen, (T, num_q_heads, head_dim), dtype)
    k_pool = _randn(gen, (nb, num_kv_heads, bs, head_dim), dtype)
    v_pool = _randn(gen, v_pool_shape(nb, num_kv_heads, head_dim, bs), dtype)
    used = np.zeros(nb, dtype=bool)
    for b, L in enumerate(lens.tolist()):
        used[tables[b, :math.ceil(L / bs)]] = True
    unused = torch.from_numpy(np.nonzero(~used)[0])
    k_pool[unused] = float("nan")
    v_pool[unused] = float("nan")
    _poison_tails(k_pool, v_pool, tables, lens, bs)
    k_new = _randn(gen, (T, num_kv_heads, head_dim), dtype)
    v_new = _randn(gen, (T, num_kv_heads, head_dim), dtype)
    slots = np.empty(T, dtype=np.int32)
    qs = np.zeros(S + 1, dtype=np.int32)
    qs[1:] = np.cumsum(chunks)
    for b in range(S):
        for i in range(int(chunks[b])):
            pos = int(contexts[b]) + i
            blk = int(tables[b, pos // bs])
            slots[qs[b] + i] = blk * bs + pos % bs
            k_pool[blk, :, pos % bs, :] = float("nan")
            set_v_slot(v_pool, blk, pos % bs, float("nan"))
    case = Case(name or f"prefill_{seed}", dtype, q, k_pool, v_pool, torch.from_numpy(tables),
                torch.from_numpy(lens.astype(np.int32)), 1.0 / math.sqrt(head_dim), 0,
                poison)
    case.k_new, case.v_new = k_new, v_new
    case.slot_mapping = torch.from_numpy(slots)
    case.query_start = torch.from_numpy(qs)
    return case


def prefill_step_8b(num_chunks: int = 8, chunk: int = 512, block_size: int = BLOCK) -> Case:
    """One chunked-prefill step on an 8B-shaped layer (bf16, 32/8 heads,
    D = 128): ``num_chunks`` prompts, each at a different point of its
    prefill, contribute one ``chunk``-token piece; prompt s has s * chunk
    tokens cached (the pieces of one 4,096-token prompt at 8 x 512, side
    by side)."""
    contexts = [s * chunk for s in range(num_chunks)]
    return prefill_case(SEED_BASE + 6, [chunk] * num_chunks, contexts, 32, 8, 128, "bf16",
                        block_size=block_size, name="prefill_step_llama3_8b_8x512")


LATENT_DIM = 576      # 512-element compressed KV + 64-element positional key
LATENT_VALUE_DIM = 512
LATENT_BLOCK = 64     # the latent kernels' page size


@dataclass
class LatentCase:
    """Inputs of a latent (MLA-style) decode batch."""

    q: torch.Tensor             # [B, H, 576]
    kv_pool: torch.Tensor       # [NB, block, 576]
    block_tables: torch.Tensor  # int32 [B, MB]
    seq_lens: torch.Tensor      # int32 [B]
    scale: float
    dtype: str = "bf16"

    def to(self, device) -> "LatentCase":
        return LatentCase(self.q.to(device), self.kv_pool.to(device),
                          self.block_tables.to(device), self.seq_lens.to(device), self.scale,
                          self.dtype)

    def kv_bytes(self) -> int:
        elem = 4 if self.dtype == "f32" else 2
        return int(self.seq_lens.to(torch.int64).sum()) * self.kv_pool.shape[2] * elem


def latent_case(seed, lens, num_heads=128, block_size=LATENT_BLOCK, dtype="bf16",
                scale=None) -> LatentCase:
    """A latent decode batch: random block placement (seeded permutation of
    a pool of exactly the needed blocks plus a poison block), N(0, 1) values,
    NaN in unused blocks and in the tail slots of each last block. The scale
    defaults to 1 / sqrt(576), the softmax scale of attention with head dim
    576."""
    lens = np.asarray(lens, dtype=np.int64)
    rng = np.random.default_rng([seed, 9])
    gen = torch.Generator().manual_seed(seed)
    tables, nb, poison = place_blocks(lens, rng, block_size=block_size)
    q = _randn(gen, (len(lens), num_heads, LATENT_DIM), dtype)
    kv = _randn(gen, (nb, block_size, LATENT_DIM), dtype)
    used = np.zeros(nb, dtype=bool)
    for b, L in enumerate(lens.tolist()):
        used[tables[b, :math.ceil(L / block_size)]] = True
    kv[torch.from_numpy(np.nonzero(~used)[0])] = float("nan")
    for b, L in enumerate(lens.tolist()):
        if L % block_size:
            kv[int(tables[b, L // block_size]), L % block_size:, :] = float("nan")
    return LatentCase(q, kv, torch.from_numpy(tables), torch.from_numpy(lens.astype(np.int32)),
                      scale if scale is not None else 1.0 / math.sqrt(LATENT_DIM), dtype)


def latent_decode_batch(batch: int = 256) -> LatentCase:
    """A DeepSeek-V3-shaped MLA decode layer: 128 heads over one 576-element
    latent per token, 64-token pages, bf16, with the 70B serving batch's
    length mix (B = 256, lognormal, median 1,024, sigma 1, clipped to
    [16, 8192])."""
    return latent_case(SEED_BASE + 7, config4_lens(batch=batch))


def permute_physical(case: Case, seed: int) -> Case:
    """The same logical contents under another physical placement:
    pool'[pi(i)] = pool[i] and table' = pi(table)."""
    rng = np.random.default_rng([seed, 2])
    nb = case.num_blocks
    pi = torch.from_numpy(rng.permutation(nb))
    inv = torch.empty_like(pi)
    inv[pi] = torch.arange(nb)
    k = case.k_pool[inv]
    v = case.v_pool[inv]
    tables = pi[case.block_tables.to(torch.long)].to(torch.int32)
    out = Case(case.name + "_perm", case.dtype, case.q, k, v, tables,
               case.seq_lens, case.scale, case.partition_tokens,
               int(pi[case.poison_block]) if case.poison_block >= 0 else -1,
               meta=dict(case.meta))
    if case.slot_mapping is not None:
        s = case.slot_mapping.to(torch.long)
        valid = s >= 0
        ns = torch.where(valid, pi[torch.clamp(s // BLOCK, min=0)] * BLOCK + s % BLOCK, s)
        out.k_new, out.v_new = case.k_new, case.v_new
        out.slot_mapping = ns.to(torch.int32)
    return out


def contiguous_cache(case: Case):
    """The same K/V values as a paged case (16-token blocks), laid out as an
    unpaged cache: k [B, Hkv, Lmax, D] with token t of row b at [b, :, t],
    v [B, Hkv, Lmax // 16, D, 16] with it at [b, :, t // 16, :, t % 16],
    Lmax = 16 * max_blocks_per_seq. Each row's blocks are copied whole
    (through its table), so slots past its length keep the pool's poison,
    and slots past its last block hold poison too. Works on the case's
    device; a layout change only."""
    if case.block_size != BLOCK:
        raise ValueError("contiguous_cache takes 16-token blocks")
    B, Hkv, D = case.num_seqs, case.num_kv_heads, case.head_dim
    mb = case.max_blocks_per_seq
    dev, dt = case.k_pool.device, case.k_pool.dtype
    nan = float("nan")
    k = torch.full((B, Hkv, mb * BLOCK, D), nan, dtype=dt, device=dev)
    v = torch.full((B, Hkv, mb, D, BLOCK), nan, dtype=dt, device=dev)
    lens = case.seq_lens.cpu().numpy()
    for b in range(B):
        nb = math.ceil(int(lens[b]) / BLOCK)
        if nb == 0:
            continue
        blk = case.block_tables[b, :nb].long()
        k[b, :, :nb * BLOCK, :] = case.k_pool[blk].permute(1, 0, 2, 3).reshape(Hkv, nb * BLOCK, D)
        v[b, :, :nb] = case.v_pool[blk].permute(1, 0, 2, 3)
    return k, v
