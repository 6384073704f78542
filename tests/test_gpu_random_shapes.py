"""Seeded random shapes for the decode, chunked-prefill and latent paths on
the GPU against the float64 oracle, to the same bars as the fixed cases.

Lengths are drawn half from block and tile boundaries (0, 1, 15, 16, 17,
31, 32, 33, 63, 64, 65, ...) and half uniformly; block sizes, head
geometries (group sizes 1, 2, 3, 4, 8 and 16), dtypes, decode kernels and
partition lengths, batch sizes and chunk/context splits vary with the seed,
within what the library accepts (blocks other than 16 tokens only through
the balanced split). Each case prints its draw before the GPU call, so a
failure names it."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_55_amd as pk
import workloads as wl
from parity import bits_equal, compare, gpu_out_f64, oracle_prefill, oracle_step, run_step
from workloads import to_numpy

pytestmark = pytest.mark.gpu

EDGE = [0, 1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def draw_len(rng, hi):
    return int(rng.choice(EDGE)) if rng.random() < 0.5 else int(rng.integers(0, hi + 1))


DECODE_HEADS = [(32, 8, 128), (8, 8, 64), (16, 1, 128), (64, 8, 128), (12, 4, 64), (32, 2, 64)]


@pytest.mark.parametrize("seed", range(24))
def test_decode_random_shapes(seed):
    rng = np.random.default_rng([5501, seed])
    hq, hkv, d = DECODE_HEADS[seed % len(DECODE_HEADS)]
    bs = int(rng.choice([8, 16, 32, 64, 128, 256]))
    if bs == 16:  # any dtype, the library's kernel choice, a drawn partition length
        dtype = "f32" if seed % 3 == 0 else "bf16"
        kernel, part = "auto", int(rng.choice([0, 16, 48, 512]))
    else:  # other block sizes go through the balanced split (bf16, one partition)
        dtype, kernel, part = "bf16", "mfma", 0
    batch = int(rng.integers(1, 41))
    lens = [draw_len(rng, 1500) for _ in range(batch)]
    with_write = bool(seed % 2)
    print(f"decode seed={seed} heads={hq}/{hkv} D={d} {dtype} bs={bs} kernel={kernel} "
          f"partition={part} B={batch} write={with_write} lens={lens}", flush=True)
    c = wl.random_case(5501 + seed, batch, hq, hkv, d, dtype, lens=lens, with_write=with_write,
                       block_size=bs)
    ref, k_ref, v_ref = oracle_step(c)
    out, k, v = run_step(c, kernel=kernel, partition_tokens=part)
    assert bits_equal(k, k_ref) and bits_equal(v, v_ref)
    compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), dtype)


PREFILL_HEADS = [(32, 8, 128), (8, 8, 64), (16, 1, 128), (64, 8, 128), (24, 8, 64)]


@pytest.mark.parametrize("seed", range(20))
def test_prefill_random_shapes(seed):
    rng = np.random.default_rng([5502, seed])
    hq, hkv, d = PREFILL_HEADS[seed % len(PREFILL_HEADS)]
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    nseq = int(rng.integers(1, 7))
    chunks = [int(rng.choice([0, 1, 2, 15, 16, 17, 33])) if rng.random() < 0.4
              else int(rng.integers(1, 300)) for _ in range(nseq)]
    if sum(chunks) == 0:
        chunks[0] = 1
    contexts = [draw_len(rng, 1200) for _ in range(nseq)]
    print(f"prefill seed={seed} heads={hq}/{hkv} D={d} bs={bs} chunks={chunks} "
          f"contexts={contexts}", flush=True)
    c = wl.prefill_case(5502 + seed, chunks, contexts, hq, hkv, d, block_size=bs)
    ref, k_ref, v_ref = oracle_prefill(c)
    dc = c.to("cuda")
    pk.pa_write_kv(dc.k_new, dc.v_new, dc.slot_mapping, dc.k_pool, dc.v_pool)
    out = pk.pa_prefill(dc.q, dc.k_pool, dc.v_pool, dc.block_tables, dc.seq_lens,
                        dc.query_start, c.scale)
    assert bits_equal(dc.k_pool, k_ref) and bits_equal(dc.v_pool, v_ref)
    compare(gpu_out_f64(out), ref, np.ones(c.q.shape[0], dtype=np.int64), "bf16")


# Seeds 3 and 7 once put one element past the bf16 bar (1.045x, 1.10x) in
# rows merged from bf16 piece records; the records have a quarter of that
# rounding since (fp16, scaled per head).
LATENT_SEEDS = list(range(10))


@pytest.mark.parametrize("seed", LATENT_SEEDS)
def test_latent_random_shapes(seed):
    rng = np.random.default_rng([5503, seed])
    batch = int(rng.integers(1, 61))
    lens = [draw_len(rng, 2500) for _ in range(batch)]
    if max(lens) == 0:
        lens[0] = 1
    print(f"latent seed={seed} B={batch} lens={lens}", flush=True)
    c = wl.latent_case(5503 + seed, lens)
    ref = oracle.latent_decode(to_numpy(c.q), to_numpy(c.kv_pool), to_numpy(c.block_tables),
                               to_numpy(c.seq_lens), c.scale, c.dtype)
    d = c.to("cuda")
    out = pk.pa_latent_decode(d.q, d.kv_pool, d.block_tables, d.seq_lens, c.scale)
    torch.cuda.synchronize()
    compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), "bf16")
