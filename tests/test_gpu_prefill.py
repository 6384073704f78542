"""pa_prefill (chunked-prefill paged attention) on the GPU against the oracle
on the same seeded inputs: each chunk's K/V is appended with pa_write_kv,
then every query row is compared with the float64 oracle to the bf16 bar
(per-row RMS). Poisoned memory (unused blocks, tail slots) must never leak
into a result."""

import numpy as np
import pytest
import torch

import paged_kv_cache_55_amd as pk
import workloads as wl
from parity import bits_equal, compare, gpu_out_f64, oracle_prefill
from workloads import to_numpy

pytestmark = pytest.mark.gpu


def gpu_prefill(c):
    d = c.to("cuda")
    pk.pa_write_kv(d.k_new, d.v_new, d.slot_mapping, d.k_pool, d.v_pool)
    out = pk.pa_prefill(d.q, d.k_pool, d.v_pool, d.block_tables, d.seq_lens, d.query_start,
                        c.scale)
    torch.cuda.synchronize()
    return out, d.k_pool, d.v_pool


def check(c):
    ref, k_ref, v_ref = oracle_prefill(c)
    out, k, v = gpu_prefill(c)
    assert bits_equal(k, k_ref) and bits_equal(v, v_ref)
    rows = np.ones(c.q.shape[0], dtype=np.int64)  # every query row is real
    return compare(gpu_out_f64(out), ref, rows, "bf16")


@pytest.mark.parametrize("chunks,contexts", [
    ([37, 1, 64, 5], [100, 40, 0, 300]),          # mixed chunk sizes and offsets
    ([1, 1, 1, 1, 1], [0, 15, 16, 17, 2000]),    # decode rows only
    ([200], [0]),                                # a whole prompt in one piece
    ([16, 0, 33, 128], [16, 5, 0, 1000]),        # an idle row; block-aligned offsets
    ([300, 1, 1, 7], [3000, 4095, 10, 0]),       # chunk and decode rows together
])
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (64, 8, 128), (8, 8, 64), (16, 1, 128)])
def test_prefill_small(chunks, contexts, hq, hkv, d):
    c = wl.prefill_case(900 + sum(chunks) + hq, chunks, contexts, hq, hkv, d)
    check(c)


def test_prefill_item_ending_before_its_sequence():
    """A 216-token chunk after 2 cached tokens, 64-token blocks: the first
    column block's items end before the sequence does and have an odd tile
    count. The padding tile that completes their last pair is not loaded;
    its stage's older contents (here once a poisoned tail slot) must be
    masked by the wave's last position, not only by L."""
    check(wl.prefill_case(5507, [216], [2], 32, 8, 128, block_size=64))


@pytest.mark.parametrize("bs", [64, 256])
def test_prefill_block_sizes(bs):
    c = wl.prefill_case(950 + bs, [100, 3, 250], [60, 700, 1], 32, 8, 128, block_size=bs)
    check(c)


def test_prefill_step_8b_full_size():
    """The measured workload: 8 prompts, a 512-token chunk each, with 0 ..
    3,584 tokens already cached."""
    worst = check(wl.prefill_step_8b())
    print(f"prefill 8x512 worst ratio {worst:.3f}")


def test_one_token_chunks_match_the_decode_kernel():
    """Decode rows through pa_prefill meet the bar, as pa_decode (balanced
    split) does on the same rows."""
    c = wl.prefill_case(961, [1] * 24, list(range(5, 2400, 100)), 32, 8, 128)
    out_p, k, v = gpu_prefill(c)
    d = c.to("cuda")
    out_d = pk.pa_decode(d.q, k, v, d.block_tables, d.seq_lens, c.scale, partition_tokens=0,
                         kernel="mfma")
    torch.cuda.synchronize()
    ref, _, _ = oracle_prefill(c)
    compare(gpu_out_f64(out_p), ref, np.ones(24), "bf16")
    compare(gpu_out_f64(out_d), ref, np.ones(24), "bf16")


def test_prefill_4096_sequences():
    """The most sequences a call takes: 4,096 rows with 0-90 cached tokens,
    most appending one token (decode rows), 512 idle and 256 appending
    seven; every query row is compared with the oracle."""
    rng = np.random.default_rng(1102)
    contexts = rng.integers(0, 91, size=4096)
    chunks = np.ones(4096, dtype=np.int64)
    chunks[rng.choice(4096, 512, replace=False)] = 0
    chunks[rng.choice(4096, 256, replace=False)] = 7
    check(wl.prefill_case(1102, chunks.tolist(), contexts.tolist(), 32, 8, 128))


def test_prefill_rejects_unsupported():
    c = wl.prefill_case(971, [4], [4], 8, 2, 64, block_size=8).to("cuda")
    with pytest.raises(pk.PagedKVError):
        pk.pa_prefill(c.q, c.k_pool, c.v_pool, c.block_tables, c.seq_lens, c.query_start,
                      c.scale)
