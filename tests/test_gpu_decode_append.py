"""pa_decode_append (one decode step: the KV append of every row's new token,
then paged decode attention) on the GPU against the oracle's write-then-decode
on the same seeded inputs. Outputs must meet the bf16 / fp32 bar and the pools
must match bit for bit, poison included, so a slot read before its new token
landed would show up as NaN."""

import numpy as np
import pytest
import torch

import paged_kv_cache_55_amd as pk
import workloads as wl
from parity import bits_equal, compare, gpu_out_f64, oracle_step

pytestmark = pytest.mark.gpu


def run_fused(c, kernel="auto", partition_tokens=0):
    d = c.to("cuda")
    out = pk.pa_decode_append(d.q, d.k_new, d.v_new, d.slot_mapping, d.k_pool, d.v_pool,
                              d.block_tables, d.seq_lens, c.scale,
                              partition_tokens=partition_tokens, kernel=kernel)
    torch.cuda.synchronize()
    return out, d.k_pool, d.v_pool


def check(c, kernel="auto", partition_tokens=0):
    pk.validate(c.num_blocks, c.block_tables, c.seq_lens, c.slot_mapping, append_rows=True)
    ref, k_ref, v_ref = oracle_step(c)
    out, k, v = run_fused(c, kernel, partition_tokens)
    assert bits_equal(k, k_ref) and bits_equal(v, v_ref)
    return compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), c.dtype)


@pytest.mark.parametrize("kernel,partition", [("mfma", 0), ("mfma", 512), ("valu", 512)])
def test_config2_step(kernel, partition):
    worst = check(wl.config2(), kernel, partition)
    print(f"config2 fused {kernel} part={partition} worst ratio {worst:.3f}")


@pytest.mark.parametrize("lens,hq,hkv,d", [
    ([1] * 64, 32, 8, 128),                          # every pair is its new block
    ([0, 5, 0, 17, 1, 300, 16, 0, 33], 32, 8, 128),  # padded rows, block edges
    ([4096, 1, 2, 2000, 8192, 15], 64, 8, 128),      # G = 8, long and tiny rows
    (list(range(1, 200, 7)), 16, 1, 64),             # G = 16, D = 64
    ([20] * 300, 32, 8, 128),                        # many short rows per wave
    ([70000], 2, 1, 128),                            # one pair over hundreds of waves
])
def test_balanced_fused_edges(lens, hq, hkv, d):
    c = wl.random_case(500 + len(lens), len(lens), hq, hkv, d, "bf16", lens=lens,
                       with_write=True)
    check(c, "mfma", 0)


def test_rows_without_a_new_token():
    """Rows whose slot is negative append nothing; their newest token is
    already in the pool."""
    c = wl.random_case(531, 40, 32, 8, 128, "bf16", max_len=700, min_len=1, with_write=True)
    slots = c.slot_mapping.numpy().copy()
    for b in range(0, 40, 3):
        s = int(slots[b])
        blk, off = divmod(s, 16)
        c.k_pool[blk, :, off, :] = c.k_new[b]
        c.v_pool[blk, :, :, off] = c.v_new[b]
        slots[b] = -1
    c.slot_mapping = torch.from_numpy(slots)
    check(c, "mfma", 0)


def test_f32_step_uses_the_append_kernel():
    c = wl.random_case(541, 6, 4, 2, 64, "f32", max_len=90, with_write=True)
    check(c)


def test_fused_matches_separate_calls_bitwise():
    """The fused step computes the same bits as pa_write_kv + pa_decode."""
    c = wl.config2()
    out_f, k_f, v_f = run_fused(c, "mfma", 0)
    d = c.to("cuda")
    pk.pa_write_kv(d.k_new, d.v_new, d.slot_mapping, d.k_pool, d.v_pool)
    out_s = pk.pa_decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.seq_lens, c.scale,
                         partition_tokens=0, kernel="mfma")
    torch.cuda.synchronize()
    assert torch.equal(k_f.view(torch.int16), d.k_pool.view(torch.int16))
    assert torch.equal(v_f.view(torch.int16), d.v_pool.view(torch.int16))
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))

