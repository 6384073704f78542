"""pa_decode_contiguous (decode over an unpaged cache, no table) on the GPU
against the oracle's contiguous_cache_decode on the same seeded values, to
the bf16 bar; and bit for bit against pa_decode over the paged pool holding
the same values (the balanced split cuts the same tiles in both, so paging
changes where bytes live and nothing else [cs2680 Lecture 10, section 10.3
"Step three"])."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_55_amd as pk
import workloads as wl
from parity import compare, gpu_out_f64
from workloads import to_numpy

pytestmark = pytest.mark.gpu


def _appended(c):
    """The case with its pending KV append applied on the host by the
    oracle's write_kv (so the newest slots hold their tokens, not poison)."""
    if c.slot_mapping is None:
        return c
    k, v = oracle.write_kv(to_numpy(c.k_pool), to_numpy(c.v_pool), to_numpy(c.k_new),
                           to_numpy(c.v_new), to_numpy(c.slot_mapping))
    as_t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)  # noqa: E731
    return dataclasses.replace(c, k_pool=as_t(k), v_pool=as_t(v), k_new=None, v_new=None,
                               slot_mapping=None)


def _check(c, rows=None):
    c = _appended(c)
    d = c.to("cuda")
    k, v = wl.contiguous_cache(d)
    print(f"contiguous case B={c.num_seqs} G={c.num_q_heads // c.num_kv_heads} "
          f"D={c.head_dim} Lmax={k.shape[2]}", flush=True)
    out = pk.pa_decode_contiguous(d.q, k, v, d.seq_lens, c.scale)
    paged = pk.pa_decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.seq_lens, c.scale,
                         partition_tokens=0, kernel="mfma")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), paged.view(torch.int16))
    sel = list(range(c.num_seqs)) if rows is None else rows
    ref = oracle.contiguous_cache_decode(to_numpy(c.q), to_numpy(k), to_numpy(v),
                                         to_numpy(c.seq_lens), c.scale, c.dtype, rows=sel)
    return compare(gpu_out_f64(out, sel), ref, c.seq_lens.numpy()[sel], "bf16")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_contiguous_small(D, G):
    lens = [0, 1, 15, 16, 17, 33, 100, 255, 257, 600]
    _check(wl.random_case(800 + D + G, len(lens), G * 2, 2, D, "bf16", lens=lens,
                          extra_table_cols=3))


@pytest.mark.parametrize("lens", [[8000], [1] * 64, [4096, 1, 0, 2000, 33, 0, 8192, 15]])
def test_contiguous_edges(lens):
    _check(wl.random_case(820 + len(lens), len(lens), 32, 8, 128, "bf16", lens=lens))


def test_contiguous_8b_layer_full():
    _check(wl.config2())


def test_contiguous_70b_layer_full():
    worst = _check(wl.config4())
    print(f"contiguous 70B batch worst ratio {worst:.3f}")
