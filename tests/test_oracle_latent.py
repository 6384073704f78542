"""Pins of the latent (MLA-style) decode oracle (``oracle.latent_decode``) to
things other than itself:

* brute force: scalar loops with their own table walk and math.exp;
* a library routine: torch's scaled_dot_product_attention in float64, every
  head over the one shared latent (keys: all 576 elements; values: the first
  512);
* a reduction: with the value width equal to the latent width, latent decode
  is the grouped-query decode oracle with one KV head (K = V = the latent)
  and all heads in its group;
* special cases with closed forms: one token, identical latents, a sequence
  of length 0;
* planted mistakes: values taken from the wrong slice, scores that drop the
  64 positional elements, a block-table off-by-one and a missing scale must
  each fail a pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa
import workloads as wl
from workloads import to_numpy


def run(c, fn=None, **kw):
    return (fn or oracle.latent_decode)(to_numpy(c.q), to_numpy(c.kv_pool),
                                        to_numpy(c.block_tables), to_numpy(c.seq_lens),
                                        c.scale, c.dtype, **kw)


def brute_force(c, value_dim=512):
    q = oa.as_f64(to_numpy(c.q), c.dtype)
    kv = oa.as_f64(to_numpy(c.kv_pool), c.dtype)
    bt, lens = to_numpy(c.block_tables), to_numpy(c.seq_lens)
    bs = kv.shape[1]
    B, H, C = q.shape
    out = np.zeros((B, H, value_dim))
    for b in range(B):
        L = int(lens[b])
        for h in range(H):
            if L == 0:
                continue
            rows = [kv[int(bt[b][t // bs]), t % bs] for t in range(L)]
            sc = [c.scale * math.fsum(float(q[b, h, d]) * float(r[d]) for d in range(C))
                  for r in rows]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = math.fsum(w)
            for d in range(value_dim):
                out[b, h, d] = math.fsum(wt * float(r[d]) for wt, r in zip(w, rows)) / tot
    return out


def test_brute_force():
    c = wl.latent_case(21, [1, 70, 0, 130], num_heads=2, block_size=64)
    np.testing.assert_allclose(run(c), brute_force(c), rtol=0, atol=1e-12)


def test_brute_force_f32_small_blocks():
    c = wl.latent_case(22, [5, 33, 17], num_heads=3, block_size=16, dtype="f32")
    np.testing.assert_allclose(run(c), brute_force(c), rtol=0, atol=1e-12)


def sdpa(c, value_dim=512):
    q = oa.as_f64(to_numpy(c.q), c.dtype)
    kv = oa.as_f64(to_numpy(c.kv_pool), c.dtype)
    bt, lens = to_numpy(c.block_tables), to_numpy(c.seq_lens)
    bs = kv.shape[1]
    B, H, C = q.shape
    out = np.zeros((B, H, value_dim))
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        lat = np.concatenate([kv[int(bt[b][j])] for j in range(math.ceil(L / bs))])[:L]
        k = torch.from_numpy(lat)[None, None].expand(1, H, L, C)
        v = torch.from_numpy(lat[:, :value_dim].copy())[None, None].expand(1, H, L, value_dim)
        qt = torch.from_numpy(q[b])[None, :, None, :]          # [1, H, 1, C]
        o = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=c.scale)
        out[b] = o[0, :, 0].numpy()
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sdpa(dtype):
    c = wl.latent_case(23, [1, 64, 65, 300, 0, 1000], num_heads=16, dtype=dtype)
    np.testing.assert_allclose(run(c), sdpa(c), rtol=0, atol=1e-12)


def test_full_value_width_is_one_kv_head_decode():
    """value_dim = 576: the grouped-query oracle with Hkv = 1, G = H, K = V =
    the latent (V in its [NB, 1, D, block] layout). The first 512 columns
    are the latent decode's output."""
    c = wl.latent_case(24, [3, 64, 129, 500], num_heads=8)
    kv = to_numpy(c.kv_pool)                             # [NB, bs, 576]
    k_pool = kv[:, None, :, :]                           # [NB, 1, bs, 576]
    v_pool = np.ascontiguousarray(np.swapaxes(kv, 1, 2))[:, None]  # [NB, 1, 576, bs]
    ref = oracle.paged_decode(to_numpy(c.q), k_pool, v_pool, to_numpy(c.block_tables),
                              to_numpy(c.seq_lens), c.scale, c.dtype, block_size=64)
    full = run(c, value_dim=576)
    np.testing.assert_allclose(full, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(run(c), ref[:, :, :512], rtol=0, atol=1e-12)


def test_closed_forms():
    c = wl.latent_case(25, [1, 40, 0], num_heads=4)
    out = run(c)
    kv = oa.as_f64(to_numpy(c.kv_pool), c.dtype)
    bt = to_numpy(c.block_tables)
    # one token: every head returns that token's first 512 latent elements
    np.testing.assert_array_equal(out[0], np.broadcast_to(kv[bt[0, 0], 0, :512], (4, 512)))
    # a sequence of length 0 is zeros
    assert np.all(out[2] == 0.0)
    # identical latents: the output is that latent whatever the scores
    pool = c.kv_pool.clone()
    pool[int(bt[1, 0]), :40] = pool[int(bt[1, 0]), 0]
    c2 = wl.LatentCase(c.q, pool, c.block_tables, c.seq_lens, c.scale, c.dtype)
    same = run(c2)[1]
    lat = oa.as_f64(to_numpy(pool), c.dtype)[bt[1, 0], 0, :512]
    np.testing.assert_allclose(same, np.broadcast_to(lat, (4, 512)), rtol=0, atol=1e-12)


def test_sampled_rows_and_placement():
    c = wl.latent_case(26, [200, 7, 64, 129], num_heads=4)
    full = run(c)
    np.testing.assert_array_equal(run(c, rows=[3, 1]), full[[3, 1]])
    # the same logical contents in a different physical placement
    c2 = wl.latent_case(26, [200, 7, 64, 129], num_heads=4)
    nb = c2.kv_pool.shape[0]
    perm = torch.from_numpy(np.random.default_rng(5).permutation(nb))
    inv = torch.argsort(perm)
    pool = c2.kv_pool[perm]                 # new block j holds old block perm[j]
    tables = inv[c2.block_tables.long()].to(torch.int32)
    c3 = wl.LatentCase(c2.q, pool, tables, c2.seq_lens, c2.scale, c2.dtype)
    np.testing.assert_array_equal(run(c3), full)


# ---- planted mistakes: each must fail the brute-force pin -----------------

def _latent_mutant(value_slice=slice(0, 512), score_dims=576, table_shift=0, use_scale=True):
    def f(q, kv_pool, block_tables, seq_lens, scale, dtype, value_dim=512, rows=None):
        B, H, C = q.shape
        bs = kv_pool.shape[1]
        out = np.zeros((B, H, value_dim))
        for b in range(B):
            L = int(seq_lens[b])
            if L == 0:
                continue
            t = np.arange(L)
            j = np.minimum(t // bs + table_shift, block_tables.shape[1] - 1)
            lat = oa.as_f64(kv_pool[block_tables[b][j], t % bs], dtype)
            qb = oa.as_f64(q[b], dtype)
            sc = (scale if use_scale else 1.0) * (qb[:, :score_dims] @ lat[:, :score_dims].T)
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            out[b] = (p @ lat[:, value_slice]) / p.sum(axis=1, keepdims=True)
        return out
    return f


@pytest.mark.parametrize("mutant", [dict(value_slice=slice(64, 576)), dict(score_dims=512),
                                    dict(table_shift=1), dict(use_scale=False)])
def test_planted_mistake_is_caught(mutant):
    c = wl.latent_case(27, [70, 130], num_heads=2, dtype="f32")
    got = run(c, fn=_latent_mutant(**mutant))
    ref = brute_force(c)
    err = np.nanmax(np.abs(got - ref)) if np.isfinite(got).all() else np.inf
    assert err > 1e-3
