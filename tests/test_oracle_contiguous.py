"""Pins of the oracle's decode over an unpaged (contiguous) KV cache,
``contiguous_cache_decode``, to things other than itself:

* a library routine: torch's scaled_dot_product_attention in float64 on the
  per-sequence K/V that the test lays into the caches itself;
* brute force: scalar loops over the caches' own indexing (tiny inputs);
* the pages' invariant that paging moves bytes but not results: on the same
  values, the contiguous cache gives exactly (bitwise) what the paged pool
  gives [cs2680 Lecture 10, §10.3 "Step three"; llm-serving.xyz "KV-cache
  systems", paragraph on the price of paging];
* poison past each sequence's length is never read;
* planted mistakes in the cache indexing fail a pin.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.attention as oa
import workloads as wl
from test_oracle_pins import np_case, sdpa_reference
from workloads import to_numpy

LMAX = 256  # 16 tiles of 16 tokens


def lay_out(K_list, V_list, lmax=LMAX):
    """Caches (float32, NaN past each length) holding per-sequence K/V
    [Hkv, L, D]: k [B, Hkv, Lmax, D], v [B, Hkv, Lmax // 16, D, 16]."""
    B = len(K_list)
    Hkv, _, D = K_list[0].shape
    k = np.full((B, Hkv, lmax, D), np.nan, dtype=np.float32)
    v = np.full((B, Hkv, lmax // 16, D, 16), np.nan, dtype=np.float32)
    for b in range(B):
        for t in range(K_list[b].shape[1]):
            k[b, :, t, :] = K_list[b][:, t, :]
            v[b, :, t // 16, :, t % 16] = V_list[b][:, t, :]
    return k, v


def random_lists(seed, B=3, Hkv=2, D=16, max_len=70):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len, size=B)
    K_list = [rng.standard_normal((Hkv, L, D)).astype(np.float32) for L in lens]
    V_list = [rng.standard_normal((Hkv, L, D)).astype(np.float32) for L in lens]
    return rng, lens, K_list, V_list


def sdpa_error(seed, B=3, Hq=8, Hkv=2, D=16, max_len=70):
    rng, lens, K_list, V_list = random_lists(seed, B, Hkv, D, max_len)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    k, v = lay_out(K_list, V_list)
    scale = 1.0 / math.sqrt(D)
    got = oa.contiguous_cache_decode(q, k, v, lens.astype(np.int32), scale, "f32")
    err = np.abs(got - sdpa_reference(q, K_list, V_list, scale))
    return float("inf") if np.isnan(err).any() else float(np.max(err))


@pytest.mark.parametrize("seed", range(3))
def test_sdpa_library(seed):
    assert sdpa_error(900 + seed) < 1e-12


def test_brute_force_scalar_loops():
    rng, lens, K_list, V_list = random_lists(910, B=2, Hkv=2, D=6, max_len=40)
    Hq = 4
    q = rng.standard_normal((2, Hq, 6)).astype(np.float32)
    k, v = lay_out(K_list, V_list)
    scale = 0.3
    got = oracle.contiguous_cache_decode(q, k, v, lens.astype(np.int32), scale, "f32")
    for b in range(2):
        L = int(lens[b])
        for h in range(Hq):
            kv = h // (Hq // 2)
            s = [scale * sum(float(q[b, h, d]) * float(k[b, kv, t, d]) for d in range(6))
                 for t in range(L)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            for d in range(6):
                num = sum(w[t] * float(v[b, kv, t // 16, d, t % 16]) for t in range(L))
                assert abs(got[b, h, d] - num / sum(w)) < 1e-12


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_and_contiguous_are_bitwise_equal(dtype):
    """The same values in a paged pool (seeded random placement) and in a
    contiguous cache laid out here by a walk of the tables."""
    c = wl.random_case(920, 5, 8, 2, 32, dtype, max_len=200)
    a = np_case(c)
    B, Hkv, D = c.num_seqs, c.num_kv_heads, c.head_dim
    lmax = 16 * c.max_blocks_per_seq
    nan = np.float32("nan") if dtype == "f32" else np.uint16(0x7FC0)
    store = a["k_pool"].dtype
    k = np.full((B, Hkv, lmax, D), nan, dtype=store)
    v = np.full((B, Hkv, lmax // 16, D, 16), nan, dtype=store)
    for b in range(B):
        for t in range(int(a["seq_lens"][b])):
            blk = int(a["block_tables"][b, t // 16])
            k[b, :, t, :] = a["k_pool"][blk, :, t % 16, :]
            v[b, :, t // 16, :, t % 16] = a["v_pool"][blk, :, :, t % 16]
    paged = oracle.paged_decode(**a)
    contig = oracle.contiguous_cache_decode(a["q"], k, v, a["seq_lens"], c.scale, dtype)
    assert np.array_equal(paged, contig)


def test_zero_length_rows_and_poison_unread():
    rng, lens, K_list, V_list = random_lists(930, B=3)
    k, v = lay_out(K_list, V_list)
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    lens32 = lens.astype(np.int32)
    lens32[1] = 0
    out = oracle.contiguous_cache_decode(q, k, v, lens32, 0.25, "f32")
    assert np.all(np.isfinite(out)) and not out[1].any()


# --------------------------------------------------------------------------
# planted mistakes in the cache indexing
# --------------------------------------------------------------------------

_DECODE = oa.decode_contiguous


def _mut_v_tile_swapped(q, k_cache, v_cache, seq_lens, scale, dtype, rows=None):
    out = np.zeros(q.shape)
    for b in range(q.shape[0]):
        L = int(seq_lens[b])
        t = np.arange(L)
        K = oa.as_f64(k_cache[b, :, :L, :], dtype)
        V = oa.as_f64(v_cache[b, :, t % 16, :, t // 16], dtype).transpose(1, 0, 2)
        out[b] = _DECODE(oa.as_f64(q[b], dtype), K, V, scale)
    return out


def _mut_past_length(q, k_cache, v_cache, seq_lens, scale, dtype, rows=None):
    return _ORIG(q, k_cache, v_cache, np.asarray(seq_lens) + 1, scale, dtype, rows)


def _mut_plain_transposed_v(q, k_cache, v_cache, seq_lens, scale, dtype, rows=None):
    B, Hkv, T, D, _ = v_cache.shape
    flat = v_cache.reshape(B, Hkv, D, T * 16)  # V read as [B, Hkv, D, Lmax]
    out = np.zeros(q.shape)
    for b in range(B):
        L = int(seq_lens[b])
        K = oa.as_f64(k_cache[b, :, :L, :], dtype)
        V = oa.as_f64(flat[b, :, :, :L], dtype).transpose(0, 2, 1)
        out[b] = _DECODE(oa.as_f64(q[b], dtype), K, V, scale)
    return out


def _mut_k_for_v(q, k_cache, v_cache, seq_lens, scale, dtype, rows=None):
    out = np.zeros(q.shape)
    for b in range(q.shape[0]):
        L = int(seq_lens[b])
        K = oa.as_f64(k_cache[b, :, :L, :], dtype)
        out[b] = _DECODE(oa.as_f64(q[b], dtype), K, K, scale)
    return out


_ORIG = oa.contiguous_cache_decode
MUTATIONS = {"v_tile_swapped": _mut_v_tile_swapped, "past_length": _mut_past_length,
             "plain_transposed_v": _mut_plain_transposed_v, "k_for_v": _mut_k_for_v}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    assert sdpa_error(940) < 1e-12
    monkeypatch.setattr(oa, "contiguous_cache_decode", MUTATIONS[name])
    assert sdpa_error(940) > 1e-6, f"mutation {name} went unnoticed"
