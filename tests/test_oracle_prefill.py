"""Pins of the chunked-prefill oracle (``oracle.paged_prefill``) to things
other than itself:

* brute force: scalar loops with their own table walk and causal test;
* a library routine: torch's scaled_dot_product_attention in float64 with an
  explicit mask (query i of a chunk of n over L keys sees keys 0 .. L - n + i);
* reductions: a one-token chunk is the decode step; splitting a prompt into
  chunks changes nothing (bitwise);
* planted mistakes: a causal off-by-one and chunk positions counted from 0
  instead of from the cached length must each fail a pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa
import workloads as wl
from workloads import to_numpy


def args_of(c):
    return dict(q=to_numpy(c.q), k_pool=None, v_pool=None,
                block_tables=to_numpy(c.block_tables), seq_lens=to_numpy(c.seq_lens),
                query_start=to_numpy(c.query_start), scale=c.scale, dtype=c.dtype,
                block_size=c.block_size)


def written_pools(c):
    """Host pools after the chunk's append (the oracle's own write)."""
    return oracle.write_kv(to_numpy(c.k_pool), to_numpy(c.v_pool), to_numpy(c.k_new),
                           to_numpy(c.v_new), to_numpy(c.slot_mapping), block_size=c.block_size)


def run_oracle(c, fn=None):
    k, v = written_pools(c)
    a = args_of(c)
    a["k_pool"], a["v_pool"] = k, v
    return (fn or oracle.paged_prefill)(**a)


def brute_force(c):
    """Scalar loops: own table walk, own causal test, math.exp."""
    k, v = written_pools(c)
    q = oa.as_f64(to_numpy(c.q), c.dtype)
    kf, vf = oa.as_f64(k, c.dtype), oa.as_f64(v, c.dtype)
    bt, lens, qs = to_numpy(c.block_tables), to_numpy(c.seq_lens), to_numpy(c.query_start)
    bs = c.block_size
    T, Hq, D = q.shape
    Hkv = kf.shape[1]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    for s in range(len(lens)):
        n = int(qs[s + 1] - qs[s])
        L = int(lens[s])
        for i in range(n):
            row = int(qs[s]) + i
            pos = L - n + i
            for h in range(Hq):
                kv = h // G
                sc = []
                for t in range(L):
                    if t > pos:
                        break
                    blk, sl = int(bt[s][t // bs]), t % bs
                    sc.append(c.scale * sum(float(q[row, h, d]) * float(kf[blk, kv, sl, d])
                                            for d in range(D)))
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = sum(w)
                for d in range(D):
                    acc = 0.0
                    for t, wt in enumerate(w):
                        blk, sl = int(bt[s][t // bs]), t % bs
                        acc += wt * float(vf[blk, kv, d, sl])
                    out[row, h, d] = acc / tot
    return out


TINY = [([3, 1, 5], [0, 17, 9]), ([1, 1], [30, 0]), ([6, 2, 4], [16, 1, 33])]


@pytest.mark.parametrize("chunks,contexts", TINY)
def test_brute_force(chunks, contexts):
    c = wl.prefill_case(11, chunks, contexts, 4, 2, 8, "f32")
    np.testing.assert_allclose(run_oracle(c), brute_force(c), rtol=0, atol=1e-12)


def sdpa(c):
    k, v = written_pools(c)
    lens, qs = to_numpy(c.seq_lens), to_numpy(c.query_start)
    q = oa.as_f64(to_numpy(c.q), c.dtype)
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D))
    for s in range(len(lens)):
        n, L = int(qs[s + 1] - qs[s]), int(lens[s])
        K, V = oa.gather_sequence(k, v, to_numpy(c.block_tables)[s], L, c.dtype, c.block_size)
        G = Hq // K.shape[0]
        kt = torch.from_numpy(K).repeat_interleave(G, dim=0)[None]   # [1, Hq, L, D]
        vt = torch.from_numpy(V).repeat_interleave(G, dim=0)[None]
        qt = torch.from_numpy(q[qs[s]:qs[s + 1]].transpose(1, 0, 2).copy())[None]  # [1, Hq, n, D]
        allowed = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed,
                                                             scale=c.scale)
        out[qs[s]:qs[s + 1]] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("bs", [16, 8, 64])
def test_sdpa_with_bottom_right_causal_mask(bs):
    c = wl.prefill_case(12 + bs, [37, 1, 64, 5], [100, 40, 0, 300], 8, 2, 32, "bf16",
                        block_size=bs)
    np.testing.assert_allclose(run_oracle(c), sdpa(c), rtol=0, atol=1e-12)


def test_one_token_chunks_are_the_decode_step():
    c = wl.prefill_case(13, [1, 1, 1, 1], [0, 15, 16, 400], 8, 2, 32, "bf16")
    k, v = written_pools(c)
    dec = oracle.paged_decode(to_numpy(c.q), k, v, to_numpy(c.block_tables),
                              to_numpy(c.seq_lens), c.scale, c.dtype)
    np.testing.assert_array_equal(run_oracle(c), dec)


def test_chunking_changes_nothing():
    """One 300-token prompt prefilled in one piece, or as 128 + 128 + 44 in
    three steps over the same cache, gives the same outputs, bit for bit."""
    whole = wl.prefill_case(14, [300], [0], 8, 2, 32, "bf16")
    k, v = written_pools(whole)
    a = args_of(whole)
    a["k_pool"], a["v_pool"] = k, v
    ref = oracle.paged_prefill(**a)
    got = np.zeros_like(ref)
    for start, n in ((0, 128), (128, 128), (256, 44)):
        a2 = dict(a, q=a["q"][start:start + n], seq_lens=np.array([start + n], np.int32),
                  query_start=np.array([0, n], np.int32))
        got[start:start + n] = oracle.paged_prefill(**a2)
    np.testing.assert_array_equal(got, ref)


# ---- planted mistakes: each must fail the brute-force pin -----------------

def _prefill_mutant(shift_pos=0, from_zero=False):
    def f(q, k_pool, v_pool, block_tables, seq_lens, query_start, scale, dtype,
          block_size=oa.BLOCK_SIZE, seqs=None):
        T, Hq, D = q.shape
        out = np.zeros((T, Hq, D))
        for s in range(len(seq_lens)):
            r0, r1 = int(query_start[s]), int(query_start[s + 1])
            n, L = r1 - r0, int(seq_lens[s])
            K, V = oa.gather_sequence(k_pool, v_pool, block_tables[s], L, dtype, block_size)
            for i in range(n):
                p = (i if from_zero else L - n + i) + shift_pos
                p = max(0, min(L - 1, p))
                out[r0 + i] = oa.decode_contiguous(oa.as_f64(q[r0 + i], dtype), K[:, :p + 1],
                                                   V[:, :p + 1], scale)
        return out
    return f


@pytest.mark.parametrize("mutant", [dict(shift_pos=-1), dict(shift_pos=1),
                                    dict(from_zero=True)])
def test_planted_mistake_is_caught(mutant):
    c = wl.prefill_case(15, [3, 5], [4, 9], 4, 2, 8, "f32")
    err = np.max(np.abs(run_oracle(c, _prefill_mutant(**mutant)) - brute_force(c)))
    assert err > 1e-3
