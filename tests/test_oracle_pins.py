"""Pins of the attention oracle to things other than itself.

* brute force: scalar loops with their own table walk (tiny inputs);
* a library routine: torch's scaled_dot_product_attention in float64 on
  contiguous K/V that the test scatters into a pool through a table;
* closed forms: L = 1, scale = 0, identical keys, one dominant key;
* invariants from the pages: any physical placement gives the same result,
  paged equals contiguous, shared blocks equal private copies, padded rows
  are zero, poisoned (never referenced) memory is never read;
* planted mistakes: plausible bugs put into the oracle must fail a pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa
import workloads as wl
from workloads import to_numpy

B16 = oa.BLOCK_SIZE
_GATHER = oa.gather_sequence
_DECODE = oa.decode_contiguous


def np_case(case):
    return dict(q=to_numpy(case.q), k_pool=to_numpy(case.k_pool),
                v_pool=to_numpy(case.v_pool),
                block_tables=to_numpy(case.block_tables),
                seq_lens=to_numpy(case.seq_lens), scale=case.scale,
                dtype=case.dtype)


# --------------------------------------------------------------------------
# contiguous K/V scattered into a pool by the test itself
# --------------------------------------------------------------------------

def scatter_pool(K_list, V_list, rng, extra_blocks=3, block_size=B16):
    """Pools (float32) holding per-sequence contiguous K/V [Hkv, L, D]
    at random physical blocks of ``block_size`` tokens; returns
    (k_pool, v_pool, tables, lens)."""
    B16 = block_size  # noqa: N806 (the block size this pool uses)
    lens = [k.shape[1] for k in K_list]
    Hkv, _, D = K_list[0].shape
    nblk = [math.ceil(L / B16) for L in lens]
    nb = sum(nblk) + extra_blocks
    perm = rng.permutation(nb)
    k_pool = np.full((nb, Hkv, B16, D), np.nan, dtype=np.float32)
    v_pool = np.full(wl.v_pool_shape(nb, Hkv, D, B16), np.nan, dtype=np.float32)
    mb = max(1, max(nblk))
    tables = np.full((len(lens), mb), perm[-1], dtype=np.int32)
    i = 0
    for b, L in enumerate(lens):
        for j in range(nblk[b]):
            tables[b, j] = perm[i]
            i += 1
        for t in range(L):
            blk = tables[b, t // B16]
            k_pool[blk, :, t % B16, :] = K_list[b][:, t, :]
            slot = t % B16
            if v_pool.ndim == 5:  # a dim-major V tile per 16 slots
                v_pool[blk, :, slot // 16, :, slot % 16] = V_list[b][:, t, :]
            else:
                v_pool[blk, :, :, slot] = V_list[b][:, t, :]
    return k_pool, v_pool, tables, np.array(lens, dtype=np.int32)


def sdpa_reference(q, K_list, V_list, scale):
    """torch SDPA (float64, CPU) per sequence; K/V heads repeated for GQA."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = K_list[b].shape[1]
        if L == 0:
            continue
        Hkv = K_list[b].shape[0]
        G = Hq // Hkv
        qt = torch.from_numpy(q[b].astype(np.float64))[None, :, None, :]
        kt = torch.from_numpy(K_list[b].astype(np.float64)).repeat_interleave(G, dim=0)[None]
        vt = torch.from_numpy(V_list[b].astype(np.float64)).repeat_interleave(G, dim=0)[None]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        out[b] = o[0, :, 0, :].numpy()
    return out


def sdpa_error(seed, B=3, Hq=8, Hkv=2, D=32, max_len=70, block_size=B16):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len, size=B)
    K_list = [rng.standard_normal((Hkv, L, D)).astype(np.float32) for L in lens]
    V_list = [rng.standard_normal((Hkv, L, D)).astype(np.float32) for L in lens]
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    k_pool, v_pool, tables, lens32 = scatter_pool(K_list, V_list, rng, block_size=block_size)
    got = oracle.paged_decode(q, k_pool, v_pool, tables, lens32, scale, "f32",
                              block_size=block_size)
    ref = sdpa_reference(q, K_list, V_list, scale)
    err = np.abs(got - ref)
    return float("inf") if np.isnan(err).any() else float(np.max(err))


def brute_error(seed, B=3, Hq=4, Hkv=2, D=8, max_len=40, dtype="f32", block_size=B16):
    case = wl.random_case(seed, B, Hq, Hkv, D, dtype, max_len=max_len, block_size=block_size)
    a = np_case(case)
    got = oracle.paged_decode(**a, block_size=block_size)
    ref = oracle.brute_force_decode(**a, block_size=block_size)
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed,G", [(1, 1), (2, 2), (3, 4), (4, 2), (5, 1)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_brute_force_tiny(seed, G, dtype):
    Hkv = 2
    assert brute_error(seed, Hq=G * Hkv, Hkv=Hkv, dtype=dtype) < 1e-12


@pytest.mark.parametrize("bs", [8, 32, 64, 256])
def test_brute_force_other_block_sizes(bs):
    """Blocks of other sizes (the block-size sweep): the table walk indexes
    block t // bs at slot t % bs."""
    assert brute_error(70 + bs, Hq=8, Hkv=2, max_len=300, dtype="bf16", block_size=bs) < 1e-12


@pytest.mark.parametrize("bs", [8, 32, 256])
def test_sdpa_library_other_block_sizes(bs):
    assert sdpa_error(30 + bs, max_len=600, block_size=bs) < 1e-12


def test_brute_force_config1():
    a = np_case(wl.config1())
    got = oracle.paged_decode(**a)
    ref = oracle.brute_force_decode(**a)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("seed", [10, 11, 12])
def test_sdpa_library_gqa(seed):
    assert sdpa_error(seed) < 1e-12


def test_sdpa_library_mha_and_d128():
    assert sdpa_error(20, B=2, Hq=4, Hkv=4, D=128, max_len=50) < 1e-12


def test_sdpa_library_config2_sample():
    """Config 2's real shapes on a sample of three sequences."""
    case = wl.config2(batch=64)
    a = np_case(case)
    rows = [0, 17, 63]
    K_list, V_list = [], []
    for b in rows:
        K, V = oracle.gather_sequence(a["k_pool"], a["v_pool"], a["block_tables"][b],
                                      a["seq_lens"][b] - 1, "bf16")
        # the newest token is poisoned until the write; attend over L - 1
        K_list.append(K)
        V_list.append(V)
    lens_m1 = a["seq_lens"].copy()
    lens_m1[rows] -= 1
    got = oracle.paged_decode(a["q"], a["k_pool"], a["v_pool"], a["block_tables"],
                              lens_m1, a["scale"], "bf16", rows=rows)
    ref = sdpa_reference(oa.as_f64(a["q"][rows], "bf16"), K_list, V_list, a["scale"])
    assert np.max(np.abs(got - ref)) < 1e-12


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_single_token_returns_its_value_exactly():
    a = np_case(wl.config1())
    out = oracle.paged_decode(**a)
    # row 0 has L = 1: every head returns V of token 0 of its KV head
    blk = a["block_tables"][0, 0]
    for h in range(4):
        kv = h // 2
        np.testing.assert_array_equal(out[0, h], oa.as_f64(a["v_pool"][blk, kv, :, 0], "f32"))


def test_zero_scale_is_mean_of_values():
    case = wl.random_case(30, 2, 4, 2, 16, "f32", min_len=1, max_len=60)
    a = np_case(case)
    a["scale"] = 0.0
    out = oracle.paged_decode(**a)
    for b in range(2):
        L = int(a["seq_lens"][b])
        _, V = oracle.gather_sequence(a["k_pool"], a["v_pool"], a["block_tables"][b], L, "f32")
        # by construction of the pool: independent mean via the test's own walk
        vals = np.stack([[a["v_pool"][a["block_tables"][b][t // 16], kv, :, t % 16]
                          for t in range(L)] for kv in range(2)]).astype(np.float64)
        mean = vals.mean(axis=1)
        for h in range(4):
            np.testing.assert_allclose(out[b, h], mean[h // 2], rtol=0, atol=1e-12)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(31)
    Hkv, D, L = 2, 16, 37
    key = rng.standard_normal((Hkv, 1, D)).astype(np.float32)
    K = np.repeat(key, L, axis=1)
    V = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    q = rng.standard_normal((1, 4, D)).astype(np.float32)
    k_pool, v_pool, tables, lens = scatter_pool([K], [V], rng)
    out = oracle.paged_decode(q, k_pool, v_pool, tables, lens, 0.7, "f32")
    for h in range(4):
        np.testing.assert_allclose(out[0, h], V[h // 2].astype(np.float64).mean(axis=0), atol=1e-12)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(32)
    Hkv, D, L, j = 1, 16, 45, 29
    q = rng.standard_normal((1, 2, D)).astype(np.float32)
    K = np.zeros((Hkv, L, D), dtype=np.float32)
    # key j is aligned with both query heads' sum, large
    K[0, j] = 50.0 * (q[0, 0] + q[0, 1])
    V = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    k_pool, v_pool, tables, lens = scatter_pool([K], [V], rng)
    out = oracle.paged_decode(q, k_pool, v_pool, tables, lens, 1.0, "f32")
    for h in range(2):
        if float(q[0, h] @ (q[0, 0] + q[0, 1])) > 1.0:
            np.testing.assert_allclose(out[0, h], V[0, j], atol=1e-9)


# --------------------------------------------------------------------------
# invariants stated by the pages
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_physical_placement_invariance_bitwise(dtype):
    case = wl.random_case(40, 4, 8, 2, 32, dtype, max_len=120)
    perm = wl.permute_physical(case, 7)
    a, b = np_case(case), np_case(perm)
    np.testing.assert_array_equal(oracle.paged_decode(**a), oracle.paged_decode(**b))


@pytest.mark.parametrize("bs", [16, 8, 64, 256])
def test_paged_equals_contiguous_bitwise(bs):
    rng = np.random.default_rng(41)
    Hkv, D = 2, 32
    lens = [5, 16, 33, 64, 300]
    K_list = [rng.standard_normal((Hkv, L, D)).astype(np.float32) for L in lens]
    V_list = [rng.standard_normal((Hkv, L, D)).astype(np.float32) for L in lens]
    q = rng.standard_normal((5, 4, D)).astype(np.float32)
    k_pool, v_pool, tables, lens32 = scatter_pool(K_list, V_list, rng, block_size=bs)
    paged = oracle.paged_decode(q, k_pool, v_pool, tables, lens32, 0.3, "f32", block_size=bs)
    for b in range(5):
        contig = oracle.decode_contiguous(q[b].astype(np.float64),
                                          K_list[b].astype(np.float64),
                                          V_list[b].astype(np.float64), 0.3)
        np.testing.assert_array_equal(paged[b], contig)


def test_shared_blocks_equal_private_copies():
    case = wl.config3()
    a = np_case(case)
    k2, v2 = oracle.write_kv(*oracle.copy_blocks(a["k_pool"], a["v_pool"],
                                                 to_numpy(case.block_mapping)),
                             to_numpy(case.k_new), to_numpy(case.v_new),
                             to_numpy(case.slot_mapping))
    rows = [1, 2]
    shared = oracle.paged_decode(a["q"], k2, v2, a["block_tables"], a["seq_lens"],
                                 a["scale"], "bf16", rows=rows)
    # give row 1 and 2 private copies of the 128 prefix blocks
    nb = k2.shape[0]
    tables = a["block_tables"].copy()
    k3 = np.concatenate([k2, np.zeros((256, *k2.shape[1:]), k2.dtype)])
    v3 = np.concatenate([v2, np.zeros((256, *v2.shape[1:]), v2.dtype)])
    nxt = nb
    for r in rows:
        for j in range(128):
            k3[nxt] = k2[tables[r, j]]
            v3[nxt] = v2[tables[r, j]]
            tables[r, j] = nxt
            nxt += 1
    private = oracle.paged_decode(a["q"], k3, v3, tables, a["seq_lens"], a["scale"],
                                  "bf16", rows=rows)
    np.testing.assert_array_equal(shared, private)


def test_gqa_equals_mha_on_repeated_heads():
    case = wl.random_case(42, 3, 8, 2, 16, "f32", max_len=90)
    a = np_case(case)
    gqa = oracle.paged_decode(**a)
    a2 = dict(a)
    a2["k_pool"] = np.repeat(a["k_pool"], 4, axis=1)
    a2["v_pool"] = np.repeat(a["v_pool"], 4, axis=1)
    mha = oracle.paged_decode(**a2)
    # the grouped and per-head products sum in different orders (BLAS)
    np.testing.assert_allclose(gqa, mha, rtol=0, atol=1e-13)


def test_padded_rows_are_zero_and_poison_unread():
    case = wl.random_case(43, 5, 4, 2, 16, "f32", lens=[0, 7, 0, 16, 33])
    a = np_case(case)
    out = oracle.paged_decode(**a)
    assert np.all(out[[0, 2]] == 0.0)
    assert np.all(np.isfinite(out))
    assert np.isnan(a["k_pool"][case.poison_block]).all()


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_bf16_widening_matches_torch():
    x = torch.randn(4096, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    ours = oa.as_f64(to_numpy(x), "bf16")
    np.testing.assert_array_equal(ours, x.to(torch.float64).numpy())


def test_bf16_rounding_matches_torch():
    g = torch.Generator().manual_seed(2)
    x = torch.randn(20000, generator=g, dtype=torch.float32) * 3
    # exact ties and specials
    specials = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),
                             0.0, -0.0, float("inf"), -float("inf"), 3.0e38,
                             1e-40, -1e-40], dtype=torch.float32)
    x = torch.cat([x, specials])
    ours = oa.round_to_bf16_bits(x.numpy().astype(np.float64))
    ref = to_numpy(x.to(torch.bfloat16))
    np.testing.assert_array_equal(ours, ref)
    nan_bits = oa.round_to_bf16_bits(np.array([np.nan]))
    assert (int(nan_bits[0]) & 0x7F80) == 0x7F80 and (int(nan_bits[0]) & 0x7F) != 0


# --------------------------------------------------------------------------
# cache maintenance by construction
# --------------------------------------------------------------------------

def test_write_kv_moves_exact_bits_and_nothing_else():
    rng = np.random.default_rng(50)
    k = rng.integers(0, 2 ** 16, size=(6, 2, 16, 8), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(6, 2, 8, 16), dtype=np.uint16)
    kn = rng.integers(0, 2 ** 16, size=(3, 2, 8), dtype=np.uint16)
    vn = rng.integers(0, 2 ** 16, size=(3, 2, 8), dtype=np.uint16)
    slots = np.array([5 * 16 + 3, -1, 0 * 16 + 15], dtype=np.int32)
    k2, v2 = oracle.write_kv(k, v, kn, vn, slots)
    for h in range(2):
        for d in range(8):
            assert k2[5, h, 3, d] == kn[0, h, d] and v2[5, h, d, 3] == vn[0, h, d]
            assert k2[0, h, 15, d] == kn[2, h, d] and v2[0, h, d, 15] == vn[2, h, d]
    mask_k = np.ones(k.shape, bool)
    mask_k[5, :, 3, :] = False
    mask_k[0, :, 15, :] = False
    mask_v = np.ones(v.shape, bool)
    mask_v[5, :, :, 3] = False
    mask_v[0, :, :, 15] = False
    np.testing.assert_array_equal(k2[mask_k], k[mask_k])
    np.testing.assert_array_equal(v2[mask_v], v[mask_v])


def test_copy_blocks_duplicates_whole_blocks():
    rng = np.random.default_rng(51)
    k = rng.integers(0, 2 ** 16, size=(6, 2, 16, 8), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(6, 2, 8, 16), dtype=np.uint16)
    k2, v2 = oracle.copy_blocks(k, v, np.array([[1, 4], [2, 0]], dtype=np.int32))
    np.testing.assert_array_equal(k2[4], k[1])
    np.testing.assert_array_equal(v2[4], v[1])
    np.testing.assert_array_equal(k2[0], k[2])
    for i in (1, 2, 3, 5):
        np.testing.assert_array_equal(k2[i], k[i])
        np.testing.assert_array_equal(v2[i], v[i])


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin
# --------------------------------------------------------------------------

def _gather_wrong_slot(k_pool, v_pool, table_row, seq_len, dtype, block_size=16):
    L = int(seq_len)
    t = np.arange(L)
    phys = np.asarray(table_row)[t // block_size]
    slot = (t + 1) % block_size  # off by one inside the block
    K = oa.as_f64(k_pool[phys, :, slot, :], dtype).transpose(1, 0, 2)
    V = oa.as_f64(v_pool[phys, :, :, slot], dtype).transpose(1, 0, 2)
    return K, V


def _gather_v_token_major(k_pool, v_pool, table_row, seq_len, dtype, block_size=16):
    L = int(seq_len)
    t = np.arange(L)
    phys = np.asarray(table_row)[t // block_size]
    slot = t % block_size
    K = oa.as_f64(k_pool[phys, :, slot, :], dtype).transpose(1, 0, 2)
    # V read as if it were token-major: wrong layout
    vv = v_pool.reshape(v_pool.shape[0], v_pool.shape[1], block_size, -1)
    V = oa.as_f64(vv[phys, :, slot, :], dtype).transpose(1, 0, 2)
    return K, V


def _gather_drops_last(k_pool, v_pool, table_row, seq_len, dtype, block_size=16):
    return _GATHER(k_pool, v_pool, table_row, max(int(seq_len) - 1, 1), dtype,
                   block_size)


def _decode_head_modulo(q_b, K, V, scale):
    Hq, D = q_b.shape
    Hkv, L, _ = K.shape
    out = np.zeros((Hq, D))
    for h in range(Hq):
        kv = h % Hkv  # interleaved instead of contiguous groups
        s = scale * (K[kv] @ q_b[h])
        p = np.exp(s - s.max())
        out[h] = (p @ V[kv]) / p.sum()
    return out


def _decode_no_scale(q_b, K, V, scale):
    return _DECODE(q_b, K, V, 1.0)


def _decode_k_for_v(q_b, K, V, scale):
    return _DECODE(q_b, K, K, scale)


MUTATIONS = {
    "wrong_slot": ("gather_sequence", _gather_wrong_slot),
    "v_token_major": ("gather_sequence", _gather_v_token_major),
    "drops_last_token": ("gather_sequence", _gather_drops_last),
    "head_modulo": ("decode_contiguous", _decode_head_modulo),
    "no_scale": ("decode_contiguous", _decode_no_scale),
    "k_for_v": ("decode_contiguous", _decode_k_for_v),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    assert sdpa_error(60, B=3, Hq=4, Hkv=2, D=16, max_len=40) < 1e-12
    monkeypatch.setattr(oa, attr, fn)
    assert sdpa_error(60, B=3, Hq=4, Hkv=2, D=16, max_len=40) > 1e-6, \
        f"mutation {name} went unnoticed"
