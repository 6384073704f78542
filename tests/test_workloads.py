"""The seeded input generators: determinism, shapes, placement, poison."""

import math

import numpy as np
import torch

import workloads as wl
from workloads import to_numpy


def _valid_mask(case):
    """Boolean [NB, 16] marking slots some sequence references."""
    nb = case.num_blocks
    m = np.zeros((nb, 16), bool)
    for b, L in enumerate(case.seq_lens.tolist()):
        for t in range(L):
            m[int(case.block_tables[b, t // 16]), t % 16] = True
    return m


def _check_poison(case, written_slots=()):
    m = _valid_mask(case)
    for s in written_slots:
        if s >= 0:
            m[s // 16, s % 16] = False
    k = case.k_pool.float()
    v = case.v_pool.float()
    kv_nan = torch.isnan(k).all(dim=3).all(dim=1).numpy()          # [NB, 16]
    vv_nan = torch.isnan(v).all(dim=2).all(dim=1).numpy()          # [NB, 16]
    assert not np.isnan(k.numpy()[m.nonzero()[0], :, m.nonzero()[1], :]).any()
    assert (kv_nan == ~m).all() and (vv_nan == ~m).all()


def test_config1_layout_and_poison():
    c = wl.config1()
    assert c.dtype == "f32" and tuple(c.q.shape) == (4, 4, 64)
    assert tuple(c.k_pool.shape) == (32, 2, 16, 64)
    assert tuple(c.v_pool.shape) == (32, 2, 64, 16)
    assert c.seq_lens.tolist() == [1, 17, 33, 50]
    used = {int(c.block_tables[b, j]) for b in range(4)
            for j in range(math.ceil(c.seq_lens[b].item() / 16))}
    assert len(used) == 10
    _check_poison(c)
    assert c.scale == 1.0 / 8.0


def test_config2_shapes_lengths_and_write_slots():
    c = wl.config2()
    L = c.seq_lens.numpy()
    assert L.min() >= 128 and L.max() <= 4096 and len(L) == 64
    assert c.num_blocks == sum(math.ceil(x / 16) for x in L) + 1
    s = c.slot_mapping.numpy()
    for b in range(64):
        pos = L[b] - 1
        assert s[b] == int(c.block_tables[b, pos // 16]) * 16 + pos % 16
    _check_poison(c, written_slots=s)


def test_deterministic():
    a, b = wl.config2(), wl.config2()
    assert torch.equal(a.block_tables, b.block_tables)
    assert torch.equal(a.q.view(torch.int16), b.q.view(torch.int16))
    assert torch.equal(a.k_pool.view(torch.int16), b.k_pool.view(torch.int16))


def test_config3_admission_fork_and_cow():
    c = wl.config3()
    m = c.meta
    assert m["admitted"] == [True] * 7 + [False]
    assert m["used_after_admission"] == 247 and m["free_after_admission"] == 9
    assert m["refcount_prefix_after_fork"] == 8
    assert m["refcount_last_after_fork"] == 2
    assert len(m["cow_pairs"]) == 1
    assert m["refcount_after_cow"] == {"src": 1, "dst": 1}
    assert m["free_after_step"] == 8
    assert c.seq_lens.tolist() == [2306] * 8
    assert c.block_tables.shape == (8, 145)
    # all eight share the 128 prompt blocks
    assert (c.block_tables[:, :128] == c.block_tables[0, :128]).all()
    src, dst = m["cow_pairs"][0]
    assert int(c.block_tables[0, 144]) == src and int(c.block_tables[7, 144]) == dst
    assert int(c.slot_mapping[7]) == dst * 16 + 1
    assert int(c.slot_mapping[0]) == src * 16 + 1
    assert torch.isnan(c.k_pool[dst].float()).all()   # filled only by the copy


def test_config4_lengths():
    L = wl.config4_lens()
    assert len(L) == 256 and L.min() >= 16 and L.max() <= 8192
    assert 700 < np.median(L) < 1500


def test_config5_specs():
    for bk in wl.C5_BUCKETS:
        s = wl.config5_spec(bk)
        assert s.block_tables.shape == (bk, 512)
        assert bk // 2 + 1 <= s.n_real <= bk
        assert (s.seq_lens[s.n_real:] == 0).all()
        assert (s.seq_lens[:s.n_real] >= 1).all() and (s.seq_lens <= 8192).all()
        assert s.num_blocks == sum(math.ceil(int(x) / 16) for x in s.seq_lens) + 1


def test_permutation_relabels_consistently():
    c = wl.random_case(3, 4, 8, 2, 32, "f32", max_len=100, with_write=True)
    p = wl.permute_physical(c, 9)
    for b in range(4):
        for t in range(int(c.seq_lens[b]) - 1):
            i0, i1 = int(c.block_tables[b, t // 16]), int(p.block_tables[b, t // 16])
            assert torch.equal(c.k_pool[i0, :, t % 16], p.k_pool[i1, :, t % 16])
            assert torch.equal(c.v_pool[i0, :, :, t % 16], p.v_pool[i1, :, :, t % 16])


def test_latent_case_layout_and_poison():
    c = wl.latent_case(31, [1, 64, 65, 0, 200], num_heads=8)
    assert c.q.shape == (5, 8, wl.LATENT_DIM)
    nb, bs, C = c.kv_pool.shape
    assert (bs, C) == (wl.LATENT_BLOCK, wl.LATENT_DIM)
    used = np.zeros((nb, bs), bool)
    for b, L in enumerate(c.seq_lens.tolist()):
        for t in range(L):
            used[int(c.block_tables[b, t // bs]), t % bs] = True
    nan = torch.isnan(c.kv_pool.float()).all(dim=2).numpy()
    assert np.array_equal(nan, ~used)          # every unread slot is poison, no read slot is
    assert nb == sum(math.ceil(L / bs) for L in c.seq_lens.tolist()) + 1
    b = wl.latent_decode_batch()
    assert b.q.shape == (256, 128, 576) and b.kv_pool.dtype == torch.bfloat16
    assert np.array_equal(b.seq_lens.numpy(), wl.config4_lens())


def test_contiguous_cache_layout():
    """The unpaged cache holds each row's tokens in order (checked against the
    table walk) and poison everywhere past the row's length."""
    c = wl.random_case(77, 6, 8, 2, 32, "bf16", lens=[0, 1, 15, 16, 17, 70])
    k, v = wl.contiguous_cache(c)
    kp, vp = to_numpy(c.k_pool), to_numpy(c.v_pool)
    kc, vc = to_numpy(k), to_numpy(v)
    bt = to_numpy(c.block_tables)
    for b, L in enumerate(c.seq_lens.tolist()):
        for t in range(L):
            blk = bt[b, t // 16]
            assert np.array_equal(kc[b, :, t, :], kp[blk, :, t % 16, :])
            assert np.array_equal(vc[b, :, t // 16, :, t % 16], vp[blk, :, :, t % 16])
        assert np.all(kc[b, :, L:, :] == 0x7FC0)
        tt = np.arange(L, kc.shape[2])
        assert np.all(vc[b, :, tt // 16, :, tt % 16] == 0x7FC0)
