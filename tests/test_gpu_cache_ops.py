"""pa_write_kv and pa_copy_blocks on the GPU: bit-exact against the oracle on
NaN-poisoned pools (every untouched slot must keep its poison bits)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_55_amd as pk
import workloads as wl
from workloads import to_numpy
from parity import bits_equal

pytestmark = pytest.mark.gpu


def _write_case(seed, nb, hkv, d, dtype, T, skip_every=0):
    rng = np.random.default_rng(seed)
    gen = torch.Generator().manual_seed(seed)
    td = wl.TORCH_DTYPE[dtype]
    k = torch.full((nb, hkv, 16, d), float("nan"), dtype=td)
    v = torch.full((nb, hkv, d, 16), float("nan"), dtype=td)
    kn = torch.randn((T, hkv, d), generator=gen).to(td)
    vn = torch.randn((T, hkv, d), generator=gen).to(td)
    slots = rng.choice(nb * 16, size=T, replace=False).astype(np.int32)
    if skip_every:
        slots[::skip_every] = -1
    return k, v, kn, vn, torch.from_numpy(slots)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hkv,d", [(2, 64), (8, 128), (1, 128)])
def test_write_kv_bit_exact(dtype, hkv, d):
    k, v, kn, vn, slots = _write_case(7 + hkv + d, 40, hkv, d, dtype, 37, skip_every=5)
    k_ref, v_ref = oracle.write_kv(to_numpy(k), to_numpy(v), to_numpy(kn), to_numpy(vn),
                                   to_numpy(slots))
    kg, vg = k.cuda(), v.cuda()
    pk.pa_write_kv(kn.cuda(), vn.cuda(), slots.cuda(), kg, vg)
    torch.cuda.synchronize()
    assert bits_equal(kg, k_ref) and bits_equal(vg, v_ref)


def test_write_kv_many_tokens():
    """More (token, head) pairs than one launch covers at once: the kernel's
    grid-stride loop takes the rest."""
    k, v, kn, vn, slots = _write_case(11, 2600, 8, 64, "bf16", 40000, skip_every=7)
    k_ref, v_ref = oracle.write_kv(to_numpy(k), to_numpy(v), to_numpy(kn), to_numpy(vn),
                                   to_numpy(slots))
    kg, vg = k.cuda(), v.cuda()
    pk.pa_write_kv(kn.cuda(), vn.cuda(), slots.cuda(), kg, vg)
    torch.cuda.synchronize()
    assert bits_equal(kg, k_ref) and bits_equal(vg, v_ref)


def test_write_kv_config2_tokens():
    c = wl.config2()
    k_ref, v_ref = oracle.write_kv(to_numpy(c.k_pool), to_numpy(c.v_pool), to_numpy(c.k_new),
                                   to_numpy(c.v_new), to_numpy(c.slot_mapping))
    d = c.to("cuda")
    pk.pa_write_kv(d.k_new, d.v_new, d.slot_mapping, d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    assert bits_equal(d.k_pool, k_ref) and bits_equal(d.v_pool, v_ref)


def test_write_kv_zero_tokens_is_noop():
    k, v, kn, vn, slots = _write_case(3, 4, 2, 64, "bf16", 1)
    kg, vg = k.cuda(), v.cuda()
    pk.pa_write_kv(kn[:0].cuda(), vn[:0].cuda(), slots[:0].cuda(), kg, vg)
    torch.cuda.synchronize()
    assert bits_equal(kg, to_numpy(k))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_copy_blocks_bit_exact(dtype):
    rng = np.random.default_rng(11)
    gen = torch.Generator().manual_seed(11)
    td = wl.TORCH_DTYPE[dtype]
    nb, hkv, d = 30, 8, 128
    k = torch.randn((nb, hkv, 16, d), generator=gen).to(td)
    v = torch.randn((nb, hkv, d, 16), generator=gen).to(td)
    k[::3] = float("nan")
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:6], perm[6:12]], axis=1).astype(np.int32)
    k_ref, v_ref = oracle.copy_blocks(to_numpy(k), to_numpy(v), pairs)
    kg, vg = k.cuda(), v.cuda()
    pk.pa_copy_blocks(kg, vg, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert bits_equal(kg, k_ref) and bits_equal(vg, v_ref)


def test_copy_then_write_config3():
    c = wl.config3()
    k_ref, v_ref = oracle.copy_blocks(to_numpy(c.k_pool), to_numpy(c.v_pool),
                                      to_numpy(c.block_mapping))
    k_ref, v_ref = oracle.write_kv(k_ref, v_ref, to_numpy(c.k_new), to_numpy(c.v_new),
                                   to_numpy(c.slot_mapping))
    d = c.to("cuda")
    pk.pa_copy_blocks(d.k_pool, d.v_pool, d.block_mapping)
    pk.pa_write_kv(d.k_new, d.v_new, d.slot_mapping, d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    assert bits_equal(d.k_pool, k_ref) and bits_equal(d.v_pool, v_ref)
