"""Blocks of other than 16 tokens (the block-size sweep) on the GPU: the
balanced-split decode, the fused decode step, KV append and block copy at
8 .. 256 tokens per block, and the contiguous placement, against the oracle
on the same seeded inputs (poisoned memory included)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_55_amd as pk
import workloads as wl
from parity import bits_equal, compare, gpu_out_f64, oracle_step, run_step
from workloads import to_numpy

pytestmark = pytest.mark.gpu

SIZES = [8, 32, 64, 128, 256]


@pytest.mark.parametrize("bs", SIZES)
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (64, 8, 128), (16, 2, 64)])
def test_decode_block_sizes(bs, hq, hkv, d):
    lens = [0, 1, bs - 1, bs, bs + 1, 15, 17, 700, 3000, 2 * bs + 9]
    c = wl.random_case(800 + bs + hq, len(lens), hq, hkv, d, "bf16", lens=lens, block_size=bs)
    pk.validate(c.num_blocks, c.block_tables, c.seq_lens, block_size=bs)
    ref, _, _ = oracle_step(c)
    out, _, _ = run_step(c, kernel="mfma", partition_tokens=0)
    compare(gpu_out_f64(out), ref, lens, "bf16")


@pytest.mark.parametrize("bs", [8, 64, 256])
def test_config2_shape_block_sizes(bs):
    c = wl.config2(block_size=bs)
    ref, k_ref, v_ref = oracle_step(c)
    out, k, v = run_step(c, kernel="mfma", partition_tokens=0)
    assert bits_equal(k, k_ref) and bits_equal(v, v_ref)
    compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), "bf16")


@pytest.mark.parametrize("bs", [16, 64])
def test_contiguous_placement(bs):
    c = wl.config2(block_size=bs, placement="contiguous")
    ref, _, _ = oracle_step(c)
    out, _, _ = run_step(c, kernel="mfma", partition_tokens=0)
    compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), "bf16")


@pytest.mark.parametrize("bs", [8, 32])
def test_fused_step_block_sizes(bs):
    c = wl.random_case(850 + bs, 40, 32, 8, 128, "bf16", min_len=1, max_len=900,
                       with_write=True, block_size=bs)
    pk.validate(c.num_blocks, c.block_tables, c.seq_lens, c.slot_mapping,
                append_rows=True, block_size=bs)
    ref, k_ref, v_ref = oracle_step(c)
    d = c.to("cuda")
    out = pk.pa_decode_append(d.q, d.k_new, d.v_new, d.slot_mapping, d.k_pool, d.v_pool,
                              d.block_tables, d.seq_lens, c.scale, partition_tokens=0,
                              kernel="mfma")
    torch.cuda.synchronize()
    assert bits_equal(d.k_pool, k_ref) and bits_equal(d.v_pool, v_ref)
    compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), "bf16")


@pytest.mark.parametrize("bs", [8, 64, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_write_and_copy_block_sizes(bs, dtype):
    rng = np.random.default_rng(bs)
    gen = torch.Generator().manual_seed(bs)
    td = wl.TORCH_DTYPE[dtype]
    nb, hkv, d, T = 12, 4, 128, 50
    k = torch.full((nb, hkv, bs, d), float("nan"), dtype=td)
    v = torch.full(wl.v_pool_shape(nb, hkv, d, bs), float("nan"), dtype=td)
    kn = torch.randn((T, hkv, d), generator=gen).to(td)
    vn = torch.randn((T, hkv, d), generator=gen).to(td)
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int32)
    slots[::6] = -1
    k_ref, v_ref = oracle.write_kv(to_numpy(k), to_numpy(v), to_numpy(kn), to_numpy(vn),
                                   slots, block_size=bs)
    kg, vg = k.cuda(), v.cuda()
    pk.pa_write_kv(kn.cuda(), vn.cuda(), torch.from_numpy(slots).cuda(), kg, vg)
    torch.cuda.synchronize()
    assert bits_equal(kg, k_ref) and bits_equal(vg, v_ref)
    pairs = np.array([[0, 7], [3, 11]], dtype=np.int32)
    k_ref2, v_ref2 = oracle.copy_blocks(k_ref, v_ref, pairs)
    pk.pa_copy_blocks(kg, vg, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert bits_equal(kg, k_ref2) and bits_equal(vg, v_ref2)


def test_other_block_sizes_reject_fixed_partitions():
    c = wl.random_case(870, 3, 8, 2, 64, "bf16", max_len=100, block_size=32).to("cuda")
    with pytest.raises(pk.PagedKVError):
        pk.pa_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.seq_lens, c.scale,
                     partition_tokens=512, kernel="mfma")
