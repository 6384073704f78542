"""pa_decode on the GPU against the float64 oracle on the same seeded inputs.

Covers the five configurations (configuration 4 and the first and last
layers of the 32-layer step at every bucket on every row), small random cases that span several tiles and
partitions with ragged tails, every supported head group and head dim, both
decode kernels, padded rows, poisoned memory, run-to-run determinism,
placement invariance and sharing exactness (bitwise).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_55_amd as pk
import workloads as wl
from workloads import to_numpy
from parity import (bits_equal, compare, gpu_out_f64, oracle_config5_rows, oracle_inputs,
                    oracle_step, run_step)

pytestmark = pytest.mark.gpu

BF16_KERNELS = ["mfma", "valu"]


def _kernels(dtype):
    return BF16_KERNELS if dtype == "bf16" else ["valu"]


# --------------------------------------------------------------------------
# configuration 1: tiny fp32
# --------------------------------------------------------------------------

@pytest.mark.parametrize("partition", [0, 16, 32, 512])
def test_config1_fp32(partition):
    c = wl.config1()
    ref, _, _ = oracle_step(c)
    out, _, _ = run_step(c, partition_tokens=partition)
    compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), "f32")


def test_config1_single_token_row_is_its_value():
    c = wl.config1()
    out, _, _ = run_step(c)
    blk = int(c.block_tables[0, 0])
    o = out.cpu()
    for h in range(4):
        np.testing.assert_allclose(o[0, h].numpy(), c.v_pool[blk, h // 2, :, 0].numpy(),
                                   rtol=0, atol=1e-6)


# --------------------------------------------------------------------------
# small random cases: tiles, partitions, ragged tails
# --------------------------------------------------------------------------

CASES = []
for dtype in ("f32", "bf16"):
    for D in (64, 128):
        for G in (1, 2, 4, 8, 16):
            CASES.append((dtype, D, G))


@pytest.mark.parametrize("dtype,D,G", CASES)
def test_random_small(dtype, D, G):
    Hkv = 2
    lens = [0, 1, 15, 16, 17, 33, 100, 255, 257, 600]
    c = wl.random_case(100 + D + G, len(lens), G * Hkv, Hkv, D, dtype, lens=lens,
                       extra_table_cols=3)
    ref, _, _ = oracle_step(c)
    for kernel in _kernels(dtype):
        for part in (0, 16, 48, 256):
            out, _, _ = run_step(c, kernel=kernel, partition_tokens=part)
            compare(gpu_out_f64(out), ref, lens, dtype)


@pytest.mark.parametrize("seed", range(4))
def test_random_lengths_bf16(seed):
    c = wl.random_case(200 + seed, 9, 32, 8, 128, "bf16", max_len=1100, with_write=True)
    ref, _, _ = oracle_step(c)
    for kernel in BF16_KERNELS:
        out, _, _ = run_step(c, kernel=kernel, partition_tokens=512)
        compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), "bf16")


# --------------------------------------------------------------------------
# configuration 2: 8B-shaped layer, write then decode, full batch
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def config2_ref():
    c = wl.config2()
    ref, k, v = oracle_step(c)
    return c, ref, k, v


@pytest.mark.parametrize("kernel", BF16_KERNELS)
@pytest.mark.parametrize("partition", [512, 256, 0])
def test_config2_full(config2_ref, kernel, partition):
    c, ref, k_ref, v_ref = config2_ref
    out, k, v = run_step(c, kernel=kernel, partition_tokens=partition)
    assert bits_equal(k, k_ref) and bits_equal(v, v_ref)
    worst = compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), "bf16")
    print(f"config2 {kernel} part={partition} worst ratio {worst:.3f}")


# --------------------------------------------------------------------------
# configuration 3: copy-on-write over a shared prefix
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", BF16_KERNELS)
def test_config3_cow(kernel):
    c = wl.config3()
    ref, k_ref, v_ref = oracle_step(c)
    out, k, v = run_step(c, kernel=kernel)
    assert bits_equal(k, k_ref) and bits_equal(v, v_ref)
    compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), "bf16")
    # sequence 0 and its fork differ only in the last token
    assert not torch.equal(out[0], out[7])


def test_config3_sharing_is_exact():
    """Shared prefix blocks and private copies of them give identical bits."""
    c = wl.config3()
    out_shared, k, v = run_step(c)
    nb = c.num_blocks
    tables = c.block_tables.clone()
    extra_k = torch.empty((128 * 2, *c.k_pool.shape[1:]), dtype=c.k_pool.dtype, device="cuda")
    extra_v = torch.empty((128 * 2, *c.v_pool.shape[1:]), dtype=c.v_pool.dtype, device="cuda")
    nxt = 0
    for r in (1, 2):
        for j in range(128):
            extra_k[nxt] = k[tables[r, j]]
            extra_v[nxt] = v[tables[r, j]]
            tables[r, j] = nb + nxt
            nxt += 1
    k2 = torch.cat([k, extra_k]).contiguous()
    v2 = torch.cat([v, extra_v]).contiguous()
    d = c.to("cuda")
    out_private = pk.pa_decode(d.q, k2, v2, tables.cuda(), d.seq_lens, c.scale,
                               partition_tokens=c.partition_tokens)
    torch.cuda.synchronize()
    assert torch.equal(out_shared.view(torch.int16), out_private.view(torch.int16))


# --------------------------------------------------------------------------
# configuration 4: 70B-shaped layer, full size, every row
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def config4_ref():
    c = wl.config4()
    return c, oracle.paged_decode(**oracle_inputs(c))


@pytest.mark.parametrize("kernel,partition", [("mfma", 512), ("mfma", 0), ("valu", 512)])
def test_config4_full_batch(config4_ref, kernel, partition):
    """Every one of the 256 rows against the oracle (about 10 s of oracle work,
    shared by the three kernel variants)."""
    c, ref = config4_ref
    out, _, _ = run_step(c, kernel=kernel, partition_tokens=partition)
    worst = compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), "bf16")
    print(f"config4 {kernel} part={partition} worst ratio {worst:.3f} over 256 rows")


@pytest.mark.parametrize("lens", [
    [8000],                                     # one pair cut into many pieces
    [0, 5, 0, 0, 17, 1, 0, 300, 16, 0],         # tiny pairs, padded rows between
    [4096, 1, 1, 1, 2000, 33, 0, 8192, 15],     # mixed
    [1] * 64,                                   # one block per pair
])
def test_balanced_split_edges(lens):
    c = wl.random_case(400 + len(lens), len(lens), 32, 8, 128, "bf16", lens=lens)
    ref, _, _ = oracle_step(c)
    for part in (0, 512):
        out, _, _ = run_step(c, kernel="mfma", partition_tokens=part)
        compare(gpu_out_f64(out), ref, lens, "bf16")


# --------------------------------------------------------------------------
# configuration 5: bucketed step with padded rows, per-layer pools
# --------------------------------------------------------------------------

def _c5_check(bucket, layers, rows=None, partitions=(512, 0)):
    """Each layer of the 32-layer step (its own pool) decoded with every
    split in `partitions`, against one oracle pass over the selected rows
    (all rows by default); padded rows must be exact zeros."""
    spec = wl.config5_spec(bucket)
    bt = torch.from_numpy(spec.block_tables).cuda()
    lens = torch.from_numpy(spec.seq_lens).cuda()
    sel = list(range(bucket)) if rows is None else rows
    for layer in layers:
        q, k, v = wl.config5_layer(spec, layer, "cuda")
        print(f"config5 bucket {bucket} layer {layer} rows {len(sel)}", flush=True)
        ref = oracle_config5_rows(spec, q, k, v, sel)
        for partition in partitions:
            out = pk.pa_decode(q, k, v, bt, lens, 1.0 / math.sqrt(128),
                               partition_tokens=partition)
            torch.cuda.synchronize()
            worst = compare(gpu_out_f64(out, sel), ref, spec.seq_lens[sel], "bf16")
            print(f"  split {partition}: worst ratio {worst:.3f}", flush=True)
            pad = out[spec.n_real:]
            assert torch.count_nonzero(pad.view(torch.int16)) == 0
            del out
        del q, k, v


@pytest.mark.parametrize("bucket", [1, 2, 4, 8])
def test_config5_small_buckets_all_rows(bucket):
    _c5_check(bucket, layers=[0, 1, 2, 31])


@pytest.mark.parametrize("bucket", [64, 256])
def test_config5_large_buckets_all_rows(bucket):
    """Every row (real and padded) of the first and last layers."""
    _c5_check(bucket, layers=[0, 31])


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kernel,partition", [("mfma", 512), ("mfma", 0), ("valu", 512)])
def test_deterministic_and_placement_invariant(kernel, partition):
    c = wl.random_case(300, 12, 32, 8, 128, "bf16", max_len=2000)
    out1, _, _ = run_step(c, kernel=kernel, partition_tokens=partition)
    out2, _, _ = run_step(c, kernel=kernel, partition_tokens=partition)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    p = wl.permute_physical(c, 3)
    out3, _, _ = run_step(p, kernel=kernel, partition_tokens=partition)
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))


def test_kernels_agree_within_tolerance():
    c = wl.random_case(301, 6, 64, 8, 128, "bf16", max_len=3000)
    ref, _, _ = oracle_step(c)
    a, _, _ = run_step(c, kernel="mfma")
    b, _, _ = run_step(c, kernel="valu")
    compare(gpu_out_f64(a), ref, c.seq_lens.numpy(), "bf16")
    compare(gpu_out_f64(b), ref, c.seq_lens.numpy(), "bf16")


@pytest.mark.parametrize("lens,hq,hkv", [
    ([8000], 32, 2),     # G = 16: each pair cut into 32 pieces
    ([70000], 2, 1),     # one pair cut into > 256 pieces (many merge batches)
])
def test_balanced_many_pieces(lens, hq, hkv):
    c = wl.random_case(450 + hq, len(lens), hq, hkv, 128, "bf16", lens=lens)
    ref, _, _ = oracle_step(c)
    out, _, _ = run_step(c, kernel="mfma", partition_tokens=0)
    compare(gpu_out_f64(out), ref, lens, "bf16")


@pytest.mark.parametrize("lens", [[70000], [70000, 3, 0, 2000]])
def test_fixed_many_partitions(lens):
    """512-token partitions: a 70,000-token row is 137 partitions, merged in
    the decode kernel by the last one to finish over several rounds of
    loads (each thread of a 4-dim unit takes up to 16 partitions a round)."""
    c = wl.random_case(455 + len(lens), len(lens), 32, 8, 128, "bf16", lens=lens)
    ref, _, _ = oracle_step(c)
    out, _, _ = run_step(c, kernel="mfma", partition_tokens=512)
    compare(gpu_out_f64(out), ref, lens, "bf16")


@pytest.mark.parametrize("partition", [256, 64])
def test_fixed_partials_at_extreme_magnitudes(partition):
    """The fixed split at outputs far from 1: V scaled by 1e-6 .. 3e4 per
    KV head, so that heads of one row differ by ten orders of magnitude
    through the partials and their merge; every row meets the oracle's
    bar."""
    lens = [3000, 700, 1, 1800, 0, 257]
    c = wl.random_case(492, len(lens), 32, 8, 128, "bf16", lens=lens)
    gains = torch.tensor([1e-6, 1e-3, 1.0, 30.0, 1e3, 3e4, 1.0, 0.5]).view(1, 8, 1, 1)
    c.v_pool = (c.v_pool.float() * gains).to(c.v_pool.dtype)  # NaN poison stays NaN
    ref, _, _ = oracle_step(c)
    out, _, _ = run_step(c, kernel="mfma", partition_tokens=partition)
    compare(gpu_out_f64(out), ref, np.asarray(lens), "bf16")


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 8, 128), (16, 1, 128), (32, 8, 64)])
def test_fixed_merge_batch_boundaries(hq, hkv, d):
    """The merge of a row's partitions gives each unit (4 dims of one head)
    T = 256 / units threads (at least 1; units = G D / 4), each loading up to
    4, 8 or 16 partitions a round. Rows of 64-token partitions at the edges
    of each batch size and of the first round, exact and one token past
    (one partition more), for T = 1 (two passes over the units), 2, 4 and 8."""
    units = hq // hkv * d // 4
    T = 1 if units >= 256 else 256 // units
    parts = sorted({2, 4 * T, 4 * T + 1, 8 * T, 8 * T + 1, 16 * T, 16 * T + 1, 32 * T + 1})
    lens = [p * 64 + e for p in parts for e in (0, 1)]
    c = wl.random_case(457 + T, len(lens), hq, hkv, d, "bf16", lens=lens)
    ref, _, _ = oracle_step(c)
    out, _, _ = run_step(c, kernel="mfma", partition_tokens=64)
    compare(gpu_out_f64(out), ref, lens, "bf16")


@pytest.fixture(scope="module")
def max_batch():
    """4,096 rows (the most a call takes) of 0-90 tokens, a quarter empty."""
    rng = np.random.default_rng(1101)
    lens = rng.integers(0, 91, size=4096)
    lens[rng.choice(4096, 1024, replace=False)] = 0
    c = wl.random_case(1101, 4096, 32, 8, 128, "bf16", lens=lens.tolist())
    return c, oracle_step(c)[0], lens


@pytest.mark.parametrize("kernel,partition", [("mfma", 0), ("mfma", 512), ("valu", 512),
                                              ("auto", pk.PARTITION_AUTO)])
def test_max_batch_4096_rows(max_batch, kernel, partition):
    """The most rows a call takes: the work lists' prefixes over 4,096 rows
    fill their LDS share and each balanced range holds many whole rows.
    Every row is compared with the oracle, and the empty rows are exactly
    zero."""
    c, ref, lens = max_batch
    out, _, _ = run_step(c, kernel=kernel, partition_tokens=partition)
    compare(gpu_out_f64(out), ref, lens, "bf16")
    empty = torch.from_numpy(lens == 0).to(out.device)
    assert torch.count_nonzero(out[empty].view(torch.int16)) == 0


@pytest.mark.parametrize("lens,partition", [
    ([5000], 256),              # one row, 20 slots per KV head, the last partition partial
    ([0, 1000, 4096, 1], 512),  # a padded row, a partition end at a row end, a one-token row
    ([512, 0, 3000], 512),
])
def test_fixed_slot_grid(lens, partition):
    """While every (row, partition, KV head) slot fits on a compute unit of
    its own, the fixed split gives each slot a workgroup and builds no work
    list: slots past a row's end exit, and slot 0 of a padded row writes its
    zeros. The same call with a block table wide enough to need the work
    list (columns past every row's end, never read) gives the same bits,
    and both meet the oracle's bar."""
    c = wl.random_case(480 + len(lens), len(lens), 32, 8, 128, "bf16", lens=lens)
    ref, _, _ = oracle_step(c)
    d = c.to("cuda")
    wide = torch.cat([d.block_tables, torch.zeros((len(lens), 2000), dtype=torch.int32,
                                                  device="cuda")], dim=1).contiguous()
    outs = []
    for bt in (d.block_tables, wide):
        out = torch.full_like(d.q, float("nan"))
        pk.pa_decode(d.q, d.k_pool, d.v_pool, bt, d.seq_lens, c.scale, out,
                     partition_tokens=partition, kernel="mfma")
        torch.cuda.synchronize()
        compare(gpu_out_f64(out), ref, np.asarray(lens), "bf16")
        for b, L in enumerate(lens):
            if L == 0:
                assert torch.count_nonzero(out[b].view(torch.int16)) == 0
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("partition", [0, 512, 64])
def test_workspace_reuse_across_calls(partition):
    """The piece counters of the balanced split and the partition counters
    of the fixed split return to zero: one workspace serves a sequence of
    different batches, each repeated bit for bit."""
    cases = [wl.random_case(500 + i, 7, 32, 8, 128, "bf16", max_len=3000) for i in range(3)]
    refs = [oracle_step(c)[0] for c in cases]
    dims = pk.make_dims(7, 32, 8, 128, max(c.max_blocks_per_seq for c in cases),
                        max(c.num_blocks for c in cases), pk.PA_BF16, partition, "mfma")
    ws = torch.zeros(pk.pa_decode_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    first = {}
    for rep in range(3):
        for i, (c, ref) in enumerate(zip(cases, refs)):
            d = c.to("cuda")
            out = pk.pa_decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.seq_lens, c.scale,
                               partition_tokens=partition, kernel="mfma", workspace=ws)
            torch.cuda.synchronize()
            compare(gpu_out_f64(out), ref, c.seq_lens.numpy(), "bf16")
            if rep == 0:
                first[i] = out.clone()
            else:
                assert torch.equal(out.view(torch.int16), first[i].view(torch.int16))


def test_abi_error_reaches_python():
    c = wl.random_case(302, 2, 8, 2, 64, "bf16", max_len=600).to("cuda")
    with pytest.raises(pk.PagedKVError):
        pk.pa_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.seq_lens, c.scale,
                     partition_tokens=16,
                     workspace=torch.empty(8, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        pk.pa_decode(c.q.float(), c.k_pool, c.v_pool, c.block_tables, c.seq_lens, c.scale)


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 9, 40])
def test_auto_split_is_the_documented_choice(B):
    """PA_PARTITION_AUTO gives bit for bit the split it documents: fixed
    partitions of 256 tokens for one row, 192 for two, 320 for three or
    four, 384 for five to eight, the balanced split above; and meets the
    oracle's bar."""
    c = wl.random_case(470 + B, B, 32, 8, 128, "bf16", max_len=3000)
    ref, _, _ = oracle_step(c)
    auto, _, _ = run_step(c, kernel="mfma", partition_tokens=pk.PARTITION_AUTO)
    chosen, _, _ = run_step(c, kernel="mfma",
                            partition_tokens={1: 256, 2: 192, 3: 320, 4: 320}.get(
                                B, 384 if B <= 8 else 0))
    assert torch.equal(auto.view(torch.int16), chosen.view(torch.int16))
    compare(gpu_out_f64(auto), ref, c.seq_lens.numpy(), "bf16")
