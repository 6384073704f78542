"""The C ABI library without a GPU: it loads, exports what the header
declares, and rejects bad host-visible arguments before launching anything.

Every call here returns before the library touches the HIP runtime, so
these run on a machine without a GPU.
"""

import ctypes
import glob
import os
import re

import numpy as np
import pytest

import paged_kv_cache_55_amd as pk
from paged_kv_cache_55_amd import build as pkbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkbuild.LIB_PATH):
        pkbuild.build()
    return pk.load_library()


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(pa_[a-z_0-9]+)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(pk.SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert pk.pa_status_string(pk.PA_OK) == "ok"
    assert "invalid" in pk.pa_status_string(pk.PA_ERR_INVALID_ARG)
    assert "unsupported" in pk.pa_status_string(pk.PA_ERR_UNSUPPORTED)
    assert "launch" in pk.pa_status_string(pk.PA_ERR_LAUNCH)
    assert "gfx950" in pk.pa_version()


def dims(**kw):
    base = dict(num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                max_blocks_per_seq=256, num_blocks=9000, dtype=pk.PA_BF16,
                partition_tokens=512, kernel="auto")
    base.update(kw)
    return pk.make_dims(**base)


def test_workspace_size(lib):
    d = dims()
    nparts = 4096 // 512
    rows = 64 * 32 * nparts
    align = lambda x: (x + 255) // 256 * 256
    # fixed split: int32 partition counters per (sequence, KV head), then
    # fp32 m, l and unnormalised outputs per (sequence, query head, partition)
    assert pk.pa_decode_workspace_bytes(d) == \
        align(64 * 8 * 4) + 2 * align(rows * 4) + rows * 128 * 4
    assert pk.pa_decode_workspace_bytes(dims(kernel="valu")) == \
        align(64 * 8 * 4) + 2 * align(rows * 4) + rows * 128 * 4
    # balanced split (matrix-core kernel, partition_tokens = 0): int32
    # counters per (sequence, KV head), then one fp32 record (G x D outputs,
    # G maxima, G sums, padded to 4 floats) per piece slot, two slots per
    # wave of at most 256 four-wave workgroups
    slots = 2 * 4 * 256
    assert pk.pa_decode_workspace_bytes(dims(partition_tokens=0)) == \
        align(64 * 8 * 4) + slots * (4 * 128 + 8) * 4
    # G = 1: 2 floats of (m, l) padded to 4
    assert pk.pa_decode_workspace_bytes(dims(partition_tokens=0, num_q_heads=8)) == \
        align(64 * 8 * 4) + slots * (128 + 4) * 4
    # G = 3: 6 floats padded to 8
    assert pk.pa_decode_workspace_bytes(dims(partition_tokens=0, num_q_heads=24)) == \
        align(64 * 8 * 4) + slots * (3 * 128 + 8) * 4
    assert pk.pa_decode_workspace_bytes(dims(partition_tokens=0, kernel="valu")) == 0
    assert pk.pa_decode_workspace_bytes(dims(partition_tokens=4096)) == 0
    assert pk.pa_decode_workspace_bytes(dims(max_blocks_per_seq=32)) == 0
    assert pk.pa_decode_workspace_bytes(dims(head_dim=96)) == 0  # invalid -> 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails first


def decode_status(lib, d, q=FAKE, ws=None, wsb=0, scale=0.1):
    return lib.pa_decode(q, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(scale), FAKE,
                         ctypes.byref(d), ws, ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), pk.PA_ERR_UNSUPPORTED),
    (dict(num_q_heads=33), pk.PA_ERR_INVALID_ARG),
    (dict(num_q_heads=8 * 17), pk.PA_ERR_UNSUPPORTED),
    (dict(num_seqs=0), pk.PA_ERR_INVALID_ARG),
    (dict(num_seqs=4097), pk.PA_ERR_UNSUPPORTED),
    (dict(num_kv_heads=0), pk.PA_ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=0), pk.PA_ERR_INVALID_ARG),
    (dict(num_blocks=0), pk.PA_ERR_INVALID_ARG),
    (dict(partition_tokens=100), pk.PA_ERR_INVALID_ARG),
    (dict(partition_tokens=-16), pk.PA_ERR_INVALID_ARG),
    (dict(dtype=7), pk.PA_ERR_INVALID_ARG),
    (dict(dtype=pk.PA_F32, kernel="mfma"), pk.PA_ERR_UNSUPPORTED),
])
def test_decode_rejects_bad_dims(lib, kw, status):
    assert decode_status(lib, dims(**kw)) == status


@pytest.mark.parametrize("bs", [0, 4, 12, 24, 512, -16])
def test_decode_rejects_bad_block_size(lib, bs):
    d = dims(partition_tokens=0)
    d.block_size = bs
    assert decode_status(lib, d) == pk.PA_ERR_INVALID_ARG


@pytest.mark.parametrize("bs", [8, 32, 64, 128, 256])
def test_other_block_sizes_need_the_balanced_split(lib, bs):
    # fixed partitions and the vector-ALU kernel take 16-token blocks only
    for kw in (dict(partition_tokens=512), dict(partition_tokens=0, kernel="valu")):
        d = dims(**kw)
        d.block_size = bs
        assert decode_status(lib, d) == pk.PA_ERR_UNSUPPORTED
    d = dims(partition_tokens=0, block_size=bs)
    assert pk.pa_decode_workspace_bytes(d) > 0


def test_decode_rejects_bad_kernel_code(lib):
    d = dims()
    d.kernel = 9
    assert decode_status(lib, d) == pk.PA_ERR_INVALID_ARG


def test_decode_rejects_null_and_small_workspace(lib):
    d = dims()
    assert decode_status(lib, d, q=None) == pk.PA_ERR_INVALID_ARG
    assert decode_status(lib, d, ws=None) == pk.PA_ERR_INVALID_ARG
    need = pk.pa_decode_workspace_bytes(d)
    assert decode_status(lib, d, ws=FAKE, wsb=need - 1) == pk.PA_ERR_INVALID_ARG
    assert decode_status(lib, d, scale=float("nan")) == pk.PA_ERR_INVALID_ARG
    assert lib.pa_decode(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE,
                         None, None, 0, None) == pk.PA_ERR_INVALID_ARG


def test_write_and_copy_reject_bad_args(lib):
    d = dims()
    assert lib.pa_write_kv(FAKE, FAKE, FAKE, -1, FAKE, FAKE, ctypes.byref(d), None) == pk.PA_ERR_INVALID_ARG
    assert lib.pa_write_kv(None, FAKE, FAKE, 4, FAKE, FAKE, ctypes.byref(d), None) == pk.PA_ERR_INVALID_ARG
    assert lib.pa_write_kv(None, None, None, 0, None, None, ctypes.byref(d), None) == pk.PA_OK
    assert lib.pa_copy_blocks(FAKE, FAKE, None, 2, ctypes.byref(d), None) == pk.PA_ERR_INVALID_ARG
    assert lib.pa_copy_blocks(FAKE, FAKE, FAKE, -3, ctypes.byref(d), None) == pk.PA_ERR_INVALID_ARG
    assert lib.pa_copy_blocks(None, None, None, 0, ctypes.byref(d), None) == pk.PA_OK
    bad = dims(head_dim=80)
    assert lib.pa_copy_blocks(FAKE, FAKE, FAKE, 1, ctypes.byref(bad), None) == pk.PA_ERR_UNSUPPORTED


# --------------------------------------------------------------------------
# host validator
# --------------------------------------------------------------------------

def test_validator_accepts_good_inputs():
    import workloads as wl
    c = wl.config2()
    pk.validate(c.num_blocks, c.block_tables, c.seq_lens, c.slot_mapping)
    c3 = wl.config3()
    pk.validate(c3.num_blocks, c3.block_tables, c3.seq_lens, c3.slot_mapping, c3.block_mapping)


def test_append_rejects_null_new_tokens(lib):
    d = dims(partition_tokens=0)
    st = lib.pa_decode_append(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              ctypes.c_float(0.1), FAKE, ctypes.byref(d), FAKE,
                              ctypes.c_size_t(1 << 30), None)
    assert st == pk.PA_ERR_INVALID_ARG


def prefill_status(lib, d, tokens=8, q=FAKE, qs=FAKE, scale=0.1):
    return lib.pa_prefill(q, FAKE, FAKE, FAKE, FAKE, qs, tokens, ctypes.c_float(scale), FAKE,
                          ctypes.byref(d), None)


def test_prefill_host_checks(lib):
    assert prefill_status(lib, dims(dtype=pk.PA_F32)) == pk.PA_ERR_UNSUPPORTED
    assert prefill_status(lib, dims(block_size=8)) == pk.PA_ERR_UNSUPPORTED
    assert prefill_status(lib, dims(), qs=None) == pk.PA_ERR_INVALID_ARG
    assert prefill_status(lib, dims(), tokens=-1) == pk.PA_ERR_INVALID_ARG
    assert prefill_status(lib, dims(num_q_heads=12)) == pk.PA_ERR_INVALID_ARG
    for bad in (0.0, -0.1, float("inf"), float("nan")):
        assert prefill_status(lib, dims(), scale=bad) == pk.PA_ERR_INVALID_ARG
    assert prefill_status(lib, dims(), tokens=0) == pk.PA_OK  # nothing to do, nothing launched


def test_validator_fused_step_contract():
    import workloads as wl
    c = wl.config2()
    pk.validate(c.num_blocks, c.block_tables, c.seq_lens, c.slot_mapping, append_rows=True)
    bad = c.slot_mapping.clone()
    bad[3] += 1  # not the slot of position L - 1
    with pytest.raises(ValueError):
        pk.validate(c.num_blocks, c.block_tables, c.seq_lens, bad, append_rows=True)
    lens = c.seq_lens.clone()
    lens[5] = 0  # a padded row may not append
    with pytest.raises(ValueError):
        pk.validate(c.num_blocks, c.block_tables, lens, c.slot_mapping, append_rows=True)


@pytest.mark.parametrize("case", ["len", "entry", "dup_slot", "slot_range", "dst_src", "dup_dst"])
def test_validator_rejects(case):
    bt = np.array([[0, 1, 2]], dtype=np.int32)
    lens = np.array([40], dtype=np.int32)
    kw = dict(num_blocks=4, block_tables=bt, seq_lens=lens)
    if case == "len":
        kw["seq_lens"] = np.array([49], dtype=np.int32)
    elif case == "entry":
        kw["block_tables"] = np.array([[0, 1, 9]], dtype=np.int32)
    elif case == "dup_slot":
        kw["slot_mapping"] = np.array([5, -1, 5], dtype=np.int32)
    elif case == "slot_range":
        kw["slot_mapping"] = np.array([64], dtype=np.int32)
    elif case == "dst_src":
        kw["block_mapping"] = np.array([[0, 1], [1, 2]], dtype=np.int32)
    elif case == "dup_dst":
        kw["block_mapping"] = np.array([[0, 3], [1, 3]], dtype=np.int32)
    with pytest.raises(ValueError):
        pk.validate(**kw)


# --------------------------------------------------------------------------
# latent (MLA-style) decode
# --------------------------------------------------------------------------

def latent_dims(**kw):
    base = dict(num_seqs=256, max_blocks_per_seq=128, num_blocks=7000)
    base.update(kw)
    return pk.make_latent_dims(**base)


def test_latent_workspace_size(lib):
    align = lambda x: (x + 255) // 256 * 256
    B = 256
    rec = 128 * 512 * 2 + 3 * 128 * 4  # scaled output (fp16), then max, sum, scale (fp32)
    off_rec = align(2 * B * 4)  # piece descriptors [B][2], then the records
    assert pk.pa_latent_workspace_bytes(latent_dims()) == off_rec + 2 * 256 * rec
    assert pk.pa_latent_workspace_bytes(latent_dims(num_heads=64)) == 0
    assert pk.pa_latent_workspace_bytes(latent_dims(num_seqs=0)) == 0


def latent_status(lib, d, q=FAKE, ws=FAKE, wsb=None, scale=0.05):
    if wsb is None:
        wsb = pk.pa_latent_workspace_bytes(d) or (1 << 30)
    return lib.pa_latent_decode(q, FAKE, FAKE, FAKE, ctypes.c_float(scale), FAKE,
                                ctypes.byref(d), ws, ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("kw,status", [
    (dict(num_seqs=0), pk.PA_ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=0), pk.PA_ERR_INVALID_ARG),
    (dict(num_blocks=0), pk.PA_ERR_INVALID_ARG),
    (dict(value_dim=600), pk.PA_ERR_INVALID_ARG),
    (dict(dtype=7), pk.PA_ERR_INVALID_ARG),
    (dict(dtype=pk.PA_F32), pk.PA_ERR_UNSUPPORTED),
    (dict(num_heads=64), pk.PA_ERR_UNSUPPORTED),
    (dict(latent_dim=512, value_dim=512), pk.PA_ERR_UNSUPPORTED),
    (dict(value_dim=576), pk.PA_ERR_UNSUPPORTED),
    (dict(block_size=16), pk.PA_ERR_UNSUPPORTED),
    (dict(num_seqs=5000), pk.PA_ERR_UNSUPPORTED),
])
def test_latent_rejects_bad_dims(lib, kw, status):
    assert latent_status(lib, latent_dims(**kw)) == status


def test_latent_rejects_null_and_small_workspace(lib):
    d = latent_dims()
    need = pk.pa_latent_workspace_bytes(d)
    assert latent_status(lib, d, q=None) == pk.PA_ERR_INVALID_ARG
    assert latent_status(lib, d, ws=None) == pk.PA_ERR_INVALID_ARG
    assert latent_status(lib, d, wsb=need - 1) == pk.PA_ERR_INVALID_ARG
    assert latent_status(lib, d, scale=float("inf")) == pk.PA_ERR_INVALID_ARG
    assert lib.pa_latent_decode(FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, None, FAKE,
                                ctypes.c_size_t(need), None) == pk.PA_ERR_INVALID_ARG


def test_latent_write_rejects_bad_args(lib):
    d = latent_dims()
    assert lib.pa_latent_write(FAKE, FAKE, -1, FAKE, ctypes.byref(d), None) == pk.PA_ERR_INVALID_ARG
    assert lib.pa_latent_write(None, FAKE, 3, FAKE, ctypes.byref(d), None) == pk.PA_ERR_INVALID_ARG
    assert lib.pa_latent_write(None, None, 0, None, ctypes.byref(d), None) == pk.PA_OK
    bad = latent_dims(block_size=32)
    assert lib.pa_latent_write(FAKE, FAKE, 3, FAKE, ctypes.byref(bad), None) == pk.PA_ERR_UNSUPPORTED


# --------------------------------------------------------------------------
# allocation-free decode: its checks run before the library touches the GPU
# --------------------------------------------------------------------------

def noalloc_status(lib, d, q=FAKE, scale=0.1):
    return lib.pa_decode_noalloc(q, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(scale), FAKE,
                                 ctypes.byref(d), None)


def test_noalloc_rejects_workspaces_beyond_its_scratch(lib):
    # fixed split at 16-token partitions: 64 x 32 x 256 partials of 128 fp32
    big = dims(partition_tokens=16)
    assert pk.pa_decode_workspace_bytes(big) > pk.NOALLOC_SCRATCH_BYTES
    assert noalloc_status(lib, big) == pk.PA_ERR_UNSUPPORTED
    # the balanced split fits at every supported head group and the largest batch
    for g in (1, 4, 8, 16):
        d = dims(partition_tokens=0, num_seqs=4096, num_q_heads=8 * g)
        assert 0 < pk.pa_decode_workspace_bytes(d) <= pk.NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_bad_args_like_pa_decode(lib):
    assert noalloc_status(lib, dims(head_dim=96)) == pk.PA_ERR_UNSUPPORTED
    assert noalloc_status(lib, dims(num_seqs=0)) == pk.PA_ERR_INVALID_ARG
    assert noalloc_status(lib, dims(partition_tokens=0), q=None) == pk.PA_ERR_INVALID_ARG
    assert noalloc_status(lib, dims(partition_tokens=0), scale=float("nan")) == \
        pk.PA_ERR_INVALID_ARG


def contiguous_status(lib, d, tables_unused=None):
    return lib.pa_decode_contiguous(FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE,
                                    ctypes.byref(d), FAKE, ctypes.c_size_t(1 << 30), None)


def test_contiguous_takes_the_balanced_split_only(lib):
    assert contiguous_status(lib, dims(partition_tokens=512)) == pk.PA_ERR_UNSUPPORTED
    assert contiguous_status(lib, dims(partition_tokens=0, kernel="valu")) == \
        pk.PA_ERR_UNSUPPORTED
    assert contiguous_status(lib, dims(partition_tokens=0, block_size=32)) == \
        pk.PA_ERR_UNSUPPORTED
    assert contiguous_status(lib, dims(partition_tokens=0, head_dim=96)) == \
        pk.PA_ERR_UNSUPPORTED
    assert lib.pa_decode_contiguous(None, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE,
                                    ctypes.byref(dims(partition_tokens=0)), FAKE,
                                    ctypes.c_size_t(1 << 30), None) == pk.PA_ERR_INVALID_ARG


# the fixed partition PA_PARTITION_AUTO documents for 1 .. 8 rows
AUTO_PARTITION = {1: 256, 2: 192, 3: 320, 4: 320, 5: 384, 6: 384, 7: 384, 8: 384}


def test_auto_partition_follows_the_dims(lib):
    """PA_PARTITION_AUTO: fixed partitions of 256 tokens for one row, 192
    for two, 320 for three or four and 384 for five to eight; larger batches
    (and any block size but 16) the balanced split; the vector-ALU kernel
    takes 512-token partitions."""
    ws = pk.pa_decode_workspace_bytes
    for B in (1, 2, 3, 4, 5, 8, 9, 256):
        auto = ws(dims(num_seqs=B, partition_tokens=pk.PARTITION_AUTO))
        expect = ws(dims(num_seqs=B, partition_tokens=AUTO_PARTITION.get(B, 0)))
        assert auto == expect, B
        if B <= 8:  # the workspace size tells the chosen partition from its neighbours
            for other in (192, 256, 320, 384, 512):
                if other != AUTO_PARTITION[B]:
                    assert ws(dims(num_seqs=B, partition_tokens=other)) != auto, (B, other)
    assert ws(dims(num_seqs=4, block_size=32, partition_tokens=pk.PARTITION_AUTO)) == \
        ws(dims(num_seqs=4, block_size=32, partition_tokens=0))
    for B in (1, 64):
        assert ws(dims(num_seqs=B, kernel="valu", partition_tokens=pk.PARTITION_AUTO)) == \
            ws(dims(num_seqs=B, kernel="valu", partition_tokens=512))
    assert ws(dims(partition_tokens=-2)) == 0  # invalid


def test_contiguous_auto_is_the_balanced_split(lib):
    # small batch: AUTO would pick the fixed split for the paged call, but the
    # unpaged cache has the balanced split only; still accepted (the call
    # fails only at the fake pointers' launch, which a host test never reaches)
    d = dims(num_seqs=4, partition_tokens=pk.PARTITION_AUTO)
    assert lib.pa_decode_contiguous(None, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE,
                                    ctypes.byref(d), FAKE, ctypes.c_size_t(1 << 30),
                                    None) == pk.PA_ERR_INVALID_ARG
