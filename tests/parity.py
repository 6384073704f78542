"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, compare.

Tolerances (spec bar):
  f32   max |gpu - oracle| <= 2e-3 over every element;
  bf16  for every row b (a sequence in decode, a query token in prefill) and
        element e:
            |gpu - oracle| <= 2e-2 * RMS(oracle[b]) + 2^-8 * |oracle[b, e]|,
        the RMS taken over all query heads and dims of the row and the oracle
        unrounded (float64). The first term is the arithmetic budget,
        relative to the row's own output RMS (output magnitudes scale like
        sqrt(e / L), so rows of different lengths are normalised by their
        own RMS); the second is the bf16 output format's own rounding (half
        an ulp is at most 2^-8 of the value), which even the correctly
        rounded exact result needs on rows with a few large elements.
  Padded rows (L = 0) must be exact zeros (bitwise).
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import paged_kv_cache_55_amd as pk
from workloads import to_numpy

F32_ATOL = 2e-3
BF16_RMS_RTOL = 2e-2
BF16_ROUNDING = 2.0 ** -8


def gpu_out_f64(out: torch.Tensor, rows=None) -> np.ndarray:
    o = out.detach()
    if rows is not None:
        o = o[torch.as_tensor(rows, dtype=torch.long, device=o.device)]
    return o.float().cpu().numpy().astype(np.float64)


def compare(got: np.ndarray, ref: np.ndarray, lens, dtype: str) -> float:
    """Assert the bar; returns the worst ratio error / allowed (diagnostic)."""
    lens = np.asarray(lens)
    assert got.shape == ref.shape
    worst = 0.0
    for i, L in enumerate(lens.tolist()):
        if L == 0:
            assert np.all(got[i] == 0.0), f"row {i}: padded row not zero"
            continue
        assert np.all(np.isfinite(got[i])), f"row {i}: non-finite output"
        err = np.abs(got[i] - ref[i])
        if dtype == "f32":
            allowed = np.full(err.shape, F32_ATOL)
        else:
            rms = float(np.sqrt(np.mean(ref[i] ** 2)))
            allowed = BF16_RMS_RTOL * rms + BF16_ROUNDING * np.abs(ref[i])
        ratio = err / allowed
        k = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        worst = max(worst, float(ratio[k]))
        assert ratio[k] <= 1.0, (f"row {i} (L={L}): err {err[k]:.3e} > allowed "
                                 f"{allowed[k]:.3e} at {k}")
    return worst


def oracle_inputs(case, k_pool=None, v_pool=None):
    return dict(q=to_numpy(case.q),
                k_pool=to_numpy(case.k_pool) if k_pool is None else k_pool,
                v_pool=to_numpy(case.v_pool) if v_pool is None else v_pool,
                block_tables=to_numpy(case.block_tables),
                seq_lens=to_numpy(case.seq_lens), scale=case.scale,
                dtype=case.dtype)


def run_step(case, kernel="auto", partition_tokens=None, device="cuda"):
    """copy_blocks -> write_kv -> decode on the GPU; returns (out, k, v)."""
    d = case.to(device)
    if d.block_mapping is not None and d.block_mapping.numel():
        pk.pa_copy_blocks(d.k_pool, d.v_pool, d.block_mapping)
    if d.slot_mapping is not None:
        pk.pa_write_kv(d.k_new, d.v_new, d.slot_mapping, d.k_pool, d.v_pool)
    pt = case.partition_tokens if partition_tokens is None else partition_tokens
    out = pk.pa_decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.seq_lens, case.scale,
                       partition_tokens=pt, kernel=kernel)
    torch.cuda.synchronize()
    return out, d.k_pool, d.v_pool


def oracle_step(case, rows=None):
    """The oracle's copy -> write -> decode; returns (out, k, v) on the host."""
    a = oracle_inputs(case)
    k, v = a["k_pool"], a["v_pool"]
    if case.block_mapping is not None and case.block_mapping.numel():
        k, v = oracle.copy_blocks(k, v, to_numpy(case.block_mapping))
    if case.slot_mapping is not None:
        k, v = oracle.write_kv(k, v, to_numpy(case.k_new), to_numpy(case.v_new),
                               to_numpy(case.slot_mapping), block_size=case.block_size)
    a["k_pool"], a["v_pool"] = k, v
    return oracle.paged_decode(**a, rows=rows, block_size=case.block_size), k, v


def bits_equal(gpu_t: torch.Tensor, host: np.ndarray) -> bool:
    """Bitwise equality (NaN payloads included)."""
    g = np.ascontiguousarray(to_numpy(gpu_t))
    h = np.ascontiguousarray(host)
    return g.shape == h.shape and np.array_equal(g.view(np.uint8), h.view(np.uint8))


def oracle_prefill(case):
    """The oracle's chunk append then chunked-prefill attention; returns
    (out, k, v) on the host."""
    k, v = oracle.write_kv(to_numpy(case.k_pool), to_numpy(case.v_pool), to_numpy(case.k_new),
                           to_numpy(case.v_new), to_numpy(case.slot_mapping),
                           block_size=case.block_size)
    out = oracle.paged_prefill(to_numpy(case.q), k, v, to_numpy(case.block_tables),
                               to_numpy(case.seq_lens), to_numpy(case.query_start), case.scale,
                               case.dtype, block_size=case.block_size)
    return out, k, v


def oracle_config5_rows(spec, q, k, v, rows):
    """The oracle on rows `rows` of one layer of the 32-layer step, whose
    tensors live on the device: host copies are made of just the blocks
    those rows reference (the oracle walks the remapped tables)."""
    need = sorted({int(spec.block_tables[b, j]) for b in rows
                   for j in range(math.ceil(int(spec.seq_lens[b]) / 16))} | {spec.poison_block})
    remap = np.full(spec.num_blocks, -1, dtype=np.int64)
    remap[need] = np.arange(len(need))
    idx = torch.tensor(need, dtype=torch.long, device=k.device)
    kh, vh = to_numpy(k[idx]), to_numpy(v[idx])
    tables = remap[spec.block_tables[rows]]
    tables[tables < 0] = remap[spec.poison_block]  # entries past each row's end
    return oracle.paged_decode(to_numpy(q)[rows], kh, vh, tables.astype(np.int32),
                               spec.seq_lens[rows], 1.0 / math.sqrt(128), "bf16")
