"""The parity check itself, on the CPU: it accepts the exact result rounded
once to the output dtype and rejects a result that is off by a little more
than the bar, so a GPU parity pass means what the bar says."""

import numpy as np
import pytest
import torch

import workloads as wl
from parity import BF16_ROUNDING, BF16_RMS_RTOL, F32_ATOL, compare, oracle_prefill, oracle_step


def _bf16_round(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).double().numpy()


@pytest.fixture(scope="module")
def mixed_lengths():
    # one short row among long ones: output magnitudes differ by ~ sqrt(L)
    c = wl.random_case(71, 4, 8, 2, 64, "bf16", lens=[17, 900, 1500, 0])
    ref, _, _ = oracle_step(c)
    return c, ref


def test_bf16_bar_accepts_correct_rounding(mixed_lengths):
    c, ref = mixed_lengths
    got = _bf16_round(ref)
    worst = compare(got, ref, c.seq_lens.numpy(), "bf16")
    assert 0.0 < worst < 1.0


def test_bf16_bar_rejects_error_above_row_rms(mixed_lengths):
    c, ref = mixed_lengths
    got = ref.copy()
    row = 2  # a long row: its own RMS is small
    rms = float(np.sqrt(np.mean(ref[row] ** 2)))
    got[row, 3, 5] += 1.1 * (BF16_RMS_RTOL * rms + BF16_ROUNDING * abs(ref[row, 3, 5]))
    with pytest.raises(AssertionError):
        compare(got, ref, c.seq_lens.numpy(), "bf16")


def test_bf16_bar_allows_exactly_the_rounding_budget(mixed_lengths):
    c, ref = mixed_lengths
    got = ref.copy()
    row = 1
    rms = float(np.sqrt(np.mean(ref[row] ** 2)))
    got[row, 0, 7] += 0.99 * (BF16_RMS_RTOL * rms + BF16_ROUNDING * abs(ref[row, 0, 7]))
    compare(got, ref, c.seq_lens.numpy(), "bf16")


def test_prefill_rows_need_the_rounding_allowance():
    """On a whole 200-token prompt, correct rounding of the exact result
    alone exceeds 2e-2 x RMS on some rows; with the rounding term it is
    inside the bar."""
    c = wl.prefill_case(1132, [200], [0], 32, 8, 128)
    ref, _, _ = oracle_prefill(c)
    rounded = _bf16_round(ref)
    err = np.abs(rounded - ref).reshape(len(ref), -1).max(1)
    rms = np.sqrt((ref.reshape(len(ref), -1) ** 2).mean(1))
    assert (err > BF16_RMS_RTOL * rms).any()
    compare(rounded, ref, np.ones(len(ref)), "bf16")


def test_padded_row_must_be_exact_zero(mixed_lengths):
    c, ref = mixed_lengths
    got = ref.copy()
    got[3, 0, 0] = 1e-30
    with pytest.raises(AssertionError):
        compare(got, ref, c.seq_lens.numpy(), "bf16")


def test_non_finite_output_rejected(mixed_lengths):
    c, ref = mixed_lengths
    got = ref.copy()
    got[1, 0, 0] = np.nan
    with pytest.raises(AssertionError):
        compare(got, ref, c.seq_lens.numpy(), "bf16")


def test_f32_bar_is_absolute():
    c = wl.config1()
    ref, _, _ = oracle_step(c)
    lens = c.seq_lens.numpy()
    compare(ref + 0.9 * F32_ATOL, ref, lens, "f32")
    with pytest.raises(AssertionError):
        compare(ref + 1.1 * F32_ATOL, ref, lens, "f32")
