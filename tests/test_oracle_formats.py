"""Pins of the oracle's number formats: E4M3FN codec and block-scaled FP8 quantisation.

The blueprint's training box names "block-scaled FP8" (archdiff.com, "Qwen3.5-397B-A17B vs
DeepSeek-V4-Pro", blueprint diagram).  The pages fix neither the FP8 variant nor the scale
rule; the oracle reads them as OCP E4M3FN (round to nearest even, saturating at +-448) with
one fp32 scale = group max / 448 per 128 values.  These tests pin the codec against torch's
independent float8_e4m3fn implementation and the quantiser against closed forms and
invariants.  Whether the models' own kernels use exactly this rule is "parity unpinned".
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_decode_all_256_codes_match_torch_table():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # closed-form landmarks of the format
    assert ours[0x7E] == 448.0                      # largest finite: 1.75 * 2^8
    assert ours[0x08] == 2.0 ** -6                  # smallest normal
    assert ours[0x01] == 2.0 ** -9                  # smallest subnormal
    assert ours[0x38] == 1.0                        # exponent field 7 = bias
    assert ours[0xB8] == -1.0


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(v, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_round_matches_torch_on_every_bf16_value_in_range():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    with np.errstate(invalid="ignore"):
        vals = bits.astype(np.uint32).view(np.float32).astype(np.float64)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448.0)]
    ours = oracle.e4m3_round(vals)
    assert np.array_equal(ours, _torch_e4m3(vals))


def test_round_ties_to_even_and_saturation():
    rng = np.random.default_rng(7)
    codes = np.arange(0x7E, dtype=np.uint8)           # every positive finite code
    v = oracle.e4m3_value(codes)
    mids = (v[:-1] + v[1:]) / 2                        # exact midpoints
    ours = oracle.e4m3_round(mids)
    lo_even = (codes[:-1] % 2) == 0
    assert np.array_equal(ours, np.where(lo_even, v[:-1], v[1:]))
    assert np.array_equal(ours, _torch_e4m3(mids))
    # random fp32 values, both signs
    r = (rng.standard_normal(20000) * rng.choice([1e-3, 0.1, 1, 30, 300], 20000)).astype(np.float32)
    r = r.astype(np.float64)
    assert np.array_equal(oracle.e4m3_round(r), _torch_e4m3(r))
    # saturation beyond the largest finite value
    assert list(oracle.e4m3_round(np.array([448.5, 463.9, 464.0, 1e9, -500.0]))) == \
        [448.0, 448.0, 448.0, 448.0, -448.0]
    # subnormal ties: 2^-10 sits between 0 and 2^-9 -> 0 (even); 3*2^-10 -> 2^-8 (even code 2)
    assert oracle.e4m3_round(np.array([2.0 ** -10]))[0] == 0.0
    assert oracle.e4m3_round(np.array([3 * 2.0 ** -10]))[0] == 2.0 ** -8


def test_encode_inverts_decode():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_value(codes)), codes)


def test_quant_closed_forms():
    # a group whose largest magnitude is 448 has scale exactly 1: codes are plain E4M3 roundings
    x = np.zeros((1, 128))
    x[0, 0] = 448.0
    x[0, 1:] = np.linspace(-3.3, 3.3, 127)
    codes, scales, xdq = oracle.quant_rows(x, 128)
    assert scales[0, 0] == 1.0
    assert np.array_equal(xdq[0], oracle.e4m3_round(x[0]))
    # an all-zero group: scale 1, every code +0
    codes, scales, xdq = oracle.quant_rows(np.zeros((2, 256)), 128)
    assert np.all(scales == 1.0) and np.all(codes == 0) and np.all(xdq == 0)
    # scale = amax / 448 rounded to fp32, and the max element lands on +-448 * scale
    x = np.zeros((1, 128))
    x[0, 5] = -3.0
    x[0, 9] = 1.0
    codes, scales, xdq = oracle.quant_rows(x, 128)
    assert scales[0, 0] == np.float32(3.0 / 448.0)
    assert abs(xdq[0, 5] / float(scales[0, 0])) == 448.0


def test_quant_invariants_random():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 512)) * rng.choice([1e-4, 1.0, 50.0], (16, 1))
    x = x.astype(np.float32).astype(np.float64)
    codes, scales, xdq = oracle.quant_rows(x, 128)
    g = x.reshape(16, 4, 128)
    s = scales.astype(np.float64)
    q = xdq.reshape(16, 4, 128) / s[..., None]
    # every q is an E4M3 value, and the group's largest element maps to 448 in magnitude
    assert np.array_equal(oracle.e4m3_round(q.ravel()), q.ravel())
    imax = np.abs(g).argmax(-1)
    top = np.take_along_axis(np.abs(q), imax[..., None], -1)[..., 0]
    assert np.all(np.abs(top - 448.0) <= 16.0)
    # relative rounding error of E4M3 in the normal range is at most 2^-4
    big = np.abs(q) >= 2.0 ** -6
    err = np.abs(xdq.reshape(16, 4, 128) - g)[big] / np.abs(g[big])
    assert err.max() <= 2.0 ** -4 * (1 + 1e-6)
    # codes decode to the stored values
    assert np.array_equal(oracle.e4m3_value(codes).reshape(q.shape), q)


@pytest.mark.parametrize("bits", [0x3F80, 0xC040, 0x0001, 0x7F7F])
def test_bf16_value(bits):
    u = np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]
    assert oracle.bf16_value(np.array([bits], dtype=np.uint16))[0] == float(u)
    assert math.isfinite(float(u))


# ------------------------------------------------------------------ MXFP4 (E2M1 + E8M0)
# OCP Microscaling Formats (MX) v1.0: the FP4 E2M1 element values of the 16 codes (sign in
# bit 3), and the E8M0 scale 2^(code - 127).  The blueprint's training box names MXFP4.
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_matches_the_ocp_table():
    got = oracle.e2m1_value(np.arange(16))
    assert got[:8].tolist() == OCP_E2M1
    assert got[8:].tolist() == [-v for v in OCP_E2M1]
    assert math.copysign(1.0, got[8]) == -1.0      # code 8 is -0


def test_e8m0_decode_matches_torch_on_every_finite_code():
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(oracle.e8m0_value(codes), ref)
    assert math.isnan(oracle.e8m0_value(np.array([255]))[0])
