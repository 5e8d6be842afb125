"""Pins of the read-copy quantisers against the published format tables and a
library cast (torch's float8_e4m3fn), plus brute-force nearest-value rounding."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (e4m3_encode, e4m3_decode, e2m1_encode, e2m1_decode,
                    quantize_fp8_blocks, dequantize_fp8_blocks,
                    quantize_mxfp4_blocks, dequantize_mxfp4_blocks)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_e4m3_named_points():
    for p in _load("ocp_e4m3fn_points.json")["points"]:
        code = int(p["code"], 16)
        got = e4m3_decode(np.array([code], np.uint8))[0]
        if p["value"] == "nan":
            assert np.isnan(got)
        else:
            assert got == p["value"] and math.copysign(1, got) == math.copysign(1, p["value"])
            assert e4m3_encode(np.array([p["value"]]))[0] == code


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_e4m3_encode_matches_torch_in_range():
    """torch's float32 -> float8_e4m3fn cast rounds to nearest even; compare where it does not overflow."""
    finite = e4m3_decode(np.arange(256, dtype=np.uint8))
    vals = np.unique(finite[np.isfinite(finite)])
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(5)
    x = np.concatenate([vals, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01])
    x = x.astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(x.astype(np.float64)), ref)


def test_e4m3_saturates():
    assert e4m3_encode(np.array([465.0, 1e30, -500.0])).tolist() == [0x7E, 0x7E, 0xFE]


def _nearest_even(x, mags, codes):
    """Brute force: nearest magnitude, ties to the even code; saturate above the max."""
    out = []
    for v in x:
        a = abs(v)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        pick = best[0] if len(best) == 1 else [b for b in best if codes[b] % 2 == 0][0]
        c = codes[pick] | (8 if math.copysign(1, v) < 0 else 0)
        out.append(c)
    return np.array(out, np.uint8)


def test_e2m1_table_and_rounding():
    g = _load("ocp_e2m1_values.json")
    mags = np.array(g["e2m1_magnitudes_by_code"])
    np.testing.assert_array_equal(e2m1_decode(np.arange(8)), mags)
    np.testing.assert_array_equal(e2m1_decode(np.arange(8) | 8), -mags)
    codes = np.arange(8)
    grid = np.concatenate([np.linspace(-7, 7, 2801), (mags[:-1] + mags[1:]) / 2,
                           -(mags[:-1] + mags[1:]) / 2, [6.5, -9.0, 100.0]])
    np.testing.assert_array_equal(e2m1_encode(grid), _nearest_even(grid, mags, codes))


def test_mxfp4_shared_scale_definition():
    g = _load("ocp_e2m1_values.json")
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((64, 32)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    x[3, :] = 0.0
    x[4, :] = 0.0
    x[4, 7] = 4.0          # power-of-two amax
    x[5, 0] = -1e-40       # denormal amax candidate is dominated by others in that row
    x[6, :] = 0.0
    x[6, 3] = 2.0 ** -130  # tiny block: exponent clamps to -126
    packed, e8 = quantize_mxfp4_blocks(x)
    for r in range(64):
        amax = float(np.max(np.abs(x[r].astype(np.float64))))
        if amax == 0:
            assert e8[r, 0] == 1          # 2^-126, the smallest scale used
            continue
        E = math.floor(math.log2(amax)) - g["e2m1_emax"]
        assert int(e8[r, 0]) == max(min(E, 127), -126) + g["e8m0_bias"]
    deq = dequantize_mxfp4_blocks(packed, e8)
    assert deq.shape == x.shape
    # every element within half a step of its binade (or clipped to 6 * 2^E)
    scale = np.ldexp(1.0, e8.astype(np.int64) - 127)[:, :1]
    err = np.abs(deq - x.astype(np.float64)) / scale
    assert np.all((err <= 1.0) | (np.abs(x / scale) > 6))


def test_fp8_block_quantiser_properties():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((16, 4, 128)) * 0.3).astype(np.float32)
    x[0, 0, :32] = 0.0
    codes, scales = quantize_fp8_blocks(x)
    assert codes.shape == x.shape and scales.shape == (16, 4, 4)
    assert scales[0, 0, 0] == 0 and np.all(codes[0, 0, :32] == 0)
    amax = np.max(np.abs(x.reshape(16, 4, 4, 32)), axis=-1)
    np.testing.assert_array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    deq = dequantize_fp8_blocks(codes, scales)
    # relative error of a normal E4M3 value is at most 2^-4; absolute floor from subnormals
    s = np.repeat(scales, 32, axis=-1).astype(np.float64)
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), s * 2.0 ** -10) * (1 + 1e-6))
    # the block maximum maps to +-448 (up to one float32 rounding of x / scale)
    top = np.take_along_axis(np.abs(deq.reshape(16, 4, 4, 32)),
                             np.argmax(np.abs(x.reshape(16, 4, 4, 32)), axis=-1)[..., None], -1)[..., 0]
    nz = amax > 0
    np.testing.assert_allclose(top[nz], amax[nz], rtol=2.0 ** -4)


def test_mxfp4_packing_low_nibble_first():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0      # E = 0 - 2 = -2 -> 1.0 / 0.25 = 4 -> code 6
    x[0, 1] = -0.5     # -0.5 / 0.25 = -2 -> code 4 | 8 = 12
    packed, e8 = quantize_mxfp4_blocks(x)
    assert e8[0, 0] == 125
    assert packed[0, 0] == (6 | (12 << 4))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_ambiguity_bound_covers_brute_force_perturbations(fmt):
    """Random perturbations of the float32 input within +-delta never change a dequantised
    value by more than read_copy_ambiguity's bound; delta = 0 gives a zero bound."""
    from oracle import read_copy_ambiguity, read_copy_dequant
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((8, 64)) * 0.3).astype(np.float32)
    x[0, :32] = np.float32(2.0) ** np.arange(-16, 16)       # block maxima on powers of two
    x[1, 5] = np.float32(448.0)
    delta = 2e-5 * np.max(np.abs(x), axis=-1, keepdims=True)      # per row, as per tile in use
    bound = read_copy_ambiguity(fmt, x, delta)
    assert np.all(read_copy_ambiguity(fmt, x, 0.0) == 0)
    base = read_copy_dequant(fmt, x)
    worst_seen = 0.0
    for trial in range(300):
        dx = rng.uniform(-delta, delta, x.shape)
        if trial % 3 == 0:
            dx = np.sign(dx) * delta                           # corners
        xp = (x.astype(np.float64) + dx).astype(np.float32)
        dev = np.abs(read_copy_dequant(fmt, xp) - base)
        assert np.all(dev <= bound * (1 + 1e-12) + 1e-30)
        worst_seen = max(worst_seen, float(np.max(dev)))
    assert worst_seen > 0                                       # some perturbation did flip a code
