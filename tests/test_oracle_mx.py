"""Pins for the oracle's MX codecs and quantiser (CPU only).

Each check ties the oracle to something other than itself: hand-decoded elements and hand-quantised
blocks from the OCP MX v1.0 definitions (tests/golden), and torch's own float8 casts (a library
routine written independently of the oracle)."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.split("#", 1)[0].strip()
            if ln:
                yield ln


def test_codec_hand_examples():
    n = 0
    for ln in _lines("mx_codec_examples.txt"):
        fmt, sb, code, val = ln.split()
        c, s, v = int(code, 16), int(sb), float(val)
        got = (mx.E4M3_TABLE if fmt == "e4m3" else mx.E2M1_TABLE)[c] * mx.E8M0_TABLE[s]
        assert got == v and math.copysign(1, got) == math.copysign(1, v), ln
        n += 1
    assert n >= 30


def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(mx.E4M3_TABLE), nan)
    assert np.array_equal(mx.E4M3_TABLE[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mx.E4M3_TABLE[~nan]), np.signbit(ref[~nan]))


def test_e8m0_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(ref[255]) and np.isnan(mx.E8M0_TABLE[255])
    assert np.array_equal(mx.E8M0_TABLE[:255], ref[:255])


def test_e2m1_table_by_hand():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(mx.E2M1_TABLE[:8]) == mags
    assert list(mx.E2M1_TABLE[8:]) == [-m for m in mags]
    assert np.signbit(mx.E2M1_TABLE[8])


def test_quantize_hand_blocks():
    n = 0
    for ln in _lines("mx_quant_examples.txt"):
        fmt, vals, sb, codes = [p.strip() for p in ln.split("|")]
        x = np.zeros(32)
        v = [float(t) for t in vals.split()]
        x[:len(v)] = v
        c, s = mx.quantize(x[None, :], fmt)
        want = [int(t, 16) for t in codes.split()]
        assert int(s[0, 0]) == int(sb), ln
        assert list(c[0, :len(want)]) == want, ln
        assert np.all(c[0, len(want):] == 0), ln
        n += 1
    assert n >= 15


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_quantize_round_trip_on_grid(fmt):
    # Blocks whose values are already codes * 2^se, with the largest magnitude in the top binade of
    # the element format, must come back unchanged (codes compared with +0 == -0).
    rng = np.random.default_rng(1)
    top = {"e4m3": list(range(0x78, 0x7F)), "e2m1": [4, 5, 6, 7]}[fmt]
    nmax = {"e4m3": 0x7F, "e2m1": 8}[fmt]
    sign = {"e4m3": 0x80, "e2m1": 0x8}[fmt]
    for _ in range(200):
        codes = rng.integers(0, nmax, size=32)
        codes[rng.integers(0, 32)] = rng.choice(top)
        codes = codes | np.where(rng.random(32) < 0.5, sign, 0)
        se = int(rng.integers(-100, 100))
        x = mx.decode(codes, fmt) * 2.0 ** se
        c, s = mx.quantize(x[None], fmt)
        assert int(s[0, 0]) == se + 127
        zero = mx.decode(codes, fmt) == 0
        assert np.array_equal(c[0][~zero], codes[~zero].astype(np.uint8))


def test_e4m3_elements_match_torch_cast():
    # After the shared scaling, in-range elements must round exactly as torch's float8_e4m3fn cast
    # (round to nearest even); torch does not saturate, so out-of-range values are excluded.
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4000, 32)) * np.exp(rng.uniform(-20, 20, size=(4000, 1)))
    c, s = mx.quantize(x, "e4m3")
    se = s.astype(np.int64) - 127
    v = x / np.ldexp(1.0, np.repeat(se, 32, axis=1))
    inr = np.abs(v) <= 448
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # v is exact in fp32 only when it has <= 24 significant bits; the normal draws do not, so compare
    # against the fp64 value rounded by torch via fp32 only where the fp32 rounding is exact.
    exact32 = v.astype(np.float32).astype(np.float64) == v
    sel = inr & exact32
    a = c[sel] & 0x7F
    b = ref[sel] & 0x7F
    assert np.array_equal(a, b)
    # And on values that are exact in fp32 by construction (bf16 inputs, the activation case):
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    c2, s2 = mx.quantize(xb, "e4m3")
    v2 = xb / np.ldexp(1.0, np.repeat(s2.astype(np.int64) - 127, 32, axis=1))
    ref2 = torch.from_numpy(v2.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    m2 = np.abs(v2) <= 448
    assert np.array_equal(c2[m2] & 0x7F, ref2[m2] & 0x7F)
    assert np.all(c2[~m2] & 0x7F == 0x7E)          # saturated


def test_all_bf16_values_quantise_within_half_ulp():
    # Exhaustive over every finite bf16 value, each in its own block (so it sets the scale):
    # the element must land within half a step of its binade (or saturate at 448 * 2^se).
    bits = np.arange(65536, dtype=np.uint32)
    vals32 = (bits << 16).view(np.float32)
    vals = vals32[np.isfinite(vals32)].astype(np.float64)
    blocks = np.zeros((vals.size, 32))
    blocks[:, 0] = vals
    c, s = mx.quantize(blocks, "e4m3")
    q = mx.dequantize(c, s, "e4m3")[:, 0]
    se = s[:, 0].astype(np.int64) - 127
    nz = vals != 0
    a = np.abs(vals[nz])
    e = np.floor(np.log2(a))
    # E4M3 step in the top binade is 2^(e-3) for a in [2^e, 2^(e+1)); saturation caps at 1.75*2^e.
    bound = np.where(a <= 1.75 * 2.0 ** e, 2.0 ** (e - 4), a - 1.75 * 2.0 ** e)
    err = np.abs(q[nz] - vals[nz])
    tiny = se[nz] == -127                      # clamped scale: subnormal element grid
    assert np.all(err[~tiny] <= bound[~tiny])
    assert np.all(q[~nz] == 0)


def test_round_to_bf16_matches_torch():
    # On fp32 inputs a single rounding to bf16 is what torch's fp32 -> bf16 cast does (RNE).
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, size=100000))
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(mx.round_to_bf16(x32.astype(np.float64)), ref)


def test_round_to_bf16_is_one_rounding_of_the_exact_value():
    # Hand-worked: 1 + 2^-8 + 2^-30 lies just above the midpoint between the bf16 neighbours 1 and
    # 1 + 2^-7, so it rounds up. Rounding to fp32 first would land exactly on the midpoint
    # (2^-30 is below half an fp32 ulp at 1) and the tie would go to the even neighbour, 1.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert mx.round_to_bf16(np.array([v]))[0] == 1.0 + 2.0 ** -7
    assert mx.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0          # exact tie: even
    assert mx.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert mx.round_to_bf16(np.array([-(1.0 + 2.0 ** -8 + 2.0 ** -30)]))[0] == -(1.0 + 2.0 ** -7)
    # below the smallest normal (2^-126) the grid step stays 2^-133
    assert mx.round_to_bf16(np.array([2.0 ** -133 * 1.5]))[0] == 2.0 ** -132
    assert mx.round_to_bf16(np.array([2.0 ** -130 + 2.0 ** -134]))[0] == 2.0 ** -130


def test_round_to_bf16_against_bit_formula():
    # Independent form: the bf16 neighbours of v are the fp64 values whose low 45 mantissa bits are
    # zero; the nearest one (ties to the even 8-bit significand) is chosen by comparing distances.
    rng = np.random.default_rng(5)
    v = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, size=20000))
    u = v.view(np.uint64)
    lo = (u & ~np.uint64((1 << 45) - 1)).view(np.float64)             # toward zero
    hi = ((u | np.uint64((1 << 45) - 1)) + np.uint64(1)).view(np.float64)  # away from zero
    d_lo, d_hi = np.abs(v - lo), np.abs(hi - v)
    lo_even = ((lo.view(np.uint64) >> np.uint64(45)) & np.uint64(1)) == 0
    want = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo_even, lo, hi)))
    assert np.array_equal(mx.round_to_bf16(v), want)


def test_dequantize_inverts_scale_layout():
    codes = np.full((2, 64), 0x38, dtype=np.uint8)      # all 1.0
    scales = np.array([[127, 128], [120, 0]], dtype=np.uint8)
    d = mx.dequantize(codes, scales, "e4m3")
    assert np.all(d[0, :32] == 1.0) and np.all(d[0, 32:] == 2.0)
    assert np.all(d[1, :32] == 2.0 ** -7) and np.all(d[1, 32:] == 2.0 ** -127)
