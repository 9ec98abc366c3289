"""Pins of the CPU oracle: each check compares the oracle with something other
than itself -- landmark values of the number formats (``tests/golden/``),
library routines (torch's fp8/bf16 casts and rms_norm, numpy's complex
multiply), brute force over every representable value, closed forms and
invariants of rotation and normalisation, and an inverse (physical slot ->
token) scan of the page table.

Every pin is a plain function taking an ``oracle.Oracle`` and raising
AssertionError on failure, so the same pins run against the committed oracle
(``test_oracle_*.py``) and against deliberately broken builds of it
(``test_oracle_mutations.py``).
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# -- independent number-format helpers (test side) ------------------------------


def fp8_values_torch() -> np.ndarray:
    """The 256 E4M3FN codes decoded by torch (a library routine)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def fp8_midpoint_dist(v: np.ndarray):
    """(distance, midpoint): |v|'s distance from the nearest rounding midpoint
    between two adjacent finite E4M3FN magnitudes (the values torch decodes
    for codes 0x00..0x7E), and that midpoint.  Above 448 saturation decides,
    so there is no midpoint: distance +inf.  NaN stays NaN."""
    mags = np.unique(fp8_values_torch()[:0x7F])
    mids = (mags[1:] + mags[:-1]) / 2
    a = np.abs(np.asarray(v, np.float64))
    i = np.clip(np.searchsorted(mids, a), 1, mids.size - 1)
    with np.errstate(invalid="ignore"):
        lo, hi = np.abs(a - mids[i - 1]), np.abs(a - mids[i])
        mid = np.where(lo <= hi, mids[i - 1], mids[i])
        d = np.minimum(lo, hi)
    d = np.where(a > 448.0, np.inf, d)
    return np.where(np.isnan(a), np.nan, d), mid


def fp8_midpoint_rel(v: np.ndarray) -> np.ndarray:
    """fp8_midpoint_dist's distance relative to the midpoint."""
    d, mid = fp8_midpoint_dist(v)
    return d / mid


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns decoded by numpy's float16 (a library routine)."""
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def elem_to_f64(a: np.ndarray) -> np.ndarray:
    """An element-typed array as float64: uint16 holds bf16 bits, float16 and
    float32 are numpy's own."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


def ulp_f16(v: np.ndarray) -> np.ndarray:
    """Spacing of binary16 values at |v| (11 significant bits, quantum >= 2^-24)."""
    _, e = np.frexp(np.maximum(np.abs(v), 2.0 ** -14))
    return np.ldexp(1.0, e - 1 - 10)


def ulp_f32(v: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.maximum(np.abs(v), 2.0 ** -126))
    return np.ldexp(1.0, e - 1 - 23)


def ulp_of(a: np.ndarray):
    """The spacing function of an element-typed array's type."""
    return {np.dtype(np.uint16): ulp_bf16, np.dtype(np.float16): ulp_f16,
            np.dtype(np.float32): ulp_f32}[np.asarray(a).dtype]


def fp8_to_f64(codes: np.ndarray) -> np.ndarray:
    return fp8_values_torch()[np.asarray(codes, np.uint8)]


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (8 significant bits, quantum >= 2^-133)."""
    _, e = np.frexp(np.maximum(np.abs(v), 2.0 ** -126))
    return np.ldexp(1.0, e - 1 - 7)


def ulp_fp8(v: np.ndarray) -> np.ndarray:
    """Spacing of E4M3FN values at |v| (4 significant bits, quantum >= 2^-9)."""
    _, e = np.frexp(np.maximum(np.abs(v), 2.0 ** -6))
    return np.ldexp(1.0, e - 1 - 3)


def assert_correctly_rounded(got: np.ndarray, ref: np.ndarray, ulp_fn, what: str,
                             sat: float | None = None, abs_tol=None) -> None:
    """|got - ref| <= ulp(ref)/2: got is a nearest representable value of ref.
    With ``sat``, references beyond +-sat must come back as +-sat.  abs_tol
    (same shape as ref): the reference's own binary64 error, added to the
    bound (where a cancellation leaves the reference a residue near zero)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = np.zeros_like(ref) if abs_tol is None else np.broadcast_to(abs_tol, ref.shape)
    if sat is not None:
        over = np.abs(ref) > sat
        assert np.all(got[over] == np.sign(ref[over]) * sat), f"{what}: saturation"
        got, ref, tol = got[~over], ref[~over], tol[~over]
    err = np.abs(got - ref)
    bound = 0.5 * ulp_fn(ref) * (1.0 + 1e-12) + tol
    bad = err > bound
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} values not correctly rounded; "
            f"first ref={ref.ravel()[i]!r} got={got.ravel()[i]!r}")


def fp8_encode_bruteforce(v: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3FN code by exhaustive search (ties -> even code),
    magnitudes clamped to 448, sign taken from the sign bit."""
    v = np.asarray(v, np.float64).ravel()
    mags = fp8_values_torch()[:0x7F]          # codes 0x00..0x7E, increasing
    codes = np.arange(0x7F)
    out = np.empty(v.size, np.uint8)
    for s in range(0, v.size, 4096):
        a = np.minimum(np.abs(v[s:s + 4096]), 448.0)
        d = np.abs(a[:, None] - mags[None, :])
        cand = d == d.min(axis=1, keepdims=True)
        even = cand & (codes[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[s:s + 4096] = pick.astype(np.uint8) | (
            np.signbit(v[s:s + 4096]).astype(np.uint8) << 7)
    return out


def bf16_encode_bruteforce(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 to each fp64 value (ties -> even pattern) among the
    patterns around numpy's fp32 rounding of it, by direct comparison."""
    v = np.asarray(v, np.float64).ravel()
    t = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    cands = np.stack([t - 1, t, t + 1, t + 2], axis=1)
    sign = (t & 0x8000)
    mag = cands & 0x7FFF
    mag = np.clip(mag, 0, 0x7F80)
    pats = (mag | sign[:, None]).astype(np.uint16)
    vals = bf16_to_f64(pats)
    d = np.abs(vals - v[:, None])
    cand = d == d.min(axis=1, keepdims=True)
    even = cand & (pats % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return pats[np.arange(v.size), pick]


def read_golden(name: str):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def all_finite_bf16() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_to_f64(bits)
    return v[np.isfinite(v)]


# -- codec pins -------------------------------------------------------------------


def pin_fp8_decode(orc):
    """Oracle decode == torch decode for all 256 codes, and == the OCP table."""
    ref = fp8_values_torch()
    got = np.array([orc.e4m3fn_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "fp8 NaN codes"
    assert np.array_equal(got[~nan], ref[~nan]), "fp8 decode vs torch"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "fp8 -0"
    for row in read_golden("e4m3fn_landmarks.txt"):
        if row[0] == "decode":
            code, val = int(row[1], 16), float(row[2])
            d = orc.e4m3fn_decode(code)
            assert (math.isnan(val) and math.isnan(d)) or (
                d == val and math.copysign(1, d) == math.copysign(1, val)), row


def pin_fp8_encode_landmarks(orc):
    for row in read_golden("e4m3fn_landmarks.txt"):
        if row[0] == "encode":
            val, code = float(row[1]), int(row[2], 16)
            assert orc.e4m3fn_encode(val) == code, row


def fp8_sweep_values(rng) -> np.ndarray:
    """Every finite bf16 value at several scales, every midpoint between
    neighbouring fp8 magnitudes and its fp64 neighbours, and the saturation
    and subnormal edges."""
    bf = all_finite_bf16()
    bf = bf[np.abs(bf) < 1e6]
    mags = fp8_values_torch()[:0x7F]
    mids = (mags[1:] + mags[:-1]) / 2.0
    pts = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    edges = np.array([447.0, 448.0, 449.0, 463.9, 464.0, 464.1, 479.9, 480.0,
                      1e6, 1e30, 2.0 ** -10, 2.0 ** -11, 2.0 ** -9, 0.0])
    scaled = [bf, bf / np.float64(np.float32(0.05)), bf * 2.0 ** -7]
    sweep = np.concatenate(scaled + [pts, -pts, edges, -edges,
                                     rng.standard_normal(20000) * 100])
    return sweep


def pin_fp8_encode_bruteforce(orc, n_limit: int | None = None):
    rng = np.random.Generator(np.random.PCG64(7))
    v = fp8_sweep_values(rng)
    if n_limit is not None:
        v = v[rng.permutation(v.size)[:n_limit]]
    got = orc.e4m3fn_encode_array(v)
    ref = fp8_encode_bruteforce(v)
    bad = got != ref
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"fp8 encode: {int(bad.sum())} mismatches; first "
                             f"v={v[i]!r} got={got[i]:#04x} ref={ref[i]:#04x}")


def pin_fp8_encode_torch(orc):
    """In range (|v| <= 448) the oracle equals torch's fp32 -> e4m3fn cast."""
    rng = np.random.Generator(np.random.PCG64(8))
    mag = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000))
    v = (mag * np.where(rng.random(mag.size) < 0.5, -1, 1)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3fn_encode_array(v.astype(np.float64))
    assert np.array_equal(got, ref), f"fp8 vs torch: {int((got != ref).sum())} differ"


def pin_bf16_landmarks(orc):
    for row in read_golden("bf16_landmarks.txt"):
        if row[0] == "decode":
            code, val = int(row[1], 16), float(row[2])
            d = orc.bf16_decode(code)
            assert d == val and math.copysign(1, d) == math.copysign(1, val), row
        else:
            val, code = float(row[1]), int(row[2], 16)
            assert orc.bf16_encode(val) == code, row


def pin_bf16_encode_torch(orc):
    """For fp32 inputs the oracle equals torch's fp32 -> bf16 cast (RNE)."""
    rng = np.random.Generator(np.random.PCG64(9))
    bits = rng.integers(0, 2 ** 32, size=30000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_encode_array(f.astype(np.float64))
    assert np.array_equal(got, ref), f"bf16 vs torch: {int((got != ref).sum())} differ"


def pin_bf16_encode_bruteforce(orc):
    """For fp64 inputs between bf16 values (and at their midpoints) the oracle
    returns the nearest pattern, ties to even, with no double rounding."""
    rng = np.random.Generator(np.random.PCG64(10))
    base = rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))
    pats = (base.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    lo = bf16_to_f64(pats)
    hi = bf16_to_f64(pats + np.uint16(1))    # next pattern: next larger magnitude
    mid = (lo + hi) / 2.0
    v = np.concatenate([base, mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf),
                        lo + (hi - lo) * (0.5 + 2.0 ** -30)])
    v = v[np.isfinite(v) & (np.abs(v) < 1e38)]
    got = orc.bf16_encode_array(v)
    ref = bf16_encode_bruteforce(v)
    bad = got != ref
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"bf16 encode: {int(bad.sum())} mismatches; first "
                             f"v={v[i]!r} got={got[i]:#06x} ref={ref[i]:#06x}")


def pin_f16_decode(orc):
    """Every binary16 pattern decodes as numpy's float16 does (NaN patterns
    to NaN), signed zeros included."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = f16_to_f64(bits)
    got = np.array([orc.f16_decode(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "f16 NaN patterns"
    assert np.array_equal(got[~nan], ref[~nan]), "f16 decode values"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "f16 decode signs"


def pin_f16_landmarks(orc):
    for row in read_golden("f16_landmarks.txt"):
        if row[0] == "decode":
            code, val = int(row[1], 16), float(row[2])
            d = orc.f16_decode(code)
            assert d == val and math.copysign(1, d) == math.copysign(1, val), row
        else:
            val, code = float(row[1]), int(row[2], 16)
            assert orc.f16_encode(val) == code, (row, hex(orc.f16_encode(val)))


def pin_f16_encode_numpy(orc):
    """For fp64 inputs over the whole range (subnormals, overflow to
    infinity included) the oracle equals numpy's float64 -> float16 cast,
    which rounds to nearest even in one step."""
    rng = np.random.Generator(np.random.PCG64(11))
    v = rng.standard_normal(40000) * np.exp(rng.uniform(-22, 13, 40000))
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = orc.f16_encode_array(v)
    bad = got != ref
    assert not bad.any(), f"f16 vs numpy: {int(bad.sum())} differ, first v={v[bad][0]!r}"


def pin_f16_encode_bruteforce(orc):
    """At every midpoint between adjacent finite binary16 values (and one
    fp64 step either side of it) the oracle returns the nearest pattern, ties
    to the even pattern, by direct comparison with both neighbours."""
    lo_bits = np.arange(0, 0x7BFF, dtype=np.uint16)          # finite, next one finite
    lo, hi = f16_to_f64(lo_bits), f16_to_f64(lo_bits + np.uint16(1))
    mid = (lo + hi) / 2.0
    for v, want in ((mid, np.where(lo_bits % 2 == 0, lo_bits, lo_bits + 1)),
                    (np.nextafter(mid, 0), lo_bits), (np.nextafter(mid, np.inf), lo_bits + 1)):
        got = orc.f16_encode_array(v)
        assert np.array_equal(got, want.astype(np.uint16)), "f16 positive midpoints"
        got_n = orc.f16_encode_array(-v)
        assert np.array_equal(got_n, (want | 0x8000).astype(np.uint16)), "f16 negative midpoints"
    # past the largest finite value: below 65520 stays 65504, from 65520 on infinity
    assert orc.f16_encode(np.nextafter(65520.0, 0)) == 0x7BFF
    assert orc.f16_encode(65520.0) == 0x7C00 and orc.f16_encode(-1e300) == 0xFC00


# -- RoPE row pins -------------------------------------------------------------------


def _angle_row(dim, pos, theta, dtype=np.float32):
    return workloads.freqs_table(pos + 1, dim, theta)[pos].astype(dtype)


def pin_rope_pos0_identity(orc):
    """Row 0 of the table is (1, 0, 1, 0, ...): rotation by 0 is the identity."""
    rng = np.random.Generator(np.random.PCG64(11))
    for dim in (2, 64, 128):
        x = rng.standard_normal(dim)
        row0 = workloads.freqs_table(4, dim, 10000.0)[0]
        for inter in (0, 1):
            assert np.array_equal(orc.rope_row(x, row0, inter), x), (dim, inter)


def pin_rope_complex(orc):
    """Rotate-half pairs (i, i+d/2) and interleaved pairs (2i, 2i+1), each
    multiplied as complex numbers by cos + i sin (numpy complex128)."""
    rng = np.random.Generator(np.random.PCG64(12))
    for dim in (2, 8, 64, 128):
        for pos in (1, 7, 1000):
            x = rng.standard_normal(dim)
            fr = _angle_row(dim, pos, 10000.0)
            w = fr[0::2].astype(np.float64) + 1j * fr[1::2].astype(np.float64)
            h = dim // 2
            z = (x[:h] + 1j * x[h:]) * w
            ref = np.concatenate([z.real, z.imag])
            got = orc.rope_row(x, fr, 0)
            assert np.allclose(got, ref, rtol=1e-15, atol=1e-15), ("half", dim, pos)
            z = (x[0::2] + 1j * x[1::2]) * w
            ref = np.empty(dim)
            ref[0::2], ref[1::2] = z.real, z.imag
            got = orc.rope_row(x, fr, 1)
            assert np.allclose(got, ref, rtol=1e-15, atol=1e-15), ("inter", dim, pos)


def pin_rope_pair_norm(orc):
    """|rotated pair|^2 = |pair|^2 (cos^2 + sin^2) holds exactly in fp64 up to
    rounding: a dropped term or a wrong sign breaks it."""
    rng = np.random.Generator(np.random.PCG64(13))
    dim = 64
    for inter in (0, 1):
        for pos in (3, 4095):
            x = rng.standard_normal(dim)
            fr = _angle_row(dim, pos, 10000.0).astype(np.float64)
            y = orc.rope_row(x, fr.astype(np.float32), inter)
            idx = (np.arange(0, dim, 2), np.arange(1, dim, 2)) if inter else (
                np.arange(dim // 2), np.arange(dim // 2, dim))
            n_in = (x[idx[0]] ** 2 + x[idx[1]] ** 2) * (fr[0::2] ** 2 + fr[1::2] ** 2)
            n_out = y[idx[0]] ** 2 + y[idx[1]] ** 2
            assert np.allclose(n_out, n_in, rtol=1e-13), (inter, pos)


def pin_rope_textbook_2d(orc):
    """dim = 2: (1, 0) rotated by theta lands on (cos, sin); (0, 1) on
    (-sin, cos) -- the counter-clockwise rotation matrix."""
    fr = np.array([0.6, 0.8], np.float32)
    c, s = float(fr[0]), float(fr[1])
    for inter in (0, 1):
        assert np.array_equal(orc.rope_row(np.array([1.0, 0.0]), fr, inter), [c, s])
        assert np.array_equal(orc.rope_row(np.array([0.0, 1.0]), fr, inter), [-s, c])


def pin_rope_inverse(orc):
    """Rotating by the table row with negated sines undoes the rotation up to
    the fp32 rounding of cos/sin."""
    rng = np.random.Generator(np.random.PCG64(14))
    dim = 128
    x = rng.standard_normal(dim)
    for inter in (0, 1):
        fr = _angle_row(dim, 777, 500000.0)
        inv = fr.copy()
        inv[1::2] = -inv[1::2]
        back = orc.rope_row(orc.rope_row(x, fr, inter), inv, inter)
        assert np.allclose(back, x, rtol=0, atol=1e-6), inter


def pin_rope_relative_position(orc):
    """<rope_m q, rope_n k> = <rope_(m-n) q, k> (fp32 table: to ~1e-6)."""
    rng = np.random.Generator(np.random.PCG64(15))
    dim = 64
    tab = workloads.freqs_table(512, dim, 10000.0)
    q, k = rng.standard_normal(dim), rng.standard_normal(dim)
    for inter in (0, 1):
        for m, n in ((10, 3), (300, 299), (511, 0)):
            lhs = orc.rope_row(q, tab[m], inter) @ orc.rope_row(k, tab[n], inter)
            rhs = orc.rope_row(q, tab[m - n], inter) @ k
            assert abs(lhs - rhs) <= 1e-5 * np.linalg.norm(q) * np.linalg.norm(k), (
                inter, m, n, lhs, rhs)


def pin_rope_interleaved_permutation(orc):
    """Interleaved rotation of P x equals P (rotate-half rotation of x), where
    P sends element i to 2i and element i + d/2 to 2i + 1 (bit-exact)."""
    rng = np.random.Generator(np.random.PCG64(16))
    for dim in (64, 128):
        x = rng.standard_normal(dim)
        fr = _angle_row(dim, 123, 10000.0)
        h = dim // 2
        perm = np.empty(dim, np.int64)
        perm[0::2] = np.arange(h)
        perm[1::2] = np.arange(h, dim)
        assert np.array_equal(orc.rope_row(x[perm], fr, 1), orc.rope_row(x, fr, 0)[perm])


# -- RMSNorm row pins ----------------------------------------------------------------


def pin_rmsnorm_closed_forms(orc):
    rng = np.random.Generator(np.random.PCG64(17))
    n = 512
    x = rng.standard_normal(n) * 3.0
    ms = float(np.mean(x * x))
    ones = np.ones(n)
    for eps in (0.0, 1e-6, 0.25, 10.0):
        y = orc.rmsnorm_row(x, ones, eps)
        rms = math.sqrt(float(np.mean(y * y)))
        assert abs(rms - math.sqrt(ms / (ms + eps))) <= 1e-14, eps
    # scale invariance (eps = 0)
    y1 = orc.rmsnorm_row(x, ones, 0.0)
    assert np.allclose(orc.rmsnorm_row(x * 37.5, ones, 0.0), y1, rtol=1e-14, atol=0)
    assert np.array_equal(orc.rmsnorm_row(x * 4.0, ones, 0.0), y1)
    # constant row c: y_k = c g_k / sqrt(c^2 + eps)
    g = rng.uniform(0.5, 1.5, n)
    for c in (-2.5, 0.125, 3.0):
        y = orc.rmsnorm_row(np.full(n, c), g, 0.01)
        assert np.allclose(y, c * g / math.sqrt(c * c + 0.01), rtol=1e-14), c
    # inv_rms alone
    assert abs(orc.inv_rms(x, 0.5) - 1 / math.sqrt(ms + 0.5)) <= 1e-15


def pin_rmsnorm_torch(orc):
    """Equal to torch.nn.functional.rms_norm in float64."""
    rng = np.random.Generator(np.random.PCG64(18))
    for n in (8, 128, 512):
        x = rng.standard_normal(n)
        g = rng.uniform(0.5, 1.5, n)
        for eps in (1e-6, 0.3):
            ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (n,),
                                               weight=torch.from_numpy(g), eps=eps).numpy()
            assert np.allclose(orc.rmsnorm_row(x, g, eps), ref, rtol=1e-14, atol=1e-15)


# -- composite (entry point) pins -----------------------------------------------------


def slot_owners(row_offsets, cache_lengths, page_table, page_size):
    """Inverse scan of the page table: for every physical (page, offset) that
    holds one of this step's tokens, that token and its cache slot."""
    owners = {}
    B = row_offsets.size - 1
    for b in range(B):
        c, n = int(cache_lengths[b]), int(row_offsets[b + 1] - row_offsets[b])
        for col, page in enumerate(page_table[b]):
            if page == workloads.UNUSED_PAGE:
                continue
            for off in range(page_size):
                slot = col * page_size + off
                if c <= slot < c + n:
                    key = (int(page), off)
                    assert key not in owners, f"page table maps {key} twice"
                    owners[key] = (int(row_offsets[b]) + slot - c, slot)
    return owners


def _complex_rope(x, cs, sn, interleaved):
    """x [..., d] fp64, cs/sn broadcastable to [..., d/2]."""
    w = cs + 1j * sn
    out = np.empty_like(x)
    if interleaved:
        z = (x[..., 0::2] + 1j * x[..., 1::2]) * w
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
    else:
        h = x.shape[-1] // 2
        z = (x[..., :h] + 1j * x[..., h:]) * w
        out[..., :h], out[..., h:] = z.real, z.imag
    return out


def mla_reference(case):
    """Independent fp64 reference for a fused MLA case: numpy complex RoPE and
    torch's float64 rms_norm, tokens located by the inverse page-table scan.
    Returns (q_ref [T,H,R], y_ref [T,W], owners)."""
    S = case.meta["page_size"]
    owners = slot_owners(case.row_offsets, case.cache_lengths, case.page_table, S)
    assert len(owners) == case.T, "some token has no slot"
    pos = np.empty(case.T, np.int64)
    for (page, off), (t, slot) in owners.items():
        pos[t] = slot
    fr = elem_to_f64(case.freqs[pos])
    cs, sn = fr[:, 0::2], fr[:, 1::2]
    q_ref = _complex_rope(elem_to_f64(case.q), cs[:, None, :], sn[:, None, :], False)
    x = bf16_to_f64(case.latent)
    Dn = case.Dn
    y_ref = np.empty_like(x)
    y_ref[:, :Dn] = torch.nn.functional.rms_norm(
        torch.from_numpy(x[:, :Dn].copy()), (Dn,),
        weight=torch.from_numpy(elem_to_f64(case.gamma)), eps=case.epsilon).numpy()
    y_ref[:, Dn:] = _complex_rope(x[:, Dn:], cs, sn, False)
    return q_ref, y_ref, owners


def run_mla(orc, case, q_out_dtype=None):
    q_out = np.zeros(case.q.shape, case.q.dtype if q_out_dtype is None else q_out_dtype)
    cache = case.cache.copy()
    ts = None if case.token_scales is None else case.token_scales.copy()
    orc.mla_rope_rmsnorm_quant(q_out, case.q, case.latent, case.row_offsets,
                               case.cache_lengths, case.page_table, case.freqs,
                               case.gamma, case.epsilon, cache, case.layer_idx,
                               case.scale_mode, case.tensor_scale, ts)
    return q_out, cache, ts


def check_mla_against_reference(case, q_out, cache, ts):
    q_ref, y_ref, owners = mla_reference(case)
    assert_correctly_rounded(elem_to_f64(q_out), q_ref, ulp_of(q_out), "q_rope_output")
    L = case.layer_idx
    expect = case.cache.copy()
    written = np.zeros(case.cache.shape[:3], bool)
    for (page, off), (t, slot) in owners.items():
        written[L, page, off] = True
        row = cache[L, page, off, 0]
        if case.cache.dtype == np.uint16:
            assert_correctly_rounded(bf16_to_f64(row), y_ref[t], ulp_bf16, f"row {t}")
        else:
            if case.scale_mode == "per_tensor":
                s = float(case.tensor_scale)
            else:
                amax = float(np.max(np.abs(y_ref[t])))
                s = float(np.float32(amax / 448.0))
                got_s = float(ts[L, page, off, 0])
                assert got_s == s or abs(got_s - s) <= 2.0 ** -23 * s, (t, got_s, s)
                s = got_s
                if amax > 0:
                    assert np.any((row & 0x7F) == 0x7E), f"row {t}: no +-448 code"
            if s == 0.0:
                assert np.all((row & 0x7F) == 0), f"row {t}: zero scale"
            else:
                assert_correctly_rounded(fp8_to_f64(row), y_ref[t] / s, ulp_fp8,
                                         f"fp8 row {t}", sat=448.0)
        expect[L, page, off] = cache[L, page, off]
    # every byte outside the new tokens' rows is unchanged
    assert np.array_equal(cache, expect), "bytes outside the new rows changed"
    if ts is not None:
        keep = ~written
        assert np.array_equal(ts[keep].view(np.uint32),
                              case.token_scales[keep].view(np.uint32)), "scales outside"


def small_mla_cases():
    """Small cases covering ragged batches, prior lengths, page crossings,
    zero-length requests, both scale modes and a bf16 cache."""
    yield workloads.mla_tiny()
    yield workloads.build_mla("mla_small_decode", 2001, [1] * 9, [0, 5, 15, 16, 17, 31, 32, 47, 63],
                              H=8, page_size=16, max_seq_len=64, spare_pages=3,
                              scale_mode="per_tensor", tensor_scale=0.05)
    yield workloads.build_mla("mla_small_ragged", 2002, [7, 0, 13, 1, 0, 20], [3, 9, 0, 30, 0, 2],
                              H=16, page_size=8, max_seq_len=64, spare_pages=5,
                              latent_sigma=2.0, scale_mode="per_tensor", tensor_scale=0.05)
    yield workloads.build_mla("mla_small_token", 2003, [1, 1, 1, 9, 12], [40, 0, 100, 0, 3],
                              H=4, page_size=16, max_seq_len=128, spare_pages=2,
                              outlier_p=0.01, scale_mode="per_token")
    yield workloads.build_mla("mla_small_bf16", 2004, [4, 6], [2, 0], H=4,
                              page_size=4, max_seq_len=16, spare_pages=2,
                              scale_mode="none", cache_dtype="bf16")


def pin_mla_composite(orc):
    for case in small_mla_cases():
        q_out, cache, ts = run_mla(orc, case)
        check_mla_against_reference(case, q_out, cache, ts)


def dtype_mla_cases():
    """Small MLA cases over the element types the pages parameterise: q_rope
    (dtype) bf16 / fp16, freqs_cis (freq_dtype) fp32 / bf16 / fp16, gamma
    (gamma_dtype) bf16 / fp16 / fp32, with an fp8 (tensor and token scale)
    or bf16 cache; each with its q output types."""
    specs = [("f16", "f32", "bf16", "per_tensor", "fp8"), ("bf16", "bf16", "f32", "per_token", "fp8"),
             ("f16", "f16", "f16", "none", "bf16"), ("bf16", "f16", "bf16", "per_tensor", "fp8"),
             ("f16", "bf16", "f32", "per_token", "fp8")]
    for k, (qd, fd, gd, mode, cache) in enumerate(specs):
        yield workloads.build_mla(f"mla_types_{qd}_{fd}_{gd}", 2100 + k, [5, 0, 9, 3], [2, 7, 0, 30],
                                  H=6, page_size=8, max_seq_len=64, spare_pages=3,
                                  outlier_p=0.02, scale_mode=mode, tensor_scale=0.05,
                                  cache_dtype=cache, q_dtype=qd, freq_dtype=fd, gamma_dtype=gd)


def pin_mla_types(orc):
    """Every q input / q output / freqs / gamma element type: q_rope_output is
    the correctly rounded value of the exact rotation in its own type (bf16,
    fp16 or fp32), the cache rows as in the bf16 case (the exact values of
    the widened inputs), and the cache rows do not depend on q's output type."""
    for case in dtype_mla_cases():
        outs = (np.uint16, np.float16, np.float32)
        caches = []
        for od in outs:
            q_out, cache, ts = run_mla(orc, case, od)
            check_mla_against_reference(case, q_out, cache, ts)
            caches.append(cache)
        assert all(np.array_equal(c, caches[0]) for c in caches), case.name


def pin_mla_f32_q(orc):
    """fp32 q output: the correctly rounded fp32 of the exact rotation, and the
    bf16 output is that value's bf16 rounding up to the double-rounding case."""
    case = list(small_mla_cases())[2]
    q32 = np.zeros(case.q.shape, np.float32)
    cache = case.cache.copy()
    orc.mla_rope_rmsnorm_quant(q32, case.q, case.latent, case.row_offsets, case.cache_lengths,
                               case.page_table, case.freqs, case.gamma, case.epsilon, cache,
                               case.layer_idx, case.scale_mode, case.tensor_scale, None)
    q_ref, _, _ = mla_reference(case)
    ulp32 = np.ldexp(1.0, np.frexp(np.maximum(np.abs(q_ref), 2.0 ** -126))[1] - 1 - 23)
    assert np.all(np.abs(q32.astype(np.float64) - q_ref) <= 0.5 * ulp32 * (1 + 1e-12)), "fp32 q"
    # the fp32 run writes the same cache rows as the bf16 run
    _, cache_b, _ = run_mla(orc, case)
    assert np.array_equal(cache, cache_b)


def expected_token_plan(case, T=None):
    """The plan a batch implies, from the inverse page-table scan: row t is
    (page, offset, slot, 1) for the physical (page, offset) that holds token
    t's slot, zeros for a token no valid page-table entry places."""
    T = case.T if T is None else T
    P = case.cache.shape[1]
    pt = case.page_table.copy()
    pt[pt >= P] = workloads.UNUSED_PAGE      # ids past the pool place nothing
    plan = np.zeros((T, 4), np.uint32)
    for (page, off), (t, slot) in slot_owners(case.row_offsets, case.cache_lengths, pt,
                                              case.meta["page_size"]).items():
        if t < T:
            plan[t] = (page, off, slot, 1)
    return plan


def run_token_plan(orc, case, T=None):
    return orc.token_plan(case.T if T is None else T, case.row_offsets, case.cache_lengths,
                          case.page_table, case.cache.shape[1], case.meta["page_size"])


def token_plan_cases():
    """The small MLA cases, plus one whose page table holds ids past the pool
    and one more row than its offsets cover."""
    yield from small_mla_cases()
    bad = workloads.build_mla("mla_small_badpages", 2011, [5, 9, 3], [14, 0, 40], H=4,
                              page_size=8, max_seq_len=64, spare_pages=2,
                              scale_mode="per_tensor", tensor_scale=0.05)
    P = bad.cache.shape[1]
    bad.page_table[0, 2] = P                 # request 0: slots 16..23 lose their page
    bad.page_table[2, 5] = P + 7             # request 2: slots 40..47
    yield bad


def pin_token_plan(orc):
    for case in token_plan_cases():
        got = run_token_plan(orc, case)
        assert np.array_equal(got, expected_token_plan(case)), case.name
    # rows past the last offset: nothing owns them
    case = workloads.mla_tiny()
    got = run_token_plan(orc, case, case.T + 3)
    assert np.array_equal(got, expected_token_plan(case, case.T + 3))
    assert not got[case.T:].any()


def run_mla_planned(orc, case, plan, q_f32=False):
    q_out = np.zeros(case.q.shape, np.float32) if q_f32 else np.zeros_like(case.q)
    cache = case.cache.copy()
    ts = None if case.token_scales is None else case.token_scales.copy()
    skipped = False
    try:
        orc.mla_rope_rmsnorm_quant_planned(q_out, case.q, case.latent, plan, case.freqs,
                                           case.gamma, case.epsilon, cache, case.layer_idx,
                                           case.scale_mode, case.tensor_scale, ts)
    except oracle.OracleError:
        skipped = True                       # some token was skipped; the rest is written
    return q_out, cache, ts, skipped


def free_plan(case, rng, skip_every=0):
    """A plan that places each token at a random distinct (page, offset) of
    the pool with a random position, unrelated to the batch's page table;
    every skip_every-th token (when > 0) is marked not placed."""
    L, P, S = case.cache.shape[:3]
    cells = rng.choice(P * S, size=case.T, replace=False)
    plan = np.zeros((case.T, 4), np.uint32)
    plan[:, 0], plan[:, 1] = cells // S, cells % S
    plan[:, 2] = rng.integers(0, case.freqs.shape[0], size=case.T)
    plan[:, 3] = 1
    if skip_every:
        plan[::skip_every, 3] = 0
    return plan


def check_mla_planned_free(case, plan, q_out, cache, ts):
    """Outputs of a planned step against the float64 reference at each
    token's planned position; rows land at the planned cells, nothing else
    changes (q of a skipped token stays zero)."""
    placed = plan[:, 3] != 0
    pos = plan[:, 2].astype(np.int64)
    fr = case.freqs[pos].astype(np.float64)
    cs, sn = fr[:, 0::2], fr[:, 1::2]
    q_ref = _complex_rope(bf16_to_f64(case.q), cs[:, None, :], sn[:, None, :], False)
    assert_correctly_rounded(bf16_to_f64(q_out[placed]), q_ref[placed], ulp_bf16, "planned q")
    assert not q_out[~placed].any(), "q written for a skipped token"
    x = bf16_to_f64(case.latent)
    Dn = case.Dn
    y_ref = np.empty_like(x)
    y_ref[:, :Dn] = torch.nn.functional.rms_norm(
        torch.from_numpy(x[:, :Dn].copy()), (Dn,),
        weight=torch.from_numpy(bf16_to_f64(case.gamma)), eps=case.epsilon).numpy()
    y_ref[:, Dn:] = _complex_rope(x[:, Dn:], cs, sn, False)
    L = case.layer_idx
    expect = case.cache.copy()
    for t in np.nonzero(placed)[0]:
        page, off = int(plan[t, 0]), int(plan[t, 1])
        row = cache[L, page, off, 0]
        if case.cache.dtype == np.uint16:
            assert_correctly_rounded(bf16_to_f64(row), y_ref[t], ulp_bf16, f"row {t}")
        else:
            if case.scale_mode == "per_tensor":
                s = float(case.tensor_scale)
            else:
                s = float(ts[L, page, off, 0])
                assert s == float(np.float32(np.max(np.abs(y_ref[t])) / 448.0)), t
            assert_correctly_rounded(fp8_to_f64(row), y_ref[t] / s, ulp_fp8, f"fp8 row {t}",
                                     sat=448.0)
        expect[L, page, off] = row
    assert np.array_equal(cache, expect), "bytes outside the planned rows changed"


def pin_mla_planned(orc):
    """The planned step: with the plan of its own batch it meets the same
    independent reference as the batch form (and equals it bit for bit);
    with a free placement, rows land at the planned cells with the planned
    positions' rotation; tokens marked not placed are skipped."""
    for case in small_mla_cases():
        plan = run_token_plan(orc, case)
        q_out, cache, ts, skipped = run_mla_planned(orc, case, plan)
        assert not skipped
        check_mla_against_reference(case, q_out, cache, ts)
        q_b, cache_b, ts_b = run_mla(orc, case)
        assert np.array_equal(q_out, q_b) and np.array_equal(cache, cache_b)
        if ts is not None:
            assert np.array_equal(ts.view(np.uint32), ts_b.view(np.uint32))
    # in place on a bf16 cache holding the rows: equals the batch in-place form
    for case in small_mla_inplace_cases():
        plan = run_token_plan(orc, case)
        cache0 = place_latent_rows(case)
        q_p = np.zeros_like(case.q)
        c_p = cache0.copy()
        orc.mla_rope_rmsnorm_quant_planned(q_p, case.q, None, plan, case.freqs, case.gamma,
                                           case.epsilon, c_p, case.layer_idx, "none")
        q_b, c_b = run_mla_inplace(orc, case)
        assert np.array_equal(q_p, q_b) and np.array_equal(c_p, c_b), case.name
    rng = np.random.default_rng(2020)
    for k, case in enumerate(small_mla_cases()):
        plan = free_plan(case, rng, skip_every=3 if k % 2 else 0)
        q_out, cache, ts, skipped = run_mla_planned(orc, case, plan)
        assert skipped == bool(k % 2 and case.T)
        check_mla_planned_free(case, plan, q_out, cache, ts)


def small_mla_inplace_cases():
    """bf16 latent caches for the in-place form: ragged prefill with page
    crossings and zero-length requests, decode rows, fp32 q in one case."""
    yield list(small_mla_cases())[4]
    yield workloads.build_mla("mla_inplace_ragged", 2011, [7, 0, 13, 1, 0, 20], [3, 9, 0, 30, 0, 2],
                              H=16, page_size=8, max_seq_len=64, spare_pages=5, latent_sigma=2.0,
                              scale_mode="none", cache_dtype="bf16")
    yield workloads.build_mla("mla_inplace_decode", 2012, [1] * 9, [0, 5, 15, 16, 17, 31, 32, 47, 63],
                              H=8, page_size=16, max_seq_len=64, spare_pages=3,
                              scale_mode="none", cache_dtype="bf16")


def place_latent_rows(case):
    """The case's bf16 cache with each new token's latent row written at its
    slot (what the in-place form expects to find there)."""
    cache = case.cache.copy()
    owners = slot_owners(case.row_offsets, case.cache_lengths, case.page_table,
                         case.meta["page_size"])
    for (page, off), (t, slot) in owners.items():
        cache[case.layer_idx, page, off, 0] = case.latent[t]
    return cache


def run_mla_inplace(orc, case, q_f32=False):
    q_out = np.zeros(case.q.shape, np.float32 if q_f32 else np.uint16)
    cache = place_latent_rows(case)
    orc.mla_rope_rmsnorm_inplace(q_out, case.q, case.row_offsets, case.cache_lengths,
                                 case.page_table, case.freqs, case.gamma, case.epsilon, cache,
                                 case.layer_idx)
    return q_out, cache


def pin_mla_inplace(orc):
    """In-place form: with the latent rows placed at their slots it gives
    exactly what the (separately pinned) buffer form gives with a bf16 cache,
    q included, and nothing else in the pool changes; rows placed elsewhere
    are not read."""
    for case in small_mla_inplace_cases():
        for q_f32 in (False, True):
            q_a, cache_a = run_mla_inplace(orc, case, q_f32)
            q_b = np.zeros(case.q.shape, np.float32 if q_f32 else np.uint16)
            cache_b = case.cache.copy()
            orc.mla_rope_rmsnorm_quant(q_b, case.q, case.latent, case.row_offsets,
                                       case.cache_lengths, case.page_table, case.freqs,
                                       case.gamma, case.epsilon, cache_b, case.layer_idx, "none")
            assert np.array_equal(q_a.view(np.uint8), q_b.view(np.uint8)), case.name
            assert np.array_equal(cache_a, cache_b), case.name
    # the rows are read from the token's own slot: garbage at the slots gives
    # a different result, garbage elsewhere does not
    case = list(small_mla_inplace_cases())[1]
    _, ref = run_mla_inplace(orc, case)
    cache = place_latent_rows(case)
    owners = slot_owners(case.row_offsets, case.cache_lengths, case.page_table,
                         case.meta["page_size"])
    used = np.zeros(cache.shape[:3], bool)
    for (page, off) in owners:
        used[case.layer_idx, page, off] = True
    cache[~used] ^= 0x5555
    orc.mla_rope_rmsnorm_inplace(np.zeros_like(case.q), case.q, case.row_offsets,
                                 case.cache_lengths, case.page_table, case.freqs, case.gamma,
                                 case.epsilon, cache, case.layer_idx)
    assert np.array_equal(cache[used], ref[used]), "rows outside the slots were read"


def pin_mla_position0(orc):
    """Tokens at position 0 come back unchanged in q (values; +-0 equal)."""
    case = workloads.build_mla("mla_pos0", 2005, [1] * 6, [0] * 6, H=8,
                               page_size=4, max_seq_len=8, spare_pages=1)
    q_out, _, _ = run_mla(orc, case)
    assert np.array_equal(bf16_to_f64(q_out), bf16_to_f64(case.q))


def pin_mla_zero_row_per_token(orc):
    """An all-zero latent row under per-token scaling stores scale 0 and zero
    codes; the non-rope part keeps each input's sign (x r g with r, g > 0)."""
    case = workloads.build_mla("mla_zero", 2006, [2], [0], H=4, page_size=4,
                               max_seq_len=8, spare_pages=1, scale_mode="per_token")
    case.latent[0, :] = 0x0000
    case.latent[0, ::3] = 0x8000
    q_out, cache, ts = run_mla(orc, case)
    page = int(case.page_table[0, 0])
    row = cache[case.layer_idx, page, 0, 0]
    assert ts[case.layer_idx, page, 0, 0] == 0.0
    assert np.all((row & 0x7F) == 0)
    Dn = case.Dn
    assert np.array_equal(row[:Dn] >> 7, (case.latent[0, :Dn] >> 15).astype(np.uint8))


# The K reference's own error with the norm: torch's rms_norm (a square
# root, a division and two products, each rounded in binary64) and the
# complex product that rotates it leave an absolute error of a few 2^-53 of
# the pair's magnitude; where the pair cancels, that is all the reference
# holds.  2^-49 x the pair magnitude bounds it with margin.
QK_REF_NORM_TOL = 2.0 ** -49


def pair_magnitude_of(v: np.ndarray, interleaved: bool) -> np.ndarray:
    """|(a, b)| of the rotation pair each element of the last axis is in."""
    out = np.empty_like(v)
    if interleaved:
        m = np.hypot(v[..., 0::2], v[..., 1::2])
        out[..., 0::2], out[..., 1::2] = m, m
    else:
        h = v.shape[-1] // 2
        m = np.hypot(v[..., :h], v[..., h:])
        out[..., :h], out[..., h:] = m, m
    return out


def qk_k_tolerance(ref: np.ndarray, case, k_norm: bool):
    """abs_tol for a K reference row (None without the norm: the rotation of
    bf16 values by fp32 / 16-bit cos and sin is exact in binary64)."""
    if not k_norm:
        return None
    return QK_REF_NORM_TOL * pair_magnitude_of(ref, case.interleaved)


def qk_reference(case, k_norm: bool):
    S = case.meta["page_size"]
    owners = slot_owners(case.row_offsets, case.cache_lengths, case.page_table, S)
    assert len(owners) == case.T
    slot_of = np.empty(case.T, np.int64)
    for (page, off), (t, slot) in owners.items():
        slot_of[t] = slot
    pos = case.position_ids.astype(np.int64) if case.position_ids is not None else slot_of
    fr = elem_to_f64(case.freqs[pos])
    cs, sn = fr[:, 0::2], fr[:, 1::2]
    q_ref = _complex_rope(elem_to_f64(case.q), cs[:, None, :], sn[:, None, :],
                          case.interleaved)
    L = case.layer_idx
    k_ref = {}
    for (page, off), (t, slot) in owners.items():
        x = bf16_to_f64(case.k_cache[L, page, off])            # [Hkv, D]
        if k_norm:
            C = case.gamma.size
            x[:, :C] = torch.nn.functional.rms_norm(
                torch.from_numpy(x[:, :C].copy()), (C,),
                weight=torch.from_numpy(bf16_to_f64(case.gamma)),
                eps=case.epsilon).numpy()
        k_ref[(page, off)] = _complex_rope(x, cs[t][None, :], sn[t][None, :],
                                           case.interleaved)
    return q_ref, k_ref


def dtype_qk_cases():
    """Q/K cases with fp16 Q (the pages' dtype of q_proj and the output) and
    bf16 / fp16 / fp32 freqs_cis (freq_dtype), both rope styles."""
    yield workloads.build_qk("qk_types_f16_bf16", 3101, [5, 0, 17, 1], [0, 4, 11, 31],
                             Hq=4, Hkv=2, D=128, page_size=16, max_seq_len=4096,
                             theta=500000.0, interleaved=True, with_position_ids=True,
                             norm_cols=128, spare_pages=3, q_dtype="f16", freq_dtype="bf16")
    yield workloads.build_qk("qk_types_f16_f16", 3102, [3, 9], [14, 0], Hq=3, Hkv=1, D=64,
                             page_size=4, max_seq_len=64, theta=10000.0,
                             interleaved=False, with_position_ids=False,
                             norm_cols=40, spare_pages=2, q_dtype="f16", freq_dtype="f16")
    yield workloads.build_qk("qk_types_bf16_f16", 3103, [6, 2], [1, 7], Hq=2, Hkv=2, D=96,
                             page_size=8, max_seq_len=64, theta=10000.0,
                             interleaved=False, with_position_ids=True,
                             norm_cols=96, spare_pages=1, q_dtype="bf16", freq_dtype="f16")


def pin_qk_types(orc):
    for case in dtype_qk_cases():
        q_out = np.zeros_like(case.q)
        k = case.k_cache.copy()
        orc.qk_rope_paged_ragged(q_out, case.q, case.row_offsets, case.cache_lengths,
                                 case.page_table, k, case.layer_idx, case.freqs,
                                 case.position_ids, case.interleaved, case.gamma, case.epsilon)
        q_ref, k_ref = qk_reference(case, True)
        assert_correctly_rounded(elem_to_f64(q_out), q_ref, ulp_of(q_out), f"{case.name} q")
        L = case.layer_idx
        for (page, off), ref in k_ref.items():
            assert_correctly_rounded(bf16_to_f64(k[L, page, off]), ref, ulp_bf16,
                                     f"{case.name} k {page},{off}",
                                     abs_tol=qk_k_tolerance(ref, case, True))


def pin_qk_norm_exact_cancellation(orc):
    """The fused K norm where a rotation pair cancels exactly ([QK]: the K
    norm, then RoPE): with cos = sin in every row and x_a g_a = x_b g_b for
    every pair (x_b / x_a = 1.2, not a power of two), the first output of each
    pair is exactly zero -- r is common to both members, so the definition's
    value is r (x_a g_a c - x_b g_b s) = 0 -- and every other value is
    correctly rounded.  Both rope styles; bf16 freqs_cis."""
    D, h = 64, 32
    for inter in (True, False):
        case = workloads.build_qk(f"qk_cancel_{int(inter)}", 3201, [4, 3], [2, 9], Hq=1, Hkv=2,
                                  D=D, page_size=4, max_seq_len=32, theta=10000.0,
                                  interleaved=inter, with_position_ids=False, norm_cols=D,
                                  spare_pages=1, freq_dtype="bf16")
        ia = np.arange(0, D, 2) if inter else np.arange(h)
        ib = ia + 1 if inter else ia + h
        case.freqs[:] = workloads.bf16_bits(np.float32(0.70703125))   # cos = sin
        case.gamma[ia] = workloads.bf16_bits(np.float32(1.5))
        case.gamma[ib] = workloads.bf16_bits(np.float32(1.25))
        rng = np.random.Generator(np.random.PCG64(3202))
        L = case.layer_idx
        owners = slot_owners(case.row_offsets, case.cache_lengths, case.page_table,
                             case.meta["page_size"])
        for (page, off) in owners:
            for head in range(2):
                kk = (rng.integers(8, 16, size=h) * 2.0 ** rng.integers(-5, 0, size=h) *
                      rng.choice([-1.0, 1.0], size=h))
                x = np.zeros(D, np.float32)
                x[ia], x[ib] = 1.25 * kk, 1.5 * kk                  # both exact in bf16
                case.k_cache[L, page, off, head] = workloads.bf16_bits(x)
        q_out = np.zeros_like(case.q)
        k = case.k_cache.copy()
        orc.qk_rope_paged_ragged(q_out, case.q, case.row_offsets, case.cache_lengths,
                                 case.page_table, k, L, case.freqs, None, inter, case.gamma,
                                 case.epsilon)
        _, k_ref = qk_reference(case, True)
        for (page, off), ref in k_ref.items():
            row = k[L, page, off]
            assert np.all(row[:, ia] & 0x7FFF == 0), f"cancelling pair not zero ({inter})"
            assert np.all(row[:, ib] & 0x7FFF != 0)
            assert_correctly_rounded(bf16_to_f64(row), ref, ulp_bf16, "cancel k",
                                     abs_tol=qk_k_tolerance(ref, case, True))


def pin_rms_norm_kv_gamma_types(orc):
    """The K-cache norm with gamma (and weight_offset) in fp16 or fp32 ([NORM]:
    gamma and weight_offset share a dtype): torch rms_norm (fp64) with the
    widened gamma + offset, each written value correctly rounded."""
    case = list(small_qk_cases())[0]
    S = case.meta["page_size"]
    owners = slot_owners(case.row_offsets, case.cache_lengths, case.page_table, S)
    L = case.layer_idx
    rng = np.random.Generator(np.random.PCG64(77))
    g32 = rng.uniform(0.5, 1.5, 100).astype(np.float32)
    for gamma in (g32.astype(np.float16), g32):
        k = case.k_cache.copy()
        orc.rms_norm_kv_cache_paged(k, L, case.row_offsets, case.cache_lengths, case.page_table,
                                    gamma, case.epsilon, 0.25, case.T, True)
        g = gamma.astype(np.float64) + 0.25
        for (page, off), (t, slot) in owners.items():
            x = bf16_to_f64(case.k_cache[L, page, off])[:, :100]
            ref = torch.nn.functional.rms_norm(torch.from_numpy(x.copy()), (100,),
                                               weight=torch.from_numpy(g),
                                               eps=case.epsilon).numpy()
            assert_correctly_rounded(bf16_to_f64(k[L, page, off][:, :100]), ref, ulp_bf16,
                                     f"kvnorm gamma {gamma.dtype}")
            assert np.array_equal(k[L, page, off][:, 100:], case.k_cache[L, page, off][:, 100:])


def small_qk_cases():
    yield workloads.build_qk("qk_small_inter", 3001, [5, 0, 17, 1], [0, 4, 11, 31],
                             Hq=4, Hkv=2, D=128, page_size=16, max_seq_len=4096,
                             theta=500000.0, interleaved=True, with_position_ids=True,
                             norm_cols=128, spare_pages=3)
    yield workloads.build_qk("qk_small_half", 3002, [3, 9], [14, 0], Hq=3, Hkv=1, D=64,
                             page_size=4, max_seq_len=64, theta=10000.0,
                             interleaved=False, with_position_ids=False,
                             norm_cols=40, spare_pages=2)
    yield workloads.build_qk("qk_small_nonorm", 3003, [6, 2], [1, 7], Hq=2, Hkv=2, D=128,
                             page_size=8, max_seq_len=64, theta=10000.0,
                             interleaved=True, with_position_ids=False,
                             norm_cols=None, spare_pages=1)
    yield workloads.build_qk("qk_small_d256", 3004, [4, 7, 0], [3, 0, 9], Hq=3, Hkv=2, D=256,
                             page_size=8, max_seq_len=128, theta=10000.0,
                             interleaved=False, with_position_ids=True,
                             norm_cols=200, spare_pages=2)
    yield workloads.build_qk("qk_small_d96", 3005, [6, 0, 9], [2, 5, 0], Hq=5, Hkv=3, D=96,
                             page_size=8, max_seq_len=128, theta=10000.0,
                             interleaved=False, with_position_ids=False,
                             norm_cols=72, spare_pages=2)
    yield workloads.build_qk("qk_small_d80", 3006, [3, 11], [7, 1], Hq=4, Hkv=1, D=80,
                             page_size=4, max_seq_len=64, theta=10000.0,
                             interleaved=True, with_position_ids=True,
                             norm_cols=80, spare_pages=2)


def pin_qk_composite(orc):
    for case in small_qk_cases():
        for use_norm in ((False, True) if case.gamma is not None else (False,)):
            q_out = np.zeros_like(case.q)
            k = case.k_cache.copy()
            orc.qk_rope_paged_ragged(q_out, case.q, case.row_offsets, case.cache_lengths,
                                     case.page_table, k, case.layer_idx, case.freqs,
                                     case.position_ids, case.interleaved,
                                     case.gamma if use_norm else None, case.epsilon)
            q_ref, k_ref = qk_reference(case, use_norm)
            assert_correctly_rounded(elem_to_f64(q_out), q_ref, ulp_of(q_out), "qk q")
            expect = case.k_cache.copy()
            L = case.layer_idx
            for (page, off), ref in k_ref.items():
                assert_correctly_rounded(bf16_to_f64(k[L, page, off]), ref, ulp_bf16,
                                         f"qk k {page},{off}",
                                         abs_tol=qk_k_tolerance(ref, case, use_norm))
                expect[L, page, off] = k[L, page, off]
            assert np.array_equal(k, expect), "K elements outside the new rows changed"


def pin_rms_norm_kv(orc):
    """In-place K RMSNorm against torch rms_norm (fp64) with gamma + offset:
    multiply_before_cast rounds once; otherwise the normalised value is
    rounded to bf16 (by the separately pinned codec) before the gamma product."""
    for case in small_qk_cases():
        C = case.gamma.size if case.gamma is not None else 48
        rng = np.random.Generator(np.random.PCG64(case.seed))
        gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, C).astype(np.float32))
        for mbc in (True, False):
            for w in (0.0, 0.25):
                for total in (case.T, max(case.T - 3, 0)):
                    k = case.k_cache.copy()
                    orc.rms_norm_kv_cache_paged(k, case.layer_idx, case.row_offsets,
                                                case.cache_lengths, case.page_table,
                                                gamma, case.epsilon, w, total, mbc)
                    S = case.meta["page_size"]
                    owners = slot_owners(case.row_offsets, case.cache_lengths,
                                         case.page_table, S)
                    L = case.layer_idx
                    expect = case.k_cache.copy()
                    g = bf16_to_f64(gamma) + w
                    for (page, off), (t, slot) in owners.items():
                        if t >= total:
                            continue
                        x = bf16_to_f64(case.k_cache[L, page, off])[:, :C]
                        if mbc:
                            ref = torch.nn.functional.rms_norm(
                                torch.from_numpy(x.copy()), (C,),
                                weight=torch.from_numpy(g), eps=case.epsilon).numpy()
                        else:
                            nrm = torch.nn.functional.rms_norm(
                                torch.from_numpy(x.copy()), (C,), eps=case.epsilon).numpy()
                            ref = bf16_to_f64(orc.bf16_encode_array(nrm)) * g
                        assert_correctly_rounded(bf16_to_f64(k[L, page, off][:, :C]), ref,
                                                 ulp_bf16, f"kvnorm {t} mbc={mbc}")
                        expect[L, page, off, :, :C] = k[L, page, off, :, :C]
                    assert np.array_equal(k, expect), "kvnorm touched other elements"


def qk_token_plan(orc, case):
    L, P, S = case.k_cache.shape[:3]
    return orc.token_plan(case.T, case.row_offsets, case.cache_lengths, case.page_table, P, S)


def pin_rms_norm_kv_planned(orc):
    """The planned K-cache norm: with the plan of its own batch it writes the
    batch form's bits (bf16 both cast orders and weight offsets, fp8 tensor and
    token scales, per-head and per-token statistic, total_seq_len short of
    the batch); with a free placement every placed cell is normalised against
    torch rms_norm in fp64 and nothing else changes."""
    def run_both(case, gamma, w, total, mbc, mode, scales, per_head):
        plan = qk_token_plan(orc, case)
        k_b, k_p = case.k_cache.copy(), case.k_cache.copy()
        s_b = None if scales is None else scales.copy()
        s_p = None if scales is None else scales.copy()
        orc.rms_norm_kv_cache_paged(k_b, case.layer_idx, case.row_offsets, case.cache_lengths,
                                    case.page_table, gamma, case.epsilon, w, total, mbc, mode,
                                    s_b, per_head)
        orc.rms_norm_kv_cache_planned(k_p, case.layer_idx, plan, gamma, case.epsilon, w, total,
                                      mbc, mode, s_p, per_head)
        assert np.array_equal(k_b, k_p), (case.name, mbc, w, total, mode, per_head)
        if s_b is not None:
            assert np.array_equal(s_b.view(np.uint32), s_p.view(np.uint32))
    for case in small_qk_cases():
        C = case.gamma.size if case.gamma is not None else 48
        rng = np.random.Generator(np.random.PCG64(case.seed))
        gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, C).astype(np.float32))
        for mbc, w, total, per_head in ((True, 0.0, case.T, True), (False, 0.25, case.T, True),
                                        (True, 0.25, max(case.T - 3, 0), False)):
            run_both(case, gamma, w, total, mbc, "none", None, per_head)
    for case in small_qk_fp8_cases():
        gamma = case.gamma if case.gamma is not None else workloads.bf16_bits(
            np.linspace(0.5, 1.5, case.k_cache.shape[-1]).astype(np.float32))
        run_both(case, gamma, 0.0, case.T, True, case.k_scale_mode, case.k_scales, True)
    # free placement on a bf16 case
    case = next(iter(small_qk_cases()))
    L, P, S, Hkv, D = case.k_cache.shape
    C = D // 2
    rng = np.random.default_rng(4040)
    gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, C).astype(np.float32))
    cells = rng.choice(P * S, size=case.T, replace=False)
    plan = np.zeros((case.T, 4), np.uint32)
    plan[:, 0], plan[:, 1], plan[:, 3] = cells // S, cells % S, 1
    plan[::4, 3] = 0
    k = case.k_cache.copy()
    try:
        orc.rms_norm_kv_cache_planned(k, case.layer_idx, plan, gamma, case.epsilon, 0.0, case.T)
    except oracle.OracleError:
        pass                                  # entries marked not placed were skipped
    expect = case.k_cache.copy()
    g = bf16_to_f64(gamma)
    for t in np.nonzero(plan[:, 3])[0]:
        page, off = int(plan[t, 0]), int(plan[t, 1])
        x = bf16_to_f64(case.k_cache[case.layer_idx, page, off])[:, :C]
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x.copy()), (C,),
                                           weight=torch.from_numpy(g), eps=case.epsilon).numpy()
        assert_correctly_rounded(bf16_to_f64(k[case.layer_idx, page, off][:, :C]), ref,
                                 ulp_bf16, f"planned kvnorm {t}")
        expect[case.layer_idx, page, off, :, :C] = k[case.layer_idx, page, off, :, :C]
    assert np.array_equal(k, expect), "planned kvnorm touched other elements"


def small_qk_fp8_cases():
    """fp8 K caches: per-tensor scale (interleaved, position ids, full-width
    norm) and per-token scales (rotate-half, partial norm width)."""
    yield workloads.build_qk("qk_fp8_tensor", 3011, [5, 0, 17, 1], [0, 4, 11, 31],
                             Hq=4, Hkv=2, D=128, page_size=16, max_seq_len=4096,
                             theta=500000.0, interleaved=True, with_position_ids=True,
                             norm_cols=128, spare_pages=3, k_dtype="fp8",
                             k_scale_mode="per_tensor")
    yield workloads.build_qk("qk_fp8_token", 3012, [3, 9], [14, 0], Hq=3, Hkv=2, D=64,
                             page_size=4, max_seq_len=64, theta=10000.0, interleaved=False,
                             with_position_ids=False, norm_cols=40, spare_pages=2,
                             k_dtype="fp8", k_scale_mode="per_token")


def k_scale_of(case, page, off):
    """Per-head dequantisation scales [Hkv] of one slot."""
    if case.k_scale_mode == "per_token":
        return case.k_scales[case.layer_idx, page, off].astype(np.float64)
    return np.full(case.k_cache.shape[3], float(case.k_scales[0]))


def check_fp8_k_rows(case, k_new, s_new, refs, what, cols=None):
    """refs: (page, off) -> fp64 [Hkv, D] expected values.  Per-tensor: codes
    are the correctly rounded values / scale; per-token: the stored scale is
    fp32(max|y| / 448) per head and codes are values / that scale.  Columns
    outside ``cols`` (per-tensor only) and every other slot are unchanged."""
    L = case.layer_idx
    expect = case.k_cache.copy()
    expect_s = None if case.k_scales is None else case.k_scales.copy()
    for (page, off), ref in refs.items():
        lo, hi = (0, ref.shape[1]) if cols is None else cols
        if case.k_scale_mode == "per_token":
            amax = np.max(np.abs(ref), axis=1)
            want_s = (amax / 448.0).astype(np.float32)
            got_s = s_new[L, page, off]
            assert np.all(np.abs(got_s.astype(np.float64) - want_s) <= 2.0 ** -23 * want_s), what
            for h in range(ref.shape[0]):
                sc = float(got_s[h])
                assert_correctly_rounded(fp8_to_f64(k_new[L, page, off, h]), ref[h] / sc,
                                         ulp_fp8, f"{what} token head {h}", sat=448.0)
            expect[L, page, off] = k_new[L, page, off]
            expect_s[L, page, off] = got_s
        else:
            sc = float(case.k_scales[0])
            assert_correctly_rounded(fp8_to_f64(k_new[L, page, off][:, lo:hi]), ref[:, lo:hi] / sc,
                                     ulp_fp8, f"{what} tensor", sat=448.0)
            expect[L, page, off, :, lo:hi] = k_new[L, page, off, :, lo:hi]
    assert np.array_equal(k_new, expect), f"{what}: K codes outside the written span changed"
    if expect_s is not None and case.k_scale_mode == "per_token":
        assert np.array_equal(s_new.view(np.uint32), expect_s.view(np.uint32)), f"{what}: scales"


def pin_qk_fp8(orc):
    for case in small_qk_fp8_cases():
        for use_norm in (False, True):
            q_out = np.zeros_like(case.q)
            k = case.k_cache.copy()
            ks = case.k_scales.copy()
            orc.qk_rope_paged_ragged(q_out, case.q, case.row_offsets, case.cache_lengths,
                                     case.page_table, k, case.layer_idx, case.freqs,
                                     case.position_ids, case.interleaved,
                                     case.gamma if use_norm else None, case.epsilon,
                                     case.k_scale_mode, ks)
            S = case.meta["page_size"]
            owners = slot_owners(case.row_offsets, case.cache_lengths, case.page_table, S)
            slot_of = {t: slot for (page, off), (t, slot) in owners.items()}
            refs = {}
            for (page, off), (t, slot) in owners.items():
                pos = int(case.position_ids[t]) if case.position_ids is not None else slot
                fr = case.freqs[pos].astype(np.float64)
                x = fp8_to_f64(case.k_cache[case.layer_idx, page, off]) * \
                    k_scale_of(case, page, off)[:, None]
                if use_norm:
                    C = case.gamma.size
                    x[:, :C] = torch.nn.functional.rms_norm(
                        torch.from_numpy(x[:, :C].copy()), (C,),
                        weight=torch.from_numpy(bf16_to_f64(case.gamma)),
                        eps=case.epsilon).numpy()
                refs[(page, off)] = _complex_rope(x, fr[0::2][None, :], fr[1::2][None, :],
                                                  case.interleaved)
            check_fp8_k_rows(case, k, ks if case.k_scale_mode == "per_token" else None, refs,
                             f"qk fp8 {case.name} norm={use_norm}")
            _ = slot_of


def pin_rms_norm_kv_fp8(orc):
    for case in small_qk_fp8_cases():
        C = case.gamma.size
        k = case.k_cache.copy()
        ks = case.k_scales.copy()
        total = case.T - 2
        orc.rms_norm_kv_cache_paged(k, case.layer_idx, case.row_offsets, case.cache_lengths,
                                    case.page_table, case.gamma, case.epsilon, 0.25, total,
                                    True, case.k_scale_mode, ks)
        S = case.meta["page_size"]
        owners = slot_owners(case.row_offsets, case.cache_lengths, case.page_table, S)
        refs = {}
        g = bf16_to_f64(case.gamma) + 0.25
        for (page, off), (t, slot) in owners.items():
            if t >= total:
                continue
            x = fp8_to_f64(case.k_cache[case.layer_idx, page, off]) * \
                k_scale_of(case, page, off)[:, None]
            x[:, :C] = torch.nn.functional.rms_norm(torch.from_numpy(x[:, :C].copy()), (C,),
                                                    weight=torch.from_numpy(g),
                                                    eps=case.epsilon).numpy()
            refs[(page, off)] = x
        check_fp8_k_rows(case, k, ks if case.k_scale_mode == "per_token" else None, refs,
                         f"kvnorm fp8 {case.name}", cols=(0, C))


def small_mrope_cases():
    """Multimodal RoPE: sections over 64 pairs (D = 128), both rope styles."""
    yield workloads.build_qk("mrope_inter", 3201, [4, 0, 11, 2], [0, 3, 7, 20], Hq=3, Hkv=2,
                             D=128, page_size=8, max_seq_len=512, theta=10000.0,
                             interleaved=True, with_position_ids=True, norm_cols=None,
                             spare_pages=2, mrope_section=(16, 24, 24))
    yield workloads.build_qk("mrope_half", 3202, [6, 5], [1, 12], Hq=2, Hkv=1, D=128,
                             page_size=16, max_seq_len=512, theta=10000.0, interleaved=False,
                             with_position_ids=True, norm_cols=128, spare_pages=1,
                             mrope_section=(8, 40, 16))


def run_qk_oracle(orc, case, with_norm, position_ids=None, mrope_section="case"):
    q_out = np.zeros_like(case.q)
    k = case.k_cache.copy()
    orc.qk_rope_paged_ragged(
        q_out, case.q, case.row_offsets, case.cache_lengths, case.page_table, k,
        case.layer_idx, case.freqs,
        case.position_ids if position_ids is None else position_ids, case.interleaved,
        case.gamma if with_norm else None, case.epsilon,
        mrope_section=case.mrope_section if mrope_section == "case" else mrope_section)
    return q_out, k


def pin_mrope(orc):
    """Multimodal RoPE: with three equal position rows it is plain RoPE at that
    position (bit-exact); in general every pair is rotated by the angle of its
    section's row (numpy complex reference, correct rounding)."""
    for case in small_mrope_cases():
        with_norm = case.gamma is not None
        same = np.repeat(case.position_ids[:1], 3, axis=0)
        q1, k1 = run_qk_oracle(orc, case, with_norm, position_ids=same)
        q2, k2 = run_qk_oracle(orc, case, with_norm, position_ids=same[0].copy(),
                               mrope_section=None)
        assert np.array_equal(q1, q2) and np.array_equal(k1, k2), "equal rows != plain"
        q, k = run_qk_oracle(orc, case, with_norm)
        D = case.q.shape[2]
        s0, s1, _ = case.mrope_section
        sec = np.where(np.arange(D // 2) < s0, 0, np.where(np.arange(D // 2) < s0 + s1, 1, 2))
        pos = case.position_ids[sec, :].T.astype(np.int64)          # [T, D/2]
        fr = case.freqs.astype(np.float64)
        cs = fr[pos, 2 * np.arange(D // 2)[None, :]]
        sn = fr[pos, 2 * np.arange(D // 2)[None, :] + 1]
        q_ref = _complex_rope(bf16_to_f64(case.q), cs[:, None, :], sn[:, None, :], case.interleaved)
        assert_correctly_rounded(bf16_to_f64(q), q_ref, ulp_bf16, "mrope q")
        owners = slot_owners(case.row_offsets, case.cache_lengths, case.page_table,
                             case.meta["page_size"])
        for (page, off), (t, slot) in owners.items():
            x = bf16_to_f64(case.k_cache[case.layer_idx, page, off])
            if with_norm:
                C = case.gamma.size
                x[:, :C] = torch.nn.functional.rms_norm(
                    torch.from_numpy(x[:, :C].copy()), (C,),
                    weight=torch.from_numpy(bf16_to_f64(case.gamma)), eps=case.epsilon).numpy()
            ref = _complex_rope(x, cs[t][None, :], sn[t][None, :], case.interleaved)
            assert_correctly_rounded(bf16_to_f64(k[case.layer_idx, page, off]), ref, ulp_bf16,
                                     "mrope k")


def pin_rms_norm_kv_token(orc):
    """per_head_norm = False (reading: one statistic over all heads' first C
    columns): equals the per-head form for a single head, and matches torch
    rms_norm over the flattened heads with gamma repeated per head."""
    one = list(small_qk_cases())[1]                       # Hkv = 1
    g1 = workloads.bf16_bits(np.linspace(0.6, 1.4, 40).astype(np.float32))
    outs = []
    for per_head in (True, False):
        k = one.k_cache.copy()
        orc.rms_norm_kv_cache_paged(k, one.layer_idx, one.row_offsets, one.cache_lengths,
                                    one.page_table, g1, one.epsilon, 0.0, one.T, True,
                                    per_head_norm=per_head)
        outs.append(k)
    assert np.array_equal(outs[0], outs[1]), "single head: token norm != head norm"
    case = list(small_qk_cases())[0]                      # Hkv = 2, D = 128
    C = 100
    gamma = workloads.bf16_bits(np.linspace(0.5, 1.5, C).astype(np.float32))
    k = case.k_cache.copy()
    orc.rms_norm_kv_cache_paged(k, case.layer_idx, case.row_offsets, case.cache_lengths,
                                case.page_table, gamma, case.epsilon, 0.25, case.T, True,
                                per_head_norm=False)
    owners = slot_owners(case.row_offsets, case.cache_lengths, case.page_table,
                         case.meta["page_size"])
    H = case.k_cache.shape[3]
    g = np.tile(bf16_to_f64(gamma) + 0.25, H)
    L = case.layer_idx
    expect = case.k_cache.copy()
    for (page, off), (t, slot) in owners.items():
        x = bf16_to_f64(case.k_cache[L, page, off])[:, :C].reshape(-1)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x.copy()), (H * C,),
                                           weight=torch.from_numpy(g),
                                           eps=case.epsilon).numpy().reshape(H, C)
        assert_correctly_rounded(bf16_to_f64(k[L, page, off][:, :C]), ref, ulp_bf16, "token norm")
        expect[L, page, off, :, :C] = k[L, page, off, :, :C]
    assert np.array_equal(k, expect)


def gather_case(kind: str, seed: int = 3101):
    """A paged latent cache holding whole request contexts: ``kind`` is
    "fp8_tensor", "fp8_token" or "bf16".  Cache bytes are finite values (no
    NaN codes); per-token scales are finite and positive.  Returns the case
    and kv_row_offsets (prefix sums of prior + new lengths)."""
    mode = {"fp8_tensor": "per_tensor", "fp8_token": "per_token", "bf16": "none"}[kind]
    case = workloads.build_mla(f"gather_{kind}", seed, [3, 0, 9, 1, 20], [13, 5, 0, 30, 2],
                               H=1, page_size=8, max_seq_len=64, spare_pages=3,
                               scale_mode=mode, tensor_scale=0.05,
                               cache_dtype="bf16" if kind == "bf16" else "fp8")
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "bf16":
        case.cache[...] = workloads.bf16_bits(
            rng.standard_normal(case.cache.shape).astype(np.float32) * 3)
    else:
        nan = (case.cache & 0x7F) == 0x7F
        case.cache[nan] ^= 0x01
    if kind == "fp8_token":
        case.token_scales[...] = rng.uniform(1e-3, 2.0, case.token_scales.shape).astype(np.float32)
    ctx = case.cache_lengths.astype(np.int64) + np.diff(case.row_offsets.astype(np.int64))
    kvo = np.zeros(ctx.size + 1, np.uint32)
    kvo[1:] = np.cumsum(ctx)
    return case, kvo


def gather_owners(case, kvo):
    """Inverse page-table scan: (page, offset) -> output row of the context."""
    S = case.meta["page_size"]
    owners = {}
    for b in range(kvo.size - 1):
        L = int(kvo[b + 1] - kvo[b])
        for col, page in enumerate(case.page_table[b]):
            if page == workloads.UNUSED_PAGE:
                continue
            for off in range(S):
                slot = col * S + off
                if slot < L:
                    owners[(int(page), off)] = int(kvo[b]) + slot
    return owners


def pin_gather(orc):
    """Each output row is the cache row its slot maps to: bit-exact copies,
    correctly rounded dequantisation (code x scale -> bf16), brute-force
    nearest fp8 codes for quantisation; per-token scales travel with rows."""
    for kind in ("fp8_tensor", "fp8_token", "bf16"):
        case, kvo = gather_case(kind)
        rows = int(kvo[-1])
        W = case.cache.shape[-1]
        owners = gather_owners(case, kvo)
        assert len(owners) == rows
        L = case.layer_idx
        src = np.empty((rows, W), case.cache.dtype)
        row_scale = np.empty(rows)
        for (page, off), r in owners.items():
            src[r] = case.cache[L, page, off, 0]
            row_scale[r] = (case.token_scales[L, page, off, 0] if kind == "fp8_token"
                            else case.tensor_scale)
        scales = (case.token_scales if kind == "fp8_token" else
                  np.array([case.tensor_scale], np.float32))
        for out_fp8 in (True, False):
            out = np.zeros((rows, W), np.uint8 if out_fp8 else np.uint16)
            osc = np.full(rows, -1.0, np.float32)
            orc.mla_gather_latent_paged(out, kvo, case.page_table, case.cache, L,
                                        case.scale_mode, scales if kind != "bf16" else None,
                                        osc, out_tensor_scale=0.25)
            if kind == "bf16" and not out_fp8:
                assert np.array_equal(out, src), "bf16 copy"
            elif kind == "bf16":
                want = fp8_encode_bruteforce(bf16_to_f64(src).ravel() / 0.25).reshape(rows, W)
                assert np.array_equal(out, want), "bf16 -> fp8"
            elif out_fp8:
                assert np.array_equal(out, src), "fp8 copy"
                if kind == "fp8_token":
                    assert np.array_equal(osc, row_scale.astype(np.float32)), "scales copy"
            else:
                ref = fp8_to_f64(src) * row_scale[:, None]
                assert_correctly_rounded(bf16_to_f64(out), ref, ulp_bf16, f"dequant {kind}")


ALL_PINS = [
    pin_fp8_decode, pin_fp8_encode_landmarks, pin_fp8_encode_bruteforce,
    pin_fp8_encode_torch, pin_bf16_landmarks, pin_bf16_encode_torch,
    pin_bf16_encode_bruteforce, pin_rope_pos0_identity, pin_rope_complex,
    pin_rope_pair_norm, pin_rope_textbook_2d, pin_rope_inverse,
    pin_rope_relative_position, pin_rope_interleaved_permutation,
    pin_rmsnorm_closed_forms, pin_rmsnorm_torch, pin_mla_composite,
    pin_mla_position0, pin_mla_zero_row_per_token, pin_qk_composite,
    pin_rms_norm_kv, pin_gather, pin_qk_fp8, pin_rms_norm_kv_fp8, pin_mrope,
    pin_mla_f32_q, pin_rms_norm_kv_token, pin_mla_inplace, pin_token_plan, pin_mla_planned,
    pin_rms_norm_kv_planned, pin_f16_decode, pin_f16_landmarks, pin_f16_encode_numpy,
    pin_f16_encode_bruteforce, pin_mla_types, pin_qk_types, pin_rms_norm_kv_gamma_types,
    pin_qk_norm_exact_cancellation,
]
