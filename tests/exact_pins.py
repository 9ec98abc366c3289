"""Exact-arithmetic pins of the CPU oracle.

The oracle's contract for every value it writes: the value the method
defines, taken without any rounding, then rounded once into the output
format -- bf16 and fp32 round to nearest with ties to even; E4M3FN clamps the
magnitude to 448 and then rounds to nearest, ties to the even code; a
per-token scale is the fp32 nearest to max|y| / 448.  The pins here check
that contract against a reference with no binary rounding at all: tiny cases
are recomputed with Python's ``decimal`` module at 120 significant digits
(every binary input converts to a decimal exactly), the rounding is decided
by comparing exact distances to the neighbouring representable values, and
the oracle's bits must equal the result.

The arithmetic restated (pages: the MLA fused-kernel page, Summary and Args;
the Q/K RoPE page, Parameters; the K-cache RMSNorm page, Parameters):
  RoPE      pair (a, b) at angle with cosine c and sine s becomes
            (a c - b s, b c + a s); pairs are (i, i + d/2) for rotate-half and
            (2i, 2i+1) for the interleaved layout; c and s are columns 2i and
            2i+1 of the angle table row of the token's position
  RMSNorm   y_k = x_k g_k / sqrt(sum_j x_j^2 / n + eps), eps the fp32 value
  quantise  code = E4M3FN(y / scale)

Exact ties are real and frequent here: a rotation of bf16 inputs by fp32
angles has at most about 33 significant bits, so about one value in 2^8
sits exactly on an fp32 midpoint; at 120 digits those rotations, products
and their sums are computed without error, and such a tie is checked by the
ties-to-even rule.  A value that lies within 2^-40 (relative) of a rounding
boundary without being on it is not checked: the oracle computes in
binary64, and its own error (well under 2^-43 relative for these chains of
at most a few hundred operations) may decide such a case.  The skipped count
is bounded, so the pins cannot pass by skipping.
"""
from __future__ import annotations

import bisect
import struct
from decimal import Decimal, localcontext

import numpy as np

import oracle_pins as op
import workloads

PREC = 120
NEAR = Decimal(2) ** -40
MAX_SKIP_FRAC = 1e-3


# -- exact values of the formats ---------------------------------------------------------


def dec(x) -> Decimal:
    """Exact decimal of a binary float."""
    return Decimal(float(x))


def bf16_value(p: int) -> Decimal:
    return Decimal(struct.unpack("<f", struct.pack("<I", (int(p) & 0xFFFF) << 16))[0])


def f32_value(bits: int) -> Decimal:
    return Decimal(struct.unpack("<f", struct.pack("<I", int(bits) & 0xFFFFFFFF))[0])


def _fp8_magnitude(code: int) -> Decimal:
    """E4M3FN: 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
    subnormal with quantum 2^-9."""
    e, m = code >> 3, code & 7
    if e == 0:
        return Decimal(m) * Decimal(2) ** -9
    return Decimal(8 + m) * Decimal(2) ** (e - 10)


FP8_MAGS = [_fp8_magnitude(c) for c in range(0x7F)]      # 0x00 .. 0x7E = 448, increasing
assert FP8_MAGS[-1] == 448 and all(a < b for a, b in zip(FP8_MAGS, FP8_MAGS[1:]))


def fp8_value(code: int) -> Decimal:
    v = FP8_MAGS[int(code) & 0x7F]
    return v.copy_negate() if int(code) & 0x80 else v


# -- rounding by exact comparison ---------------------------------------------------------


OK, TIE, NEAR_TIE = 0, 1, 2


def _pick(m: Decimal, cands):
    """Nearest of the candidate (value, code) pairs to m >= 0, ties to the even
    code.  Returns (code, kind): TIE when m is exactly a midpoint of the two
    nearest candidates, NEAR_TIE when it is within NEAR * m of it but not on
    it, else OK."""
    ds = sorted((abs(v - m), code & 1, code) for v, code in set(cands))
    if len(ds) == 1:
        return ds[0][2], OK
    gap = ds[1][0] - ds[0][0]
    return ds[0][2], TIE if gap == 0 else (NEAR_TIE if gap <= NEAR * m else OK)


def round_bf16(v: Decimal):
    m = abs(v)
    t = int(np.float32(float(m)).view(np.uint32)) >> 16
    code, kind = _pick(m, [(bf16_value(p), p) for p in range(t - 1, t + 3) if 0 <= p <= 0x7F7F])
    return code | (0x8000 if v.is_signed() else 0), kind


def round_f32(v: Decimal):
    m = abs(v)
    c = np.float32(float(m))
    near_vals = {c, np.nextafter(c, np.float32(0)), np.nextafter(c, np.float32(np.inf))}
    cands = [(f32_value(int(x.view(np.uint32))), int(x.view(np.uint32))) for x in near_vals]
    code, kind = _pick(m, cands)
    return code | (0x80000000 if v.is_signed() else 0), kind


def f16_value(p: int) -> Decimal:
    return Decimal(float(np.array([int(p) & 0xFFFF], np.uint16).view(np.float16)[0]))


def round_f16(v: Decimal):
    """binary16 (11 significant bits) by exact comparison with the patterns
    around numpy's rounding of the value (finite range only)."""
    m = abs(v)
    t = int(np.array([float(m)]).astype(np.float16).view(np.uint16)[0])
    code, kind = _pick(m, [(f16_value(p), p) for p in range(t - 1, t + 2) if 0 <= p <= 0x7BFF])
    return code | (0x8000 if v.is_signed() else 0), kind


def round_fp8(v: Decimal):
    m = min(abs(v), Decimal(448))
    i = bisect.bisect_left(FP8_MAGS, m)
    code, kind = _pick(m, [(FP8_MAGS[c], c) for c in (i - 1, i) if 0 <= c <= 0x7E])
    return code | (0x80 if v.is_signed() else 0), kind


class Tally:
    """Counts checked values (and among them exact ties) and skipped ones;
    collects the mismatches."""

    def __init__(self, what: str):
        self.what, self.checked, self.ties, self.skipped, self.bad = what, 0, 0, 0, []

    def check(self, got: int, want_kind, where):
        want, kind = want_kind
        if kind == NEAR_TIE:
            self.skipped += 1
            return
        self.checked += 1
        self.ties += kind == TIE
        if int(got) != want and len(self.bad) < 8:
            self.bad.append((where, hex(int(got)), hex(want)))
        elif int(got) != want:
            self.bad.append(None)

    def done(self, min_ties: int = 0):
        assert not self.bad, f"{self.what}: {len(self.bad)} values differ from the exact " \
                             f"rounding; first {[b for b in self.bad if b][:4]}"
        total = self.checked + self.skipped
        assert self.checked > 0, f"{self.what}: nothing checked"
        assert self.skipped <= max(2, MAX_SKIP_FRAC * total), \
            f"{self.what}: {self.skipped} of {total} values skipped as near ties"
        assert self.ties >= min_ties, f"{self.what}: {self.ties} exact ties, want {min_ties}"
        print(f"[exact] {self.what}: {self.checked} checked ({self.ties} exact ties), "
              f"{self.skipped} skipped", flush=True)


# -- the exact computations ---------------------------------------------------------------


def rope_exact(x, cs, sn, interleaved: bool):
    """Rotated copy of the decimal list x; cs/sn are per-pair decimal lists."""
    d = len(x)
    out = list(x)
    for i in range(d // 2):
        ia, ib = (2 * i, 2 * i + 1) if interleaved else (i, i + d // 2)
        a, b = x[ia], x[ib]
        out[ia] = a * cs[i] - b * sn[i]
        out[ib] = b * cs[i] + a * sn[i]
    return out


def inv_rms_exact(x, n_div: int, eps: Decimal) -> Decimal:
    ss = sum((v * v for v in x), Decimal(0))
    return 1 / (ss / n_div + eps).sqrt()


def angles(freqs, pos):
    row = freqs[int(pos)]
    return [dec(v) for v in row[0::2]], [dec(v) for v in row[1::2]]


def mixed_angles(case, t):
    """Per-pair cos/sin of a multimodal case: pair i of section k takes the
    angle of position row k."""
    D = case.q.shape[2]
    s0, s1, _ = case.mrope_section
    cs, sn = [], []
    for i in range(D // 2):
        k = 0 if i < s0 else (1 if i < s0 + s1 else 2)
        row = case.freqs[int(case.position_ids[k, t])]
        cs.append(dec(row[2 * i]))
        sn.append(dec(row[2 * i + 1]))
    return cs, sn


def quantise_row(y, scale_mode, tensor_scale, tally_codes, tally_scale, got_codes, got_scale,
                 where, cols=None):
    """Check the fp8 codes (and the per-token scale) written for the exact
    row y.  Returns False when the row was skipped (scale near a tie)."""
    cols = range(len(y)) if cols is None else cols
    if scale_mode == "per_token":
        amax = max(abs(v) for v in y)
        st_bits, kind = round_f32(amax / 448)
        tally_scale.check(int(np.float32(got_scale).view(np.uint32)), (st_bits, kind), where)
        if kind == NEAR_TIE:
            for _ in cols:
                tally_codes.skipped += 1
            return False
        s = f32_value(st_bits)
    else:
        s = dec(np.float32(tensor_scale))
    for k in cols:
        tally_codes.check(got_codes[k], round_fp8(y[k] if s == 0 else y[k] / s), (where, k))
    return True


def pin_mla_exact(orc):
    """Fused MLA step: q rotation (bf16 and fp32 outputs), latent RMSNorm and
    tail rotation, bf16 cache rows (from the latent buffer, or in place from
    the rows placed at their slots), fp8 codes with the tensor scale or a
    fresh per-token scale, all equal to the exact value rounded once."""
    tq = Tally("mla q")
    tq32 = Tally("mla q fp32")
    tc = Tally("mla cache")
    ts_t = Tally("mla token scale")
    runs = [(case, False) for case in op.small_mla_cases()]
    runs += [(case, True) for case in list(op.small_mla_inplace_cases())[1:]]
    with localcontext() as ctx:
        ctx.prec = PREC
        for ci, (case, in_place) in enumerate(runs):
            if in_place:
                q_out, cache = op.run_mla_inplace(orc, case)
                ts = None
            else:
                q_out, cache, ts = op.run_mla(orc, case)
            q32 = None
            if ci == 2:
                q32 = np.zeros(case.q.shape, np.float32)
                orc.mla_rope_rmsnorm_quant(q32, case.q, case.latent, case.row_offsets,
                                           case.cache_lengths, case.page_table, case.freqs,
                                           case.gamma, case.epsilon, case.cache.copy(),
                                           case.layer_idx, case.scale_mode, case.tensor_scale,
                                           None if ts is None else case.token_scales.copy())
            S = case.meta["page_size"]
            owners = op.slot_owners(case.row_offsets, case.cache_lengths, case.page_table, S)
            H, R = case.q.shape[1:]
            Dn = case.Dn
            g = [dec(v) for v in op.bf16_to_f64(case.gamma)]
            eps = dec(np.float32(case.epsilon))
            L = case.layer_idx
            for (page, off), (t, slot) in owners.items():
                cs, sn = angles(case.freqs, slot)
                for h in range(H):
                    x = [dec(v) for v in op.bf16_to_f64(case.q[t, h])]
                    y = rope_exact(x, cs, sn, False)
                    for i in range(R):
                        tq.check(q_out[t, h, i], round_bf16(y[i]), (case.name, t, h, i))
                        if q32 is not None:
                            tq32.check(int(q32[t, h, i:i + 1].view(np.uint32)[0]),
                                       round_f32(y[i]), (case.name, t, h, i))
                x = [dec(v) for v in op.bf16_to_f64(case.latent[t])]
                r = inv_rms_exact(x[:Dn], Dn, eps)
                y = [x[k] * g[k] * r for k in range(Dn)] + rope_exact(x[Dn:], cs, sn, False)
                row = cache[L, page, off, 0]
                if case.cache.dtype == np.uint16:
                    for k in range(Dn + R):
                        tc.check(row[k], round_bf16(y[k]), (case.name, t, k))
                else:
                    quantise_row(y, case.scale_mode, case.tensor_scale, tc, ts_t, row,
                                 None if ts is None else ts[L, page, off, 0], (case.name, t))
    tq.done()
    tq32.done(min_ties=50)
    tc.done()
    ts_t.done()


def pin_mla_types_exact(orc):
    """The fused MLA step over the element types the pages parameterise (q
    input bf16 / fp16, freqs_cis fp32 / bf16 / fp16, gamma bf16 / fp16 /
    fp32): fp16 and fp32 q outputs and every cache row equal the exact value
    of the widened inputs rounded once."""
    tq = Tally("mla q fp16 (element types)")
    tq32 = Tally("mla q fp32 (element types)")
    tc = Tally("mla cache (element types)")
    ts_t = Tally("mla token scale (element types)")
    with localcontext() as ctx:
        ctx.prec = PREC
        for case in op.dtype_mla_cases():
            q16, cache, ts = op.run_mla(orc, case, np.float16)
            q32, _, _ = op.run_mla(orc, case, np.float32)
            S = case.meta["page_size"]
            owners = op.slot_owners(case.row_offsets, case.cache_lengths, case.page_table, S)
            H, R = case.q.shape[1:]
            Dn = case.Dn
            g = [dec(v) for v in op.elem_to_f64(case.gamma)]
            eps = dec(np.float32(case.epsilon))
            L = case.layer_idx
            for (page, off), (t, slot) in owners.items():
                row_f = op.elem_to_f64(case.freqs[slot])
                cs, sn = [dec(v) for v in row_f[0::2]], [dec(v) for v in row_f[1::2]]
                for h in range(H):
                    x = [dec(v) for v in op.elem_to_f64(case.q[t, h])]
                    y = rope_exact(x, cs, sn, False)
                    for i in range(R):
                        tq.check(int(q16[t, h, i:i + 1].view(np.uint16)[0]), round_f16(y[i]),
                                 (case.name, t, h, i))
                        tq32.check(int(q32[t, h, i:i + 1].view(np.uint32)[0]), round_f32(y[i]),
                                   (case.name, t, h, i))
                x = [dec(v) for v in op.bf16_to_f64(case.latent[t])]
                r = inv_rms_exact(x[:Dn], Dn, eps)
                y = [x[k] * g[k] * r for k in range(Dn)] + rope_exact(x[Dn:], cs, sn, False)
                row = cache[L, page, off, 0]
                if case.cache.dtype == np.uint16:
                    for k in range(Dn + R):
                        tc.check(row[k], round_bf16(y[k]), (case.name, t, k))
                else:
                    quantise_row(y, case.scale_mode, case.tensor_scale, tc, ts_t, row,
                                 None if ts is None else ts[L, page, off, 0], (case.name, t))
    tq.done()
    tq32.done()
    tc.done()
    ts_t.done()


def _k_row(case, page, off, h, ks):
    """Decimal K row of one head: bf16 values, or fp8 code times its scale."""
    src = case.k_cache[case.layer_idx, page, off, h]
    if case.k_cache.dtype == np.uint16:
        return [dec(v) for v in op.bf16_to_f64(src)]
    if case.k_scale_mode == "per_token":
        s = dec(ks[case.layer_idx, page, off, h])
    else:
        s = dec(ks[0])
    return [fp8_value(c) * s for c in src]


def pin_qk_exact(orc):
    """Paged-ragged Q/K RoPE with and without the per-head K RMSNorm, bf16 and
    fp8 K caches (tensor and per-token scales), multimodal sections: every
    output equals the exact value rounded once."""
    tq, tk, tks = Tally("qk q"), Tally("qk k"), Tally("qk k scale")
    small = list(op.small_qk_cases())
    cases = (small[:3] + small[4:] + list(op.small_qk_fp8_cases())
             + list(op.small_mrope_cases())[1:])
    with localcontext() as ctx:
        ctx.prec = PREC
        for case in cases:
            fp8 = case.k_cache.dtype == np.uint8
            norms = (False, True) if case.gamma is not None else (False,)
            for use_norm in norms:
                q_out = np.zeros_like(case.q)
                k = case.k_cache.copy()
                ks = None if case.k_scales is None else case.k_scales.copy()
                orc.qk_rope_paged_ragged(q_out, case.q, case.row_offsets, case.cache_lengths,
                                         case.page_table, k, case.layer_idx, case.freqs,
                                         case.position_ids, case.interleaved,
                                         case.gamma if use_norm else None, case.epsilon,
                                         case.k_scale_mode if fp8 else "none", ks,
                                         mrope_section=case.mrope_section)
                S = case.meta["page_size"]
                owners = op.slot_owners(case.row_offsets, case.cache_lengths, case.page_table, S)
                Hq, D = case.q.shape[1:]
                Hkv = case.k_cache.shape[3]
                eps = dec(np.float32(case.epsilon))
                g = None if not use_norm else [dec(v) for v in op.bf16_to_f64(case.gamma)]
                L = case.layer_idx
                for (page, off), (t, slot) in owners.items():
                    if case.mrope_section is not None:
                        cs, sn = mixed_angles(case, t)
                    else:
                        pos = case.position_ids[t] if case.position_ids is not None else slot
                        cs, sn = angles(case.freqs, pos)
                    for h in range(Hq):
                        x = [dec(v) for v in op.bf16_to_f64(case.q[t, h])]
                        y = rope_exact(x, cs, sn, case.interleaved)
                        for i in range(D):
                            tq.check(q_out[t, h, i], round_bf16(y[i]),
                                     (case.name, use_norm, t, h, i))
                    for h in range(Hkv):
                        x = _k_row(case, page, off, h, case.k_scales)
                        if use_norm:
                            C = len(g)
                            r = inv_rms_exact(x[:C], C, eps)
                            x = [x[i] * g[i] * r for i in range(C)] + x[C:]
                        y = rope_exact(x, cs, sn, case.interleaved)
                        where = (case.name, use_norm, t, h)
                        if not fp8:
                            for i in range(D):
                                tk.check(k[L, page, off, h, i], round_bf16(y[i]), where + (i,))
                        else:
                            quantise_row(y, case.k_scale_mode, case.k_scales[0], tk, tks,
                                         k[L, page, off, h],
                                         ks[L, page, off, h] if case.k_scale_mode == "per_token"
                                         else None, where)
    tq.done()
    tk.done()
    tks.done()


def pin_rms_norm_kv_exact(orc):
    """In-place K-cache RMSNorm: per-head and per-token statistics, weight
    offset, both cast orders (multiply before the cast rounds once; the other
    order rounds the normalised value to bf16, then the gamma product), tokens
    past total_seq_len untouched, fp8 caches re-encoded with their scale."""
    tk, tks = Tally("kvnorm k"), Tally("kvnorm k scale")
    plans = []
    for case in list(op.small_qk_cases())[:2]:
        for mbc in (True, False):
            for per_head in (True, False):
                plans.append((case, mbc, per_head, 0.25 if mbc else -0.5))
    for case in op.small_qk_fp8_cases():
        for per_head in (True, False):
            plans.append((case, True, per_head, 0.25))
    with localcontext() as ctx:
        ctx.prec = PREC
        for case, mbc, per_head, w in plans:
            fp8 = case.k_cache.dtype == np.uint8
            rng = np.random.Generator(np.random.PCG64(case.seed + 77))
            C = int(case.gamma.size) if case.gamma is not None else 48
            gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, C).astype(np.float32))
            total = case.T - 1
            k = case.k_cache.copy()
            ks = None if case.k_scales is None else case.k_scales.copy()
            orc.rms_norm_kv_cache_paged(k, case.layer_idx, case.row_offsets, case.cache_lengths,
                                        case.page_table, gamma, case.epsilon, w, total, mbc,
                                        case.k_scale_mode if fp8 else "none", ks,
                                        per_head_norm=per_head)
            S = case.meta["page_size"]
            owners = op.slot_owners(case.row_offsets, case.cache_lengths, case.page_table, S)
            Hkv, D = case.k_cache.shape[3:]
            eps = dec(np.float32(case.epsilon))
            gw = [dec(v) + dec(np.float32(w)) for v in op.bf16_to_f64(gamma)]
            L = case.layer_idx
            for (page, off), (t, slot) in owners.items():
                if t >= total:
                    assert np.array_equal(k[L, page, off], case.k_cache[L, page, off])
                    continue
                rows = [_k_row(case, page, off, h, case.k_scales) for h in range(Hkv)]
                if not per_head:
                    r_tok = inv_rms_exact([v for x in rows for v in x[:C]], Hkv * C, eps)
                for h, x in enumerate(rows):
                    r = inv_rms_exact(x[:C], C, eps) if per_head else r_tok
                    if mbc:
                        y = [x[i] * gw[i] * r for i in range(C)] + x[C:]
                    else:
                        y = []
                        for i in range(C):
                            n_bits, kind = round_bf16(x[i] * r)
                            if kind == NEAR_TIE:
                                y.append(None)
                            else:
                                y.append(bf16_value(n_bits) * gw[i])
                        y += x[C:]
                    where = (case.name, mbc, per_head, t, h)
                    if not fp8:
                        for i in range(C):
                            if y[i] is None:
                                tk.skipped += 1
                            else:
                                tk.check(k[L, page, off, h, i], round_bf16(y[i]), where + (i,))
                        assert np.array_equal(k[L, page, off, h, C:],
                                              case.k_cache[L, page, off, h, C:]), where
                    else:
                        per_tok = case.k_scale_mode == "per_token"
                        quantise_row(y, case.k_scale_mode, case.k_scales[0], tk, tks,
                                     k[L, page, off, h],
                                     ks[L, page, off, h] if per_tok else None, where,
                                     cols=range(D) if per_tok else range(C))
    tk.done(min_ties=100)
    tks.done()


def pin_gather_exact(orc):
    """Latent gather: dequantisation (code x scale -> bf16) and quantisation
    (bf16 / scale -> E4M3FN) rounded once from the exact value."""
    t = Tally("gather")
    with localcontext() as ctx:
        ctx.prec = PREC
        for kind in ("fp8_tensor", "fp8_token", "bf16"):
            case, kvo = op.gather_case(kind, seed=3111)
            rows = int(kvo[-1])
            W = case.cache.shape[-1]
            owners = op.gather_owners(case, kvo)
            L = case.layer_idx
            scales = (case.token_scales if kind == "fp8_token" else
                      np.array([case.tensor_scale], np.float32))
            out_fp8 = kind == "bf16"
            out = np.zeros((rows, W), np.uint8 if out_fp8 else np.uint16)
            orc.mla_gather_latent_paged(out, kvo, case.page_table, case.cache, L,
                                        case.scale_mode, scales if kind != "bf16" else None,
                                        np.zeros(rows, np.float32), out_tensor_scale=0.3)
            for (page, off), r in owners.items():
                src = case.cache[L, page, off, 0]
                if kind == "bf16":
                    s = dec(np.float32(0.3))
                    for j in range(W):
                        t.check(out[r, j], round_fp8(bf16_value(src[j]) / s), (kind, r, j))
                else:
                    s = dec(case.token_scales[L, page, off, 0] if kind == "fp8_token"
                            else case.tensor_scale)
                    for j in range(W):
                        t.check(out[r, j], round_bf16(fp8_value(src[j]) * s), (kind, r, j))
    t.done()


ALL_EXACT_PINS = [pin_mla_exact, pin_qk_exact, pin_rms_norm_kv_exact, pin_gather_exact,
                  pin_mla_types_exact]
