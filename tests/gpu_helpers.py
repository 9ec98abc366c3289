"""Helpers for the GPU parity tests: move a seeded case to the device, call the
HIP library through its binding, bring results back, and compare them with the
oracle's by ordered-integer ulp distance."""
from __future__ import annotations

import numpy as np
import torch

import workloads

DEV = "cuda"


# -- host <-> device ---------------------------------------------------------------

def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_u32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(DEV)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


# numpy representation of each element type (bf16 as its uint16 bits) -> torch dtype
TORCH_OF = {np.dtype(np.uint16): torch.bfloat16, np.dtype(np.float16): torch.float16,
            np.dtype(np.float32): torch.float32}


def dev_elem(a: np.ndarray) -> torch.Tensor:
    """A bf16 (uint16 bits), fp16 or fp32 array on the device, in its type."""
    if a.dtype == np.uint16:
        return dev_bf16(a)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_elem(t: torch.Tensor) -> np.ndarray:
    """Inverse of dev_elem."""
    if t.dtype == torch.bfloat16:
        return host_bf16(t)
    return t.contiguous().cpu().numpy()


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


# -- ulp distances ---------------------------------------------------------------------

def ord_bf16(u: np.ndarray) -> np.ndarray:
    u = u.astype(np.int64)
    mag = u & 0x7FFF
    return np.where(u & 0x8000, -mag, mag)


def ord_fp8(u: np.ndarray) -> np.ndarray:
    u = u.astype(np.int64)
    mag = u & 0x7F
    return np.where(u & 0x80, -mag, mag)


def ord_f32(a: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.int64)
    mag = u & 0x7FFFFFFF
    return np.where(u & 0x80000000, -mag, mag)


def ord_f16(a: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a, np.float16).view(np.uint16).astype(np.int64)
    mag = u & 0x7FFF
    return np.where(u & 0x8000, -mag, mag)


def f16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ord_f16(a) - ord_f16(b))


def f32_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ord_f32(a) - ord_f32(b))


def bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ord_bf16(a) - ord_bf16(b))


def fp8_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Ordered-integer distance of E4M3FN codes; two NaN codes (S.1111.111,
    either sign) are equal, a NaN against a number is 1000 steps apart."""
    d = np.abs(ord_fp8(a) - ord_fp8(b))
    na, nb = (a & 0x7F) == 0x7F, (b & 0x7F) == 0x7F
    return np.where(na & nb, 0, np.where(na | nb, 1000, d))


# Parity bar.  q_rope_output: every value within 1 bf16 ulp of the oracle's
# correctly rounded result; in addition at most 0.1% may differ at all (the
# GPU's fp32 result lands on the other side of a bf16 rounding boundary only
# when the exact value is within a few fp32 ulps of it; a wrong rounding mode
# would move about half of all values).  FP8 cache bytes: within 1 code on at
# most 0.1% of written bytes, identical elsewhere.
BF16_MAX_ULP = 1
BF16_MAX_DIFF_FRAC = 1e-3
SCALE_MAX_REL = 1e-5
# The fused MLA step's quantised cache bytes: within 1 fp8 step on at most
# 0.1 % of written bytes (the stated target), and each differing code a near-tie
# as below.
FP8_MAX_DIFF_FRAC = 1e-3
# FP8 codes: identical to the oracle's, except where the oracle's exact value
# (before rounding) lies within FP8_TIE_REL of a rounding midpoint; there the
# kernel's fp32 error decides and either neighbour is right.  The kernel's
# value before rounding carries at most ~30 fp32 roundings' worth of relative
# error (lane sums of 8 squares and a 6-level DPP tree, mean, sqrt, reciprocal,
# gamma product, Kahan rotation, the scale's reciprocal and product; with a
# per-token scale the max carries the same error again): below 2^-19.
# Values with a per-token scale sit near midpoints far more often than chance,
# since r cancels from y / (max|y| / 448) and leaves a ratio of short binary
# numbers.
FP8_TIE_REL = 2.0 ** -18
# fp32 q_rope_output: the kernel forms each rotated value as a difference of
# two products with Kahan's FMA algorithm (within 1.5 ulp of the exact value);
# the oracle rounds the exact value once (within 0.5 ulp): at most 2 fp32 ulps.
F32_MAX_ULP = 2
# fp16 q output: within 1 fp16 ulp; a value differs from the correctly rounded
# one only where the exact value lies within the kernel's ~1.5 fp32 ulps of an
# fp16 rounding midpoint, about 3 x 2^-13 = 3.7e-4 of values: bar 10x that.
F16_MAX_ULP = 1
F16_MAX_DIFF_FRAC = 4e-3


def check_fp8(got: np.ndarray, want: np.ndarray, pre, what: str, abs_slack=None,
              max_frac=None) -> dict:
    """FP8 codes against the oracle's; ``pre`` holds the oracle's binary64
    values before rounding (NaN for bytes it copied), or None.  A code may
    differ by one step only where pre lies within FP8_TIE_REL x midpoint
    (+ abs_slack, same shape as pre, where the path amplifies an fp32 error
    by cancellation) of a rounding midpoint."""
    import oracle_pins
    d = fp8_ulp_diff(got, want)
    bad = d != 0
    stats = dict(max_ulp=int(d.max(initial=0)), diff_frac=float(bad.sum() / max(d.size, 1)),
                 n=d.size)
    assert stats["max_ulp"] <= 1, f"{what}: {stats}"
    if max_frac is not None:
        assert stats["diff_frac"] <= max_frac, f"{what}: {stats}"
    if bad.any():
        assert pre is not None, f"{what}: codes differ and no oracle values: {stats}"
        dist, mid = oracle_pins.fp8_midpoint_dist(pre[bad])
        window = FP8_TIE_REL * mid + (0.0 if abs_slack is None else abs_slack[bad])
        ratio = np.where(np.isnan(dist), np.inf, dist / window)
        stats["worst_window_frac"] = float(ratio.max())
        assert stats["worst_window_frac"] <= 1.0, f"{what}: a code off a near-tie differs: {stats}"
    return stats


def check_q(got: np.ndarray, want: np.ndarray, what: str, floor: int = 0) -> dict:
    """A q output of any element type against the oracle's under its type's
    bar (floor: differing values always allowed, for cases of a few hundred
    values)."""
    n = max(want.size, 1)
    if want.dtype == np.uint16:
        return check_bf16(got, want, what, max_frac=max(BF16_MAX_DIFF_FRAC, floor / n))
    if want.dtype == np.float16:
        d, max_ulp, frac = f16_ulp_diff(got, want), F16_MAX_ULP, max(F16_MAX_DIFF_FRAC, floor / n)
    else:
        d, max_ulp, frac = f32_ulp_diff(got, want), F32_MAX_ULP, 1.0
    stats = dict(max_ulp=int(d.max(initial=0)), diff_frac=float((d != 0).sum() / n), n=d.size)
    assert stats["max_ulp"] <= max_ulp, f"{what}: {stats}"
    assert stats["diff_frac"] <= frac, f"{what}: {stats}"
    return stats


def check_bf16(got: np.ndarray, want: np.ndarray, what: str, max_ulp=BF16_MAX_ULP,
               max_frac=BF16_MAX_DIFF_FRAC) -> dict:
    d = bf16_ulp_diff(got, want)
    n = max(d.size, 1)
    stats = dict(max_ulp=int(d.max(initial=0)), diff_frac=float((d != 0).sum() / n), n=d.size)
    assert stats["max_ulp"] <= max_ulp, f"{what}: {stats}"
    assert stats["diff_frac"] <= max_frac, f"{what}: {stats}"
    return stats


# -- MLA ---------------------------------------------------------------------------------

class MlaDevice:
    """Device copies of an MlaCase plus the cache descriptor."""

    def __init__(self, case: workloads.MlaCase, q_layout: str = "dense", q_f32: bool = False,
                 q_out_dtype=None):
        """q_out_dtype: numpy type of the q output (np.uint16 = bf16,
        np.float16, np.float32); default q's own type (q_f32: np.float32)."""
        import paged_kv_cache_wavefront_amd as pkv
        self.case = case
        T, H, R = case.q.shape
        out_np = np.dtype(np.float32 if q_f32 else (case.q.dtype if q_out_dtype is None
                                                     else q_out_dtype))
        out_t = TORCH_OF[out_np]
        if q_layout == "dense":
            self.q_in = dev_elem(case.q)
            self.q_out = torch.full((T, H, R), float("nan"), dtype=out_t, device=DEV)
        elif q_layout == "strided":
            # q and q_out live inside wider buffers: token stride 2*H*R + 8
            # (+ 16 for the output), head stride 2*R (the rope slice of a
            # [T, H, nope+rope] tensor).
            big = torch.zeros((T, 2 * H * R + 8), dtype=TORCH_OF[case.q.dtype], device=DEV)
            view = big[:, : 2 * H * R].view(T, H, 2 * R)[:, :, R:]
            view.copy_(dev_elem(case.q))
            self.q_in = view
            big_o = torch.zeros((T, 2 * H * R + 16), dtype=out_t, device=DEV)
            self.q_out = big_o[:, : 2 * H * R].view(T, H, 2 * R)[:, :, :R]
            self._keep = (big, big_o)
        elif q_layout == "inplace":
            if out_np != case.q.dtype:
                raise ValueError("in-place q needs one element type")
            self.q_in = dev_elem(case.q)
            self.q_out = self.q_in
        else:
            raise ValueError(q_layout)
        self.latent = dev_bf16(case.latent)
        self.offsets = dev_u32(case.row_offsets)
        self.cache_lengths = dev_u32(case.cache_lengths)
        self.page_table = dev_u32(case.page_table)
        self.freqs = dev_elem(case.freqs)
        self.gamma = dev_elem(case.gamma)
        if case.cache.dtype == np.uint16:
            self.cache = dev_bf16(case.cache)
            mode, self.scales = pkv.PKV_SCALE_NONE, None
        elif case.scale_mode == "per_tensor":
            self.cache = dev_u8(case.cache)
            mode = pkv.PKV_SCALE_PER_TENSOR
            self.scales = dev_f32(np.array([case.tensor_scale], np.float32))
        else:
            self.cache = dev_u8(case.cache)
            mode = pkv.PKV_SCALE_PER_TOKEN
            self.scales = dev_f32(case.token_scales)
        self.error_count = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.desc = pkv.paged_cache(self.cache, self.cache_lengths, self.page_table, mode,
                                    self.scales, self.error_count)

    def run(self, stream=None):
        import paged_kv_cache_wavefront_amd as pkv
        pkv.mla_rope_rmsnorm_quant(self.q_out, self.q_in, self.latent, self.offsets,
                                   self.freqs, self.gamma, self.case.epsilon, self.desc,
                                   self.case.layer_idx, stream=stream)

    def place_rows(self):
        """Write each new token's latent row into its slot of the (bf16)
        device cache, as the in-place form expects."""
        import oracle_pins
        self.cache.copy_(dev_bf16(oracle_pins.place_latent_rows(self.case)))

    def run_inplace(self, stream=None):
        import paged_kv_cache_wavefront_amd as pkv
        pkv.mla_rope_rmsnorm_inplace(self.q_out, self.q_in, self.offsets, self.freqs,
                                     self.gamma, self.case.epsilon, self.desc,
                                     self.case.layer_idx, stream=stream)

    def results(self):
        torch.cuda.synchronize()
        q = host_elem(self.q_out)
        cache = host_bf16(self.cache) if self.case.cache.dtype == np.uint16 else host_u8(self.cache)
        ts = host_f32(self.scales) if self.case.scale_mode == "per_token" else None
        return q, cache, ts, int(self.error_count.item())


def oracle_mla(orc, case, q_f32=False, q_out_dtype=None):
    """Oracle results (q_out, cache, token_scales, pre): ``pre`` holds the
    binary64 value each fp8 cache code was rounded from (None: bf16 cache).
    The q output has q_out_dtype (default q's type; q_f32: np.float32)."""
    import contextlib
    out_np = np.float32 if q_f32 else (case.q.dtype if q_out_dtype is None else q_out_dtype)
    q_out = np.zeros(case.q.shape, out_np)
    cache = case.cache.copy()
    ts = None if case.token_scales is None else case.token_scales.copy()
    probe = orc.fp8_probe(cache) if cache.dtype == np.uint8 else contextlib.nullcontext()
    with probe as pre:
        orc.mla_rope_rmsnorm_quant(q_out, case.q, case.latent, case.row_offsets,
                                   case.cache_lengths, case.page_table, case.freqs, case.gamma,
                                   case.epsilon, cache, case.layer_idx, case.scale_mode,
                                   case.tensor_scale, ts)
    return q_out, cache, ts, pre


def oracle_mla_inplace(orc, case, q_f32=False):
    """Oracle results of the in-place form, shaped like :func:`oracle_mla`."""
    import oracle_pins
    q_out, cache = oracle_pins.run_mla_inplace(orc, case, q_f32)
    return q_out, cache, None, None


def written_rows(case) -> np.ndarray:
    """Boolean [L, P, S] mask of the rows the new tokens own (inverse scan)."""
    import oracle_pins
    mask = np.zeros(case.cache.shape[:3], bool)
    for (page, off) in oracle_pins.slot_owners(case.row_offsets, case.cache_lengths,
                                               case.page_table, case.meta["page_size"]):
        mask[case.layer_idx, page, off] = True
    return mask


def compare_mla(case, gpu, orc_res, small_case_floor: int = 0, rows=None) -> dict:
    """GPU results against the oracle's under the parity bars.  With
    small_case_floor = k, the fraction bars allow at least k differing values
    (for cases of a few hundred values, where one near-tie is already more
    than 0.1 %); the per-value bars (1 step, fp8 near-ties only) still hold.
    rows: mask [L, P, S] of the cache rows the step writes (default: the new
    tokens' slots under the case's page table)."""
    q_g, cache_g, ts_g, _ = gpu
    q_o, cache_o, ts_o, pre = orc_res

    def cap(frac, n):
        return max(frac, small_case_floor / max(n, 1))
    assert q_g.dtype == q_o.dtype, (q_g.dtype, q_o.dtype)
    stats = {"q": check_q(q_g, q_o, f"q_rope_output ({q_o.dtype})", small_case_floor)}
    rows = written_rows(case) if rows is None else rows
    # untouched rows: bit-exact against the starting pool (and the oracle's)
    assert np.array_equal(cache_g[~rows], case.cache[~rows]), "cache bytes outside new rows changed"
    assert np.array_equal(cache_o[~rows], case.cache[~rows]), "oracle changed bytes outside new rows"
    wg, wo = cache_g[rows], cache_o[rows]
    if case.cache.dtype == np.uint16:
        stats["cache"] = check_bf16(wg, wo, "bf16 cache rows",
                                    max_frac=cap(BF16_MAX_DIFF_FRAC, wg.size))
    else:
        stats["cache"] = check_fp8(wg, wo, pre[rows], "fp8 cache rows",
                                   max_frac=cap(FP8_MAX_DIFF_FRAC, wg.size))
    if ts_o is not None:
        keep = ~rows
        assert np.array_equal(ts_g[keep].view(np.uint32), case.token_scales[keep].view(np.uint32)), \
            "scales outside new rows changed"
        sg, so = ts_g[rows].astype(np.float64), ts_o[rows].astype(np.float64)
        with np.errstate(invalid="ignore"):
            rel = np.abs(sg - so) / np.maximum(np.abs(so), 1e-30)
        rel[sg == so] = 0          # equal values, infinities included
        stats["scale_max_rel"] = float(rel.max(initial=0))
        assert stats["scale_max_rel"] <= SCALE_MAX_REL, stats
    return stats


# -- QK RoPE / K norm ----------------------------------------------------------------------

class QkDevice:
    def __init__(self, case: workloads.QkCase):
        import paged_kv_cache_wavefront_amd as pkv
        self.case = case
        self.q_in = dev_elem(case.q)
        self.q_out = torch.empty_like(self.q_in)
        self.offsets = dev_u32(case.row_offsets)
        self.cache_lengths = dev_u32(case.cache_lengths)
        self.page_table = dev_u32(case.page_table)
        self.freqs = dev_elem(case.freqs)
        self.pos = None if case.position_ids is None else dev_u32(case.position_ids)
        self.gamma = None if case.gamma is None else dev_bf16(case.gamma)
        self.error_count = torch.zeros(1, dtype=torch.int32, device=DEV)
        if case.k_cache.dtype == np.uint16:
            self.k = dev_bf16(case.k_cache)
            mode, self.k_scales = pkv.PKV_SCALE_NONE, None
        else:
            self.k = dev_u8(case.k_cache)
            self.k_scales = dev_f32(case.k_scales)
            mode = (pkv.PKV_SCALE_PER_TOKEN if case.k_scale_mode == "per_token"
                    else pkv.PKV_SCALE_PER_TENSOR)
        self.desc = pkv.paged_cache(self.k, self.cache_lengths, self.page_table,
                                    mode, self.k_scales, self.error_count)

    def k_host(self):
        torch.cuda.synchronize()
        k = host_bf16(self.k) if self.case.k_cache.dtype == np.uint16 else host_u8(self.k)
        ks = None if self.k_scales is None else host_f32(self.k_scales)
        return k, ks

    def rope(self, with_norm: bool):
        import paged_kv_cache_wavefront_amd as pkv
        pkv.qk_rope_paged_ragged(self.q_out, self.q_in, self.offsets, self.desc,
                                 self.case.layer_idx, self.freqs, self.pos,
                                 self.case.interleaved,
                                 self.gamma if with_norm else None, self.case.epsilon,
                                 mrope_section=self.case.mrope_section)

    def kv_norm(self, gamma: torch.Tensor, weight_offset=0.0, total=None, mbc=True,
                per_head=True):
        import paged_kv_cache_wavefront_amd as pkv
        pkv.rms_norm_kv_cache_paged(self.desc, self.case.layer_idx, gamma, self.case.epsilon,
                                    weight_offset, self.case.T if total is None else total,
                                    self.offsets, per_head, mbc)


def written_k_rows(case) -> np.ndarray:
    import oracle_pins
    mask = np.zeros(case.k_cache.shape[:3], bool)
    for (page, off) in oracle_pins.slot_owners(case.row_offsets, case.cache_lengths,
                                               case.page_table, case.meta["page_size"]):
        mask[case.layer_idx, page, off] = True
    return mask
