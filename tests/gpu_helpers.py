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


def bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ord_bf16(a) - ord_bf16(b))


def fp8_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ord_fp8(a) - ord_fp8(b))


# Parity bar.  q_rope_output: every value within 1 bf16 ulp of the oracle's
# correctly rounded result; in addition at most 0.1% may differ at all (the
# GPU's fp32 result lands on the other side of a bf16 rounding boundary only
# when the exact value is within a few fp32 ulps of it; a wrong rounding mode
# would move about half of all values).  FP8 cache bytes: within 1 code on at
# most 0.1% of written bytes, identical elsewhere.
BF16_MAX_ULP = 1
BF16_MAX_DIFF_FRAC = 1e-3
FP8_MAX_ULP = 1
FP8_MAX_DIFF_FRAC = 1e-3
SCALE_MAX_REL = 1e-5


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

    def __init__(self, case: workloads.MlaCase, q_layout: str = "dense"):
        import paged_kv_cache_wavefront_amd as pkv
        self.case = case
        T, H, R = case.q.shape
        if q_layout == "dense":
            self.q_in = dev_bf16(case.q)
            self.q_out = torch.empty_like(self.q_in)
        elif q_layout == "strided":
            # q and q_out live inside wider buffers: token stride 2*H*R + 8,
            # head stride 2*R (the rope slice of a [T, H, nope+rope] tensor).
            big = torch.zeros((T, 2 * H * R + 8), dtype=torch.bfloat16, device=DEV)
            view = big[:, : 2 * H * R].view(T, H, 2 * R)[:, :, R:]
            view.copy_(dev_bf16(case.q))
            self.q_in = view
            big_o = torch.zeros((T, 2 * H * R + 16), dtype=torch.bfloat16, device=DEV)
            self.q_out = big_o[:, : 2 * H * R].view(T, H, 2 * R)[:, :, :R]
            self._keep = (big, big_o)
        elif q_layout == "inplace":
            self.q_in = dev_bf16(case.q)
            self.q_out = self.q_in
        else:
            raise ValueError(q_layout)
        self.latent = dev_bf16(case.latent)
        self.offsets = dev_u32(case.row_offsets)
        self.cache_lengths = dev_u32(case.cache_lengths)
        self.page_table = dev_u32(case.page_table)
        self.freqs = dev_f32(case.freqs)
        self.gamma = dev_bf16(case.gamma)
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

    def results(self):
        torch.cuda.synchronize()
        q = host_bf16(self.q_out)
        cache = host_bf16(self.cache) if self.case.cache.dtype == np.uint16 else host_u8(self.cache)
        ts = host_f32(self.scales) if self.case.scale_mode == "per_token" else None
        return q, cache, ts, int(self.error_count.item())


def oracle_mla(orc, case):
    q_out = np.zeros_like(case.q)
    cache = case.cache.copy()
    ts = None if case.token_scales is None else case.token_scales.copy()
    orc.mla_rope_rmsnorm_quant(q_out, case.q, case.latent, case.row_offsets,
                               case.cache_lengths, case.page_table, case.freqs, case.gamma,
                               case.epsilon, cache, case.layer_idx, case.scale_mode,
                               case.tensor_scale, ts)
    return q_out, cache, ts


def written_rows(case) -> np.ndarray:
    """Boolean [L, P, S] mask of the rows the new tokens own (inverse scan)."""
    import oracle_pins
    mask = np.zeros(case.cache.shape[:3], bool)
    for (page, off) in oracle_pins.slot_owners(case.row_offsets, case.cache_lengths,
                                               case.page_table, case.meta["page_size"]):
        mask[case.layer_idx, page, off] = True
    return mask


def compare_mla(case, gpu, orc_res) -> dict:
    q_g, cache_g, ts_g, _ = gpu
    q_o, cache_o, ts_o = orc_res
    stats = {"q": check_bf16(q_g, q_o, "q_rope_output")}
    rows = written_rows(case)
    # untouched rows: bit-exact against the starting pool (and the oracle's)
    assert np.array_equal(cache_g[~rows], case.cache[~rows]), "cache bytes outside new rows changed"
    assert np.array_equal(cache_o[~rows], case.cache[~rows]), "oracle changed bytes outside new rows"
    wg, wo = cache_g[rows], cache_o[rows]
    if case.cache.dtype == np.uint16:
        stats["cache"] = check_bf16(wg, wo, "bf16 cache rows")
    else:
        d = fp8_ulp_diff(wg, wo)
        frac = float((d != 0).sum() / max(d.size, 1))
        stats["cache"] = dict(max_ulp=int(d.max(initial=0)), diff_frac=frac, n=d.size)
        assert stats["cache"]["max_ulp"] <= FP8_MAX_ULP, stats
        assert frac <= FP8_MAX_DIFF_FRAC, stats
    if ts_o is not None:
        keep = ~rows
        assert np.array_equal(ts_g[keep].view(np.uint32), case.token_scales[keep].view(np.uint32)), \
            "scales outside new rows changed"
        sg, so = ts_g[rows].astype(np.float64), ts_o[rows].astype(np.float64)
        rel = np.abs(sg - so) / np.maximum(np.abs(so), 1e-30)
        rel[(sg == 0) & (so == 0)] = 0
        stats["scale_max_rel"] = float(rel.max(initial=0))
        assert stats["scale_max_rel"] <= SCALE_MAX_REL, stats
    return stats


# -- QK RoPE / K norm ----------------------------------------------------------------------

class QkDevice:
    def __init__(self, case: workloads.QkCase):
        import paged_kv_cache_wavefront_amd as pkv
        self.case = case
        self.q_in = dev_bf16(case.q)
        self.q_out = torch.empty_like(self.q_in)
        self.offsets = dev_u32(case.row_offsets)
        self.cache_lengths = dev_u32(case.cache_lengths)
        self.page_table = dev_u32(case.page_table)
        self.freqs = dev_f32(case.freqs)
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

    def kv_norm(self, gamma: torch.Tensor, weight_offset=0.0, total=None, mbc=True):
        import paged_kv_cache_wavefront_amd as pkv
        pkv.rms_norm_kv_cache_paged(self.desc, self.case.layer_idx, gamma, self.case.epsilon,
                                    weight_offset, self.case.T if total is None else total,
                                    self.offsets, True, mbc)


def written_k_rows(case) -> np.ndarray:
    import oracle_pins
    mask = np.zeros(case.k_cache.shape[:3], bool)
    for (page, off) in oracle_pins.slot_owners(case.row_offsets, case.cache_lengths,
                                               case.page_table, case.meta["page_size"]):
        mask[case.layer_idx, page, off] = True
    return mask
