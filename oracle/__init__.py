"""CPU oracle for the paged-KV pre-attention path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports it, and it imports nothing from the product path.

The arithmetic lives in ``pkv_oracle.c`` (plain C, IEEE binary64, one rounding
per output); this module only loads ``liboracle.so`` with ctypes and passes
numpy arrays to it.  Every function works on host arrays and mirrors one entry
point of the method:

* :func:`mla_rope_rmsnorm_quant` -- page "mla_fused_rope_rmsnorm_quantization"
  (summary, Args) and the fused_rope_rmsnorm_quantization_kernel entry of the
  "mla_graph" module page;
* :func:`qk_rope_paged_ragged` -- page "generic_fused_qk_rope_bshd_paged_ragged";
* :func:`rms_norm_kv_cache_paged` -- page "rms_norm_kv_cache_ragged_paged";
* :func:`token_plan`, :func:`mla_rope_rmsnorm_quant_planned` and
  :func:`rms_norm_kv_cache_planned` -- the ragged / paged addressing written
  out once per batch layout, and the MLA step and the K-cache norm placed by
  it;
* :func:`mla_gather_latent_paged` -- the paged-to-contiguous latent copy and
  fp8 (de)quantisation step of mla_prefill_branch_fp8 ("mla_graph" page);
* the bf16, binary16 and FP8 E4M3FN codecs and the RoPE / RMSNorm row steps,
  exposed so that tests can pin each step on its own.

Element types: q (and q_out), freqs_cis and gamma arrays may be bf16 (bits in
a uint16 array), fp16 (numpy float16) or fp32, the dtype / out_rope_dtype /
freq_dtype / gamma_dtype parameters of the pages; the latent row is bf16 (the
MLA page's kv_input_fn yields bfloat16).

Parity status of each function: pinned by ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force and library special cases (no page
prints a worked example).  ``rms_norm_kv_cache_paged`` with
``multiply_before_cast=0`` is pinned only through the bf16 codec and the
RMSNorm row step it is built from.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_c_u16p = ctypes.POINTER(ctypes.c_uint16)
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64

SCALE_PER_TENSOR = 1
SCALE_PER_TOKEN = 2
CACHE_FP8 = 0
CACHE_BF16 = 1
# element types of q, freqs and gamma arrays, from their numpy dtype: uint16
# holds bf16 bits, float16 holds fp16 values (the same bits), float32 fp32
ELEM_BF16 = 0
ELEM_F32 = 2
ELEM_F16 = 3


def _elem_type(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return ELEM_BF16
    if a.dtype == np.float16:
        return ELEM_F16
    if a.dtype == np.float32:
        return ELEM_F32
    raise TypeError(f"element type {a.dtype} is not bf16 (uint16), fp16 or fp32")


def build() -> str:
    """Compile liboracle.so with the oracle's own Makefile (gcc, binary64)."""
    subprocess.run(["make", "-s", "-C", _HERE], check=True)
    return LIB_PATH


def load(path: str | None = None) -> ctypes.CDLL:
    """Load an oracle library (the default one, or a test-built variant)."""
    path = path or LIB_PATH
    if not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    lib.oracle_bf16_decode.restype = ctypes.c_double
    lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_encode.restype = ctypes.c_uint16
    lib.oracle_bf16_encode.argtypes = [ctypes.c_double]
    lib.oracle_f16_decode.restype = ctypes.c_double
    lib.oracle_f16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_encode.restype = ctypes.c_uint16
    lib.oracle_f16_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3fn_decode.restype = ctypes.c_double
    lib.oracle_e4m3fn_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3fn_encode_sat.restype = ctypes.c_uint8
    lib.oracle_e4m3fn_encode_sat.argtypes = [ctypes.c_double]
    lib.oracle_rope_row.restype = None
    lib.oracle_rope_row.argtypes = [_vp, _vp, _i64, _vp, ctypes.c_int]
    lib.oracle_inv_rms.restype = ctypes.c_double
    lib.oracle_inv_rms.argtypes = [_vp, _i64, ctypes.c_double]
    lib.oracle_rmsnorm_row.restype = None
    lib.oracle_rmsnorm_row.argtypes = [_vp, _vp, _i64, _vp, ctypes.c_double]
    lib.oracle_mla_rope_rmsnorm_quant.restype = ctypes.c_int
    lib.oracle_mla_rope_rmsnorm_quant.argtypes = [
        _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
        ctypes.c_int, _i64, _vp, ctypes.c_int, ctypes.c_float, _i64, _i64, _i64, _vp,
        ctypes.c_int, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_float, _vp]
    lib.oracle_token_plan.restype = ctypes.c_int
    lib.oracle_token_plan.argtypes = [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _i64]
    lib.oracle_mla_rope_rmsnorm_quant_planned.restype = ctypes.c_int
    lib.oracle_mla_rope_rmsnorm_quant_planned.argtypes = [
        _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _i64, _vp, ctypes.c_int, _i64, _vp,
        ctypes.c_int, ctypes.c_float, _i64, _i64, _i64, _vp, ctypes.c_int, _i64, _i64, _i64,
        _i64, ctypes.c_int, ctypes.c_float, _vp]
    lib.oracle_rms_norm_kv_cache_planned.restype = ctypes.c_int
    lib.oracle_rms_norm_kv_cache_planned.argtypes = [
        _vp, ctypes.c_int, ctypes.c_int, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp,
        ctypes.c_int, _i64, ctypes.c_float, ctypes.c_float, _i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_mla_rope_rmsnorm_inplace.restype = ctypes.c_int
    lib.oracle_mla_rope_rmsnorm_inplace.argtypes = [
        _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _i64, _vp, _i64, _vp, ctypes.c_int,
        _i64, _vp, ctypes.c_int, ctypes.c_float, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64]
    lib.oracle_qk_rope_paged_ragged.restype = ctypes.c_int
    lib.oracle_qk_rope_paged_ragged.argtypes = [
        _vp, _vp, ctypes.c_int, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp, ctypes.c_int,
        ctypes.c_int, _vp, _i64, _i64, _i64, _i64, _i64, _vp, ctypes.c_int, _i64, _vp, _vp,
        ctypes.c_int, _vp, _i64, ctypes.c_float]
    lib.oracle_mla_gather_latent_paged.restype = ctypes.c_int
    lib.oracle_mla_gather_latent_paged.argtypes = [
        _vp, ctypes.c_int, _vp, ctypes.c_float, _vp, _i64, _vp, _i64, _vp, ctypes.c_int,
        ctypes.c_int, _vp, _i64, _i64, _i64, _i64, _i64]
    lib.oracle_rms_norm_kv_cache_paged.restype = ctypes.c_int
    lib.oracle_rms_norm_kv_cache_paged.argtypes = [
        _vp, ctypes.c_int, ctypes.c_int, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp,
        _i64, _vp, _i64, _vp, ctypes.c_int, _i64, ctypes.c_float, ctypes.c_float, _i64,
        ctypes.c_int, ctypes.c_int]
    _declare_probe(lib)
    return lib


def _declare_probe(lib):
    lib.oracle_set_fp8_probe.argtypes = [_vp, _i64, _vp]
    lib.oracle_set_fp8_probe.restype = None


def _ptr(a: np.ndarray | None, dtype) -> int | None:
    if a is None:
        return None
    if a.dtype != np.dtype(dtype) or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"oracle wants a C-contiguous {np.dtype(dtype)} array, got "
                        f"{a.dtype} contiguous={a.flags['C_CONTIGUOUS']}")
    return a.ctypes.data


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what}: oracle precondition failed (code {rc})")


class Oracle:
    """One loaded oracle library; methods take and fill numpy arrays."""

    def __init__(self, path: str | None = None):
        self.path = path or LIB_PATH
        self.lib = load(self.path)

    # -- observation ----------------------------------------------------------
    @contextlib.contextmanager
    def fp8_probe(self, codes: np.ndarray):
        """While active, every fp8 code an entry point writes into ``codes``
        (a uint8 array passed to that call) records the binary64 value it was
        rounded from; yields that float64 array (same shape, NaN where no code
        was encoded: bytes left alone or copied as they were)."""
        if codes.dtype != np.uint8 or not codes.flags.c_contiguous:
            raise ValueError("probe needs a contiguous uint8 array")
        pre = np.full(codes.shape, np.nan)
        self.lib.oracle_set_fp8_probe(codes.ctypes.data, codes.size, pre.ctypes.data)
        try:
            yield pre
        finally:
            self.lib.oracle_set_fp8_probe(None, 0, None)

    # -- codecs and row steps --------------------------------------------------
    def bf16_decode(self, bits: int) -> float:
        return self.lib.oracle_bf16_decode(int(bits))

    def bf16_encode(self, v: float) -> int:
        return self.lib.oracle_bf16_encode(float(v))

    def f16_decode(self, bits: int) -> float:
        return self.lib.oracle_f16_decode(int(bits))

    def f16_encode(self, v: float) -> int:
        return self.lib.oracle_f16_encode(float(v))

    def f16_encode_array(self, v) -> np.ndarray:
        f = self.lib.oracle_f16_encode
        v = np.asarray(v, np.float64)
        return np.fromiter((f(float(x)) for x in v.ravel()), np.uint16,
                           count=v.size).reshape(v.shape)

    def e4m3fn_decode(self, code: int) -> float:
        return self.lib.oracle_e4m3fn_decode(int(code))

    def e4m3fn_encode(self, v: float) -> int:
        return self.lib.oracle_e4m3fn_encode_sat(float(v))

    def bf16_encode_array(self, v) -> np.ndarray:
        f = self.lib.oracle_bf16_encode
        v = np.asarray(v, np.float64)
        return np.fromiter((f(float(x)) for x in v.ravel()), np.uint16,
                           count=v.size).reshape(v.shape)

    def e4m3fn_encode_array(self, v) -> np.ndarray:
        f = self.lib.oracle_e4m3fn_encode_sat
        v = np.asarray(v, np.float64)
        return np.fromiter((f(float(x)) for x in v.ravel()), np.uint8,
                           count=v.size).reshape(v.shape)

    def rope_row(self, x, freqs_row, interleaved: bool) -> np.ndarray:
        x = np.ascontiguousarray(x, np.float64)
        fr = np.ascontiguousarray(freqs_row, np.float32)
        if fr.size < x.size:
            raise ValueError("freqs row narrower than the rotated row")
        out = np.empty_like(x)
        self.lib.oracle_rope_row(x.ctypes.data, out.ctypes.data, x.size,
                                 fr.ctypes.data, int(bool(interleaved)))
        return out

    def inv_rms(self, x, eps: float) -> float:
        x = np.ascontiguousarray(x, np.float64)
        return self.lib.oracle_inv_rms(x.ctypes.data, x.size, float(eps))

    def rmsnorm_row(self, x, g, eps: float) -> np.ndarray:
        x = np.ascontiguousarray(x, np.float64)
        g = np.ascontiguousarray(g, np.float64)
        y = np.empty_like(x)
        self.lib.oracle_rmsnorm_row(x.ctypes.data, y.ctypes.data, x.size,
                                    g.ctypes.data, float(eps))
        return y

    # -- entry points ----------------------------------------------------------
    def mla_rope_rmsnorm_quant(self, q_out, q_in, latent, row_offsets,
                               cache_lengths, page_table, freqs, gamma, epsilon,
                               cache, layer_idx, scale_mode, tensor_scale=1.0,
                               token_scales=None):
        """Fill ``q_out`` and the new rows of ``cache`` (and ``token_scales``).

        Shapes: q_in [T,H,R]; q_out the same shape; latent [T,Dn+R] u16
        (bf16); row_offsets [B+1] u32; cache_lengths [B] u32; page_table
        [B,stride] u32; freqs [max_seq,R]; gamma [Dn]; cache [L,P,S,1,Dn+R] u8
        (fp8) or u16 (bf16); token_scales [L,P,S,1] f32.  q_in, q_out, freqs
        and gamma may each be u16 (bf16 bits), float16 or float32 (q_in:
        bf16 or fp16).  ``scale_mode``: "per_tensor" | "per_token" (ignored
        for a bf16 cache).
        """
        T, H, R = q_in.shape
        W = latent.shape[1]
        Dn = W - R
        L, P, S = cache.shape[:3]
        if (cache.shape[3:] != (1, W) or q_out.shape != q_in.shape
                or latent.shape[0] != T):
            raise ValueError("inconsistent MLA shapes")
        B = row_offsets.size - 1
        cache_type = CACHE_BF16 if cache.dtype == np.uint16 else CACHE_FP8
        mode = {"per_tensor": SCALE_PER_TENSOR, "per_token": SCALE_PER_TOKEN,
                "none": 0}[scale_mode]
        rc = self.lib.oracle_mla_rope_rmsnorm_quant(
            _ptr(q_out, q_out.dtype), _elem_type(q_out), _ptr(q_in, q_in.dtype),
            _elem_type(q_in), _ptr(latent, np.uint16),
            _ptr(row_offsets, np.uint32), _ptr(cache_lengths, np.uint32), B,
            _ptr(page_table, np.uint32), page_table.shape[1],
            _ptr(freqs, freqs.dtype), _elem_type(freqs), freqs.shape[0],
            _ptr(gamma, gamma.dtype), _elem_type(gamma),
            float(epsilon), H, R, Dn, _ptr(cache, cache.dtype), cache_type, L, P, S,
            int(layer_idx), mode, float(tensor_scale),
            _ptr(token_scales, np.float32))
        _check(rc, "mla_rope_rmsnorm_quant")

    def token_plan(self, T, row_offsets, cache_lengths, page_table, num_pages, page_size):
        """Placement of each of the T new tokens: u32 [T, 4] rows (page,
        offset, position, 1), or zeros for a token without a request or a
        valid page."""
        plan = np.zeros((T, 4), np.uint32)
        rc = self.lib.oracle_token_plan(
            _ptr(plan, np.uint32), int(T), _ptr(row_offsets, np.uint32),
            _ptr(cache_lengths, np.uint32), row_offsets.size - 1, _ptr(page_table, np.uint32),
            page_table.shape[1], int(num_pages), int(page_size))
        _check(rc, "token_plan")
        return plan

    def mla_rope_rmsnorm_quant_planned(self, q_out, q_in, latent, plan, freqs, gamma,
                                       epsilon, cache, layer_idx, scale_mode,
                                       tensor_scale=1.0, token_scales=None):
        """:meth:`mla_rope_rmsnorm_quant` with each token placed by ``plan``
        (u32 [T, 4]: page, offset, position, placed flag) instead of the
        ragged batch and the page table; ``latent=None`` is the in-place form
        on a bf16 cache."""
        T, H, R = q_in.shape
        W = cache.shape[4] if latent is None else latent.shape[1]
        L, P, S = cache.shape[:3]
        if (cache.shape[3:] != (1, W) or q_out.shape != q_in.shape
                or (latent is not None and latent.shape[0] != T) or plan.shape != (T, 4)):
            raise ValueError("inconsistent MLA shapes")
        cache_type = CACHE_BF16 if cache.dtype == np.uint16 else CACHE_FP8
        mode = {"per_tensor": SCALE_PER_TENSOR, "per_token": SCALE_PER_TOKEN,
                "none": 0}[scale_mode]
        rc = self.lib.oracle_mla_rope_rmsnorm_quant_planned(
            _ptr(q_out, q_out.dtype), _elem_type(q_out), _ptr(q_in, q_in.dtype),
            _elem_type(q_in), _ptr(latent, np.uint16), _ptr(plan, np.uint32), T,
            _ptr(freqs, freqs.dtype), _elem_type(freqs), freqs.shape[0],
            _ptr(gamma, gamma.dtype), _elem_type(gamma), float(epsilon),
            H, R, W - R, _ptr(cache, cache.dtype), cache_type, L, P, S, int(layer_idx), mode,
            float(tensor_scale), _ptr(token_scales, np.float32))
        _check(rc, "mla_rope_rmsnorm_quant_planned")

    def mla_rope_rmsnorm_inplace(self, q_out, q_in, row_offsets, cache_lengths, page_table,
                                 freqs, gamma, epsilon, cache, layer_idx):
        """In-place form on a bf16 cache [L,P,S,1,Dn+R] u16 that holds the new
        tokens' latent rows at their slots; q as in
        :meth:`mla_rope_rmsnorm_quant`."""
        T, H, R = q_in.shape
        L, P, S, one, W = cache.shape
        if cache.dtype != np.uint16 or one != 1 or q_out.shape != q_in.shape:
            raise ValueError("inconsistent in-place MLA arguments")
        B = row_offsets.size - 1
        rc = self.lib.oracle_mla_rope_rmsnorm_inplace(
            _ptr(q_out, q_out.dtype), _elem_type(q_out), _ptr(q_in, q_in.dtype),
            _elem_type(q_in), _ptr(row_offsets, np.uint32),
            _ptr(cache_lengths, np.uint32), B, _ptr(page_table, np.uint32),
            page_table.shape[1], _ptr(freqs, freqs.dtype), _elem_type(freqs), freqs.shape[0],
            _ptr(gamma, gamma.dtype), _elem_type(gamma), float(epsilon), H, R, W - R,
            _ptr(cache, np.uint16),
            L, P, S, int(layer_idx))
        _check(rc, "mla_rope_rmsnorm_inplace")

    def qk_rope_paged_ragged(self, q_out, q_in, row_offsets, cache_lengths,
                             page_table, k_cache, layer_idx, freqs, position_ids,
                             interleaved, k_gamma=None, epsilon=1e-6, k_scale_mode="none",
                             k_scales=None, mrope_section=None):
        """Fill ``q_out``; rotate (and optionally K-normalise) ``k_cache``.

        Shapes: q [T,Hq,D] u16 (bf16 bits) or float16 (q_out of the same
        type); k_cache [L,P,S,Hkv,D] u16 (bf16) or u8 (fp8,
        with k_scale_mode "per_tensor" -> k_scales f32 [1], "per_token" ->
        k_scales f32 [L,P,S,Hkv], rewritten); freqs [max_seq,D] f32, float16
        or u16 (bf16);
        position_ids [T] u32 or None, or [3, T] u32 with mrope_section =
        (temporal, height, width) pair counts summing to D/2; k_gamma [C]
        u16 or None.
        """
        T, Hq, D = q_in.shape
        L, P, S, Hkv, Dk = k_cache.shape
        if Dk != D or q_out.shape != q_in.shape or q_out.dtype != q_in.dtype:
            raise ValueError("inconsistent QK shapes")
        B = row_offsets.size - 1
        k_type = CACHE_BF16 if k_cache.dtype == np.uint16 else CACHE_FP8
        mode = {"per_tensor": SCALE_PER_TENSOR, "per_token": SCALE_PER_TOKEN, "none": 0}[k_scale_mode]
        sec = None if mrope_section is None else np.asarray(mrope_section, np.int64)
        if sec is not None and (position_ids is None or position_ids.shape != (3, T)):
            raise ValueError("multimodal RoPE needs position ids of shape [3, T]")
        rc = self.lib.oracle_qk_rope_paged_ragged(
            _ptr(q_out, q_out.dtype), _ptr(q_in, q_in.dtype), _elem_type(q_in), Hq, D,
            _ptr(row_offsets, np.uint32), _ptr(cache_lengths, np.uint32), B,
            _ptr(page_table, np.uint32), page_table.shape[1], _ptr(k_cache, k_cache.dtype),
            k_type, mode, _ptr(k_scales, np.float32), L, P, S, Hkv, int(layer_idx),
            _ptr(freqs, freqs.dtype), _elem_type(freqs), freqs.shape[0],
            _ptr(position_ids, np.uint32),
            None if sec is None else sec.ctypes.data,
            int(bool(interleaved)), _ptr(k_gamma, np.uint16),
            0 if k_gamma is None else k_gamma.size, float(epsilon))
        _check(rc, "qk_rope_paged_ragged")

    def mla_gather_latent_paged(self, out, kv_row_offsets, page_table, cache, layer_idx,
                                scale_mode="none", cache_scales=None, out_scales=None,
                                out_tensor_scale=1.0):
        """Fill ``out`` [rows, W] (u8 = fp8 codes, u16 = bf16 bits) with the
        cache rows of every request's context; cache [L,P,S,1,W] u8 or u16;
        cache_scales f32 [1] (per-tensor) or [L,P,S,1] (per-token)."""
        L, P, S, one, W = cache.shape
        if one != 1 or out.shape[1] != W:
            raise ValueError("inconsistent gather shapes")
        B = kv_row_offsets.size - 1
        mode = {"per_tensor": SCALE_PER_TENSOR, "per_token": SCALE_PER_TOKEN, "none": 0}[scale_mode]
        rc = self.lib.oracle_mla_gather_latent_paged(
            _ptr(out, out.dtype), CACHE_BF16 if out.dtype == np.uint16 else CACHE_FP8,
            _ptr(out_scales, np.float32), float(out_tensor_scale),
            _ptr(kv_row_offsets, np.uint32), B, _ptr(page_table, np.uint32),
            page_table.shape[1], _ptr(cache, cache.dtype),
            CACHE_BF16 if cache.dtype == np.uint16 else CACHE_FP8, mode,
            _ptr(cache_scales, np.float32), W, L, P, S, int(layer_idx))
        _check(rc, "mla_gather_latent_paged")

    def rms_norm_kv_cache_paged(self, k_cache, layer_idx, row_offsets,
                                cache_lengths, page_table, gamma, epsilon,
                                weight_offset, total_seq_len,
                                multiply_before_cast=True, k_scale_mode="none",
                                k_scales=None, per_head_norm=True):
        """Normalise the new K rows of ``k_cache`` in place (one statistic per
        head, or per token over all heads with per_head_norm=False); fp8
        caches as in :meth:`qk_rope_paged_ragged`."""
        L, P, S, Hkv, D = k_cache.shape
        B = row_offsets.size - 1
        k_type = CACHE_BF16 if k_cache.dtype == np.uint16 else CACHE_FP8
        mode = {"per_tensor": SCALE_PER_TENSOR, "per_token": SCALE_PER_TOKEN, "none": 0}[k_scale_mode]
        rc = self.lib.oracle_rms_norm_kv_cache_paged(
            _ptr(k_cache, k_cache.dtype), k_type, mode, _ptr(k_scales, np.float32),
            L, P, S, Hkv, D, int(layer_idx),
            _ptr(row_offsets, np.uint32), _ptr(cache_lengths, np.uint32), B,
            _ptr(page_table, np.uint32), page_table.shape[1],
            _ptr(gamma, gamma.dtype), _elem_type(gamma), gamma.size, float(epsilon),
            float(weight_offset), int(total_seq_len),
            int(bool(multiply_before_cast)), int(bool(per_head_norm)))
        _check(rc, "rms_norm_kv_cache_paged")

    def rms_norm_kv_cache_planned(self, k_cache, layer_idx, plan, gamma, epsilon,
                                  weight_offset, total_seq_len, multiply_before_cast=True,
                                  k_scale_mode="none", k_scales=None, per_head_norm=True):
        """:meth:`rms_norm_kv_cache_paged` with each token t < total_seq_len
        placed by ``plan`` (u32 [T, 4]: page, offset, position, placed flag)."""
        L, P, S, Hkv, D = k_cache.shape
        k_type = CACHE_BF16 if k_cache.dtype == np.uint16 else CACHE_FP8
        mode = {"per_tensor": SCALE_PER_TENSOR, "per_token": SCALE_PER_TOKEN, "none": 0}[k_scale_mode]
        if plan.ndim != 2 or plan.shape[1] != 4 or plan.shape[0] < total_seq_len:
            raise ValueError("plan must be [>= total_seq_len, 4]")
        rc = self.lib.oracle_rms_norm_kv_cache_planned(
            _ptr(k_cache, k_cache.dtype), k_type, mode, _ptr(k_scales, np.float32),
            L, P, S, Hkv, D, int(layer_idx), _ptr(plan, np.uint32),
            _ptr(gamma, gamma.dtype), _elem_type(gamma), gamma.size, float(epsilon),
            float(weight_offset),
            int(total_seq_len), int(bool(multiply_before_cast)), int(bool(per_head_norm)))
        _check(rc, "rms_norm_kv_cache_planned")


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    """The oracle built from the committed source."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
