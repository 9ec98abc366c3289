"""Python binding of the paged-KV pre-attention library (``include/pkv.h``).

Argument marshalling only: every function here checks nothing beyond what it
needs to fill the C call, passes torch device tensors as raw pointers with
element strides, and raises :class:`PkvError` when the library returns a
non-zero status.  All computation happens in the HIP kernels of ``libpkv.so``
(built for gfx950 by ``paged_kv_cache_wavefront_amd.build``); there is no
fallback: importing the module without the built library raises.

Tensor conventions: bf16 data is ``torch.bfloat16``; q, its output,
freqs_cis and gamma may also be ``torch.float16`` or ``torch.float32`` where
the C entry point accepts that type (their ``pkv_elem_types`` is built from
the tensors' dtypes, any other dtype passing a code the library refuses with
PKV_ERR_DTYPE); the FP8 cache is
``torch.uint8`` (or ``torch.float8_e4m3fn``) holding E4M3FN codes; index
arrays are ``torch.int32`` or ``torch.uint32`` holding unsigned values; all of
them live on the same ROCm device.  Kernels are enqueued on ``stream`` (a
``torch.cuda.Stream``) or on torch's current stream.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpkv.so")

PKV_DTYPE_BF16 = 0
PKV_DTYPE_FP8_E4M3FN = 1
PKV_DTYPE_F32 = 2
PKV_DTYPE_F16 = 3
PKV_SCALE_NONE = 0
PKV_SCALE_PER_TENSOR = 1
PKV_SCALE_PER_TOKEN = 2

EXPORTED = ("mla_rope_rmsnorm_quant", "mla_rope_rmsnorm_inplace", "pkv_token_plan",
            "mla_rope_rmsnorm_quant_planned", "mla_rope_rmsnorm_inplace_planned",
            "qk_rope_paged_ragged",
            "rms_norm_kv_cache_paged", "rms_norm_kv_cache_paged_planned",
            "mla_gather_latent_paged", "mla_rope_rmsnorm_quant_noalloc", "pkv_status_string")


class PkvError(RuntimeError):
    def __init__(self, func: str, status: int, text: str):
        super().__init__(f"{func} failed: {text} (status {status})")
        self.status = status


class PagedCache(ctypes.Structure):
    """Mirror of ``pkv_paged_cache``."""

    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("num_layers", ctypes.c_uint32),
        ("num_pages", ctypes.c_uint32),
        ("page_size", ctypes.c_uint32),
        ("num_heads", ctypes.c_uint32),
        ("head_dim", ctypes.c_uint32),
        ("layer_stride", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("slot_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64),
        ("cache_lengths", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("page_table_stride", ctypes.c_uint32),
        ("scale_mode", ctypes.c_int32),
        ("scales", ctypes.c_void_p),
        ("error_count", ctypes.c_void_p),
    ]


class ElemTypes(ctypes.Structure):
    """Mirror of ``pkv_elem_types``."""

    _fields_ = [("q", ctypes.c_int32), ("q_out", ctypes.c_int32), ("freqs", ctypes.c_int32),
                ("gamma", ctypes.c_int32)]


_ELEM_CODES = {torch.bfloat16: PKV_DTYPE_BF16, torch.float16: PKV_DTYPE_F16,
               torch.float32: PKV_DTYPE_F32}


def _code(t: torch.Tensor | None, default: int) -> int:
    if t is None:
        return default
    return _ELEM_CODES.get(t.dtype, -1)  # -1: refused by the library


def _types(q=None, q_out=None, freqs=None, gamma=None) -> ElemTypes:
    """The pkv_elem_types of a call, from its tensors' dtypes (a missing tensor
    takes the library's default)."""
    return ElemTypes(_code(q, PKV_DTYPE_BF16), _code(q_out, PKV_DTYPE_BF16),
                     _code(freqs, PKV_DTYPE_F32), _code(gamma, PKV_DTYPE_BF16))


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python paged_kv_cache_wavefront_amd/build.py` "
            "(hipcc, gfx950) first -- there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    i64, u32, vp, f32 = ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_float
    cache_p = ctypes.POINTER(PagedCache)
    types_p = ctypes.POINTER(ElemTypes)
    lib.mla_rope_rmsnorm_quant.restype = ctypes.c_int
    lib.mla_rope_rmsnorm_quant.argtypes = [
        vp, i64, i64, vp, i64, i64, vp, i64, vp, u32, u32, u32, u32, u32, vp, u32, vp, f32,
        cache_p, u32, types_p, vp]
    lib.mla_rope_rmsnorm_inplace.restype = ctypes.c_int
    lib.mla_rope_rmsnorm_inplace.argtypes = [
        vp, i64, i64, vp, i64, i64, vp, u32, u32, u32, u32, u32, vp, u32, vp, f32,
        cache_p, u32, types_p, vp]
    lib.pkv_token_plan.restype = ctypes.c_int
    lib.pkv_token_plan.argtypes = [vp, vp, u32, u32, cache_p, vp]
    lib.mla_rope_rmsnorm_quant_planned.restype = ctypes.c_int
    lib.mla_rope_rmsnorm_quant_planned.argtypes = [
        vp, i64, i64, vp, i64, i64, vp, i64, vp, u32, u32, u32, u32, vp, u32, vp, f32,
        cache_p, u32, types_p, vp]
    lib.mla_rope_rmsnorm_inplace_planned.restype = ctypes.c_int
    lib.mla_rope_rmsnorm_inplace_planned.argtypes = [
        vp, i64, i64, vp, i64, i64, vp, u32, u32, u32, u32, vp, u32, vp, f32, cache_p, u32,
        types_p, vp]
    lib.qk_rope_paged_ragged.restype = ctypes.c_int
    lib.qk_rope_paged_ragged.argtypes = [
        vp, i64, i64, vp, i64, i64, u32, u32, u32, vp, u32, cache_p, u32, vp, u32, vp, vp,
        ctypes.c_int, vp, u32, f32, types_p, vp]
    lib.rms_norm_kv_cache_paged.restype = ctypes.c_int
    lib.rms_norm_kv_cache_paged.argtypes = [
        cache_p, u32, vp, u32, f32, f32, u32, vp, u32, ctypes.c_int, ctypes.c_int, types_p, vp]
    lib.rms_norm_kv_cache_paged_planned.restype = ctypes.c_int
    lib.rms_norm_kv_cache_paged_planned.argtypes = [
        cache_p, u32, vp, u32, f32, f32, u32, vp, ctypes.c_int, ctypes.c_int, types_p, vp]
    lib.mla_gather_latent_paged.restype = ctypes.c_int
    lib.mla_gather_latent_paged.argtypes = [
        vp, ctypes.c_int32, i64, vp, vp, vp, u32, u32, cache_p, u32, vp]
    lib.mla_rope_rmsnorm_quant_noalloc.restype = ctypes.c_int
    lib.mla_rope_rmsnorm_quant_noalloc.argtypes = [
        vp, i64, i64, vp, i64, i64, vp, i64, vp, u32, u32, u32, u32, u32, vp, u32, vp, f32,
        cache_p, u32, types_p, ctypes.c_int, vp]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_stream_copy.restype = ctypes.c_int
    lib.pkv_stream_copy.argtypes = [vp, vp, ctypes.c_uint64, u32, vp]
    lib.pkv_stream_mix.restype = ctypes.c_int
    lib.pkv_stream_mix.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_uint64, u32, vp]
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.pkv_status_string(int(status)).decode()


def _check(func: str, status: int) -> None:
    if status != 0:
        raise PkvError(func, status, status_string(status))


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def paged_cache(data: torch.Tensor, cache_lengths: torch.Tensor | None, page_table: torch.Tensor,
                scale_mode: int = PKV_SCALE_NONE, scales: torch.Tensor | None = None,
                error_count: torch.Tensor | None = None) -> PagedCache:
    """Describe a 5-D cache pool ``data[layer, page, slot, head, dim]`` (bf16,
    or uint8 / float8_e4m3fn for FP8), its per-request prior lengths and its
    page table ``[batch, stride]``.  ``scales``: fp32 ``[1]`` (per-tensor) or
    ``[layers, pages, page_size, heads]`` (per-token).  The returned descriptor
    keeps references to the tensors it points to."""
    if data.dim() != 5:
        raise ValueError("cache data must be [layers, pages, page_size, heads, head_dim]")
    if data.dtype == torch.bfloat16:
        dt = PKV_DTYPE_BF16
    elif data.dtype in (torch.uint8, torch.float8_e4m3fn):
        dt = PKV_DTYPE_FP8_E4M3FN
    else:
        raise TypeError(f"unsupported cache dtype {data.dtype}")
    if data.stride(4) != 1:
        raise ValueError("the head_dim axis of the cache must be contiguous")
    if page_table.dim() != 2 or page_table.stride(1) != 1:
        raise ValueError("page_table must be a row-major [batch, stride] tensor")
    L, P, S, H, D = data.shape
    desc = PagedCache(
        data=data.data_ptr(), dtype=dt, num_layers=L, num_pages=P, page_size=S,
        num_heads=H, head_dim=D, layer_stride=data.stride(0), page_stride=data.stride(1),
        slot_stride=data.stride(2), head_stride=data.stride(3),
        cache_lengths=_ptr(cache_lengths), page_table=page_table.data_ptr(),
        page_table_stride=page_table.stride(0), scale_mode=scale_mode,
        scales=_ptr(scales), error_count=_ptr(error_count))
    # the struct holds raw device pointers: keep the tensors alive with it
    desc._tensors = (data, cache_lengths, page_table, scales, error_count)
    return desc


def mla_rope_rmsnorm_quant(q_rope_output: torch.Tensor, q_rope: torch.Tensor,
                           kv_latent: torch.Tensor, input_row_offsets: torch.Tensor,
                           freqs_cis: torch.Tensor, gamma: torch.Tensor, epsilon: float,
                           kv_cache: PagedCache, layer_idx: int, stream=None) -> None:
    """Fused MLA step (C: ``mla_rope_rmsnorm_quant``).  q tensors are
    ``[tokens, heads, rope_dim]`` (rope_dim axis contiguous; q_rope bf16 or
    float16, q_rope_output bf16, float16 or float32), kv_latent
    ``[tokens, kv_norm_dim + rope_dim]`` bf16, freqs_cis ``[max_seq_len,
    rope_dim]`` and gamma ``[kv_norm_dim]`` float32, bf16 or float16."""
    T, H, R = q_rope.shape
    st = _lib.mla_rope_rmsnorm_quant(
        _ptr(q_rope_output), q_rope_output.stride(0), q_rope_output.stride(1),
        _ptr(q_rope), q_rope.stride(0), q_rope.stride(1),
        _ptr(kv_latent), kv_latent.stride(0),
        _ptr(input_row_offsets), input_row_offsets.numel() - 1, T, H, R,
        kv_latent.shape[1] - R, _ptr(freqs_cis), freqs_cis.shape[0], _ptr(gamma),
        float(epsilon), ctypes.byref(kv_cache), int(layer_idx),
        ctypes.byref(_types(q_rope, q_rope_output, freqs_cis, gamma)),
        _stream(stream))
    _check("mla_rope_rmsnorm_quant", st)


def mla_rope_rmsnorm_inplace(q_rope_output: torch.Tensor, q_rope: torch.Tensor,
                             input_row_offsets: torch.Tensor, freqs_cis: torch.Tensor,
                             gamma: torch.Tensor, epsilon: float, kv_cache: PagedCache,
                             layer_idx: int, stream=None) -> None:
    """Fused MLA step in place on a bf16 latent cache that already holds the
    new tokens' rows (C: ``mla_rope_rmsnorm_inplace``).  Shapes as for
    :func:`mla_rope_rmsnorm_quant`; the latent row width is the cache's
    head_dim."""
    T, H, R = q_rope.shape
    st = _lib.mla_rope_rmsnorm_inplace(
        _ptr(q_rope_output), q_rope_output.stride(0), q_rope_output.stride(1),
        _ptr(q_rope), q_rope.stride(0), q_rope.stride(1),
        _ptr(input_row_offsets), input_row_offsets.numel() - 1, T, H, R,
        kv_cache.head_dim - R, _ptr(freqs_cis), freqs_cis.shape[0], _ptr(gamma),
        float(epsilon), ctypes.byref(kv_cache), int(layer_idx),
        ctypes.byref(_types(q_rope, q_rope_output, freqs_cis, gamma)),
        _stream(stream))
    _check("mla_rope_rmsnorm_inplace", st)


def _check_plan(plan: torch.Tensor, rows: int, like: torch.Tensor | None, what: str) -> None:
    """A token plan is a contiguous [>= rows, 4] int32 / uint32 tensor on the
    device of the other tensors: the library writes or reads 16 bytes per
    token through its raw pointer and cannot check any of this itself."""
    if plan.dim() != 2 or plan.shape[1] != 4 or not plan.is_contiguous():
        raise ValueError("plan must be a contiguous [tokens, 4] tensor")
    if plan.dtype not in (torch.int32, torch.uint32):
        raise TypeError(f"plan must be int32 or uint32, not {plan.dtype}")
    if plan.shape[0] < rows:
        raise ValueError(f"plan has fewer rows than {what}")
    if not plan.is_cuda or (like is not None and plan.device != like.device):
        where = "a ROCm device" if like is None else str(like.device)
        raise ValueError(f"plan must live on {where}, not {plan.device}")


def pkv_token_plan(plan: torch.Tensor, input_row_offsets: torch.Tensor, kv_cache: PagedCache,
                   stream=None) -> None:
    """Write each new token's placement (C: ``pkv_token_plan``) into ``plan``,
    a contiguous ``[tokens, 4]`` int32 / uint32 tensor: (page, offset,
    position, 1), or zeros for a token without a valid placement.  The
    token count is ``plan.shape[0]``."""
    _check_plan(plan, 0, input_row_offsets, "tokens")
    st = _lib.pkv_token_plan(_ptr(plan), _ptr(input_row_offsets),
                             input_row_offsets.numel() - 1, plan.shape[0],
                             ctypes.byref(kv_cache), _stream(stream))
    _check("pkv_token_plan", st)


def mla_rope_rmsnorm_quant_planned(q_rope_output: torch.Tensor, q_rope: torch.Tensor,
                                   kv_latent: torch.Tensor, plan: torch.Tensor,
                                   freqs_cis: torch.Tensor, gamma: torch.Tensor,
                                   epsilon: float, kv_cache: PagedCache, layer_idx: int,
                                   stream=None) -> None:
    """Fused MLA step placed by a token plan (C:
    ``mla_rope_rmsnorm_quant_planned``); arguments as for
    :func:`mla_rope_rmsnorm_quant` with ``plan`` (``[tokens, 4]``, from
    :func:`pkv_token_plan`) in place of the row offsets."""
    T, H, R = q_rope.shape
    _check_plan(plan, T, q_rope, "q_rope has tokens")
    st = _lib.mla_rope_rmsnorm_quant_planned(
        _ptr(q_rope_output), q_rope_output.stride(0), q_rope_output.stride(1),
        _ptr(q_rope), q_rope.stride(0), q_rope.stride(1),
        _ptr(kv_latent), kv_latent.stride(0), _ptr(plan), T, H, R,
        kv_latent.shape[1] - R, _ptr(freqs_cis), freqs_cis.shape[0], _ptr(gamma),
        float(epsilon), ctypes.byref(kv_cache), int(layer_idx),
        ctypes.byref(_types(q_rope, q_rope_output, freqs_cis, gamma)),
        _stream(stream))
    _check("mla_rope_rmsnorm_quant_planned", st)


def mla_rope_rmsnorm_inplace_planned(q_rope_output: torch.Tensor, q_rope: torch.Tensor,
                                     plan: torch.Tensor, freqs_cis: torch.Tensor,
                                     gamma: torch.Tensor, epsilon: float, kv_cache: PagedCache,
                                     layer_idx: int, stream=None) -> None:
    """In-place fused MLA step placed by a token plan (C:
    ``mla_rope_rmsnorm_inplace_planned``); arguments as for
    :func:`mla_rope_rmsnorm_inplace` with ``plan`` in place of the row
    offsets."""
    T, H, R = q_rope.shape
    _check_plan(plan, T, q_rope, "q_rope has tokens")
    st = _lib.mla_rope_rmsnorm_inplace_planned(
        _ptr(q_rope_output), q_rope_output.stride(0), q_rope_output.stride(1),
        _ptr(q_rope), q_rope.stride(0), q_rope.stride(1), _ptr(plan), T, H, R,
        kv_cache.head_dim - R, _ptr(freqs_cis), freqs_cis.shape[0], _ptr(gamma),
        float(epsilon), ctypes.byref(kv_cache), int(layer_idx),
        ctypes.byref(_types(q_rope, q_rope_output, freqs_cis, gamma)),
        _stream(stream))
    _check("mla_rope_rmsnorm_inplace_planned", st)


def mla_rope_rmsnorm_quant_noalloc(q_rope_output: torch.Tensor, q_rope: torch.Tensor,
                                   kv_latent: torch.Tensor, input_row_offsets: torch.Tensor,
                                   freqs_cis: torch.Tensor, gamma: torch.Tensor, epsilon: float,
                                   kv_cache: PagedCache, layer_idx: int, build_plan: bool = True,
                                   stream=None) -> None:
    """The planned MLA step with its token plan in the library's static
    device array (C: ``mla_rope_rmsnorm_quant_noalloc``): ``build_plan``
    writes this batch's plan there first; without it the plan the last
    building call left on the device is used.  Arguments as for
    :func:`mla_rope_rmsnorm_quant`; nothing is allocated."""
    T, H, R = q_rope.shape
    st = _lib.mla_rope_rmsnorm_quant_noalloc(
        _ptr(q_rope_output), q_rope_output.stride(0), q_rope_output.stride(1),
        _ptr(q_rope), q_rope.stride(0), q_rope.stride(1),
        _ptr(kv_latent), kv_latent.stride(0),
        _ptr(input_row_offsets), input_row_offsets.numel() - 1, T, H, R,
        kv_latent.shape[1] - R, _ptr(freqs_cis), freqs_cis.shape[0], _ptr(gamma),
        float(epsilon), ctypes.byref(kv_cache), int(layer_idx),
        ctypes.byref(_types(q_rope, q_rope_output, freqs_cis, gamma)),
        int(bool(build_plan)), _stream(stream))
    _check("mla_rope_rmsnorm_quant_noalloc", st)


def qk_rope_paged_ragged(q_out: torch.Tensor, q_proj: torch.Tensor,
                         input_row_offsets: torch.Tensor, k_cache: PagedCache,
                         layer_idx: int, freqs_cis: torch.Tensor,
                         position_ids: torch.Tensor | None, interleaved: bool,
                         k_norm_gamma: torch.Tensor | None = None, epsilon: float = 1e-6,
                         stream=None, mrope_section=None) -> None:
    """Paged-ragged fused Q/K RoPE (C: ``qk_rope_paged_ragged``).  Q tensors
    are ``[tokens, heads, head_dim]`` bf16 or float16 (both the same);
    freqs_cis float32, bf16 or float16; K is rotated in place.
    ``mrope_section``: three ints (temporal, height, width pair counts) with
    ``position_ids`` of shape [3, tokens]."""
    T, Hq, D = q_proj.shape
    sec = None
    if mrope_section is not None:
        sec = (ctypes.c_uint32 * 3)(*[int(v) for v in mrope_section])
    st = _lib.qk_rope_paged_ragged(
        _ptr(q_out), q_out.stride(0), q_out.stride(1), _ptr(q_proj), q_proj.stride(0),
        q_proj.stride(1), T, Hq, D, _ptr(input_row_offsets), input_row_offsets.numel() - 1,
        ctypes.byref(k_cache), int(layer_idx), _ptr(freqs_cis), freqs_cis.shape[0],
        _ptr(position_ids), sec, int(bool(interleaved)), _ptr(k_norm_gamma),
        0 if k_norm_gamma is None else k_norm_gamma.numel(), float(epsilon),
        ctypes.byref(_types(q_proj, q_out, freqs_cis, k_norm_gamma)), _stream(stream))
    _check("qk_rope_paged_ragged", st)


def rms_norm_kv_cache_paged(k_cache: PagedCache, layer_idx: int, gamma: torch.Tensor,
                            epsilon: float, weight_offset: float, total_seq_len: int,
                            input_row_offsets: torch.Tensor, per_head_norm: bool = True,
                            multiply_before_cast: bool = True, stream=None) -> None:
    """In-place K-cache RMSNorm (C: ``rms_norm_kv_cache_paged``); gamma bf16,
    float16 or float32."""
    st = _lib.rms_norm_kv_cache_paged(
        ctypes.byref(k_cache), int(layer_idx), _ptr(gamma), gamma.numel(), float(epsilon),
        float(weight_offset), int(total_seq_len), _ptr(input_row_offsets),
        input_row_offsets.numel() - 1, int(bool(per_head_norm)),
        int(bool(multiply_before_cast)), ctypes.byref(_types(gamma=gamma)), _stream(stream))
    _check("rms_norm_kv_cache_paged", st)


def rms_norm_kv_cache_paged_planned(k_cache: PagedCache, layer_idx: int, gamma: torch.Tensor,
                                    epsilon: float, weight_offset: float, total_seq_len: int,
                                    plan: torch.Tensor, per_head_norm: bool = True,
                                    multiply_before_cast: bool = True, stream=None) -> None:
    """In-place K-cache RMSNorm placed by a token plan (C:
    ``rms_norm_kv_cache_paged_planned``); ``plan`` is the ``[tokens, 4]``
    tensor :func:`pkv_token_plan` wrote."""
    _check_plan(plan, int(total_seq_len), gamma, "total_seq_len")
    st = _lib.rms_norm_kv_cache_paged_planned(
        ctypes.byref(k_cache), int(layer_idx), _ptr(gamma), gamma.numel(), float(epsilon),
        float(weight_offset), int(total_seq_len), _ptr(plan), int(bool(per_head_norm)),
        int(bool(multiply_before_cast)), ctypes.byref(_types(gamma=gamma)), _stream(stream))
    _check("rms_norm_kv_cache_paged_planned", st)


def mla_gather_latent_paged(out: torch.Tensor, kv_row_offsets: torch.Tensor,
                            cache: PagedCache, layer_idx: int,
                            out_scales: torch.Tensor | None = None,
                            out_scale: torch.Tensor | None = None, stream=None) -> None:
    """Paged latent cache -> dense ``out`` [rows, head_dim] (C:
    ``mla_gather_latent_paged``).  ``out`` is bf16 (dequantise / copy) or
    uint8 / float8_e4m3fn (copy / quantise with ``out_scale``)."""
    out_dt = PKV_DTYPE_BF16 if out.dtype == torch.bfloat16 else PKV_DTYPE_FP8_E4M3FN
    st = _lib.mla_gather_latent_paged(
        _ptr(out), out_dt, out.stride(0), _ptr(out_scales), _ptr(out_scale),
        _ptr(kv_row_offsets), kv_row_offsets.numel() - 1, out.shape[0], ctypes.byref(cache),
        int(layer_idx), _stream(stream))
    _check("mla_gather_latent_paged", st)


def pkv_stream_copy(dst: torch.Tensor, src: torch.Tensor, blocks: int, stream=None) -> None:
    """Measurement helper (C: ``pkv_stream_copy``, include/pkv_bench.h): copy
    src's bytes into dst with a plain streaming kernel of ``blocks`` blocks."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    st = _lib.pkv_stream_copy(_ptr(src), _ptr(dst), nbytes, int(blocks), _stream(stream))
    _check("pkv_stream_copy", st)


def pkv_stream_mix(dst: torch.Tensor, src: torch.Tensor, read_bytes: int, write_bytes: int,
                   blocks: int, stream=None) -> None:
    """Measurement helper (C: ``pkv_stream_mix``, include/pkv_bench.h): read
    ``read_bytes`` of src and write ``write_bytes`` of dst in one streaming
    kernel, the two interleaved at that ratio; ``dst is src`` streams in
    place."""
    if read_bytes > src.numel() * src.element_size():
        raise ValueError("src smaller than read_bytes")
    if write_bytes > dst.numel() * dst.element_size():
        raise ValueError("dst smaller than write_bytes")
    st = _lib.pkv_stream_mix(_ptr(src), int(read_bytes), _ptr(dst), int(write_bytes),
                             int(blocks), _stream(stream))
    _check("pkv_stream_mix", st)
