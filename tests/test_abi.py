"""The C ABI on the CPU: the library loads, exports every function that
include/*.h declares, and rejects bad arguments on the host with the
documented status before touching the device (no kernel is launched here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, RANGE, LAUNCH = range(8)
FAKE = 0x10000          # 16-byte aligned stand-in for a device pointer (never dereferenced)


def declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:int|const char\s*\*)\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_wavefront_amd as pkv
    return pkv


def test_header_declares_entry_points():
    assert declared_functions() == sorted(["mla_rope_rmsnorm_quant", "mla_rope_rmsnorm_inplace",
                                           "pkv_token_plan", "mla_rope_rmsnorm_quant_planned",
                                           "mla_rope_rmsnorm_inplace_planned",
                                           "qk_rope_paged_ragged", "rms_norm_kv_cache_paged",
                                           "rms_norm_kv_cache_paged_planned",
                                           "mla_gather_latent_paged", "pkv_status_string",
                                           "mla_rope_rmsnorm_quant_noalloc",
                                           "pkv_stream_copy", "pkv_stream_mix"])


def test_library_exports_every_declared_function(pkv):
    lib = pkv.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared_functions()) <= exported


def test_binding_names_match_header(pkv):
    for name in declared_functions():
        if name != "pkv_status_string":
            assert callable(getattr(pkv, name)), name


def test_stream_copy_validation(pkv):
    lib = pkv.library()
    assert lib.pkv_stream_copy(None, FAKE, 16, 1, None) == NULL
    assert lib.pkv_stream_copy(FAKE, FAKE + 4096, 16, 0, None) == SHAPE
    assert lib.pkv_stream_copy(FAKE + 8, FAKE + 4096, 16, 1, None) == ALIGN
    assert lib.pkv_stream_copy(FAKE, FAKE + 4096, 24, 1, None) == ALIGN
    assert lib.pkv_stream_copy(FAKE, FAKE + 4096, 0, 1, None) == OK


def test_stream_mix_validation(pkv):
    lib = pkv.library()
    assert lib.pkv_stream_mix(None, 16, FAKE, 16, 1, None) == NULL
    assert lib.pkv_stream_mix(FAKE, 16, None, 16, 1, None) == NULL
    assert lib.pkv_stream_mix(FAKE, 16, FAKE + 4096, 16, 0, None) == SHAPE
    assert lib.pkv_stream_mix(FAKE, 32, FAKE, 16, 1, None) == SHAPE      # in place: equal counts
    assert lib.pkv_stream_mix(FAKE + 8, 16, FAKE + 4096, 16, 1, None) == ALIGN
    assert lib.pkv_stream_mix(FAKE, 24, FAKE + 4096, 16, 1, None) == ALIGN
    assert lib.pkv_stream_mix(FAKE, 16, FAKE + 4096, 40, 1, None) == ALIGN
    assert lib.pkv_stream_mix(FAKE, 4096, FAKE + 2048, 4096, 1, None) == RANGE  # overlap
    assert lib.pkv_stream_mix(FAKE + 2048, 4096, FAKE, 4096, 1, None) == RANGE
    assert lib.pkv_stream_mix(FAKE, 16 << 31, FAKE << 8, 16, 1, None) == RANGE
    assert lib.pkv_stream_mix(FAKE, 0, FAKE + 4096, 0, 1, None) == OK
    assert lib.pkv_stream_mix(FAKE, 0, FAKE, 0, 1, None) == OK


def test_status_strings(pkv):
    assert pkv.status_string(OK) == "PKV_OK"
    for code in range(1, 8):
        assert pkv.status_string(code).startswith("PKV_ERR_")
    assert "unknown" in pkv.status_string(99)


def mla_cache(pkv, **kw):
    base = dict(data=FAKE, dtype=pkv.PKV_DTYPE_FP8_E4M3FN, num_layers=2, num_pages=8,
                page_size=16, num_heads=1, head_dim=576, layer_stride=8 * 16 * 576,
                page_stride=16 * 576, slot_stride=576, head_stride=576, cache_lengths=FAKE,
                page_table=FAKE, page_table_stride=4, scale_mode=pkv.PKV_SCALE_PER_TENSOR,
                scales=FAKE, error_count=None)
    base.update(kw)
    return pkv.PagedCache(**base)


def elem_types(pkv, q=0, q_out=0, freqs=2, gamma=0):
    """A pkv_elem_types by reference (defaults: bf16 q and output, fp32 freqs,
    bf16 gamma)."""
    return ctypes.byref(pkv.ElemTypes(q, q_out, freqs, gamma))


def call_mla(pkv, cache, T=16, H=4, R=64, Dn=512, q=FAKE, qo=FAKE, lat=FAKE, qstride=4 * 64,
             layer=1, batch=2, freqs=FAKE, gamma=FAKE, max_seq=64, qo_dtype=None, qostride=None,
             types=None):
    lib = pkv.library()
    cp = None if cache is None else ctypes.byref(cache)
    qos = qstride if qostride is None else qostride
    if qo_dtype is not None:
        types = elem_types(pkv, q_out=qo_dtype)
    return lib.mla_rope_rmsnorm_quant(qo, qos, R, q, qstride, R, lat, Dn + R, FAKE, batch,
                                      T, H, R, Dn, freqs, max_seq, gamma, 1e-6, cp, layer,
                                      types, None)


def test_mla_validation(pkv):
    assert call_mla(pkv, None) == NULL
    assert call_mla(pkv, mla_cache(pkv), R=63) == SHAPE
    assert call_mla(pkv, mla_cache(pkv), R=32) == SHAPE                 # head_dim != Dn + R
    # rope_dim 32, 64, 128 and kv_norm_dim up to 512 in steps of 8 are built
    assert call_mla(pkv, mla_cache(pkv, head_dim=560), R=48) == UNSUP
    assert call_mla(pkv, mla_cache(pkv, head_dim=528), R=16) == UNSUP
    assert call_mla(pkv, mla_cache(pkv, head_dim=768), R=256) == UNSUP
    assert call_mla(pkv, mla_cache(pkv, head_dim=584), Dn=520) == UNSUP
    assert call_mla(pkv, mla_cache(pkv, head_dim=164), Dn=100) == UNSUP
    assert call_mla(pkv, mla_cache(pkv, num_heads=2)) == SHAPE
    assert call_mla(pkv, mla_cache(pkv, scale_mode=pkv.PKV_SCALE_NONE)) == DTYPE
    assert call_mla(pkv, mla_cache(pkv, dtype=pkv.PKV_DTYPE_BF16)) == DTYPE
    assert call_mla(pkv, mla_cache(pkv, dtype=7)) == DTYPE
    assert call_mla(pkv, mla_cache(pkv), layer=2) == RANGE
    assert call_mla(pkv, mla_cache(pkv, page_size=0)) == SHAPE
    assert call_mla(pkv, mla_cache(pkv), batch=0) == SHAPE
    assert call_mla(pkv, mla_cache(pkv), max_seq=0) == SHAPE
    assert call_mla(pkv, mla_cache(pkv, data=None)) == NULL
    assert call_mla(pkv, mla_cache(pkv, page_table=None)) == NULL
    assert call_mla(pkv, mla_cache(pkv, scales=None)) == NULL
    assert call_mla(pkv, mla_cache(pkv), q=None) == NULL
    assert call_mla(pkv, mla_cache(pkv), freqs=None) == NULL
    assert call_mla(pkv, mla_cache(pkv), q=FAKE + 8) == ALIGN
    assert call_mla(pkv, mla_cache(pkv), qstride=4 * 64 + 4) == ALIGN
    assert call_mla(pkv, mla_cache(pkv), gamma=FAKE + 2) == ALIGN
    # q output dtype: bf16, fp16 or fp32 (16-byte strides: multiples of 4 fp32)
    assert call_mla(pkv, mla_cache(pkv), qo_dtype=pkv.PKV_DTYPE_FP8_E4M3FN) == DTYPE
    assert call_mla(pkv, mla_cache(pkv), qo_dtype=9) == DTYPE
    assert call_mla(pkv, mla_cache(pkv), T=0, qo_dtype=pkv.PKV_DTYPE_F32,
                    qostride=4 * 64 + 4) == OK
    assert call_mla(pkv, mla_cache(pkv), qo_dtype=pkv.PKV_DTYPE_F32, qostride=4 * 64 + 2) == ALIGN
    # per-lane byte offsets are 32-bit: head strides above 2^27 elements refused
    lib = pkv.library()
    big = (1 << 27) + 8
    assert lib.mla_rope_rmsnorm_quant(FAKE, 4 * big, big, FAKE, 4 * big, big, FAKE, 576, FAKE, 2,
                                      16, 4, 64, 512, FAKE, 64, FAKE, 1e-6,
                                      ctypes.byref(mla_cache(pkv)), 1, None, None) == UNSUP
    assert call_mla(pkv, mla_cache(pkv, slot_stride=584)) == ALIGN
    assert call_mla(pkv, mla_cache(pkv, data=FAKE + 8)) == ALIGN
    # nothing to do: accepted without a launch
    assert call_mla(pkv, mla_cache(pkv), T=0) == OK


def call_mla_inplace(pkv, cache, T=16, H=4, R=64, Dn=512, q=FAKE, qo=FAKE, layer=1, batch=2,
                     gamma=FAKE, qo_dtype=0):
    lib = pkv.library()
    cp = None if cache is None else ctypes.byref(cache)
    return lib.mla_rope_rmsnorm_inplace(qo, 4 * 64, R, q, 4 * 64, R, FAKE, batch, T, H, R, Dn,
                                        FAKE, 64, gamma, 1e-6, cp, layer,
                                        elem_types(pkv, q_out=qo_dtype), None)


def test_mla_inplace_validation(pkv):
    bf16 = dict(dtype=pkv.PKV_DTYPE_BF16, scale_mode=pkv.PKV_SCALE_NONE, scales=None,
                layer_stride=8 * 16 * 576)
    assert call_mla_inplace(pkv, None) == NULL
    # the rows are read from and written to a bf16 cache only
    assert call_mla_inplace(pkv, mla_cache(pkv)) == DTYPE
    assert call_mla_inplace(pkv, mla_cache(pkv, scale_mode=pkv.PKV_SCALE_PER_TOKEN)) == DTYPE
    assert call_mla_inplace(pkv, mla_cache(pkv, dtype=pkv.PKV_DTYPE_BF16)) == DTYPE
    assert call_mla_inplace(pkv, mla_cache(pkv, **bf16), T=0) == OK
    assert call_mla_inplace(pkv, mla_cache(pkv, **bf16), layer=2) == RANGE
    assert call_mla_inplace(pkv, mla_cache(pkv, **bf16), R=32) == SHAPE
    assert call_mla_inplace(pkv, mla_cache(pkv, **bf16), gamma=None) == NULL
    assert call_mla_inplace(pkv, mla_cache(pkv, **bf16), q=FAKE + 8) == ALIGN
    assert call_mla_inplace(pkv, mla_cache(pkv, **bf16, slot_stride=580)) == ALIGN
    assert call_mla_inplace(pkv, mla_cache(pkv, **bf16), qo_dtype=pkv.PKV_DTYPE_FP8_E4M3FN) == DTYPE


def call_plan(pkv, cache, plan=FAKE, T=16, batch=2, offsets=FAKE):
    lib = pkv.library()
    cp = None if cache is None else ctypes.byref(cache)
    return lib.pkv_token_plan(plan, offsets, batch, T, cp, None)


def test_token_plan_validation(pkv):
    assert call_plan(pkv, None) == NULL
    assert call_plan(pkv, mla_cache(pkv), plan=None) == NULL
    assert call_plan(pkv, mla_cache(pkv), offsets=None) == NULL
    assert call_plan(pkv, mla_cache(pkv, cache_lengths=None)) == NULL
    assert call_plan(pkv, mla_cache(pkv, page_table=None)) == NULL
    assert call_plan(pkv, mla_cache(pkv), plan=FAKE + 4) == ALIGN
    assert call_plan(pkv, mla_cache(pkv), batch=0) == SHAPE
    assert call_plan(pkv, mla_cache(pkv, page_size=0)) == SHAPE
    assert call_plan(pkv, mla_cache(pkv, num_pages=0)) == SHAPE
    assert call_plan(pkv, mla_cache(pkv, page_table_stride=0)) == SHAPE
    # the pool is not read: no data pointer needed; nothing to do for no tokens
    assert call_plan(pkv, mla_cache(pkv), T=0, batch=0) == OK
    assert call_plan(pkv, mla_cache(pkv, data=None), T=0) == OK


def call_kv_planned(pkv, cache, plan=FAKE, T=16, gamma=FAKE, glen=128, layer=1):
    lib = pkv.library()
    cp = None if cache is None else ctypes.byref(cache)
    return lib.rms_norm_kv_cache_paged_planned(cp, layer, gamma, glen, 1e-6, 0.0, T, plan, 1, 1,
                                               None, None)


def test_kv_norm_planned_validation(pkv):
    assert call_kv_planned(pkv, None) == NULL
    assert call_kv_planned(pkv, kcache(pkv), plan=None) == NULL
    assert call_kv_planned(pkv, kcache(pkv), plan=FAKE + 4) == ALIGN
    assert call_kv_planned(pkv, kcache(pkv), gamma=None) == NULL
    assert call_kv_planned(pkv, kcache(pkv), glen=0) == SHAPE
    assert call_kv_planned(pkv, kcache(pkv), glen=129) == SHAPE
    assert call_kv_planned(pkv, kcache(pkv), layer=2) == RANGE
    # placement comes from the plan: lengths and page table may be absent
    assert call_kv_planned(pkv, kcache(pkv, cache_lengths=None, page_table=None), T=0) == OK


def test_mla_inplace_planned_validation(pkv):
    lib = pkv.library()
    bf16 = dict(dtype=pkv.PKV_DTYPE_BF16, scale_mode=pkv.PKV_SCALE_NONE, scales=None,
                cache_lengths=None, page_table=None)

    def call(cache, plan=FAKE, T=16, layer=1):
        cp = None if cache is None else ctypes.byref(cache)
        return lib.mla_rope_rmsnorm_inplace_planned(FAKE, 4 * 64, 64, FAKE, 4 * 64, 64, plan, T,
                                                    4, 64, 512, FAKE, 64, FAKE, 1e-6, cp, layer,
                                                    None, None)
    assert call(None) == NULL
    assert call(mla_cache(pkv)) == DTYPE                 # an fp8 cache cannot hold the rows
    assert call(mla_cache(pkv, **bf16), plan=None) == NULL
    assert call(mla_cache(pkv, **bf16), plan=FAKE + 4) == ALIGN
    assert call(mla_cache(pkv, **bf16), layer=2) == RANGE
    assert call(mla_cache(pkv, **bf16), T=0) == OK


def test_planned_bindings_check_plan_rows(pkv):
    """The binding refuses a plan with fewer rows than tokens (the C entry
    points take no plan length) before any device pointer is used."""
    import torch
    plan = torch.zeros((3, 4), dtype=torch.int32)
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    lat = torch.zeros((4, 576), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pkv.mla_rope_rmsnorm_quant_planned(q, q, lat, plan, None, None, 1e-6, None, 0)
    with pytest.raises(ValueError):
        pkv.rms_norm_kv_cache_paged_planned(None, 0, None, 1e-6, 0.0, 4, plan)
    with pytest.raises(ValueError):
        pkv.mla_rope_rmsnorm_quant_planned(q, q, lat, torch.zeros((4, 3), dtype=torch.int32),
                                           None, None, 1e-6, None, 0)


def test_planned_bindings_check_plan_dtype_and_device(pkv):
    """A plan of 1- or 2-byte elements would let the plan kernel write 16
    bytes per token past its end, and a host tensor would hand the kernel a
    host pointer: every plan binding refuses both before calling the
    library."""
    import torch
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    lat = torch.zeros((4, 576), dtype=torch.bfloat16)
    offs = torch.zeros(3, dtype=torch.int32)
    calls = [
        lambda p: pkv.pkv_token_plan(p, offs, None),
        lambda p: pkv.mla_rope_rmsnorm_quant_planned(q, q, lat, p, None, None, 1e-6, None, 0),
        lambda p: pkv.mla_rope_rmsnorm_inplace_planned(q, q, p, None, None, 1e-6, None, 0),
        lambda p: pkv.rms_norm_kv_cache_paged_planned(None, 0, None, 1e-6, 0.0, 4, p),
    ]
    for call in calls:
        for dt in (torch.int8, torch.int16, torch.uint8, torch.float32, torch.int64):
            with pytest.raises(TypeError):
                call(torch.zeros((4, 4), dtype=dt))
        for dt in (torch.int32, torch.uint32):   # right type, host memory
            with pytest.raises(ValueError, match="must live on"):
                call(torch.zeros((4, 4), dtype=dt))


def call_noalloc(pkv, cache, T=16, H=4, R=64, Dn=512, offs=FAKE, batch=2, build=1, layer=1):
    lib = pkv.library()
    cp = None if cache is None else ctypes.byref(cache)
    return lib.mla_rope_rmsnorm_quant_noalloc(FAKE, 4 * 64, R, FAKE, 4 * 64, R, FAKE, Dn + R,
                                              offs, batch, T, H, R, Dn, FAKE, 64, FAKE, 1e-6,
                                              cp, layer, None, build, None)


def test_noalloc_validation(pkv):
    """The allocation-free entry point refuses on the host, before it touches
    any device: too many tokens for its plan array, and every refusal of the
    planned step and of the plan build."""
    assert call_noalloc(pkv, mla_cache(pkv), T=(1 << 18) + 1) == UNSUP
    assert call_noalloc(pkv, None) == NULL
    assert call_noalloc(pkv, mla_cache(pkv), R=48) == SHAPE
    assert call_noalloc(pkv, mla_cache(pkv, head_dim=560), R=48) == UNSUP
    assert call_noalloc(pkv, mla_cache(pkv), layer=2) == RANGE
    assert call_noalloc(pkv, mla_cache(pkv, dtype=pkv.PKV_DTYPE_BF16)) == DTYPE
    assert call_noalloc(pkv, mla_cache(pkv), offs=None) == NULL        # building needs offsets
    assert call_noalloc(pkv, mla_cache(pkv), batch=0) == SHAPE
    assert call_noalloc(pkv, mla_cache(pkv, page_table=None)) == NULL
    assert call_noalloc(pkv, mla_cache(pkv, cache_lengths=None)) == NULL


def call_mla_planned(pkv, cache, T=16, H=4, R=64, Dn=512, plan=FAKE, q=FAKE, lat=FAKE,
                     layer=1, max_seq=64, qo_dtype=0):
    lib = pkv.library()
    cp = None if cache is None else ctypes.byref(cache)
    return lib.mla_rope_rmsnorm_quant_planned(FAKE, 4 * 64, R, q, 4 * 64, R, lat, Dn + R, plan,
                                              T, H, R, Dn, FAKE, max_seq, FAKE, 1e-6, cp, layer,
                                              elem_types(pkv, q_out=qo_dtype), None)


def test_mla_planned_validation(pkv):
    assert call_mla_planned(pkv, None) == NULL
    assert call_mla_planned(pkv, mla_cache(pkv), plan=None) == NULL
    assert call_mla_planned(pkv, mla_cache(pkv), plan=FAKE + 8) == ALIGN
    assert call_mla_planned(pkv, mla_cache(pkv), lat=None) == NULL
    assert call_mla_planned(pkv, mla_cache(pkv), R=32) == SHAPE
    assert call_mla_planned(pkv, mla_cache(pkv), layer=2) == RANGE
    assert call_mla_planned(pkv, mla_cache(pkv), max_seq=0) == SHAPE
    assert call_mla_planned(pkv, mla_cache(pkv, scales=None)) == NULL
    assert call_mla_planned(pkv, mla_cache(pkv, dtype=pkv.PKV_DTYPE_BF16)) == DTYPE
    assert call_mla_planned(pkv, mla_cache(pkv), qo_dtype=9) == DTYPE
    # placement comes from the plan: lengths and page table may be absent
    assert call_mla_planned(pkv, mla_cache(pkv, cache_lengths=None, page_table=None),
                            T=0) == OK
    assert call_mla_planned(pkv, mla_cache(pkv), T=0) == OK


def kcache(pkv, **kw):
    base = dict(data=FAKE, dtype=pkv.PKV_DTYPE_BF16, num_layers=2, num_pages=8, page_size=16,
                num_heads=8, head_dim=128, layer_stride=8 * 16 * 8 * 128,
                page_stride=16 * 8 * 128, slot_stride=8 * 128, head_stride=128,
                cache_lengths=FAKE, page_table=FAKE, page_table_stride=4,
                scale_mode=pkv.PKV_SCALE_NONE, scales=None, error_count=None)
    base.update(kw)
    return pkv.PagedCache(**base)


def call_qk(pkv, cache, T=16, Hq=32, D=128, gamma=None, cols=0, layer=1, q=FAKE, pos=None,
            mrope=None, types=None):
    lib = pkv.library()
    cp = None if cache is None else ctypes.byref(cache)
    sec = None if mrope is None else (ctypes.c_uint32 * 3)(*mrope)
    return lib.qk_rope_paged_ragged(FAKE, Hq * D, D, q, Hq * D, D, T, Hq, D, FAKE, 2, cp, layer,
                                    FAKE, 4096, pos, sec, 1, gamma, cols, 1e-6, types, None)


def test_qk_validation(pkv):
    assert call_qk(pkv, None) == NULL
    assert call_qk(pkv, kcache(pkv, dtype=pkv.PKV_DTYPE_FP8_E4M3FN)) == DTYPE
    assert call_qk(pkv, kcache(pkv, scale_mode=pkv.PKV_SCALE_PER_TENSOR)) == DTYPE
    assert call_qk(pkv, kcache(pkv, head_dim=72), D=72) == UNSUP
    assert call_qk(pkv, kcache(pkv, head_dim=512), D=512) == UNSUP
    for d in (80, 96):  # heads padded to 16-lane groups
        assert call_qk(pkv, kcache(pkv, head_dim=d, head_stride=d, slot_stride=8 * d,
                                  page_stride=16 * 8 * d, layer_stride=8 * 16 * 8 * d),
                       D=d, T=0) == OK
    assert call_qk(pkv, kcache(pkv, head_dim=256, head_stride=256, slot_stride=8 * 256,
                              page_stride=16 * 8 * 256, layer_stride=8 * 16 * 8 * 256),
                   D=256, T=0) == OK
    assert call_qk(pkv, kcache(pkv), D=64) == SHAPE                    # q vs cache head_dim
    big = (1 << 27) + 8
    assert call_qk(pkv, kcache(pkv, head_stride=big, slot_stride=8 * big,
                              page_stride=16 * 8 * big, layer_stride=8 * 16 * 8 * big)) == UNSUP
    assert call_qk(pkv, kcache(pkv), gamma=FAKE, cols=129) == SHAPE
    assert call_qk(pkv, kcache(pkv), gamma=FAKE, cols=0) == SHAPE
    assert call_qk(pkv, kcache(pkv), layer=5) == RANGE
    assert call_qk(pkv, kcache(pkv), q=FAKE + 4) == ALIGN
    assert call_qk(pkv, kcache(pkv), gamma=FAKE + 2, cols=128) == ALIGN
    assert call_qk(pkv, kcache(pkv), T=0) == OK
    # fp8 K caches need their scales; multimodal sections must cover D/2 pairs
    assert call_qk(pkv, kcache(pkv, dtype=pkv.PKV_DTYPE_FP8_E4M3FN,
                               scale_mode=pkv.PKV_SCALE_PER_TOKEN, head_stride=128)) == NULL
    assert call_qk(pkv, kcache(pkv), mrope=(16, 24, 23), pos=FAKE) == SHAPE
    assert call_qk(pkv, kcache(pkv), mrope=(16, 24, 24), pos=None) == NULL
    assert call_qk(pkv, kcache(pkv), mrope=(16, 24, 24), pos=FAKE, T=0) == OK


def call_norm(pkv, cache, gamma_len=128, per_head=1, T=16, gamma=FAKE, types=None):
    lib = pkv.library()
    cp = None if cache is None else ctypes.byref(cache)
    return lib.rms_norm_kv_cache_paged(cp, 1, gamma, gamma_len, 1e-6, 0.0, T, FAKE, 2,
                                       per_head, 1, types, None)


def test_kv_norm_validation(pkv):
    assert call_norm(pkv, None) == NULL
    assert call_norm(pkv, kcache(pkv, dtype=pkv.PKV_DTYPE_FP8_E4M3FN)) == DTYPE
    assert call_norm(pkv, kcache(pkv), gamma_len=0) == SHAPE
    assert call_norm(pkv, kcache(pkv), gamma_len=129) == SHAPE
    # one statistic per token: every head of the token in one wave's registers
    assert call_norm(pkv, kcache(pkv), per_head=0, T=0) == OK
    # the per-token statistic takes any head count (17 heads: two register chunks)
    assert call_norm(pkv, kcache(pkv, num_heads=17, slot_stride=17 * 128, page_stride=16 * 17 * 128,
                                  layer_stride=8 * 16 * 17 * 128), per_head=0, T=0) == OK
    assert call_norm(pkv, kcache(pkv, num_heads=17, slot_stride=17 * 128, page_stride=16 * 17 * 128,
                                  layer_stride=8 * 16 * 17 * 128), per_head=1, T=0) == OK
    assert call_norm(pkv, kcache(pkv, head_dim=512), gamma_len=128) == UNSUP
    assert call_norm(pkv, kcache(pkv, head_dim=112), gamma_len=64) == UNSUP
    d96 = dict(head_dim=96, head_stride=96, slot_stride=17 * 96, page_stride=16 * 17 * 96,
               layer_stride=8 * 16 * 17 * 96, num_heads=17)
    assert call_norm(pkv, kcache(pkv, **d96), gamma_len=96, per_head=0, T=0) == OK
    assert call_norm(pkv, kcache(pkv, **d96), gamma_len=96, per_head=1, T=0) == OK
    assert call_norm(pkv, kcache(pkv), gamma=None) == NULL
    assert call_norm(pkv, kcache(pkv), gamma=FAKE + 2) == ALIGN
    assert call_norm(pkv, kcache(pkv), T=0) == OK
    fp8 = dict(dtype=pkv.PKV_DTYPE_FP8_E4M3FN, scale_mode=pkv.PKV_SCALE_PER_TENSOR)
    assert call_norm(pkv, kcache(pkv, **fp8)) == NULL                      # no scales
    lib = pkv.library()
    c8 = kcache(pkv, scales=FAKE, **fp8)
    assert lib.rms_norm_kv_cache_paged(ctypes.byref(c8), 1, FAKE, 128, 1e-6, 0.0, 16, FAKE, 2,
                                       1, 0, None, None) == UNSUP          # fp8 needs mbc


def test_element_types_validation(pkv):
    """pkv_elem_types: the accepted q / q-output pairs, freqs and gamma types
    of each entry point, and PKV_ERR_DTYPE for every other code (checked
    before anything else about the call, so T = 0 calls show it)."""
    BF, E8, F, H = pkv.PKV_DTYPE_BF16, pkv.PKV_DTYPE_FP8_E4M3FN, pkv.PKV_DTYPE_F32, pkv.PKV_DTYPE_F16
    for q in (BF, H):
        for qo in (BF, H, F):
            for fr in (BF, H, F):
                for g in (BF, H, F):
                    t = elem_types(pkv, q, qo, fr, g)
                    assert call_mla(pkv, mla_cache(pkv), T=0, types=t) == OK
    for bad in ((F, BF, F, BF), (E8, BF, F, BF), (BF, E8, F, BF), (BF, BF, E8, BF),
                (BF, BF, F, E8), (-1, BF, F, BF), (BF, BF, 5, BF), (BF, BF, F, 4)):
        assert call_mla(pkv, mla_cache(pkv), T=0, types=elem_types(pkv, *bad)) == DTYPE
    # fp16 output rows: strides in multiples of 8 elements
    assert call_mla(pkv, mla_cache(pkv), T=0, types=elem_types(pkv, q_out=H),
                    qostride=4 * 64 + 4) == OK
    assert call_mla(pkv, mla_cache(pkv), types=elem_types(pkv, q_out=H),
                    qostride=4 * 64 + 4) == ALIGN
    # Q/K RoPE: q and its output one 16-bit type; a K-norm gamma bf16
    for q in (BF, H):
        for fr in (BF, H, F):
            assert call_qk(pkv, kcache(pkv), T=0, types=elem_types(pkv, q, q, fr)) == OK
    assert call_qk(pkv, kcache(pkv), T=0, types=elem_types(pkv, H, BF)) == DTYPE
    assert call_qk(pkv, kcache(pkv), T=0, types=elem_types(pkv, F, F)) == DTYPE
    assert call_qk(pkv, kcache(pkv), T=0, types=elem_types(pkv, freqs=E8)) == DTYPE
    assert call_qk(pkv, kcache(pkv), T=0, types=elem_types(pkv, gamma=F)) == OK
    assert call_qk(pkv, kcache(pkv), T=0, gamma=FAKE, cols=128,
                   types=elem_types(pkv, gamma=F)) == DTYPE
    # K-cache norm: any of the three gamma types
    for g in (BF, H, F):
        assert call_norm(pkv, kcache(pkv), T=0, types=elem_types(pkv, gamma=g)) == OK
    assert call_norm(pkv, kcache(pkv), T=0, types=elem_types(pkv, gamma=E8)) == DTYPE


def test_binding_element_type_codes(pkv):
    """The binding's pkv_elem_types from tensor dtypes: bf16, fp16, fp32
    codes, the defaults for an absent tensor, -1 (refused by the library)
    for any other dtype."""
    import torch
    t = pkv._types(torch.zeros(1, dtype=torch.float16), torch.zeros(1, dtype=torch.float32),
                   torch.zeros(1, dtype=torch.bfloat16), torch.zeros(1, dtype=torch.int16))
    assert (t.q, t.q_out, t.freqs, t.gamma) == (pkv.PKV_DTYPE_F16, pkv.PKV_DTYPE_F32,
                                                pkv.PKV_DTYPE_BF16, -1)
    d = pkv._types()
    assert (d.q, d.q_out, d.freqs, d.gamma) == (pkv.PKV_DTYPE_BF16, pkv.PKV_DTYPE_BF16,
                                                pkv.PKV_DTYPE_F32, pkv.PKV_DTYPE_BF16)


def call_gather(pkv, cache, out_dtype=None, stride=576, rows=32, out=FAKE, oscales=FAKE,
                oscale=FAKE, layer=1):
    lib = pkv.library()
    cp = None if cache is None else ctypes.byref(cache)
    dt = pkv.PKV_DTYPE_BF16 if out_dtype is None else out_dtype
    return lib.mla_gather_latent_paged(out, dt, stride, oscales, oscale, FAKE, 2, rows, cp,
                                       layer, None)


def test_gather_validation(pkv):
    c = lambda **kw: mla_cache(pkv, cache_lengths=None, **kw)  # noqa: E731
    assert call_gather(pkv, None) == NULL
    assert call_gather(pkv, c(), out_dtype=9) == DTYPE
    assert call_gather(pkv, c(scale_mode=pkv.PKV_SCALE_NONE)) == DTYPE
    assert call_gather(pkv, c(dtype=pkv.PKV_DTYPE_BF16)) == DTYPE      # bf16 needs NONE
    assert call_gather(pkv, c(num_heads=2)) == SHAPE
    assert call_gather(pkv, c(head_dim=100)) == ALIGN
    assert call_gather(pkv, c(head_dim=2048, slot_stride=2048)) == UNSUP
    assert call_gather(pkv, c(), stride=500) == SHAPE
    assert call_gather(pkv, c(), stride=580) == ALIGN
    assert call_gather(pkv, c(), layer=2) == RANGE
    assert call_gather(pkv, c(), out=None) == NULL
    assert call_gather(pkv, c(scales=None)) == NULL
    assert call_gather(pkv, c(scale_mode=pkv.PKV_SCALE_PER_TOKEN),
                       out_dtype=pkv.PKV_DTYPE_FP8_E4M3FN, oscales=None) == NULL
    assert call_gather(pkv, c(), out=FAKE + 8) == ALIGN
    assert call_gather(pkv, c(), rows=0) == OK


def test_product_path_does_not_reference_the_oracle():
    """The HIP library and its binding never load or import the oracle."""
    pkg = os.path.join(ROOT, "paged_kv_cache_wavefront_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text, os.path.join(dirpath, f)


def test_descriptor_keeps_its_tensors_alive(pkv):
    """A descriptor stores raw pointers; it must hold references to the tensors
    so that temporaries passed to paged_cache() are not freed and reused."""
    import gc
    import weakref

    import torch
    pt = torch.zeros((2, 4), dtype=torch.int32)
    ref = weakref.ref(pt)
    desc = pkv.paged_cache(torch.zeros((1, 2, 4, 1, 576), dtype=torch.uint8), None, pt,
                           pkv.PKV_SCALE_PER_TENSOR, torch.ones(1))
    del pt
    gc.collect()
    assert ref() is not None and desc.page_table == ref().data_ptr()


def test_headers_compile_as_c_and_cxx(tmp_path):
    """The public headers are plain C (C99) and C++ (17), warning-free, and
    declare the entry points with the argument lists the binding uses."""
    src = tmp_path / "use.c"
    T = "const pkv_elem_types*"
    src.write_text('#include <string.h>\n#include "pkv.h"\n#include "pkv_bench.h"\n'
                   "int main(void) {\n"
                   "  pkv_paged_cache c;\n"
                   "  memset(&c, 0, sizeof c);\n"
                   "  pkv_elem_types t = {PKV_DTYPE_F16, PKV_DTYPE_F32, PKV_DTYPE_BF16,"
                   " PKV_DTYPE_F16};\n"
                   "  (void)c; (void)t;\n"
                   "  int (*f1)(void*, int64_t, int64_t, const void*, int64_t, int64_t, const void*,"
                   " int64_t, const uint32_t*, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t,"
                   " const void*, uint32_t, const void*, float, const pkv_paged_cache*, uint32_t,"
                   f" {T}, void*) = mla_rope_rmsnorm_quant;\n"
                   "  int (*f10)(void*, int64_t, int64_t, const void*, int64_t, int64_t,"
                   " const uint32_t*, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t,"
                   " const void*, uint32_t, const void*, float, const pkv_paged_cache*, uint32_t,"
                   f" {T}, void*) = mla_rope_rmsnorm_inplace;\n"
                   "  const char* (*f2)(int) = pkv_status_string;\n"
                   "  int (*f4)(uint32_t*, const uint32_t*, uint32_t, uint32_t,"
                   " const pkv_paged_cache*, void*) = pkv_token_plan;\n"
                   "  int (*f5)(void*, int64_t, int64_t, const void*, int64_t, int64_t,"
                   " const void*, int64_t, const uint32_t*, uint32_t, uint32_t, uint32_t,"
                   " uint32_t, const void*, uint32_t, const void*, float,"
                   f" const pkv_paged_cache*, uint32_t, {T}, void*) ="
                   " mla_rope_rmsnorm_quant_planned;\n"
                   "  int (*f6)(const pkv_paged_cache*, uint32_t, const void*, uint32_t, float,"
                   f" float, uint32_t, const uint32_t*, int, int, {T}, void*) ="
                   " rms_norm_kv_cache_paged_planned;\n"
                   "  int (*f11)(const pkv_paged_cache*, uint32_t, const void*, uint32_t, float,"
                   f" float, uint32_t, const uint32_t*, uint32_t, int, int, {T}, void*) ="
                   " rms_norm_kv_cache_paged;\n"
                   "  int (*f12)(void*, int64_t, int64_t, const void*, int64_t, int64_t, uint32_t,"
                   " uint32_t, uint32_t, const uint32_t*, uint32_t, const pkv_paged_cache*,"
                   " uint32_t, const void*, uint32_t, const uint32_t*, const uint32_t*, int,"
                   f" const void*, uint32_t, float, {T}, void*) = qk_rope_paged_ragged;\n"
                   "  int (*f13)(void*, int32_t, int64_t, float*, const float*, const uint32_t*,"
                   " uint32_t, uint32_t, const pkv_paged_cache*, uint32_t, void*) ="
                   " mla_gather_latent_paged;\n"
                   "  int (*f7)(void*, int64_t, int64_t, const void*, int64_t, int64_t,"
                   " const uint32_t*, uint32_t, uint32_t, uint32_t, uint32_t, const void*,"
                   f" uint32_t, const void*, float, const pkv_paged_cache*, uint32_t, {T},"
                   " void*) = mla_rope_rmsnorm_inplace_planned;\n"
                   "  int (*f9)(void*, int64_t, int64_t, const void*, int64_t, int64_t,"
                   " const void*, int64_t, const uint32_t*, uint32_t, uint32_t, uint32_t,"
                   " uint32_t, uint32_t, const void*, uint32_t, const void*, float,"
                   f" const pkv_paged_cache*, uint32_t, {T}, int, void*) ="
                   " mla_rope_rmsnorm_quant_noalloc;\n"
                   "  (void)f4; (void)f5; (void)f6; (void)f7; (void)f9; (void)f10; (void)f11;\n"
                   "  (void)f12; (void)f13;\n"
                   "  int (*f3)(const void*, void*, uint64_t, uint32_t, void*) = pkv_stream_copy;\n"
                   "  int (*f8)(const void*, uint64_t, void*, uint64_t, uint32_t, void*) ="
                   " pkv_stream_mix;\n"
                   "  (void)f1; (void)f2; (void)f3; (void)f8;\n"
                   "  return 0;\n}\n")
    inc = os.path.join(ROOT, "include")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-fsyntax-only", "-I", inc, str(src)], check=True)
    cxx = tmp_path / "use.cpp"
    cxx.write_text(src.read_text())
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                    "-I", inc, str(cxx)], check=True)
