"""GPU parity over the element types the pages parameterise (q_rope / q_proj
dtype, out_rope_dtype, freq_dtype, gamma_dtype): fp16 q, bf16 / fp16 / fp32 q
outputs, bf16 / fp16 freqs_cis, fp16 / fp32 gamma, through the C ABI, against
the oracle run on the same typed inputs.  The bars are those of the bf16
path, per output type (gpu_helpers.check_q)."""
import numpy as np
import pytest
import torch

import gpu_helpers as gh
import oracle_pins
import workloads

pytestmark = pytest.mark.gpu

OUT_TYPES = {"bf16": np.uint16, "f16": np.float16, "f32": np.float32}


def _say(*a):
    print(*a, flush=True)


def _mla(orc, case, q_out, layout="dense", floor=2):
    _say(f"[types] case={case.name} seed={case.seed} T={case.T} H={case.H} q={case.q.dtype} "
         f"freqs={case.freqs.dtype} gamma={case.gamma.dtype} out={np.dtype(q_out)} "
         f"layout={layout}")
    dev = gh.MlaDevice(case, layout, q_out_dtype=q_out)
    dev.run()
    gpu = dev.results()
    assert gpu[3] == 0, f"{gpu[3]} tokens skipped"
    stats = gh.compare_mla(case, gpu, gh.oracle_mla(orc, case, q_out_dtype=q_out),
                           small_case_floor=floor)
    _say(f"[types] {case.name}: {stats}")
    return gpu


@pytest.mark.parametrize("out", list(OUT_TYPES))
@pytest.mark.parametrize("idx", range(5))
def test_mla_small_type_cases(orc, idx, out):
    """The oracle's pinned element-type cases (fp16 / bf16 q, fp32 / bf16 /
    fp16 freqs, bf16 / fp16 / fp32 gamma; fp8 tensor / token and bf16
    caches), each with every q output type."""
    case = list(oracle_pins.dtype_mla_cases())[idx]
    _mla(orc, case, OUT_TYPES[out])


@pytest.mark.parametrize("out", ["f16", "f32", "bf16"])
def test_mla_fp16_q_many_waves(orc, out):
    """fp16 q of 128 heads (four head chunks per token), bf16 freqs, fp32
    gamma, per-token fp8 cache: a ragged batch of about 1600 tokens."""
    rng = workloads.make_rng(6100)
    new = rng.integers(0, 400, size=8, endpoint=True)
    prior = rng.integers(0, 600, size=8, endpoint=True)
    case = workloads.build_mla("mla_f16q_h128", 6100, new, prior, H=128, page_size=64,
                               max_seq_len=2048, spare_pages=4, scale_mode="per_token",
                               outlier_p=0.01, rng=rng, q_dtype="f16", freq_dtype="bf16",
                               gamma_dtype="f32")
    _mla(orc, case, OUT_TYPES[out], floor=0)


@pytest.mark.parametrize("R,Dn", [(32, 256), (128, 512)])
def test_mla_types_other_dims(orc, R, Dn):
    """fp16 q, fp16 freqs and fp16 gamma at rope_dim 32 and 128, bf16 output."""
    rng = workloads.make_rng(6200 + R)
    new = rng.integers(0, 120, size=7, endpoint=True)
    prior = rng.integers(0, 200, size=7, endpoint=True)
    case = workloads.build_mla(f"mla_types_r{R}", 6200 + R, new, prior, H=40, R=R, Dn=Dn,
                               page_size=16, max_seq_len=512, spare_pages=4,
                               scale_mode="per_tensor", tensor_scale=0.05, rng=rng,
                               q_dtype="f16", freq_dtype="f16", gamma_dtype="f16")
    _mla(orc, case, np.uint16)


def test_mla_types_strided_views(orc):
    """fp16 q read from, and an fp32 output written into, the rope slices of
    wider [T, H, 2R] buffers."""
    case = workloads.build_mla("mla_types_strided", 6300, [3, 9, 0, 14], [5, 0, 2, 30], H=20,
                               page_size=8, max_seq_len=64, spare_pages=3,
                               scale_mode="per_token", q_dtype="f16", freq_dtype="bf16",
                               gamma_dtype="bf16")
    _mla(orc, case, np.float32, layout="strided")


def test_mla_types_inplace_and_planned(orc):
    """The in-place form (bf16 cache) with fp16 q and fp16 gamma, and the
    planned form with fp16 q and fp32 freqs, each against the oracle."""
    import paged_kv_cache_wavefront_amd as pkv
    rng = workloads.make_rng(6400)
    new = rng.integers(1, 60, size=6, endpoint=True)
    prior = rng.integers(0, 100, size=6, endpoint=True)
    case = workloads.build_mla("mla_types_inplace", 6400, new, prior, H=24, page_size=16,
                               max_seq_len=256, spare_pages=4, cache_dtype="bf16",
                               scale_mode="none", rng=rng, q_dtype="f16", freq_dtype="f16",
                               gamma_dtype="f16")
    _say(f"[types] in place T={case.T}")
    dev = gh.MlaDevice(case, q_out_dtype=np.float16)
    dev.place_rows()
    dev.run_inplace()
    q_o = np.zeros(case.q.shape, np.float16)
    cache_o = oracle_pins.place_latent_rows(case)
    orc.mla_rope_rmsnorm_inplace(q_o, case.q, case.row_offsets, case.cache_lengths,
                                 case.page_table, case.freqs, case.gamma, case.epsilon, cache_o,
                                 case.layer_idx)
    q_g, cache_g, _, skipped = dev.results()
    assert skipped == 0
    gh.check_q(q_g, q_o, "in-place q (fp16)")
    gh.check_bf16(cache_g, cache_o, "in-place cache")

    fcase = workloads.build_mla("mla_types_planned", 6401, new, prior, H=24, page_size=16,
                                max_seq_len=256, spare_pages=4, scale_mode="per_token",
                                rng=workloads.make_rng(6401), q_dtype="f16")
    _say(f"[types] planned T={fcase.T}")
    fdev = gh.MlaDevice(fcase, q_out_dtype=np.uint16)
    plan = torch.empty((fcase.T, 4), dtype=torch.int32, device="cuda")
    pkv.pkv_token_plan(plan, fdev.offsets, fdev.desc)
    pkv.mla_rope_rmsnorm_quant_planned(fdev.q_out, fdev.q_in, fdev.latent, plan, fdev.freqs,
                                       fdev.gamma, fcase.epsilon, fdev.desc, fcase.layer_idx)
    gh.compare_mla(fcase, fdev.results(), gh.oracle_mla(orc, fcase, q_out_dtype=np.uint16),
                   small_case_floor=2)


def _qk(orc, case, with_norm):
    from test_parity_qk import check_k_rows, oracle_qk
    _say(f"[types-qk] case={case.name} T={case.T} q={case.q.dtype} freqs={case.freqs.dtype} "
         f"norm={with_norm}")
    dev = gh.QkDevice(case)
    dev.rope(with_norm)
    q = gh.host_elem(dev.q_out)
    k, _ = dev.k_host()
    assert int(dev.error_count.item()) == 0
    q_o, k_o = oracle_qk(orc, case, with_norm)
    assert q.dtype == q_o.dtype
    stats = {"q": gh.check_q(q, q_o, f"q ({q_o.dtype})", floor=2),
             "k": check_k_rows(case, k, k_o, "k", case.gamma.size if with_norm else None,
                               max_frac=max(gh.BF16_MAX_DIFF_FRAC, 2 / max(k.size, 1)))}
    _say(f"[types-qk] {case.name}: {stats}")


@pytest.mark.parametrize("with_norm", [True, False])
@pytest.mark.parametrize("idx", range(3))
def test_qk_type_cases(orc, idx, with_norm):
    """fp16 Q with bf16 / fp16 freqs, bf16 Q with fp16 freqs; both rope styles,
    head_dim 128, 64 and 96."""
    _qk(orc, list(oracle_pins.dtype_qk_cases())[idx], with_norm)


def test_qk_fp16_llama_shape(orc):
    """The Llama-shaped batch (19k tokens, Q 32 x 128, K 8 x 128, interleaved,
    position ids, fused K norm) with fp16 Q and bf16 freqs."""
    rng = workloads.make_rng(1007)
    new = rng.integers(1, 1024, size=32, endpoint=True)
    prior = rng.integers(0, 1023, size=32, endpoint=True)
    case = workloads.build_qk("qk_generic_f16", 1007, new, prior, Hq=32, Hkv=8, D=128,
                              page_size=16, max_seq_len=131072, theta=500000.0,
                              interleaved=True, with_position_ids=True, norm_cols=128, rng=rng,
                              q_dtype="f16", freq_dtype="bf16")
    _qk(orc, case, True)


@pytest.mark.parametrize("freq", ["bf16", "f16"])
def test_qk_types_mrope_fp8_k(orc, freq):
    """Multimodal RoPE (per-pair cos / sin from three position rows, read as
    16-bit freqs) with fp16 Q and a per-token fp8 K cache."""
    from test_parity_qk import run_qk_fp8
    rng = workloads.make_rng(6500)
    new = rng.integers(20, 150, size=5, endpoint=True)
    prior = rng.integers(0, 100, size=5, endpoint=True)
    case = workloads.build_qk(f"mrope_types_{freq}", 6500, new, prior, Hq=8, Hkv=2, D=128,
                              page_size=16, max_seq_len=2048, theta=1000000.0,
                              interleaved=False, with_position_ids=True, norm_cols=96, rng=rng,
                              mrope_section=(16, 24, 24), k_dtype="fp8",
                              k_scale_mode="per_token", q_dtype="f16", freq_dtype=freq)
    run_qk_fp8(orc, case, True)


@pytest.mark.parametrize("per_head", [True, False])
@pytest.mark.parametrize("gdt", ["f16", "f32"])
def test_kv_norm_gamma_types(orc, gdt, per_head):
    """The K-cache norm with fp16 / fp32 gamma (+ weight_offset) over a partial
    width (100 of 128 columns; the tail chunk read element by element)."""
    case = list(oracle_pins.small_qk_cases())[0]
    rng = np.random.Generator(np.random.PCG64(78))
    g32 = rng.uniform(0.5, 1.5, 100).astype(np.float32)
    gamma = g32.astype(np.float16) if gdt == "f16" else g32
    _say(f"[types-kvnorm] gamma={gamma.dtype} per_head={per_head} T={case.T}")
    dev = gh.QkDevice(case)
    dev.kv_norm(gh.dev_elem(gamma), 0.25, case.T, True, per_head)
    k, _ = dev.k_host()
    assert int(dev.error_count.item()) == 0
    k_o = case.k_cache.copy()
    orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                case.page_table, gamma, case.epsilon, 0.25, case.T, True,
                                per_head_norm=per_head)
    rows = gh.written_k_rows(case)
    assert np.array_equal(k[~rows], case.k_cache[~rows])
    _say(f"[types-kvnorm] {gh.check_bf16(k[rows], k_o[rows], 'k', max_frac=2e-3)}")


def test_kv_norm_fp32_gamma_fp8_per_token(orc):
    """fp32 gamma on a per-token fp8 K cache (the head re-encoded with a fresh
    scale)."""
    from test_parity_qk import check_fp8_k
    case = list(oracle_pins.small_qk_fp8_cases())[1]
    assert case.k_scale_mode == "per_token"
    D = case.k_cache.shape[-1]
    gamma = np.random.Generator(np.random.PCG64(79)).uniform(0.5, 1.5, D).astype(np.float32)
    _say(f"[types-kvnorm8] case={case.name} T={case.T}")
    dev = gh.QkDevice(case)
    dev.kv_norm(gh.dev_elem(gamma), 0.0, case.T, True)
    k, ks = dev.k_host()
    assert int(dev.error_count.item()) == 0
    k_o = case.k_cache.copy()
    ks_o = case.k_scales.copy()
    with orc.fp8_probe(k_o) as pre:
        orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                    case.page_table, gamma, case.epsilon, 0.0, case.T, True,
                                    case.k_scale_mode, ks_o)
    _say(f"[types-kvnorm8] {check_fp8_k(case, k, ks, k_o, ks_o, pre, 'kvnorm fp8 f32 gamma')}")


def test_binding_refuses_other_dtypes(orc):
    """A q tensor of a type the library does not take (fp32 q) comes back as
    PKV_ERR_DTYPE through the binding, before any launch."""
    import paged_kv_cache_wavefront_amd as pkv
    case = list(oracle_pins.dtype_mla_cases())[0]
    dev = gh.MlaDevice(case)
    q32 = dev.q_in.float()
    with pytest.raises(pkv.PkvError) as e:
        pkv.mla_rope_rmsnorm_quant(dev.q_out, q32, dev.latent, dev.offsets, dev.freqs, dev.gamma,
                                   case.epsilon, dev.desc, case.layer_idx)
    assert e.value.status == 3
    _, cache, _, _ = dev.results()
    assert np.array_equal(cache, case.cache)
