"""GPU parity of qk_rope_paged_ragged and rms_norm_kv_cache_paged against the
CPU oracle, through the C ABI: the Llama-shaped paged-ragged workload at full
size (fused per-head K norm, and the two-call form), both rope styles, with
and without position ids, head_dim 64 and 128, partial norm widths,
weight_offset, both cast orders, and determinism."""
import numpy as np
import pytest
import torch

import gpu_helpers as gh
import oracle_pins
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def bf16_f64(u):
    return oracle_pins.bf16_to_f64(u)


def pair_magnitude(v: np.ndarray, interleaved: bool) -> np.ndarray:
    """|(a, b)| of the rotation pair each element belongs to (last axis)."""
    out = np.empty_like(v)
    if interleaved:
        m = np.hypot(v[..., 0::2], v[..., 1::2])
        out[..., 0::2], out[..., 1::2] = m, m
    else:
        h = v.shape[-1] // 2
        m = np.hypot(v[..., :h], v[..., h:])
        out[..., :h], out[..., h:] = m, m
    return out


def mixed_pair_columns(D: int, norm_cols, interleaved: bool) -> np.ndarray:
    """Boolean [D]: columns whose rotation pair has exactly one member among
    the first norm_cols (normalised) columns.  None: no K norm, no column."""
    cols = np.arange(D)
    if norm_cols is None:
        return np.zeros(D, bool)
    partner = cols ^ 1 if interleaved else (cols + D // 2) % D
    return (cols < norm_cols) != (partner < norm_cols)


def check_k_rows(case, k_gpu, k_orc, what, norm_cols=None, max_ulp=1, max_frac=None):
    """Rows the new tokens own: within max_ulp bf16 ulps of the oracle, and at
    most max_frac of the values differ at all; every other element bit-exact
    against the starting pool.  With the fused K norm over the first
    norm_cols columns, a pair that mixes a normalised and a plain member
    carries the fp32 normalisation of one member into the rotation, so there
    (only) the bound widens by NORM_SLACK x the pair's magnitude; a pair
    with both members normalised takes r after the rotation and keeps the
    plain bound."""
    rows = gh.written_k_rows(case)
    assert np.array_equal(k_gpu[~rows], case.k_cache[~rows]), f"{what}: untouched rows changed"
    g, o = k_gpu[rows], k_orc[rows]
    d = gh.bf16_ulp_diff(g, o)
    frac = float((d != 0).sum() / max(d.size, 1))
    mixed = mixed_pair_columns(g.shape[-1], norm_cols, case.interleaved)
    plain_max = int(d[..., ~mixed].max(initial=0))
    assert plain_max <= max_ulp, f"{what}: max ulp {plain_max} outside mixed pairs"
    stats = dict(max_ulp=int(d.max(initial=0)), diff_frac=frac, n=d.size,
                 mixed_cols=int(mixed.sum()))
    if mixed.any():
        of = bf16_f64(o)
        allowed = (oracle_pins.ulp_bf16(of) * max_ulp +
                   NORM_SLACK * pair_magnitude(of, case.interleaved))[..., mixed]
        err = np.abs(bf16_f64(g) - of)[..., mixed]
        worst = float(np.max(err / allowed, initial=0))
        stats["mixed_worst_frac_of_bound"] = worst
        assert worst <= 1.0, f"{what}: mixed-pair error {worst:.3f} x allowed"
    assert frac <= (gh.BF16_MAX_DIFF_FRAC if max_frac is None else max_frac), \
        f"{what}: diff frac {frac}"
    return stats


# A pair with one normalised and one plain member: the normalised member is
# scaled by its fp32 r before the rotation (relative error <= ~1.1e-6: 8-term
# lane sums + 4-level DPP tree, sqrt, divide, product), which cancellation in
# the rotation can turn into an absolute error of that size times the pair
# magnitude; 2^-18 (3.8e-6) of the pair magnitude covers it with margin.
NORM_SLACK = 2.0 ** -18


def oracle_qk(orc, case, with_norm, with_scales=False):
    """(q_out, k) or, with_scales, (q_out, k, k_scales, pre): ``pre`` holds the
    binary64 value each fp8 K code was rounded from (None: bf16 K)."""
    import contextlib
    q_out = np.zeros_like(case.q)
    k = case.k_cache.copy()
    ks = None if case.k_scales is None else case.k_scales.copy()
    probe = orc.fp8_probe(k) if k.dtype == np.uint8 else contextlib.nullcontext()
    with probe as pre:
        orc.qk_rope_paged_ragged(q_out, case.q, case.row_offsets, case.cache_lengths,
                                 case.page_table, k, case.layer_idx, case.freqs,
                                 case.position_ids, case.interleaved,
                                 case.gamma if with_norm else None, case.epsilon,
                                 case.k_scale_mode, ks, mrope_section=case.mrope_section)
    return (q_out, k, ks, pre) if with_scales else (q_out, k)


def check_fp8_k(case, k_gpu, ks_gpu, k_orc, ks_orc, pre, what, norm_cols=None):
    """fp8 K rows: codes as the oracle's but for near-ties (gh.check_fp8).
    The rotation runs on code x gamma, exact in fp32, and takes the head's
    scale and r after it, so the kernel's value before rounding is
    relative-accurate: no allowance for cancellation, except in a pair that
    mixes a normalised and a plain member (fused K norm over the first
    norm_cols columns), whose normalised member takes r before the rotation;
    there the near-tie window widens by NORM_SLACK x the pair's magnitude.
    Per-token scales within 1e-5 relative; everything else bit-exact."""
    rows = gh.written_k_rows(case)
    assert np.array_equal(k_gpu[~rows], case.k_cache[~rows]), f"{what}: untouched rows changed"
    slack = None
    mixed = mixed_pair_columns(k_gpu.shape[-1], norm_cols, case.interleaved)
    if mixed.any():
        p = np.where(np.isnan(pre[rows]), 0.0, pre[rows])
        slack = np.where(mixed, NORM_SLACK * pair_magnitude(p, case.interleaved), 0.0)
    stats = gh.check_fp8(k_gpu[rows], k_orc[rows], pre[rows], what, slack)
    if case.k_scale_mode == "per_token":
        assert np.array_equal(ks_gpu[~rows].view(np.uint32), case.k_scales[~rows].view(np.uint32))
        sg, so = ks_gpu[rows].astype(np.float64), ks_orc[rows].astype(np.float64)
        rel = np.abs(sg - so) / np.maximum(np.abs(so), 1e-30)
        stats["scale_max_rel"] = float(rel.max(initial=0))
        assert stats["scale_max_rel"] <= gh.SCALE_MAX_REL, f"{what}: {stats}"
    else:
        assert np.array_equal(ks_gpu, case.k_scales)
    return stats


def run_qk_fp8(orc, case, with_norm):
    _say(f"[qk8] case={case.name} T={case.T} mode={case.k_scale_mode} norm={with_norm}")
    dev = gh.QkDevice(case)
    dev.rope(with_norm)
    q = gh.host_elem(dev.q_out)
    k, ks = dev.k_host()
    assert int(dev.error_count.item()) == 0
    q_o, k_o, ks_o, pre = oracle_qk(orc, case, with_norm, with_scales=True)
    stats = {"q": gh.check_q(q, q_o, f"q ({q_o.dtype})"),
             "k": check_fp8_k(case, k, ks, k_o, ks_o, pre, "k",
                              case.gamma.size if with_norm else None)}
    _say(f"[qk8] {case.name}: {stats}")


@pytest.mark.parametrize("idx", range(2))
@pytest.mark.parametrize("with_norm", [True, False])
def test_fp8_k_small(orc, idx, with_norm):
    run_qk_fp8(orc, list(oracle_pins.small_qk_fp8_cases())[idx], with_norm)


@pytest.mark.parametrize("mode", ["per_tensor", "per_token"])
def test_fp8_k_llama_shape(orc, mode):
    """The Llama-shaped batch (19k tokens, Q 32 x 128, K 8 x 128, interleaved,
    position ids, fused K norm) with an fp8 K cache."""
    rng = workloads.make_rng(1005)
    new = rng.integers(1, 1024, size=32, endpoint=True)
    prior = rng.integers(0, 1023, size=32, endpoint=True)
    case = workloads.build_qk(f"qk_generic_fp8_{mode}", 1005, new, prior, Hq=32, Hkv=8, D=128,
                              page_size=16, max_seq_len=131072, theta=500000.0,
                              interleaved=True, with_position_ids=True, norm_cols=128, rng=rng,
                              k_dtype="fp8", k_scale_mode=mode)
    run_qk_fp8(orc, case, True)


@pytest.mark.parametrize("idx", range(2))
def test_mrope_small(orc, idx):
    case = list(oracle_pins.small_mrope_cases())[idx]
    run_qk(orc, case, case.gamma is not None)


def test_mrope_vision_batch(orc):
    """A Qwen2-VL-like batch: 8 requests of up to 900 tokens, Q 16 x 128, K 2 x
    128, sections (16, 24, 24), three random position rows below 4096."""
    rng = workloads.make_rng(5301)
    new = rng.integers(100, 900, size=8, endpoint=True)
    prior = rng.integers(0, 200, size=8, endpoint=True)
    case = workloads.build_qk("mrope_vision", 5301, new, prior, Hq=16, Hkv=2, D=128,
                              page_size=16, max_seq_len=4096, theta=1000000.0,
                              interleaved=False, with_position_ids=True, norm_cols=None,
                              rng=rng, mrope_section=(16, 24, 24))
    run_qk(orc, case, False)


@pytest.mark.parametrize("D", [256, 96, 80])
@pytest.mark.parametrize("mode", ["per_tensor", "per_token"])
def test_fp8_k_head_dim_256(orc, mode, D):
    """fp8 K cache with 256-wide heads (32 lanes per head: the rotate-half
    partner and the per-token max cross 16-lane rows), and with 96- and
    80-wide heads (padded 16-lane groups), fused K norm."""
    rng = workloads.make_rng(5400)
    new = rng.integers(1, 60, size=7, endpoint=True)
    prior = rng.integers(0, 80, size=7, endpoint=True)
    case = workloads.build_qk(f"qk_fp8_d{D}_{mode}", 5400, new, prior, Hq=6, Hkv=3, D=D,
                              page_size=16, max_seq_len=1024, theta=10000.0,
                              interleaved=False, with_position_ids=True, norm_cols=D, rng=rng,
                              k_dtype="fp8", k_scale_mode=mode)
    run_qk_fp8(orc, case, True)


@pytest.mark.parametrize("D", [256, 96, 80])
@pytest.mark.parametrize("per_head", [True, False])
def test_kv_norm_head_dim_256(orc, per_head, D):
    """In-place K norm with 256-wide heads, and with 96- and 80-wide heads
    (padded lane groups; 8 heads fit one wave's statistic either way)."""
    rng = workloads.make_rng(5401)
    new = rng.integers(1, 40, size=6, endpoint=True)
    prior = rng.integers(0, 60, size=6, endpoint=True)
    case = workloads.build_qk(f"kvnorm_d{D}", 5401, new, prior, Hq=2, Hkv=8, D=D, page_size=8,
                              max_seq_len=256, theta=10000.0, interleaved=False,
                              with_position_ids=False, norm_cols=None, rng=rng)
    gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, D).astype(np.float32))
    _say(f"[kvnorm{D}] T={case.T} per_head={per_head}")
    dev = gh.QkDevice(case)
    dev.kv_norm(gh.dev_bf16(gamma), 0.0, case.T, True, per_head)
    k = gh.host_bf16(dev.k)
    assert int(dev.error_count.item()) == 0
    k_o = case.k_cache.copy()
    orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                case.page_table, gamma, case.epsilon, 0.0, case.T, True,
                                per_head_norm=per_head)
    rows = gh.written_k_rows(case)
    assert np.array_equal(k[~rows], case.k_cache[~rows])
    _say(f"[kvnorm{D}] {gh.check_bf16(k[rows], k_o[rows], 'k')}")


@pytest.mark.parametrize("mode,with_norm", [("per_tensor", False), ("per_token", True)])
def test_mrope_fp8_k(orc, mode, with_norm):
    """Multimodal RoPE with an fp8 K cache (both scale modes; the per-token
    case with the fused K norm): the features combine as their oracles do."""
    rng = workloads.make_rng(5302)
    new = rng.integers(20, 200, size=6, endpoint=True)
    prior = rng.integers(0, 100, size=6, endpoint=True)
    case = workloads.build_qk(f"mrope_fp8_{mode}", 5302, new, prior, Hq=8, Hkv=2, D=128,
                              page_size=16, max_seq_len=2048, theta=1000000.0,
                              interleaved=False, with_position_ids=True,
                              norm_cols=96 if with_norm else None, rng=rng,
                              mrope_section=(16, 24, 24), k_dtype="fp8", k_scale_mode=mode)
    run_qk_fp8(orc, case, with_norm)


@pytest.mark.parametrize("idx", range(2))
def test_fp8_kv_norm(orc, idx):
    case = list(oracle_pins.small_qk_fp8_cases())[idx]
    total = case.T - 2
    _say(f"[kvnorm8] case={case.name} mode={case.k_scale_mode} total={total}")
    dev = gh.QkDevice(case)
    dev.kv_norm(dev.gamma, 0.25, total, True)
    k, ks = dev.k_host()
    assert int(dev.error_count.item()) == 0
    k_o = case.k_cache.copy()
    ks_o = case.k_scales.copy()
    with orc.fp8_probe(k_o) as pre:
        orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                    case.page_table, case.gamma, case.epsilon, 0.25, total, True,
                                    case.k_scale_mode, ks_o)
    stats = check_fp8_k(case, k, ks, k_o, ks_o, pre, "kvnorm fp8")
    _say(f"[kvnorm8] {case.name}: {stats}")


@pytest.mark.parametrize("kind", ["bf16_mbc", "bf16_two_roundings", "bf16_32_heads",
                                  "fp8_per_tensor", "fp8_per_token"])
def test_kv_norm_per_token_statistic(orc, kind):
    """per_head_norm=False: one statistic over the first len(gamma) columns of
    all of a token's heads."""
    if kind == "bf16_32_heads":
        # the most heads one wave holds at head_dim 64: 4 groups of 8
        rng = workloads.make_rng(6150)
        case = workloads.build_qk("qk_h32", 6150, rng.integers(1, 40, size=5, endpoint=True),
                                  rng.integers(0, 90, size=5, endpoint=True), Hq=32, Hkv=32,
                                  D=64, page_size=16, max_seq_len=256, theta=10000.0,
                                  interleaved=False, with_position_ids=False, norm_cols=64,
                                  rng=rng)
        mbc = True
    elif kind.startswith("bf16"):
        case = list(oracle_pins.small_qk_cases())[0]
        mbc = kind == "bf16_mbc"
    else:
        case = list(oracle_pins.small_qk_fp8_cases())[0 if kind == "fp8_per_tensor" else 1]
        mbc = True
    Hkv, D = case.k_cache.shape[3:]
    rng = workloads.make_rng(6100 + D)
    cols = D - 24
    gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, cols).astype(np.float32))
    total = case.T - 1
    _say(f"[kvnorm-tok] case={case.name} kind={kind} Hkv={Hkv} D={D} cols={cols} total={total}")
    dev = gh.QkDevice(case)
    dev.kv_norm(gh.dev_bf16(gamma), 0.125, total, mbc, per_head=False)
    k, ks = dev.k_host()
    assert int(dev.error_count.item()) == 0
    k_o = case.k_cache.copy()
    ks_o = None if case.k_scales is None else case.k_scales.copy()
    if ks_o is not None:
        with orc.fp8_probe(k_o) as pre:
            orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets,
                                        case.cache_lengths, case.page_table, gamma, case.epsilon,
                                        0.125, total, mbc, case.k_scale_mode, ks_o,
                                        per_head_norm=False)
        stats = check_fp8_k(case, k, ks, k_o, ks_o, pre, "kvnorm per-token fp8")
        _say(f"[kvnorm-tok] {stats}")
        return
    orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                case.page_table, gamma, case.epsilon, 0.125, total, mbc,
                                per_head_norm=False)
    rows = gh.written_k_rows(case)
    assert np.array_equal(k[~rows], case.k_cache[~rows])
    d = gh.bf16_ulp_diff(k[rows], k_o[rows])
    frac = float((d != 0).sum() / max(d.size, 1))
    _say(f"[kvnorm-tok] max_ulp={int(d.max())} diff_frac={frac}")
    assert int(d.max()) <= (1 if mbc else 2)
    assert frac <= gh.BF16_MAX_DIFF_FRAC
    assert np.array_equal(k[rows][..., cols:], case.k_cache[rows][..., cols:])


@pytest.mark.parametrize("D,Hkv,kmode,mbc,planned",
                         [(128, 64, "bf16", True, False), (128, 32, "bf16", False, False),
                          (64, 48, "bf16", True, True), (256, 12, "bf16", True, False),
                          (96, 20, "bf16", False, False), (128, 40, "per_tensor", True, False),
                          (128, 40, "per_token", True, True), (80, 33, "per_token", True, False)])
def test_kv_norm_per_token_statistic_many_heads(orc, D, Hkv, kmode, mbc, planned):
    """per_head_norm=False on tokens with more heads than one register chunk
    of the kernel holds (64 / (D/8) x 4 heads): the statistic is summed over
    every head first, then each chunk is normalised; every encoding, both
    cast orders, partial gamma, the planned form."""
    import paged_kv_cache_wavefront_amd as pkv
    rng = workloads.make_rng(6300 + D + Hkv)
    new = rng.integers(1, 70, size=9, endpoint=True)
    prior = rng.integers(0, 90, size=9, endpoint=True)
    fp8 = kmode != "bf16"
    case = workloads.build_qk(f"kvnorm_h{Hkv}_d{D}_{kmode}", 6300 + D + Hkv, new, prior, Hq=2,
                              Hkv=Hkv, D=D, page_size=8, max_seq_len=256, theta=10000.0,
                              interleaved=False, with_position_ids=False, norm_cols=None, rng=rng,
                              k_dtype="fp8" if fp8 else "bf16",
                              k_scale_mode=kmode if fp8 else "per_tensor")
    cols = D - 8 if D != 80 else D
    gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, cols).astype(np.float32))
    total = case.T - 1
    _say(f"[kvnorm-many] {case.name} T={case.T} cols={cols} mbc={mbc} planned={planned}")
    dev = gh.QkDevice(case)
    if planned:
        plan = torch.empty((case.T, 4), dtype=torch.int32, device="cuda")
        pkv.pkv_token_plan(plan, dev.offsets, dev.desc)
        pkv.rms_norm_kv_cache_paged_planned(dev.desc, case.layer_idx, gh.dev_bf16(gamma),
                                            case.epsilon, 0.125, total, plan, False, mbc)
    else:
        dev.kv_norm(gh.dev_bf16(gamma), 0.125, total, mbc, per_head=False)
    k, ks = dev.k_host()
    assert int(dev.error_count.item()) == 0
    k_o = case.k_cache.copy()
    ks_o = None if case.k_scales is None else case.k_scales.copy()
    if fp8:
        with orc.fp8_probe(k_o) as pre:
            orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets,
                                        case.cache_lengths, case.page_table, gamma, case.epsilon,
                                        0.125, total, mbc, case.k_scale_mode, ks_o,
                                        per_head_norm=False)
        _say(f"[kvnorm-many] {check_fp8_k(case, k, ks, k_o, ks_o, pre, 'k')}")
        return
    orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                case.page_table, gamma, case.epsilon, 0.125, total, mbc,
                                per_head_norm=False)
    rows = gh.written_k_rows(case)
    assert np.array_equal(k[~rows], case.k_cache[~rows])
    d = gh.bf16_ulp_diff(k[rows], k_o[rows])
    frac = float((d != 0).sum() / max(d.size, 1))
    _say(f"[kvnorm-many] max_ulp={int(d.max())} diff_frac={frac}")
    assert int(d.max()) <= (1 if mbc else 2)
    assert frac <= gh.BF16_MAX_DIFF_FRAC
    assert np.array_equal(k[rows][..., cols:], case.k_cache[rows][..., cols:])


def test_kv_norm_per_token_statistic_llama(orc):
    case = workloads.qk_generic()
    rng = workloads.make_rng(6200)
    gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    _say(f"[kvnorm-tok] case={case.name} T={case.T}")
    dev = gh.QkDevice(case)
    dev.kv_norm(gh.dev_bf16(gamma), 0.0, case.T, True, per_head=False)
    k = gh.host_bf16(dev.k)
    assert int(dev.error_count.item()) == 0
    k_o = case.k_cache.copy()
    orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                case.page_table, gamma, case.epsilon, 0.0, case.T, True,
                                per_head_norm=False)
    rows = gh.written_k_rows(case)
    assert np.array_equal(k[~rows], case.k_cache[~rows])
    gh.check_bf16(k[rows], k_o[rows], "kvnorm per-token llama")


def run_qk(orc, case, with_norm):
    _say(f"[qk] case={case.name} T={case.T} interleaved={case.interleaved} "
         f"pos_ids={case.position_ids is not None} norm={with_norm}")
    dev = gh.QkDevice(case)
    dev.rope(with_norm)
    q = gh.host_elem(dev.q_out)
    k, _ = dev.k_host()
    assert int(dev.error_count.item()) == 0
    q_o, k_o = oracle_qk(orc, case, with_norm)
    stats = {"q": gh.check_q(q, q_o, f"q ({q_o.dtype})")}
    stats["k"] = check_k_rows(case, k, k_o, "k", case.gamma.size if with_norm else None)
    _say(f"[qk] {case.name}: {stats}")
    return q, k


@pytest.mark.parametrize("with_norm", [True, False])
def test_llama_workload(orc, with_norm):
    run_qk(orc, workloads.qk_generic(), with_norm)


# (case index, with K norm): the third small case has no K norm gamma; the
# fourth has head_dim 256 (heads spanning 32 lanes); the fifth and sixth have
# head_dim 96 and 80 (padded 16-lane head groups, rotate-half and interleaved)
@pytest.mark.parametrize("idx,with_norm", [(0, True), (0, False), (1, True), (1, False),
                                           (2, False), (3, True), (3, False), (4, True),
                                           (4, False), (5, True), (5, False)])
def test_small_cases(orc, idx, with_norm):
    case = list(oracle_pins.small_qk_cases())[idx]
    assert with_norm is False or case.gamma is not None
    run_qk(orc, case, with_norm)


@pytest.mark.parametrize("D,interleaved,pos_ids",
                         [(128, False, True), (128, False, False), (64, True, True),
                          (64, False, False), (256, False, True), (256, True, False),
                          (96, False, True), (96, True, False), (80, False, False),
                          (80, True, True)])
def test_styles_and_dims(orc, D, interleaved, pos_ids):
    rng = workloads.make_rng(5000 + D)
    new = rng.integers(1, 200, size=12, endpoint=True)
    prior = rng.integers(0, 300, size=12, endpoint=True)
    case = workloads.build_qk(f"qk_d{D}", 5000 + D, new, prior, Hq=12, Hkv=3, D=D,
                              page_size=16, max_seq_len=2048, theta=10000.0,
                              interleaved=interleaved, with_position_ids=pos_ids,
                              norm_cols=D if D == 64 else 72, rng=rng)
    run_qk(orc, case, True)
    run_qk(orc, case, False)


@pytest.mark.parametrize("D,interleaved", [(128, False), (96, True), (64, False)])
def test_k_only(orc, D, interleaved):
    """No Q heads (num_q_heads = 0, null Q pointers): one wave per token
    rotates (and normalises) K alone; its Q lanes load nothing from Q."""
    rng = workloads.make_rng(5600 + D)
    new = rng.integers(1, 60, size=5, endpoint=True)
    prior = rng.integers(0, 100, size=5, endpoint=True)
    case = workloads.build_qk(f"qk_konly_d{D}", 5600 + D, new, prior, Hq=0, Hkv=3, D=D,
                              page_size=16, max_seq_len=512, theta=10000.0,
                              interleaved=interleaved, with_position_ids=True, norm_cols=D,
                              rng=rng)
    assert case.q.shape[1] == 0
    run_qk(orc, case, True)
    run_qk(orc, case, False)


def oracle_kv_norm(orc, case, gamma, w, total, mbc):
    k = case.k_cache.copy()
    orc.rms_norm_kv_cache_paged(k, case.layer_idx, case.row_offsets, case.cache_lengths,
                                case.page_table, gamma, case.epsilon, w, total, mbc)
    return k


@pytest.mark.parametrize("cols,w,mbc,short",
                         [(128, 0.0, True, False), (128, 0.0, False, False),
                          (40, 0.25, True, True), (100, 0.25, False, False)])
def test_kv_norm(orc, cols, w, mbc, short):
    case = workloads.qk_generic() if cols == 128 and not short else list(
        oracle_pins.small_qk_cases())[0]
    rng = workloads.make_rng(6000 + cols)
    gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, cols).astype(np.float32))
    total = case.T - 3 if short else case.T
    _say(f"[kvnorm] case={case.name} cols={cols} w={w} mbc={mbc} total={total}/{case.T}")
    dev = gh.QkDevice(case)
    dev.kv_norm(gh.dev_bf16(gamma), w, total, mbc)
    k = gh.host_bf16(dev.k)
    assert int(dev.error_count.item()) == 0
    k_o = oracle_kv_norm(orc, case, gamma, w, total, mbc)
    # multiply_before_cast=False rounds twice; a 1-ulp difference in the inner
    # rounding becomes < 2 ulps after the gamma product.
    rows = gh.written_k_rows(case)
    assert np.array_equal(k[~rows], case.k_cache[~rows])
    d = gh.bf16_ulp_diff(k[rows], k_o[rows])
    frac = float((d != 0).sum() / max(d.size, 1))
    _say(f"[kvnorm] max_ulp={int(d.max())} diff_frac={frac}")
    assert int(d.max()) <= (1 if mbc else 2)
    assert frac <= gh.BF16_MAX_DIFF_FRAC
    # columns past gamma_len and tokens past total_seq_len untouched
    assert np.array_equal(k[rows][..., cols:], case.k_cache[rows][..., cols:])


def test_two_call_form(orc):
    """K norm by rms_norm_kv_cache_paged, then RoPE without the fused norm:
    each call is checked on its own.  The norm call's K against the oracle's
    norm; the RoPE call against the oracle's RoPE applied to the GPU's own
    intermediate K (so the first call's roundings do not enter the second
    call's bar); both within one bf16 ulp, every other byte untouched."""
    case = workloads.qk_generic()
    dev = gh.QkDevice(case)
    dev.kv_norm(dev.gamma, 0.0, case.T, True)
    k_mid_gpu = gh.host_bf16(dev.k)
    rows = gh.written_k_rows(case)
    k_mid = oracle_kv_norm(orc, case, case.gamma, 0.0, case.T, True)
    assert np.array_equal(k_mid_gpu[~rows], case.k_cache[~rows])
    _say(f"[two-call] norm call: {gh.check_bf16(k_mid_gpu[rows], k_mid[rows], 'k after the norm')}")
    dev.rope(False)
    k = gh.host_bf16(dev.k)
    q = gh.host_bf16(dev.q_out)
    mid_case = workloads.QkCase(**{**case.__dict__, "k_cache": k_mid_gpu})
    q_o, k_o = oracle_qk(orc, mid_case, False)
    gh.check_bf16(q, q_o, "q")
    _say(f"[two-call] rope call: {check_k_rows(mid_case, k, k_o, 'k after the rope')}")


def test_deterministic(orc):
    case = workloads.qk_generic()
    outs = []
    for _ in range(2):
        dev = gh.QkDevice(case)
        dev.rope(True)
        outs.append((gh.host_bf16(dev.q_out), gh.host_bf16(dev.k)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
