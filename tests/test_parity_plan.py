"""GPU parity of pkv_token_plan, mla_rope_rmsnorm_quant_planned and
rms_norm_kv_cache_paged_planned against the CPU oracle, through the C ABI: the
plan bit for bit (all MLA workloads, small ragged cases, page ids past the
pool, rows past the last offset); the planned MLA step and K-cache norm
bit-identical to their batch forms on the same batch and within the parity
bars of the oracle; free placements and entries that are skipped, out of the
pool or out of the freqs table against the oracle's planned forms."""
import contextlib

import numpy as np
import pytest
import torch

import gpu_helpers as gh
import oracle
import oracle_pins
import workloads

pytestmark = pytest.mark.gpu

NAMED = ["mla_tiny", "mla_decode", "mla_mixed", "mla_prefill"]


def _say(*a):
    print(*a, flush=True)


def gpu_plan(dev, T=None):
    """The plan pkv_token_plan writes for the device copy of a case."""
    import paged_kv_cache_wavefront_amd as pkv
    T = dev.case.T if T is None else T
    plan = torch.full((T, 4), 0x5A5A5A5A, dtype=torch.int32, device=gh.DEV)
    pkv.pkv_token_plan(plan, dev.offsets, dev.desc)
    torch.cuda.synchronize()
    return plan


def run_planned(dev, plan):
    import paged_kv_cache_wavefront_amd as pkv
    pkv.mla_rope_rmsnorm_quant_planned(dev.q_out, dev.q_in, dev.latent, plan, dev.freqs,
                                       dev.gamma, dev.case.epsilon, dev.desc,
                                       dev.case.layer_idx)


def oracle_planned(orc, case, plan, q_f32=False):
    """Oracle results of the planned step, shaped like gh.oracle_mla; tokens
    the plan does not place are skipped (the oracle reports them, the rest is
    written)."""
    q_out = np.zeros(case.q.shape, np.float32) if q_f32 else np.zeros_like(case.q)
    cache = case.cache.copy()
    ts = None if case.token_scales is None else case.token_scales.copy()
    probe = orc.fp8_probe(cache) if cache.dtype == np.uint8 else contextlib.nullcontext()
    with probe as pre:
        try:
            orc.mla_rope_rmsnorm_quant_planned(q_out, case.q, case.latent, plan, case.freqs,
                                               case.gamma, case.epsilon, cache,
                                               case.layer_idx, case.scale_mode,
                                               case.tensor_scale, ts)
        except oracle.OracleError:
            pass
    return q_out, cache, ts, pre


def plan_cases():
    for name in NAMED:
        yield workloads.NAMED[name]()
    yield from oracle_pins.token_plan_cases()


@pytest.mark.parametrize("idx", range(len(NAMED) + 6))
def test_token_plan_matches_oracle(orc, idx):
    case = list(plan_cases())[idx]
    _say(f"[plan] case={case.name} seed={case.seed} T={case.T} B={case.B}")
    dev = gh.MlaDevice(case)
    got = gpu_plan(dev).cpu().numpy().view(np.uint32)
    want = oracle_pins.run_token_plan(orc, case)
    assert np.array_equal(got, want), f"{case.name}: {(got != want).any(axis=1).sum()} rows differ"
    # rows past the last offset belong to no request
    got = gpu_plan(dev, case.T + 5).cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle_pins.run_token_plan(orc, case, case.T + 5))


@pytest.mark.parametrize("name", NAMED)
def test_planned_equals_batch_form(orc, name):
    """With its own batch's plan the planned step writes exactly what the
    batch form writes, and meets the oracle's parity bars."""
    case = workloads.NAMED[name]()
    _say(f"[planned] case={case.name} seed={case.seed} T={case.T} B={case.B} H={case.H}")
    ref = gh.MlaDevice(case)
    ref.run()
    r = ref.results()
    dev = gh.MlaDevice(case)
    run_planned(dev, gpu_plan(dev))
    g = dev.results()
    assert g[3] == r[3] == 0
    assert np.array_equal(g[0].view(np.uint16), r[0].view(np.uint16)), "q_rope_output differs"
    assert np.array_equal(g[1], r[1]), "cache differs"
    if g[2] is not None:
        assert np.array_equal(g[2].view(np.uint32), r[2].view(np.uint32)), "scales differ"
    stats = gh.compare_mla(case, g, gh.oracle_mla(orc, case))
    _say(f"[planned] {case.name}: {stats}")


def free_plan_cases():
    rng = np.random.default_rng(3030)
    small = list(oracle_pins.small_mla_cases())
    for k, case in enumerate(small[:4] + [workloads.mla_decode()]):
        plan = oracle_pins.free_plan(case, rng, skip_every=0 if k == 0 else 5)
        if k >= 2 and case.T >= 8:
            P, S = case.cache.shape[1:3]
            plan[1] = (P, 0, 0, 1)                      # page past the pool
            plan[3] = (0, S, 0, 1)                      # offset past the page
            plan[6] = (0, 0, case.freqs.shape[0], 1)    # position past the freqs table
        yield case, plan


@pytest.mark.parametrize("idx", range(5))
def test_planned_free_placement(orc, idx):
    """A plan unrelated to the batch: every placed token's row lands at its
    cell with its position's rotation; skipped entries write nothing and are
    counted."""
    case, plan = list(free_plan_cases())[idx]
    _say(f"[planned-free] case={case.name} seed={case.seed} T={case.T}")
    dev = gh.MlaDevice(case)
    dev.q_out.zero_()
    run_planned(dev, gh.dev_u32(plan))
    g = dev.results()
    L, P, S = case.cache.shape[:3]
    ok = (plan[:, 3] != 0) & (plan[:, 0] < P) & (plan[:, 1] < S) & \
        (plan[:, 2] < case.freqs.shape[0])
    assert g[3] == int((~ok).sum())
    rows = np.zeros((L, P, S), bool)
    rows[case.layer_idx, plan[ok, 0], plan[ok, 1]] = True
    o = oracle_planned(orc, case, plan)
    stats = gh.compare_mla(case, g, o, small_case_floor=3, rows=rows)
    _say(f"[planned-free] {case.name}: skipped {g[3]}, {stats}")


def test_plan_reused_across_layers(orc):
    """One plan serves every layer: the planned step on layers 0 and 1 of a
    two-layer pool equals the batch form on each."""
    case = workloads.mla_tiny()
    dev, ref = gh.MlaDevice(case), gh.MlaDevice(case)
    plan = gpu_plan(dev)
    import paged_kv_cache_wavefront_amd as pkv
    for layer in range(case.cache.shape[0]):
        pkv.mla_rope_rmsnorm_quant_planned(dev.q_out, dev.q_in, dev.latent, plan, dev.freqs,
                                           dev.gamma, case.epsilon, dev.desc, layer)
        pkv.mla_rope_rmsnorm_quant(ref.q_out, ref.q_in, ref.latent, ref.offsets, ref.freqs,
                                   ref.gamma, case.epsilon, ref.desc, layer)
    g, r = dev.results(), ref.results()
    assert np.array_equal(g[1], r[1]) and np.array_equal(g[0].view(np.uint16),
                                                         r[0].view(np.uint16))


def _kv_planned_cases():
    """(case, gamma width, weight offset, total, multiply_before_cast, per_head)"""
    yield workloads.qk_generic(), 128, 0.0, None, True, True
    small = list(oracle_pins.small_qk_cases())
    yield small[0], 48, 0.25, -3, False, True
    yield small[1], None, 0.0, None, True, False
    for case in oracle_pins.small_qk_fp8_cases():
        yield case, None, 0.0, None, True, True


@pytest.mark.parametrize("idx", range(3 + len(list(oracle_pins.small_qk_fp8_cases()))))
def test_kv_norm_planned_equals_batch_form(orc, idx):
    """The K-cache norm placed by its batch's plan writes the batch form's bits
    (bf16 both cast orders, weight offset, short total_seq_len, per-token
    statistic, fp8 tensor and token scales), and meets the oracle's planned
    form on the same call."""
    import paged_kv_cache_wavefront_amd as pkv
    case, cols, w, short, mbc, per_head = list(_kv_planned_cases())[idx]
    D = case.k_cache.shape[-1]
    cols = cols or (case.gamma.size if case.gamma is not None else D)
    gamma = workloads.bf16_bits(workloads.make_rng(7000 + idx).uniform(0.5, 1.5, cols)
                                .astype(np.float32))
    total = case.T + short if short else case.T
    _say(f"[kv-planned] case={case.name} T={case.T} total={total} cols={cols} w={w} "
         f"mbc={mbc} per_head={per_head} k={case.k_scale_mode}")
    ref, dev = gh.QkDevice(case), gh.QkDevice(case)
    g = gh.dev_bf16(gamma)
    ref.kv_norm(g, w, total, mbc, per_head)
    plan = torch.zeros((case.T, 4), dtype=torch.int32, device=gh.DEV)
    pkv.pkv_token_plan(plan, dev.offsets, dev.desc)
    pkv.rms_norm_kv_cache_paged_planned(dev.desc, case.layer_idx, g, case.epsilon, w, total, plan,
                                        per_head, mbc)
    (k_r, s_r), (k_p, s_p) = ref.k_host(), dev.k_host()
    assert int(dev.error_count.item()) == int(ref.error_count.item()) == 0
    assert np.array_equal(k_p, k_r), "planned K norm differs from the batch form"
    if s_r is not None:
        assert np.array_equal(s_p.view(np.uint32), s_r.view(np.uint32))
    # the planned form against the oracle's planned form, bit for bit where
    # the oracle's float64 result is not within a hair of a rounding boundary
    k_o = case.k_cache.copy()
    s_o = None if case.k_scales is None else case.k_scales.copy()
    orc.rms_norm_kv_cache_planned(k_o, case.layer_idx, oracle_pins.qk_token_plan(orc, case),
                                  gamma, case.epsilon, w, total, mbc, case.k_scale_mode, s_o,
                                  per_head)
    rows = gh.written_k_rows(case)
    assert np.array_equal(k_p[~rows], case.k_cache[~rows])
    if case.k_cache.dtype == np.uint16:
        d = gh.bf16_ulp_diff(k_p[rows], k_o[rows])
        assert int(d.max(initial=0)) <= (1 if mbc else 2)
        assert float((d != 0).sum() / max(d.size, 1)) <= max(gh.BF16_MAX_DIFF_FRAC, 3 / d.size)
    else:
        d = gh.fp8_ulp_diff(k_p[rows], k_o[rows])
        assert int(d.max(initial=0)) <= 1
        assert float((d != 0).sum() / max(d.size, 1)) <= max(gh.FP8_MAX_DIFF_FRAC, 3 / d.size)


def test_kv_norm_planned_skips(orc):
    """Entries not marked placed, or naming a page or offset outside the pool,
    are skipped and counted; the other tokens are normalised at their cells."""
    import paged_kv_cache_wavefront_amd as pkv
    case = list(oracle_pins.small_qk_cases())[0]
    dev = gh.QkDevice(case)
    plan = torch.zeros((case.T, 4), dtype=torch.int32, device=gh.DEV)
    pkv.pkv_token_plan(plan, dev.offsets, dev.desc)
    L, P, S = case.k_cache.shape[:3]
    h = plan.cpu().numpy().view(np.uint32).copy()
    h[0, 3] = 0
    h[1, 0] = P
    h[2, 1] = S
    plan.copy_(torch.from_numpy(h.view(np.int32)))
    gamma = workloads.bf16_bits(np.linspace(0.5, 1.5, 64).astype(np.float32))
    pkv.rms_norm_kv_cache_paged_planned(dev.desc, case.layer_idx, gh.dev_bf16(gamma),
                                        case.epsilon, 0.0, case.T, plan)
    k, _ = dev.k_host()
    assert int(dev.error_count.item()) == 3
    k_o = case.k_cache.copy()
    try:
        orc.rms_norm_kv_cache_planned(k_o, case.layer_idx, h, gamma, case.epsilon, 0.0, case.T)
    except oracle.OracleError:
        pass
    d = gh.bf16_ulp_diff(k, k_o)
    assert int(d.max(initial=0)) <= 1
    assert float((d != 0).sum() / d.size) <= max(gh.BF16_MAX_DIFF_FRAC, 3 / d.size)


def _inplace_cases():
    yield from oracle_pins.small_mla_inplace_cases()
    yield workloads.mla_prefill_inplace()


@pytest.mark.parametrize("idx", range(len(list(oracle_pins.small_mla_inplace_cases())) + 1))
def test_inplace_planned_equals_batch_form(orc, idx):
    """The in-place step placed by its batch's plan reads and writes exactly
    what the batch in-place form does, and meets the oracle's parity bars."""
    import paged_kv_cache_wavefront_amd as pkv
    case = list(_inplace_cases())[idx]
    _say(f"[inplace-planned] case={case.name} seed={case.seed} T={case.T} H={case.H}")
    ref, dev = gh.MlaDevice(case), gh.MlaDevice(case)
    ref.place_rows()
    dev.place_rows()
    ref.run_inplace()
    plan = gpu_plan(dev)
    pkv.mla_rope_rmsnorm_inplace_planned(dev.q_out, dev.q_in, plan, dev.freqs, dev.gamma,
                                         case.epsilon, dev.desc, case.layer_idx)
    g, r = dev.results(), ref.results()
    assert g[3] == r[3] == 0
    assert np.array_equal(g[0].view(np.uint16), r[0].view(np.uint16)), "q_rope_output differs"
    assert np.array_equal(g[1], r[1]), "cache differs"
    stats = gh.compare_mla(case, g, gh.oracle_mla_inplace(orc, case), small_case_floor=3)
    _say(f"[inplace-planned] {case.name}: {stats}")
