"""Seeded random sweeps over the configuration space of every entry point,
each case against the oracle through the C ABI: batch shape, head counts and
dims, page sizes, q layouts and output dtype, cache dtype and scale mode, rope
style, position ids and mRoPE sections, K-norm width, weight offset, cast
order, per-head or per-token statistic, total_seq_len, gather dtypes.  Every
case prints its configuration before it runs."""
import numpy as np
import pytest

import gpu_helpers as gh
import workloads

pytestmark = pytest.mark.gpu

N_CASES = 16


def _say(*a):
    print(*a, flush=True)


def _frac_cap(n: int) -> float:
    # The fraction bar catches a wrong rounding mode, which moves about half
    # of all values; on a tiny case it still allows up to three to differ.
    return max(gh.BF16_MAX_DIFF_FRAC, 3.0 / max(n, 1))


def _lengths(rng, B, new_max, prior_max):
    new = rng.integers(0, new_max, size=B, endpoint=True)
    new[rng.integers(0, B)] = max(1, int(new.max()))        # at least one new token
    prior = rng.integers(0, prior_max, size=B, endpoint=True)
    return new, prior


@pytest.mark.parametrize("seed", range(N_CASES))
def test_mla_random(orc, seed):
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 40))
    new, prior = _lengths(rng, B, 24, 300)
    H = int(rng.choice([1, 3, 8, 15, 16, 17, 24, 31, 32, 40, 64, 100, 128]))
    page = int(rng.choice([8, 16, 32, 64, 128]))
    kind = str(rng.choice(["fp8_tensor", "fp8_token", "bf16"]))
    layout = str(rng.choice(["dense", "strided", "inplace"]))
    q_f32 = layout == "dense" and bool(rng.random() < 0.3)
    max_seq = int((prior + new).max()) + int(rng.integers(1, 50))
    layers = int(rng.integers(1, 3, endpoint=True))
    layer = int(rng.integers(0, layers))
    cfg = dict(B=B, T=int(new.sum()), H=H, page=page, kind=kind, layout=layout, q_f32=q_f32,
               max_seq=max_seq, layers=layers, layer=layer)
    _say(f"[rand-mla] seed={seed} {cfg}")
    case = workloads.build_mla(
        f"rand_mla_{seed}", 9000 + seed, new, prior, H=H, page_size=page, max_seq_len=max_seq,
        spare_pages=int(rng.integers(1, 6)), latent_sigma=float(rng.choice([0.5, 1.0, 2.0, 4.0])),
        outlier_p=float(rng.choice([0.0, 0.01])),
        scale_mode="per_token" if kind == "fp8_token" else "per_tensor",
        tensor_scale=float(rng.choice([0.02, 0.05, 0.2, 1.0])),
        cache_dtype="bf16" if kind == "bf16" else "fp8", num_layers=layers, layer_idx=layer,
        rng=rng)
    dev = gh.MlaDevice(case, layout, q_f32)
    dev.run()
    gpu = dev.results()
    assert gpu[3] == 0
    _say(f"[rand-mla] {gh.compare_mla(case, gpu, gh.oracle_mla(orc, case, q_f32), 3)}")
    # the planned form, with the plan of this batch, writes the same bits
    import torch
    import paged_kv_cache_wavefront_amd as pkv
    pdev = gh.MlaDevice(case, layout, q_f32)
    plan = torch.empty((case.T, 4), dtype=torch.int32, device=gh.DEV)
    pkv.pkv_token_plan(plan, pdev.offsets, pdev.desc)
    pkv.mla_rope_rmsnorm_quant_planned(pdev.q_out, pdev.q_in, pdev.latent, plan, pdev.freqs,
                                       pdev.gamma, case.epsilon, pdev.desc, case.layer_idx)
    planned = pdev.results()
    for got, want in zip(planned[:3], gpu[:3]):
        assert (got is None) == (want is None)
        if got is not None:
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), "planned differs"
    assert planned[3] == 0


def _random_qk(rng, seed):
    B = int(rng.integers(1, 30))
    new, prior = _lengths(rng, B, 20, 200)
    D = int(rng.choice([64, 80, 96, 128, 256]))
    Hq = int(rng.choice([1, 2, 5, 8, 16, 31, 32, 40]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    page = int(rng.choice([8, 16, 32]))
    interleaved = bool(rng.random() < 0.5)
    mrope = None
    if D >= 128 and rng.random() < 0.3:
        cut = np.sort(rng.integers(0, D // 2, size=2, endpoint=True))
        mrope = (int(cut[0]), int(cut[1] - cut[0]), int(D // 2 - cut[1]))
    pos_ids = mrope is not None or bool(rng.random() < 0.5)
    norm = rng.choice([0, 1, 2])
    norm_cols = None if norm == 0 else (D if norm == 1 else int(rng.integers(1, D)))
    k_dtype = str(rng.choice(["bf16", "fp8"]))
    k_mode = str(rng.choice(["per_tensor", "per_token"]))
    max_seq = int((prior + new).max()) + int(rng.integers(1, 300))
    layers = int(rng.integers(1, 3, endpoint=True))
    layer = int(rng.integers(0, layers))
    cfg = dict(B=B, T=int(new.sum()), D=D, Hq=Hq, Hkv=Hkv, page=page, interleaved=interleaved,
               mrope=mrope, pos_ids=pos_ids, norm_cols=norm_cols, k=k_dtype,
               k_mode=k_mode if k_dtype == "fp8" else None, layers=layers, layer=layer)
    case = workloads.build_qk(f"rand_qk_{seed}", 9100 + seed, new, prior, Hq=Hq, Hkv=Hkv, D=D,
                              page_size=page, max_seq_len=max_seq,
                              theta=float(rng.choice([1e4, 5e5, 1e6])), interleaved=interleaved,
                              with_position_ids=pos_ids, norm_cols=norm_cols, rng=rng,
                              spare_pages=int(rng.integers(1, 6)), k_dtype=k_dtype,
                              k_scale_mode=k_mode, k_scale=float(rng.choice([0.02, 0.05, 0.2])),
                              mrope_section=mrope, num_layers=layers, layer_idx=layer)
    return case, cfg


@pytest.mark.parametrize("seed", range(N_CASES))
def test_qk_random(orc, seed):
    from test_parity_qk import check_fp8_k, check_k_rows, oracle_qk
    rng = np.random.default_rng(9100 + seed)
    case, cfg = _random_qk(rng, seed)
    with_norm = case.gamma is not None
    _say(f"[rand-qk] seed={seed} {cfg}")
    dev = gh.QkDevice(case)
    dev.rope(with_norm)
    q = gh.host_bf16(dev.q_out)
    k, ks = dev.k_host()
    assert int(dev.error_count.item()) == 0
    q_o, k_o, ks_o, pre = oracle_qk(orc, case, with_norm, with_scales=True)
    stats = {"q": gh.check_bf16(q, q_o, "q", max_frac=_frac_cap(q.size))}
    if case.k_cache.dtype == np.uint8:
        stats["k"] = check_fp8_k(case, k, ks, k_o, ks_o, pre, "k",
                                 case.gamma.size if with_norm else None)
    else:
        n = int(gh.written_k_rows(case).sum()) * case.k_cache[0, 0, 0].size
        stats["k"] = check_k_rows(case, k, k_o, "k", case.gamma.size if with_norm else None,
                                  max_frac=_frac_cap(n))
    _say(f"[rand-qk] {stats}")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_kv_norm_random(orc, seed):
    from test_parity_qk import check_fp8_k
    rng = np.random.default_rng(9200 + seed)
    case, cfg = _random_qk(rng, seed)
    Hkv, D = case.k_cache.shape[3:]
    C = int(rng.integers(1, D, endpoint=True))
    w = float(rng.choice([0.0, 0.25, -0.5, 1.0]))
    fp8 = case.k_cache.dtype == np.uint8
    mbc = True if fp8 else bool(rng.random() < 0.5)
    per_head = bool(rng.random() < 0.6)
    total = case.T - int(rng.integers(0, min(3, case.T - 1), endpoint=True))
    _say(f"[rand-kvnorm] seed={seed} {cfg} C={C} w={w} mbc={mbc} per_head={per_head} "
         f"total={total}")
    gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, C).astype(np.float32))
    dev = gh.QkDevice(case)
    dev.kv_norm(gh.dev_bf16(gamma), w, total, mbc, per_head)
    k, ks = dev.k_host()
    assert int(dev.error_count.item()) == 0
    # the planned form, with the plan of this batch, writes the same bits
    import torch
    import paged_kv_cache_wavefront_amd as pkv
    pdev = gh.QkDevice(case)
    plan = torch.empty((case.T, 4), dtype=torch.int32, device=gh.DEV)
    pkv.pkv_token_plan(plan, pdev.offsets, pdev.desc)
    pkv.rms_norm_kv_cache_paged_planned(pdev.desc, case.layer_idx, gh.dev_bf16(gamma),
                                        case.epsilon, w, total, plan, per_head, mbc)
    k_p, ks_p = pdev.k_host()
    assert np.array_equal(k_p, k), "planned K norm differs"
    if ks is not None:
        assert np.array_equal(ks_p.view(np.uint32), ks.view(np.uint32))
    k_o = case.k_cache.copy()
    ks_o = None if case.k_scales is None else case.k_scales.copy()
    if fp8:
        with orc.fp8_probe(k_o) as pre:
            orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                        case.page_table, gamma, case.epsilon, w, total, mbc,
                                        case.k_scale_mode, ks_o, per_head_norm=per_head)
        # rows of tokens past total_seq_len stay as they were on both sides
        _say(f"[rand-kvnorm] {check_fp8_k(case, k, ks, k_o, ks_o, pre, 'k')}")
        return
    orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                case.page_table, gamma, case.epsilon, w, total, mbc,
                                per_head_norm=per_head)
    rows = gh.written_k_rows(case)
    assert np.array_equal(k[~rows], case.k_cache[~rows])
    d = gh.bf16_ulp_diff(k[rows], k_o[rows])
    frac = float((d != 0).sum() / max(d.size, 1))
    _say(f"[rand-kvnorm] max_ulp={int(d.max(initial=0))} diff_frac={frac:.2e}")
    assert int(d.max(initial=0)) <= (1 if mbc else 2)
    assert frac <= _frac_cap(d.size)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_gather_random(orc, seed):
    from test_parity_gather import finite_pool, run_gather
    rng = np.random.default_rng(9300 + seed)
    B = int(rng.integers(1, 40))
    new, prior = _lengths(rng, B, 8, 200)
    kind = str(rng.choice(["fp8_tensor", "fp8_token", "bf16"]))
    page = int(rng.choice([8, 16, 64, 128]))
    case = workloads.build_mla(f"rand_gather_{seed}", 9300 + seed, new, prior, H=1,
                               page_size=page, max_seq_len=int((prior + new).max()) + 1,
                               spare_pages=int(rng.integers(1, 6)),
                               scale_mode="per_token" if kind == "fp8_token" else "per_tensor",
                               tensor_scale=float(rng.choice([0.02, 0.05, 1.0])),
                               cache_dtype="bf16" if kind == "bf16" else "fp8", rng=rng)
    finite_pool(case, 9300 + seed)
    ctx = case.cache_lengths.astype(np.int64) + np.diff(case.row_offsets.astype(np.int64))
    kvo = np.zeros(B + 1, np.uint32)
    kvo[1:] = np.cumsum(ctx)
    out_fp8 = bool(rng.random() < 0.5)
    _say(f"[rand-gather] seed={seed} B={B} rows={int(kvo[-1])} kind={kind} page={page} "
         f"out_fp8={out_fp8}")
    run_gather(orc, case, kvo, out_fp8, out_scale=float(rng.choice([0.01, 0.25, 2.0])))
