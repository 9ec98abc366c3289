"""GPU parity with page sizes that are not powers of two (the general
division of a slot by the page size; powers of two take a shift) and with
head-chunk counts that are not powers of two, for every entry point, through
the C ABI against the oracle."""
import numpy as np
import pytest
import torch

import gpu_helpers as gh
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("page,mode", [(12, "per_token"), (24, "per_tensor"), (100, "bf16")])
def test_mla_page_sizes(orc, page, mode):
    """Ragged batch over pages of 12, 24 and 100 slots (slots cross many page
    boundaries), batch and planned forms; 80 heads: three head chunks."""
    import paged_kv_cache_wavefront_amd as pkv
    rng = workloads.make_rng(8100 + page)
    new = rng.integers(0, 90, size=9, endpoint=True)
    prior = rng.integers(0, 250, size=9, endpoint=True)
    case = workloads.build_mla(f"mla_page{page}", 8100 + page, new, prior, H=80, page_size=page,
                               max_seq_len=512, spare_pages=5,
                               scale_mode="per_token" if mode == "per_token" else "per_tensor",
                               tensor_scale=0.05, cache_dtype="bf16" if mode == "bf16" else "fp8",
                               rng=rng)
    _say(f"[pages] mla page={page} mode={mode} T={case.T}")
    dev = gh.MlaDevice(case)
    dev.run()
    gpu = dev.results()
    assert gpu[3] == 0
    _say(f"[pages] {gh.compare_mla(case, gpu, gh.oracle_mla(orc, case))}")
    pdev = gh.MlaDevice(case)
    plan = torch.empty((case.T, 4), dtype=torch.int32, device="cuda")
    pkv.pkv_token_plan(plan, pdev.offsets, pdev.desc)
    pkv.mla_rope_rmsnorm_quant_planned(pdev.q_out, pdev.q_in, pdev.latent, plan, pdev.freqs,
                                       pdev.gamma, case.epsilon, pdev.desc, case.layer_idx)
    pgpu = pdev.results()
    assert np.array_equal(pgpu[0], gpu[0]) and np.array_equal(pgpu[1], gpu[1]), \
        "planned form differs from the batch form"


@pytest.mark.parametrize("page,D,Hq", [(12, 128, 40), (24, 256, 40), (48, 96, 20)])
def test_qk_page_sizes(orc, page, D, Hq):
    """Q/K RoPE with the fused K norm over pages of 12, 24 and 48 slots; 40 Q
    heads of 128 and of 256 (three and five head chunks), 20 of 96."""
    from test_parity_qk import run_qk
    rng = workloads.make_rng(8200 + page)
    new = rng.integers(1, 60, size=7, endpoint=True)
    prior = rng.integers(0, 150, size=7, endpoint=True)
    case = workloads.build_qk(f"qk_page{page}", 8200 + page, new, prior, Hq=Hq, Hkv=3, D=D,
                              page_size=page, max_seq_len=1024, theta=10000.0,
                              interleaved=page == 24, with_position_ids=page == 48, norm_cols=D,
                              spare_pages=3, rng=rng)
    run_qk(orc, case, True)


@pytest.mark.parametrize("page", [12, 24])
def test_kv_norm_page_sizes(orc, page):
    """In-place K norm (per-head and per-token statistic) over pages of 12 and
    24 slots."""
    rng = workloads.make_rng(8300 + page)
    new = rng.integers(1, 50, size=6, endpoint=True)
    prior = rng.integers(0, 100, size=6, endpoint=True)
    case = workloads.build_qk(f"kvn_page{page}", 8300 + page, new, prior, Hq=1, Hkv=8, D=128,
                              page_size=page, max_seq_len=512, theta=10000.0,
                              interleaved=False, with_position_ids=False, norm_cols=None,
                              spare_pages=3, rng=rng)
    gamma = workloads.bf16_bits(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    for per_head in (True, False):
        dev = gh.QkDevice(case)
        dev.kv_norm(gh.dev_bf16(gamma), 0.0, case.T, True, per_head)
        k, _ = dev.k_host()
        assert int(dev.error_count.item()) == 0
        k_o = case.k_cache.copy()
        orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                    case.page_table, gamma, case.epsilon, 0.0, case.T, True,
                                    per_head_norm=per_head)
        rows = gh.written_k_rows(case)
        assert np.array_equal(k[~rows], case.k_cache[~rows])
        _say(f"[pages] kv_norm page={page} per_head={per_head}: "
             f"{gh.check_bf16(k[rows], k_o[rows], 'k')}")


def test_gather_page_size_24(orc):
    """Whole contexts gathered (fp8 -> bf16 and fp8 -> fp8) from pages of 24
    slots."""
    from test_parity_gather import run_gather, finite_pool
    rng = workloads.make_rng(8400)
    new = np.ones(7, np.int64)
    prior = rng.integers(0, 200, size=7, endpoint=True)
    case = workloads.build_mla("gather_page24", 8400, new, prior, H=1, page_size=24,
                               max_seq_len=int((prior + new).max()) + 1, spare_pages=3,
                               scale_mode="per_token", rng=rng)
    finite_pool(case, 8401)
    ctx = case.cache_lengths.astype(np.int64) + 1
    kvo = np.zeros(ctx.size + 1, np.uint32)
    kvo[1:] = np.cumsum(ctx)
    for out_fp8 in (False, True):
        run_gather(orc, case, kvo, out_fp8)
