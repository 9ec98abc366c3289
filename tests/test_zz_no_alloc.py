"""mla_rope_rmsnorm_quant_noalloc against mla_rope_rmsnorm_quant_planned (the
entry point it varies, with a torch-allocated plan from pkv_token_plan),
through the C ABI: two calls in a row, the second with a smaller batch, each
bit-identical to the existing entry point's outputs (q, every cache byte,
per-token scales, skip count) and within the parity bars of the oracle; then
a call that reuses the last plan for another layer, and the refusals."""
import numpy as np
import pytest
import torch

import gpu_helpers as gh
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _case(name, seed, n_req, max_new, H, mode):
    rng = workloads.make_rng(seed)
    new = rng.integers(1, max_new, size=n_req, endpoint=True)
    prior = rng.integers(0, 400, size=n_req, endpoint=True)
    return workloads.build_mla(name, seed, new, prior, H=H, page_size=32, max_seq_len=2048,
                               spare_pages=6, scale_mode=mode, tensor_scale=0.05, rng=rng)


def _planned_reference(case, layer=None):
    """Outputs of the existing planned entry point on fresh device copies."""
    import paged_kv_cache_wavefront_amd as pkv
    dev = gh.MlaDevice(case)
    plan = torch.empty((case.T, 4), dtype=torch.int32, device="cuda")
    pkv.pkv_token_plan(plan, dev.offsets, dev.desc)
    pkv.mla_rope_rmsnorm_quant_planned(dev.q_out, dev.q_in, dev.latent, plan, dev.freqs,
                                       dev.gamma, case.epsilon, dev.desc,
                                       case.layer_idx if layer is None else layer)
    return dev.results()


def _noalloc(case, build_plan, layer=None):
    import paged_kv_cache_wavefront_amd as pkv
    dev = gh.MlaDevice(case)
    pkv.mla_rope_rmsnorm_quant_noalloc(dev.q_out, dev.q_in, dev.latent, dev.offsets, dev.freqs,
                                       dev.gamma, case.epsilon, dev.desc,
                                       case.layer_idx if layer is None else layer, build_plan)
    return dev.results()


def _same(a, b, what):
    for i, name in enumerate(("q", "cache", "token scales", "skipped")):
        x, y = a[i], b[i]
        if isinstance(x, np.ndarray):
            assert x.dtype == y.dtype and np.array_equal(x.view(np.uint8), y.view(np.uint8)), \
                f"{what}: {name} differs from the planned entry point"
        else:
            assert x == y, f"{what}: {name} {x} != {y}"


def test_noalloc_matches_planned_entry_point(orc):
    big = _case("noalloc_big", 7001, 24, 300, 40, "per_token")
    small = _case("noalloc_small", 7002, 5, 60, 16, "per_tensor")
    assert small.T < big.T
    for case in (big, small):              # two calls in a row, the second smaller
        _say(f"[noalloc] case={case.name} T={case.T} H={case.H} build_plan=1")
        got = _noalloc(case, True)
        _same(got, _planned_reference(case), case.name)
        assert got[3] == 0
        _say(f"[noalloc] {case.name}: {gh.compare_mla(case, got, gh.oracle_mla(orc, case))}")
    # the other layer of the last batch, from the plan the last call built
    _say(f"[noalloc] case={small.name} layer 0, build_plan=0")
    _same(_noalloc(small, False, layer=0), _planned_reference(small, layer=0),
          "reused plan, layer 0")


def test_noalloc_refusals():
    import paged_kv_cache_wavefront_amd as pkv
    case = _case("noalloc_refuse", 7003, 3, 20, 8, "per_tensor")
    dev = gh.MlaDevice(case)
    _noalloc(case, True)                   # a plan of case.T tokens on this device
    bigger = _case("noalloc_refuse_big", 7004, 20, 200, 8, "per_tensor")
    assert bigger.T > case.T
    bdev = gh.MlaDevice(bigger)
    before = (gh.host_bf16(bdev.q_out), gh.host_u8(bdev.cache))
    with pytest.raises(pkv.PkvError) as err:   # reuse asks for more tokens than were built
        pkv.mla_rope_rmsnorm_quant_noalloc(bdev.q_out, bdev.q_in, bdev.latent, bdev.offsets,
                                           bdev.freqs, bdev.gamma, bigger.epsilon, bdev.desc,
                                           bigger.layer_idx, False)
    assert err.value.status == 2
    torch.cuda.synchronize()
    assert np.array_equal(gh.host_u8(bdev.cache), before[1])  # nothing was enqueued
    # more tokens than the array holds: refused before any device work
    lib = pkv.library()
    st = lib.mla_rope_rmsnorm_quant_noalloc(
        dev.q_out.data_ptr(), 0, 64, dev.q_in.data_ptr(), 0, 64, dev.latent.data_ptr(), 576,
        dev.offsets.data_ptr(), 2, (1 << 18) + 1, 8, 64, 512, dev.freqs.data_ptr(), 64,
        dev.gamma.data_ptr(), 1e-6, dev.desc, 1, None, 1, None)
    assert st == 5
    # zero tokens: nothing enqueued
    st = lib.mla_rope_rmsnorm_quant_noalloc(
        dev.q_out.data_ptr(), 0, 64, dev.q_in.data_ptr(), 0, 64, dev.latent.data_ptr(), 576,
        dev.offsets.data_ptr(), 2, 0, 8, 64, 512, dev.freqs.data_ptr(), 64,
        dev.gamma.data_ptr(), 1e-6, dev.desc, 1, None, 1, None)
    assert st == 0
