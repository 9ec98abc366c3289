"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph): every
replay, with eager work and synchronisations between replays, must reproduce
the eager result bit for bit.  The MLA call is out of place, so replays are
idempotent; the in-place K paths and the in-place MLA form are replayed on a
fresh copy of their cache each time."""
import numpy as np
import pytest
import torch

import gpu_helpers as gh
import workloads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["mla_tiny", "mla_prefill", "mla_mixed"])
def test_mla_graph_replays(name):
    case = workloads.NAMED[name]()
    print(f"[graph] {name} T={case.T}", flush=True)
    eager = gh.MlaDevice(case)
    eager.run()
    want = eager.results()
    dev = gh.MlaDevice(case)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dev.run()          # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dev.run()
    for rep in range(3):
        dev.q_out.zero_()                       # eager work between replays
        junk = torch.ones(1 << 20, device="cuda") * rep
        torch.cuda.synchronize()
        g.replay()
        got = dev.results()
        assert np.array_equal(got[0], want[0]), f"replay {rep}: q differs"
        assert np.array_equal(got[1], want[1]), f"replay {rep}: cache differs"
        if got[2] is not None:
            assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
        del junk


@pytest.mark.parametrize("name", ["mla_decode", "mla_mixed"])
def test_planned_graph_replays(name):
    """A model step as a caller would capture it: the plan build, then the
    planned MLA step on two layers, all inside one graph; every replay (the
    plan cleared between replays) equals the batch form run eagerly."""
    import paged_kv_cache_wavefront_amd as pkv
    case = workloads.NAMED[name]()
    print(f"[graph] planned {name} T={case.T}", flush=True)
    eager = gh.MlaDevice(case)
    layers = range(case.cache.shape[0])
    for layer in layers:
        pkv.mla_rope_rmsnorm_quant(eager.q_out, eager.q_in, eager.latent, eager.offsets,
                                   eager.freqs, eager.gamma, case.epsilon, eager.desc, layer)
    want = eager.results()
    dev = gh.MlaDevice(case)
    plan = torch.zeros((case.T, 4), dtype=torch.int32, device="cuda")

    def step():
        pkv.pkv_token_plan(plan, dev.offsets, dev.desc)
        for layer in layers:
            pkv.mla_rope_rmsnorm_quant_planned(dev.q_out, dev.q_in, dev.latent, plan, dev.freqs,
                                               dev.gamma, case.epsilon, dev.desc, layer)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()             # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        dev.q_out.zero_()                       # eager work between replays
        plan.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = dev.results()
        assert np.array_equal(got[0], want[0]), f"replay {rep}: q differs"
        assert np.array_equal(got[1], want[1]), f"replay {rep}: cache differs"
        if got[2] is not None:
            assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
        assert got[3] == 0


def test_qk_graph_replays():
    case = workloads.qk_generic()
    eager = gh.QkDevice(case)
    eager.rope(True)
    want_q, want_k = gh.host_bf16(eager.q_out), gh.host_bf16(eager.k)
    dev = gh.QkDevice(case)
    k0 = dev.k.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dev.rope(True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dev.rope(True)
    for rep in range(3):
        dev.k.copy_(k0)                         # K is rotated in place: restore it
        dev.q_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gh.host_bf16(dev.q_out), want_q), f"replay {rep}: q"
        assert np.array_equal(gh.host_bf16(dev.k), want_k), f"replay {rep}: k"


@pytest.mark.parametrize("planned", [False, True])
def test_kv_norm_graph_replays(planned):
    """The K-cache norm inside a graph (planned: the plan build and the norm
    placed by it, both captured); K restored before every replay."""
    import paged_kv_cache_wavefront_amd as pkv
    case = workloads.qk_generic()
    eager = gh.QkDevice(case)
    eager.kv_norm(eager.gamma, 0.25, case.T, True, per_head=False)
    want = gh.host_bf16(eager.k)
    dev = gh.QkDevice(case)
    k0 = dev.k.clone()
    plan = torch.zeros((case.T, 4), dtype=torch.int32, device="cuda")

    def step():
        if planned:
            pkv.pkv_token_plan(plan, dev.offsets, dev.desc)
            pkv.rms_norm_kv_cache_paged_planned(dev.desc, case.layer_idx, dev.gamma,
                                                case.epsilon, 0.25, case.T, plan, False, True)
        else:
            dev.kv_norm(dev.gamma, 0.25, case.T, True, per_head=False)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        dev.k.copy_(k0)                         # normalised in place: restore it
        plan.zero_()
        junk = torch.ones(1 << 20, device="cuda") * rep
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gh.host_bf16(dev.k), want), f"replay {rep}: k"
        del junk


def test_mla_inplace_graph_replays():
    """The in-place MLA form inside a graph: the latent rows are placed again
    before every replay (the step overwrites them)."""
    import oracle_pins
    case = list(oracle_pins.small_mla_inplace_cases())[1]
    eager = gh.MlaDevice(case)
    eager.place_rows()
    eager.run_inplace()
    want = eager.results()
    dev = gh.MlaDevice(case)
    placed = gh.dev_bf16(oracle_pins.place_latent_rows(case))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dev.cache.copy_(placed)
        dev.run_inplace()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dev.run_inplace()
    for rep in range(3):
        dev.cache.copy_(placed)                 # rewritten in place: put the rows back
        dev.q_out.zero_()
        junk = torch.ones(1 << 20, device="cuda") * rep
        torch.cuda.synchronize()
        g.replay()
        got = dev.results()
        assert np.array_equal(got[0], want[0]), f"replay {rep}: q differs"
        assert np.array_equal(got[1], want[1]), f"replay {rep}: cache differs"
        del junk


def test_gather_graph_replays():
    import oracle_pins
    import paged_kv_cache_wavefront_amd as pkv
    case, kvo = oracle_pins.gather_case("fp8_token")
    cache = gh.dev_u8(case.cache)
    scales = gh.dev_f32(case.token_scales)
    desc = pkv.paged_cache(cache, None, gh.dev_u32(case.page_table), pkv.PKV_SCALE_PER_TOKEN,
                           scales)
    kv = gh.dev_u32(kvo)
    rows = int(kvo[-1])
    out = torch.zeros((rows, 576), dtype=torch.bfloat16, device="cuda")
    pkv.mla_gather_latent_paged(out, kv, desc, case.layer_idx)
    torch.cuda.synchronize()
    want = gh.host_bf16(out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkv.mla_gather_latent_paged(out, kv, desc, case.layer_idx)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gh.host_bf16(out), want), f"replay {rep}: gather"
