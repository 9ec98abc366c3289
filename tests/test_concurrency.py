"""Two entry points on two streams at once, and several host threads calling
at once: the library keeps no state between calls, so concurrent launches on
different streams (on disjoint outputs) give the same results as one after
the other."""
import numpy as np
import pytest
import torch

import gpu_helpers as gh
import oracle_pins
import workloads

pytestmark = pytest.mark.gpu


def test_mla_and_qk_on_two_streams(orc):
    mcase = workloads.mla_mixed()
    qcase = workloads.qk_generic()
    mdev, qdev = gh.MlaDevice(mcase), gh.QkDevice(qcase)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        mdev.run(stream=s1)
    with torch.cuda.stream(s2):
        import paged_kv_cache_wavefront_amd as pkv
        pkv.qk_rope_paged_ragged(qdev.q_out, qdev.q_in, qdev.offsets, qdev.desc,
                                 qcase.layer_idx, qdev.freqs, qdev.pos, qcase.interleaved,
                                 qdev.gamma, qcase.epsilon, stream=s2)
    s1.synchronize()
    s2.synchronize()
    print("[concurrency]", gh.compare_mla(mcase, mdev.results(), gh.oracle_mla(orc, mcase)),
          flush=True)
    q = gh.host_bf16(qdev.q_out)
    q_o = np.zeros_like(qcase.q)
    k_o = qcase.k_cache.copy()
    orc.qk_rope_paged_ragged(q_o, qcase.q, qcase.row_offsets, qcase.cache_lengths,
                             qcase.page_table, k_o, qcase.layer_idx, qcase.freqs,
                             qcase.position_ids, qcase.interleaved, qcase.gamma, qcase.epsilon)
    gh.check_bf16(q, q_o, "q")
    from test_parity_qk import check_k_rows
    check_k_rows(qcase, gh.host_bf16(qdev.k), k_o, "k", qcase.gamma.size)


def test_same_entry_point_two_streams(orc):
    """Two MLA calls on two streams into different caches and outputs."""
    cases = [list(oracle_pins.small_mla_cases())[i] for i in (1, 3)]
    devs = [gh.MlaDevice(c) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for d, s in zip(devs, streams):
        with torch.cuda.stream(s):
            d.run(stream=s)
    for s in streams:
        s.synchronize()
    for c, d in zip(cases, devs):
        gh.compare_mla(c, d.results(), gh.oracle_mla(orc, c))


def test_host_threads():
    """Several host threads calling entry points at once, each on its own
    stream (ctypes releases the GIL during the call, so the host-side
    validation and launch code runs concurrently): every output is
    bit-identical to a single-threaded launch of the same call."""
    import threading
    import paged_kv_cache_wavefront_amd as pkv
    mcases = [list(oracle_pins.small_mla_cases())[i] for i in (1, 2, 3)]
    mdevs = [gh.MlaDevice(c) for c in mcases]
    gcase, kvo = oracle_pins.gather_case("fp8_token")
    gdesc = pkv.paged_cache(gh.dev_u8(gcase.cache), None, gh.dev_u32(gcase.page_table),
                            pkv.PKV_SCALE_PER_TOKEN, gh.dev_f32(gcase.token_scales))
    gkv = gh.dev_u32(kvo)
    gout = torch.zeros((int(kvo[-1]), gcase.cache.shape[-1]), dtype=torch.bfloat16,
                       device="cuda")

    def gather(stream=None):
        pkv.mla_gather_latent_paged(gout, gkv, gdesc, gcase.layer_idx, stream=stream)

    # single-threaded references
    ref = []
    for d in mdevs:
        d.run()
        ref.append(d.results())
    gather()
    torch.cuda.synchronize()
    gref = gout.clone()
    for d in mdevs:
        d.q_out.zero_()
    gout.zero_()
    torch.cuda.synchronize()

    jobs = [(lambda s, d=d: d.run(stream=s)) for d in mdevs] + [gather]
    errors = []

    def worker(job):
        try:
            s = torch.cuda.Stream()
            for _ in range(10):
                job(s)
            s.synchronize()
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a host thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for d, r in zip(mdevs, ref):
        got = d.results()
        assert np.array_equal(got[0], r[0]) and np.array_equal(got[1], r[1])
        # scales compared as bits: untouched slots hold random bytes, NaNs among them
        assert (got[2] is None and r[2] is None) or np.array_equal(got[2].view(np.uint32),
                                                                   r[2].view(np.uint32))
    assert torch.equal(gout.view(torch.int16), gref.view(torch.int16))
