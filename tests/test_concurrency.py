"""Two entry points on two streams at once: the library keeps no state
between calls, so concurrent launches on different streams (on disjoint
outputs) give the same results as one after the other."""
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
    from test_parity_qk import NORM_SLACK, check_k_rows
    check_k_rows(qcase, gh.host_bf16(qdev.k), k_o, "k", NORM_SLACK)


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
