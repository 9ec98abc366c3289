"""Host-side pieces of bench.py (CPU only): the byte model's terms, the
buffer-rotation count, the token-balanced split of the multi-threaded oracle
leg, and the single-GPU refusal."""
import os
import subprocess
import sys

import numpy as np

import oracle_pins
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_token_chunks_cover_every_token_once_with_its_slot():
    for case in list(oracle_pins.small_mla_cases()) + [workloads.mla_prefill()]:
        for n in (1, 3, 8, 16):
            seen = {}
            for ro, cl, pt in bench.token_chunks(case, n):
                assert pt.shape[0] == cl.size == ro.size - 1
                for b in range(cl.size):
                    for t in range(int(ro[b]), int(ro[b + 1])):
                        assert t not in seen
                        seen[t] = (int(cl[b]) + t - int(ro[b]), pt[b].tobytes())
            offs = case.row_offsets.astype(np.int64)
            assert len(seen) == case.T
            for b in range(case.B):
                for t in range(int(offs[b]), int(offs[b + 1])):
                    slot = int(case.cache_lengths[b]) + t - int(offs[b])
                    assert seen[t] == (slot, case.page_table[b].tobytes())


def test_chunked_oracle_equals_whole_batch(orc):
    case = list(oracle_pins.small_mla_cases())[2]
    q1, c1, _ = oracle_pins.run_mla(orc, case)
    q2 = np.zeros_like(case.q)
    c2 = case.cache.copy()
    for ro, cl, pt in bench.token_chunks(case, 5):
        orc.mla_rope_rmsnorm_quant(q2, case.q, case.latent, ro, cl, pt, case.freqs, case.gamma,
                                   case.epsilon, c2, case.layer_idx, case.scale_mode,
                                   case.tensor_scale, None)
    assert np.array_equal(q1, q2) and np.array_equal(c1, c2)


def test_mla_byte_model():
    """The prefill byte count: 34 496 B per token plus the shared terms."""
    case = workloads.mla_prefill()
    per_tok = 2 * 128 * 64 * 2 + 576 * 2 + 576
    assert per_tok == 34496
    shared = bench.mla_bytes(case) - case.T * per_tok
    assert 0 < shared < (1 << 20)
    inplace = workloads.mla_prefill_inplace()
    # bf16 row written instead of fp8; no per-tensor scale read
    assert bench.mla_bytes(inplace) - bench.mla_bytes(case) == case.T * 576 - 4


def test_rotation_count():
    assert bench.rotation_count(600 << 20, 700 << 20) == 2
    assert bench.rotation_count(1 << 20, 1 << 20) == 64            # capped
    assert bench.rotation_count(1 << 20, 1 << 20, cap=256) == 256
    assert bench.rotation_count(100 << 20, 5 << 30) == 2            # budget-bound, at least 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_written_bytes_split():
    """The read / write split of each workload's bytes, which sizes the matched
    stream: prefill writes q (16 KiB) and the fp8 row (576 B) per token."""
    case = workloads.mla_prefill()
    assert bench.written_bytes("mla_prefill", case) == case.T * (2 * 128 * 64 + 576)
    assert 0 < bench.mla_bytes(case) - bench.written_bytes("mla_prefill", case)
    mixed = workloads.mla_mixed()
    assert bench.written_bytes("mla_mixed", mixed) == mixed.T * (2 * 16 * 64 + 576 + 4)
    qk = workloads.qk_generic()
    assert bench.written_bytes("qk_generic", qk) == qk.T * (32 * 128 * 2 + 8 * 128 * 2)
    assert bench.written_bytes("kv_norm", qk) * 2 < bench.kv_norm_bytes(qk, 128) + qk.T * 8 + 300
    assert bench.written_bytes("gather", None, rows=10) == 11520


def test_grid_blocks_follow_the_launch_policy():
    """The grids the launch code sizes: 32 heads per MLA wave (16 for at most
    16 heads), 16 Q heads of 128 per Q/K wave, one wave per K-norm token, 6
    gather rows per wave; four waves per block."""
    assert bench.grid_blocks("mla_prefill", workloads.mla_prefill()) == workloads.mla_prefill().T
    assert bench.grid_blocks("mla_decode", workloads.mla_decode()) == 256
    assert bench.grid_blocks("mla_mixed", workloads.mla_mixed()) == 2064
    qk = workloads.qk_generic()
    assert bench.grid_blocks("qk_generic", qk) == -(-2 * qk.T // 4)
    assert bench.grid_blocks("kv_norm", qk) == -(-qk.T // 4)
    assert bench.grid_blocks("gather", None, rows=1022807) == -(-170468 // 4)


def test_cpu_model_names_the_processor():
    name = bench.cpu_model()
    assert name and name != "unknown"


def test_typed_workloads_byte_model():
    """The fp16-q prefill and fp16-Q Q/K siblings move the same q bytes as
    their bf16 twins; only the freqs rows (bf16: half the bytes) and gamma
    (fp32: twice) differ, and the written bytes are the same."""
    a, b = workloads.mla_prefill(), workloads.mla_prefill_f16()
    R, Dn = a.R, a.Dn
    pos = len({int(p) for c, n in zip(a.cache_lengths, np.diff(a.row_offsets.astype(np.int64)))
               for p in range(int(c), int(c) + int(n))})
    assert bench.mla_bytes(b) - bench.mla_bytes(a) == -pos * R * 2 + Dn * 2
    assert bench.written_bytes("mla_prefill_f16", b) == bench.written_bytes("mla_prefill", a)
    assert bench.grid_blocks("mla_prefill_f16", b) == bench.grid_blocks("mla_prefill", a)
    q, qh = workloads.qk_generic(), workloads.qk_generic_f16()
    assert bench.qk_bytes(q, True) - bench.qk_bytes(qh, True) == q.T * 128 * 2
    assert bench.written_bytes("qk_generic_f16", qh) == bench.written_bytes("qk_generic", q)
    assert "fp16 q" in bench.io_dtypes("mla_prefill_f16", b)
