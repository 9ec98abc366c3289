"""Benchmark of the fused MLA pre-attention step on one MI355X.

Default workload: DeepSeek-V3-shaped prefill -- 8 requests with new lengths
U{512..4096} (seeded; 17108 tokens), no prior cache, 128 query heads x rope
64, latent 512 + 64, FP8 E4M3FN paged cache (page size 128) with per-tensor
scale 0.05.  One step = one mla_rope_rmsnorm_quant launch over the whole
batch (q RoPE, latent RMSNorm + RoPE, FP8 quantisation, paged store), inputs
resident in HBM.  Prints one JSON line.

Consecutive steps rotate over enough output-buffer sets that each cycle
writes at least 1 GiB of distinct memory, so no step rewrites lines the
previous one left dirty in the Infinity Cache (``buffer_rotation`` names the
sets).  Also reported: 20 isolated launches after a 512 MiB read that
flushes the caches (``cold_us_p10_p50_p90``); a plain streaming copy timed in
the same run (``measured_copy``); a stream of the workload's own read and
written bytes, rotated and timed the same way (``matched_stream``, with the
workload's fraction of it in ``pct_of_matched_stream``); the cost of an empty
launch on the workload's grid (``launch_floor_us``); and (``siblings``) the
other workloads and entry points, each timed the same way with the same
fields -- MLA decode (256 x 1 token, 128 heads), mixed prefill + decode with
per-token scales (16 heads), both of them again placed by a token plan built
once before the timed launches (mla_rope_rmsnorm_quant_planned; the plan
build's own time beside them, and seven alternating repetitions against the
batch form in ``vs_batch_form_us``), the same prefill batch in place on a
bf16 latent cache (mla_rope_rmsnorm_inplace), the Llama-shaped paged-ragged
Q/K RoPE with fused per-head K norm, the in-place K-cache RMSNorm (also placed
by a token plan) and the paged latent gather.

``cpu_baseline`` is the oracle on the same inputs on N host threads (N = the
cores in the process's affinity mask, at most the 16 a GPU's share of the
host holds), checked bit for bit against a single-threaded run whose rate is
reported beside it; the line also carries ``parity``: one launch of the timed
entry point compared with the oracle's outputs of that run.

``--calibrate-copy`` runs a plain elementwise copy of known size instead (the
reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E peak, GB/s
METRIC = "fused MLA RoPE+RMSNorm+FP8 cache-write: tokens/s and effective HBM GB/s (% of peak)"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_cache_wavefront_amd", "csrc")
# sources that decide what a workload's launch does: its kernel file (kernel
# and launch policy) plus the shared device helpers and argument structs
COMMON_SOURCES = ("pkv_device.h", "pkv_internal.h")
KERNEL_OF = {"mla_prefill": "mla_rope_rmsnorm_quant.hip", "mla_decode": "mla_rope_rmsnorm_quant.hip",
             "mla_mixed": "mla_rope_rmsnorm_quant.hip", "mla_tiny": "mla_rope_rmsnorm_quant.hip",
             "mla_prefill_inplace": "mla_rope_rmsnorm_quant.hip",
             "mla_prefill_f16": "mla_rope_rmsnorm_quant.hip",
             "qk_generic_f16": "qk_rope_paged_ragged.hip",
             "mla_decode_planned": "mla_rope_rmsnorm_quant.hip",
             "mla_mixed_planned": "mla_rope_rmsnorm_quant.hip",
             "kv_norm_planned": "rms_norm_kv_cache_paged.hip",
             "qk_generic": "qk_rope_paged_ragged.hip", "kv_norm": "rms_norm_kv_cache_paged.hip",
             "gather": "mla_gather_latent_paged.hip"}


def kernel_source_hash(workload: str = "mla_prefill") -> str:
    h = hashlib.sha256()
    for name in (KERNEL_OF[workload],) + COMMON_SOURCES:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# -- algorithmic bytes (what the method must move, read + written) ---------------------

def mla_bytes(case, planned: bool = False) -> int:
    """q in + q out (H x R x 2 each for bf16 or fp16; the output takes q's
    type) + latent row in (W x 2, from its buffer or, in place, from the
    cache) + cache row out (W x 1 fp8 / W x 2 bf16, + 4 for a per-token scale)
    per token; once per launch: freqs rows of the distinct positions (R
    values each, 4 or 2 bytes), gamma, offsets, prior lengths, the page-table
    entries read, the per-tensor scale.  Planned: a 16-byte plan entry per
    token replaces the offsets, prior lengths and page-table entries."""
    T, H, R, W = case.T, case.H, case.R, case.latent.shape[1]
    out_b = 2 if case.cache.dtype == np.uint16 else 1
    qb = case.q.itemsize
    per_tok = 2 * H * R * qb + W * 2 + W * out_b + (4 if case.scale_mode == "per_token" else 0)
    pos = np.concatenate([np.arange(c, c + n) for c, n in
                          zip(case.cache_lengths.astype(np.int64),
                              np.diff(case.row_offsets.astype(np.int64)))]) if T else np.zeros(0)
    S = case.meta["page_size"]
    pages_read = len({(b, int(p) // S) for b, (c, n) in enumerate(
        zip(case.cache_lengths, np.diff(case.row_offsets.astype(np.int64))))
        for p in range(int(c), int(c) + int(n))})
    chain = 16 * T if planned else (case.B + 1) * 4 + case.B * 4 + 4 * pages_read
    shared = (len(np.unique(pos)) * R * case.freqs.itemsize + case.Dn * case.gamma.itemsize + chain
              + (4 if case.scale_mode == "per_tensor" else 0))
    return T * per_tok + shared


def plan_bytes(case) -> int:
    """pkv_token_plan: offsets, prior lengths and the page-table entries read,
    16 bytes written per token."""
    S = case.meta["page_size"]
    pages_read = len({(b, int(p) // S) for b, (c, n) in enumerate(
        zip(case.cache_lengths, np.diff(case.row_offsets.astype(np.int64))))
        for p in range(int(c), int(c) + int(n))})
    return (case.B + 1) * 4 + case.B * 4 + 4 * pages_read + 16 * case.T


def qk_bytes(case, with_norm: bool) -> int:
    """Q in + out, K rows in + out (in place), one position id and one freqs
    row per token; gamma, offsets, prior lengths and page-table entries once."""
    T, Hq, D = case.q.shape
    Hkv = case.k_cache.shape[3]
    per_tok = (2 * Hq * D * case.q.itemsize + 2 * Hkv * D * 2 + D * case.freqs.itemsize
               + (4 if case.position_ids is not None else 0))
    shared = (case.B + 1) * 4 + case.B * 4 + T * 4 // case.meta["page_size"] + \
        (case.gamma.size * 2 if with_norm else 0)
    return T * per_tok + shared


def gather_bytes(rows: int, batch: int, page_size: int, in_bytes=576, out_bytes=1152) -> int:
    """Each context row read from the cache and written to the dense buffer,
    plus the offsets and one page-table entry per page of context."""
    return rows * (in_bytes + out_bytes) + (batch + 1) * 4 + 4 * (-(-rows // page_size))


def written_bytes(name: str, case, rows: int = 0) -> int:
    """The part of a workload's algorithmic bytes that is written (the rest
    is read): q out and the cache rows (MLA), Q out and the K rows (Q/K RoPE),
    the normalised K columns (K norm), the dense rows (gather)."""
    if name.startswith("mla_"):
        T, H, R, W = case.T, case.H, case.R, case.latent.shape[1]
        out_b = 2 if case.cache.dtype == np.uint16 else 1
        return T * (case.q.itemsize * H * R + W * out_b + (4 if case.scale_mode == "per_token" else 0))
    if name.startswith("qk_generic"):
        T, Hq, D = case.q.shape
        return T * (Hq * D * case.q.itemsize + case.k_cache.shape[3] * D * 2)
    if name.startswith("kv_norm"):
        return case.T * case.k_cache.shape[3] * 128 * 2
    if name == "gather":
        return rows * 1152
    raise ValueError(name)


def kv_norm_bytes(case, cols: int, planned: bool = False) -> int:
    """The first cols columns of every K head read and written back; gamma;
    offsets and prior lengths (planned: a 16-byte plan entry per token)."""
    T = case.T
    Hkv = case.k_cache.shape[3]
    chain = 16 * T if planned else (case.B + 1) * 4 + case.B * 4
    return T * 2 * Hkv * cols * 2 + chain + cols * 2


# -- timing ------------------------------------------------------------------------------

def time_launches(fn, steps: int, warmup: int, spread_samples: int = 20):
    """Warm up, then time exactly `steps` back-to-back launches bracketed by
    device syncs, with one pair of HIP events (on the launch stream: torch's
    current stream) around the timed region.  Returns (wall seconds, average
    seconds per launch from the events, per-launch durations from a separate,
    untimed pass with an event pair around each launch)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg = e0.elapsed_time(e1) * 1e-3 / steps
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(spread_samples)]
    for a, b in pairs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    durs = np.array([a.elapsed_time(b) for a, b in pairs]) * 1e-3
    return wall, avg, durs


def time_graph(fn, steps: int, warmup: int, replays: int = 5, min_launches: int = 100):
    """Seconds per launch when max(steps, min_launches) launches are captured
    in one HIP graph (torch.cuda.CUDAGraph) and replayed: the kernels back to
    back with no host launch overhead between them.  The median over
    `replays` replays, each bracketed by its own event pair (a few-microsecond
    kernel needs the longer graph and the median to settle)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(1, warmup)):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    n = max(steps, min_launches)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3 / n)
    return float(np.median(times))


def profiled_traffic(name: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"{name}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not (m_b and m_h):
        return None
    return float(m_b.group(1)) if m_h.group(1) == kernel_source_hash(name) else None


def time_cold(fn, samples: int = 20, flush_mib: int = 512):
    """Per-launch durations with cold caches: before each sampled launch, a
    reduction reads flush_mib MiB of other data (more than the 256 MiB
    Infinity Cache and the L2s together), outside the event pair around the
    launch.  Reading rather than writing leaves no dirty lines behind, so the
    timed launch pays no write-back of the flush."""
    import torch
    junk = torch.ones((flush_mib << 20) // 4, dtype=torch.int32, device="cuda")
    acc = torch.zeros((), dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(samples)]
    for a, b in pairs:
        acc += junk.sum()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    del junk
    return np.array([a.elapsed_time(b) for a, b in pairs]) * 1e-3


# -- workloads -------------------------------------------------------------------------

def measure(fn, tokens, nbytes, steps, warmup, graph=True):
    wall, avg, durs = time_launches(fn, steps, warmup)
    r = dict(T=tokens, bytes=nbytes, wall=wall, durs=durs, avg=avg, med=float(np.median(durs)))
    r["cold_durs"] = time_cold(fn)
    r["graph_avg"] = time_graph(fn, steps, warmup) if graph else None
    return r


def summarize(name, r, steps, use_graph=False):
    """use_graph: quote throughput from the graph-replay time (short kernels,
    where eager timing would measure the host's launch overhead)."""
    t = r["graph_avg"] if use_graph and r["graph_avg"] else r["avg"]
    gbps = r["bytes"] / t / 1e9
    out = {"workload": name, "tokens": r["T"], "bytes_per_launch": r["bytes"],
           "timed_as": "hip graph replay" if use_graph else "eager launches",
           "kernel_us_avg": round(t * 1e6, 2),
           "eager_us_avg": round(r["avg"] * 1e6, 2),
           "eager_us_p10_p50_p90": [round(float(np.percentile(r["durs"], q)) * 1e6, 2)
                                    for q in (10, 50, 90)],
           "cold_us_p10_p50_p90": [round(float(np.percentile(r["cold_durs"], q)) * 1e6, 2)
                                   for q in (10, 50, 90)],
           "graph_us_avg": round(r["graph_avg"] * 1e6, 2) if r["graph_avg"] else None,
           "tokens_per_s": round(r["T"] / t, 1),
           "buffer_rotation": r.get("sets"),
           "effective_GBps": round(gbps, 1), "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2)}
    return out


# Buffer rotation.  Consecutive steps write different memory: a step that
# rewrote the previous step's output buffer would find part of it still in
# the 256 MiB Infinity Cache as dirty lines and overwrite them there, so
# some of its writes would never reach HBM.  Each workload cycles over
# enough output sets that the distinct bytes written per cycle reach
# ROTATE_BYTES, within a device-memory budget for the copies.
ROTATE_BYTES = 1 << 30
ROTATE_BUDGET = 8 << 30


def rotation_count(written_bytes: int, set_bytes: int, cap: int = 64) -> int:
    want = -(-ROTATE_BYTES // max(written_bytes, 1))
    fit = max(2, ROTATE_BUDGET // max(set_bytes, 1))
    return int(max(2, min(want, fit, cap)))


def cycle(fns):
    """One callable that runs fns[0], fns[1], ... in turn."""
    state = {"i": 0}

    def step():
        fns[state["i"] % len(fns)]()
        state["i"] += 1
    return step


def alternate(batch, planned, steps, warmup, reps: int = 7) -> dict:
    """The batch and planned forms of one step on the same buffers, timed by
    graph replay in turn, reps times each: the per-repetition figures, their
    medians and spreads, and the planned form's gain with the range of the
    per-repetition gains (a gain is settled only when that range excludes
    zero)."""
    ab = {"batch": [], "planned": []}
    for _ in range(reps):
        ab["batch"].append(time_graph(batch, steps, warmup) * 1e6)
        ab["planned"].append(time_graph(planned, steps, warmup) * 1e6)
    b, p = np.array(ab["batch"]), np.array(ab["planned"])
    gain = b - p
    return {"batch": round(float(np.median(b)), 2), "planned": round(float(np.median(p)), 2),
            "batch_min_max": [round(float(b.min()), 2), round(float(b.max()), 2)],
            "planned_min_max": [round(float(p.min()), 2), round(float(p.max()), 2)],
            "gain_us_median": round(float(np.median(gain)), 2),
            "gain_us_min_max": [round(float(gain.min()), 2), round(float(gain.max()), 2)],
            "settled": bool(gain.min() > 0 or gain.max() < 0),
            "how": f"graph replay, batch and planned forms alternating, {reps} repetitions "
                   "of the median of 5 replays each"}


def matched_stream(read_b: int, write_b: int, inplace: bool, sets: int, rotate_reads: bool,
                   use_graph: bool, steps: int, warmup: int) -> dict:
    """A plain stream of a workload's own traffic (pkv_stream_mix): the same
    bytes read and written, interleaved at the same ratio (in place when the
    workload rewrites what it reads), over the same number of rotating output
    buffers (and input buffers, where the workload rotates its inputs too),
    timed the same way as the workload (graph replay or eager launches); the
    best of a sweep of grid sizes.  Its time is what moving those bytes
    costs here with no address chain, no arithmetic and no lane geometry."""
    import torch
    import paged_kv_cache_wavefront_amd as pkv
    r16 = -(-read_b // 16) * 16
    w16 = r16 if inplace else -(-write_b // 16) * 16
    if inplace:
        bufs = [torch.empty(r16, dtype=torch.uint8, device="cuda") for _ in range(sets)]
        pairs = [(b, b) for b in bufs]
    else:
        srcs = [torch.empty(max(r16, 16), dtype=torch.uint8, device="cuda")
                for _ in range(sets if rotate_reads else 1)]
        dsts = [torch.empty(max(w16, 16), dtype=torch.uint8, device="cuda") for _ in range(sets)]
        pairs = [(srcs[i % len(srcs)], d) for i, d in enumerate(dsts)]
    per = {}
    for blocks in (256, 1024, 4096, 16384, 65536):
        fn = cycle([(lambda s_, d_: lambda: pkv.pkv_stream_mix(d_, s_, r16, w16, blocks))(s_, d_)
                    for s_, d_ in pairs])
        if use_graph:
            t = time_graph(fn, steps, warmup)
        else:
            _, t, _ = time_launches(fn, steps, warmup, spread_samples=1)
        per[blocks] = t
    best = min(per, key=per.get)
    del pairs
    return {"read_bytes": r16, "write_bytes": w16, "in_place": inplace, "buffer_sets": sets,
            "inputs_rotate": bool(rotate_reads or inplace),
            "us": round(per[best] * 1e6, 2), "blocks": best,
            "GBps": round((r16 + w16) / per[best] / 1e9, 1),
            "us_by_blocks": {b: round(v * 1e6, 2) for b, v in per.items()},
            "timed_as": "hip graph replay" if use_graph else "eager launches"}


_FLOOR = {}


def launch_floor(blocks: int) -> float:
    """Graph-replay time (us) of an almost empty launch (a 16-byte
    pkv_stream_mix) of `blocks` blocks of 256 threads: the fixed cost of a
    launch of that grid, below which no kernel of that grid can go."""
    if blocks not in _FLOOR:
        import torch
        import paged_kv_cache_wavefront_amd as pkv
        a = torch.empty(16, dtype=torch.uint8, device="cuda")
        b = torch.empty(16, dtype=torch.uint8, device="cuda")
        _FLOOR[blocks] = round(
            time_graph(lambda: pkv.pkv_stream_mix(b, a, 16, 16, blocks), 100, 3) * 1e6, 2)
    return _FLOOR[blocks]


def grid_blocks(name: str, case, rows: int = 0) -> int:
    """Blocks of 256 threads (4 waves) the entry point launches for a
    workload, as its launch code sizes the grid: MLA one wave per token and
    chunk of 32 heads (16 for at most 16 heads); Q/K RoPE one per token and
    chunk of 16 heads of 128; K norm and the token plan one per token; gather
    one per 6 rows."""
    if name.startswith("mla_"):
        hpw = 32 if case.H > 16 else 16
        waves = case.T * -(-case.H // hpw)
    elif name.startswith("qk_generic"):
        waves = case.T * -(-int(case.q.shape[1]) // 16)
    elif name.startswith("kv_norm"):
        waves = case.T
    elif name == "gather":
        waves = -(-rows // 6)
    else:
        raise ValueError(name)
    return -(-waves // 4)


def with_references(name, r, case, steps, warmup, use_graph):
    """The workload's figures beside a matched stream of its own traffic and
    the empty-launch floor of its grid (both measured now, in this run)."""
    total = r["bytes"]
    w = written_bytes(name, case, r["T"] if name == "gather" else 0)
    spec = r["stream_spec"]
    ms = matched_stream(total - w, w, spec["in_place"], spec["sets"], spec["rotate_reads"],
                        use_graph, steps, warmup)
    t = r["graph_avg"] if use_graph and r["graph_avg"] else r["avg"]
    blocks = grid_blocks(name, case, r["T"] if name == "gather" else 0)
    return {"matched_stream": ms,
            "pct_of_matched_stream": round(100.0 * ms["us"] * 1e-6 / t, 1),
            "launch_floor_us": launch_floor(blocks), "grid_blocks": blocks}


def run_workload(name, steps, warmup):
    """(summary, label, case) for one named workload of any entry point; the
    summary's "sets" is the number of buffer sets the steps rotate over."""
    import torch
    import workloads
    import paged_kv_cache_wavefront_amd as pkv
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_helpers as gh
    if name == "mla_prefill_inplace":
        case = workloads.NAMED[name]()
        written = case.q.size * 2 + case.T * case.latent.shape[1] * 2
        set_bytes = 2 * case.q.nbytes + case.cache.nbytes
        n = rotation_count(written, set_bytes)
        devs = [gh.MlaDevice(case) for _ in range(n)]
        for d in devs:
            d.place_rows()
        fns = [d.run_inplace for d in devs]
        how = f"{n} sets of q, q_out and bf16 cache pool"
        spec = dict(in_place=False, sets=n, rotate_reads=True)
        r = measure(cycle(fns), case.T, mla_bytes(case), steps, warmup)
        label = name
    elif name.startswith("mla_") and name.endswith("_planned"):
        # one plan per batch layout, built before the timed region (every
        # layer of a model step reuses it); the plan build is timed on its own
        case = workloads.NAMED[name[: -len("_planned")]]()
        dev = gh.MlaDevice(case)
        plan = torch.empty((case.T, 4), dtype=torch.int32, device="cuda")
        pkv.pkv_token_plan(plan, dev.offsets, dev.desc)
        n = rotation_count(case.q.size * 2, case.q.size * 2, cap=256)
        outs = [dev.q_out] + [torch.empty_like(dev.q_out) for _ in range(n - 1)]

        def make(o):
            return lambda: pkv.mla_rope_rmsnorm_quant_planned(o, dev.q_in, dev.latent, plan,
                                                              dev.freqs, dev.gamma,
                                                              case.epsilon, dev.desc,
                                                              case.layer_idx)
        fns = [make(o) for o in outs]
        plans = [torch.empty_like(plan) for _ in range(4)]

        def make_plan(p):
            return lambda: pkv.pkv_token_plan(p, dev.offsets, dev.desc)
        build = measure(cycle([make_plan(p) for p in plans]), case.T, plan_bytes(case), steps,
                        warmup)
        devs = (dev, outs, plan, plans)
        how = (f"{n} q_out buffers (one cache pool and one plan; the new rows are "
               f"{case.T * 576} bytes)")
        spec = dict(in_place=False, sets=n, rotate_reads=False)
        r = measure(cycle(fns), case.T, mla_bytes(case, planned=True), steps, warmup)
        r["plan_build"] = {"entry_point": "pkv_token_plan", "timed_as": "hip graph replay",
                           "us": round(build["graph_avg"] * 1e6, 2),
                           "bytes": plan_bytes(case)}
        # the batch form on the same buffers, the two graph-replay timings
        # alternating (figures of separate runs drift by a few tenths of a us)
        batch = cycle([(lambda o: lambda: pkv.mla_rope_rmsnorm_quant(
            o, dev.q_in, dev.latent, dev.offsets, dev.freqs, dev.gamma, case.epsilon, dev.desc,
            case.layer_idx))(o) for o in outs])
        planned_fn = cycle(fns)
        r["vs_batch_form"] = alternate(batch, planned_fn, steps, warmup)
        label = f"{name} (plan built once, outside the timed launches)"
    elif name.startswith("mla_"):
        case = workloads.NAMED[name]()
        q_out_bytes = case.q.nbytes
        written = q_out_bytes + case.T * case.latent.shape[1]
        set_bytes = 2 * q_out_bytes + case.latent.nbytes + case.cache.nbytes
        n = rotation_count(written, set_bytes)
        if n * written >= ROTATE_BYTES:
            # whole device sets: inputs, outputs and cache pool
            devs = [gh.MlaDevice(case) for _ in range(n)]
            fns = [d.run for d in devs]
            how = f"{n} sets of q, q_out, latent and cache pool"
            spec = dict(in_place=False, sets=n, rotate_reads=True)
        else:
            # the pool is large and the new rows few: rotate q_out only
            n = rotation_count(q_out_bytes, q_out_bytes, cap=256)
            dev = gh.MlaDevice(case)
            outs = [dev.q_out] + [torch.empty_like(dev.q_out) for _ in range(n - 1)]

            def make(o):
                return lambda: pkv.mla_rope_rmsnorm_quant(o, dev.q_in, dev.latent, dev.offsets,
                                                          dev.freqs, dev.gamma, case.epsilon,
                                                          dev.desc, case.layer_idx)
            fns = [make(o) for o in outs]
            devs = (dev, outs)
            how = f"{n} q_out buffers (one cache pool; its new rows are {case.T * 576} bytes)"
            spec = dict(in_place=False, sets=n, rotate_reads=False)
        r = measure(cycle(fns), case.T, mla_bytes(case), steps, warmup)
        label = name
    elif name.startswith("qk_generic"):
        case = workloads.NAMED[name]()
        written = case.q.nbytes + int(gh.written_k_rows(case).sum()) * case.k_cache[0, 0, 0].nbytes
        set_bytes = 2 * case.q.nbytes + case.k_cache.nbytes
        n = rotation_count(written, set_bytes)
        devs = [gh.QkDevice(case) for _ in range(n)]
        fns = [(lambda d: (lambda: d.rope(True)))(d) for d in devs]
        how = f"{n} sets of q, q_out and K pool"
        spec = dict(in_place=False, sets=n, rotate_reads=True)
        r = measure(cycle(fns), case.T, qk_bytes(case, True), steps, warmup)
        label = f"{name} (interleaved, position ids, fused per-head K norm; Q {case.q.dtype}, freqs {case.freqs.dtype})"
    elif name in ("kv_norm", "kv_norm_planned"):
        planned = name == "kv_norm_planned"
        case = workloads.qk_generic()
        written = int(gh.written_k_rows(case).sum()) * case.k_cache[0, 0, 0].nbytes
        n = rotation_count(written, case.k_cache.nbytes)
        base = gh.QkDevice(case)
        descs = []
        pools = [base.k] + [base.k.clone() for _ in range(n - 1)]
        for pool in pools:
            descs.append(pkv.paged_cache(pool, base.cache_lengths, base.page_table,
                                         pkv.PKV_SCALE_NONE, None, base.error_count))

        def make(dsc):
            return lambda: pkv.rms_norm_kv_cache_paged(dsc, case.layer_idx, base.gamma,
                                                       case.epsilon, 0.0, case.T, base.offsets,
                                                       True, True)
        plan = torch.empty((case.T, 4), dtype=torch.int32, device="cuda")
        pkv.pkv_token_plan(plan, base.offsets, descs[0])

        def make_planned(dsc):
            return lambda: pkv.rms_norm_kv_cache_paged_planned(dsc, case.layer_idx, base.gamma,
                                                               case.epsilon, 0.0, case.T, plan,
                                                               True, True)
        fns = [(make_planned if planned else make)(d) for d in descs]
        devs = (base, pools, descs, plan)
        how = f"{n} K pools"
        spec = dict(in_place=True, sets=n, rotate_reads=True)
        r = measure(cycle(fns), case.T, kv_norm_bytes(case, 128, planned), steps, warmup)
        label = "qk_generic K cache (8 heads x 128, gamma 128)"
        if planned:
            label += ", placed by a token plan built once"
            batch, planned_fn = cycle([make(d) for d in descs]), cycle(fns)
            r["vs_batch_form"] = alternate(batch, planned_fn, steps, warmup)
    elif name == "gather":
        case = workloads.mla_decode()
        ctx = case.cache_lengths.astype(np.int64) + 1
        kvo = np.zeros(ctx.size + 1, np.uint32)
        kvo[1:] = np.cumsum(ctx)
        rows = int(kvo[-1])
        cache = gh.dev_u8(case.cache)
        desc = pkv.paged_cache(cache, None, gh.dev_u32(case.page_table), pkv.PKV_SCALE_PER_TENSOR,
                               gh.dev_f32(np.array([case.tensor_scale], np.float32)))
        kv = gh.dev_u32(kvo)
        n = rotation_count(rows * 1152, rows * 1152)
        outs = [torch.empty((rows, 576), dtype=torch.bfloat16, device="cuda") for _ in range(n)]

        def make(o):
            return lambda: pkv.mla_gather_latent_paged(o, kv, desc, case.layer_idx)
        fns = [make(o) for o in outs]
        devs = (cache, kv, outs, desc)
        how = f"{n} output buffers"
        spec = dict(in_place=False, sets=n, rotate_reads=False)
        r = measure(cycle(fns), rows, gather_bytes(rows, case.B, case.meta["page_size"]), steps,
                    warmup)
        label = f"gather of {case.B} request contexts ({rows} rows) fp8 -> bf16"
    else:
        raise ValueError(name)
    r["keep"] = devs
    r["sets"] = how
    r["stream_spec"] = spec
    return r, label, case


def measure_siblings(main, steps, warmup):
    out = {}
    for name, entry in (("mla_decode", "mla_rope_rmsnorm_quant"),
                        ("mla_mixed", "mla_rope_rmsnorm_quant"),
                        ("mla_decode_planned", "mla_rope_rmsnorm_quant_planned"),
                        ("mla_mixed_planned", "mla_rope_rmsnorm_quant_planned"),
                        ("mla_prefill_inplace", "mla_rope_rmsnorm_inplace"),
                        ("mla_prefill_f16", "mla_rope_rmsnorm_quant"),
                        ("qk_generic", "qk_rope_paged_ragged"),
                        ("qk_generic_f16", "qk_rope_paged_ragged"),
                        ("kv_norm", "rms_norm_kv_cache_paged"),
                        ("kv_norm_planned", "rms_norm_kv_cache_paged_planned"),
                        ("gather", "mla_gather_latent_paged")):
        if name == main:
            continue
        log(f"[bench] sibling {name}")
        r, label, case = run_workload(name, steps, warmup)
        out[name] = {"entry_point": entry, **summarize(label, r, steps, use_graph=True),
                     "traffic": profiled_traffic(name),
                     **with_references(name, r, case, steps, warmup, use_graph=True)}
        if "plan_build" in r:
            out[name]["plan_build"] = r["plan_build"]
        if "vs_batch_form" in r:
            out[name]["vs_batch_form_us"] = r["vs_batch_form"]
        del r
    return out


def token_chunks(case, n: int):
    """Split the batch into n sub-batches of (nearly) equal token counts for
    the multi-threaded oracle leg.  A request cut in two keeps its slots: the
    later part's prior length is where the earlier part ends.  Returns
    (row_offsets, cache_lengths, page_table) per chunk; token indices stay
    absolute, so every chunk writes its own rows of the shared outputs."""
    offs = case.row_offsets.astype(np.int64)
    clens = case.cache_lengths.astype(np.int64)
    bounds = np.linspace(0, int(offs[-1]), n + 1).astype(np.int64)
    chunks = []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        ro, cl, rows = [int(lo)], [], []
        for b in range(offs.size - 1):
            s, e = max(int(offs[b]), int(lo)), min(int(offs[b + 1]), int(hi))
            if s >= e:
                continue
            ro.append(e)
            cl.append(int(clens[b]) + s - int(offs[b]))
            rows.append(b)
        if rows:
            chunks.append((np.array(ro, np.uint32), np.array(cl, np.uint32),
                           np.ascontiguousarray(case.page_table[rows])))
    return chunks


def cpu_model() -> str:
    """The host CPU's name: /proc/cpuinfo's model name, with lscpu's when that
    is longer, and the family / model / stepping numbers (some hosts report
    only a family name such as "AMD EPYC")."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k = k.strip()
            if k in ("model name", "cpu family", "model", "stepping") and k not in info:
                info[k] = v.strip()
    except OSError:
        pass
    name = info.get("model name", "unknown")
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                alt = line.split(":", 1)[1].strip()
                if len(alt) > len(name):
                    name = alt
    except (OSError, subprocess.SubprocessError):
        pass
    ids = ", ".join(f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info)
    return f"{name} ({ids})" if ids else name


# Host threads for the multi-threaded oracle leg: the cores this process may
# run on, capped at the host CPU share of one GPU on the boxes this runs on
# (16 threads; OMP_NUM_THREADS carries the same figure there).
CPU_SHARE = 16


def cpu_baseline(case, budget_s=10.0):
    """The oracle (C, binary64) on the same host arrays, as it stands: called
    from N host threads at once on N token-balanced slices of the batch
    (ctypes releases the GIL, so the calls run in parallel) for about
    budget_s -- the reported figure, cores = N -- and single-threaded over the
    whole workload for about budget_s / 2 (``single_thread``); the threaded
    outputs are checked bit for bit against the single-threaded run."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    orc = oracle.default()
    q_out = np.zeros_like(case.q)
    bytes_per_token = mla_bytes(case) / max(case.T, 1)  # the same byte model as the GPU line

    def whole(cache):
        orc.mla_rope_rmsnorm_quant(q_out, case.q, case.latent, case.row_offsets,
                                   case.cache_lengths, case.page_table, case.freqs, case.gamma,
                                   case.epsilon, cache, case.layer_idx, case.scale_mode,
                                   case.tensor_scale, None)

    tokens, t0 = 0, time.perf_counter()
    runs = 0
    while True:
        cache = case.cache.copy()
        t1 = time.perf_counter()
        whole(cache)
        runs += 1
        tokens += case.T
        spent = time.perf_counter() - t0
        if spent >= budget_s / 2 or (time.perf_counter() - t1) * (runs + 1) > 1.5 * budget_s:
            break
    single_s = time.perf_counter() - t0
    single = {"value": round(tokens / single_s, 1), "unit": "tokens/s", "cores": 1,
              "GBps": round(tokens / single_s * bytes_per_token / 1e9, 3),
              "sample": f"whole workload ({case.T} tokens) x {runs} run(s), {single_s:.1f} s, "
                        "one thread"}

    affinity = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    share = int(omp) if omp.isdigit() and int(omp) > 0 else CPU_SHARE
    n = max(1, min(affinity, share))
    chunks = token_chunks(case, n)
    q_par = np.zeros_like(case.q)

    def part(args, cache):
        ro, cl, pt = args
        orc.mla_rope_rmsnorm_quant(q_par, case.q, case.latent, ro, cl, pt, case.freqs,
                                   case.gamma, case.epsilon, cache, case.layer_idx,
                                   case.scale_mode, case.tensor_scale, None)

    tokens, runs = 0, 0
    with ThreadPoolExecutor(len(chunks)) as ex:
        t0 = time.perf_counter()
        while True:
            cache_par = case.cache.copy()
            list(ex.map(lambda c: part(c, cache_par), chunks))
            runs += 1
            tokens += case.T
            if time.perf_counter() - t0 >= budget_s:
                break
        par_s = time.perf_counter() - t0
    same = bool(np.array_equal(q_par, q_out) and np.array_equal(cache_par, cache))
    out = {"value": round(tokens / par_s, 1), "unit": "tokens/s", "cores": len(chunks),
           "kind": "oracle",
           "sample": f"whole workload ({case.T} tokens) x {runs} run(s), {par_s:.1f} s, "
                     f"{len(chunks)} host threads on token-balanced slices",
           "GBps": round(tokens / par_s * bytes_per_token / 1e9, 3),
           "cpu_model": cpu_model(), "affinity_cores": affinity,
           "threads_cap": f"min(affinity {affinity}, host CPU share of one GPU {share})",
           "same_bits_as_single_thread": same,
           "single_thread": single}
    return out, (q_out, cache)


ELEM_NAME = {np.dtype(np.uint16): "bf16", np.dtype(np.float16): "fp16", np.dtype(np.float32): "fp32"}


def io_dtypes(name: str, case) -> str:
    """The element types a workload's launch reads and writes."""
    if name == "gather":
        return "fp8 e4m3fn cache rows in, bf16 rows out"
    q, fr = ELEM_NAME[case.q.dtype], ELEM_NAME[case.freqs.dtype]
    if not name.startswith("mla_"):
        return f"{q} Q in and out, bf16 K rows in place, {fr} freqs" if name.startswith("qk_") \
            else "bf16 K rows in place, bf16 gamma"
    g = ELEM_NAME[case.gamma.dtype]
    if name == "mla_prefill_inplace":
        return f"{q} q in and out; bf16 latent rows read and rewritten in the cache; {fr} freqs, {g} gamma"
    return f"{q} q in and out; bf16 latent in; fp8 e4m3fn cache rows out; {fr} freqs, {g} gamma"


def parity_stats(case, oracle_out):
    """One launch of the timed entry point on fresh device copies of the
    workload, compared with the oracle's outputs from the CPU baseline (same
    inputs): q within bf16 steps, cache codes within fp8 steps on the new
    rows, every other cache byte unchanged.  Reported, not asserted (the
    tests hold the bars)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_helpers as gh
    dev = gh.MlaDevice(case)
    dev.run()
    q, cache, _, skipped = dev.results()
    q_o, cache_o = oracle_out
    rows = gh.written_rows(case)
    dq = gh.f16_ulp_diff(q, q_o) if q_o.dtype == np.float16 else gh.bf16_ulp_diff(q, q_o)
    dc = gh.fp8_ulp_diff(cache[rows], cache_o[rows]) if cache.dtype == np.uint8 else \
        gh.bf16_ulp_diff(cache[rows], cache_o[rows])
    return {"q_max_ulp": int(dq.max(initial=0)),
            "q_diff_frac": float((dq != 0).sum() / max(dq.size, 1)),
            "cache_max_step": int(dc.max(initial=0)),
            "cache_diff_frac": float((dc != 0).sum() / max(dc.size, 1)),
            "untouched_ok": bool(np.array_equal(cache[~rows], case.cache[~rows])),
            "skipped_tokens": int(skipped),
            "against": "the oracle's outputs of the cpu_baseline run"}


def calibrate_copy(steps, warmup, mib=1024):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    wall, avg, durs = time_launches(lambda: torch.neg(src, out=dst), steps, warmup)
    nbytes = 2 * n * 4
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "bytes_written": n * 4,
                      "kernel_us_avg": round(avg * 1e6, 2),
                      "GBps": round(nbytes / avg / 1e9, 1)}))


def measured_copy(steps, warmup, mib=300):
    """A plain streaming copy on the same GPU (pkv_stream_copy: 16-byte
    non-temporal loads and stores, mib MiB each way, about the prefill step's
    byte volume), the best over a sweep of grid sizes: the bandwidth a
    read-and-write stream of that size reaches here, for context."""
    import torch
    import paged_kv_cache_wavefront_amd as pkv
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    per = {}
    for blocks in (1024, 4096, 16384, 65536):
        _, avg, _ = time_launches(lambda: pkv.pkv_stream_copy(dst, src, blocks), steps, warmup,
                                  spread_samples=1)
        per[blocks] = round(2 * src.numel() / avg / 1e9, 1)
    best = max(per, key=per.get)
    return {"GBps": per[best], "bytes_per_copy": 2 * src.numel(), "blocks": best,
            "GBps_by_blocks": per,
            "how": f"pkv_stream_copy of {mib} MiB, device to device, average of {steps} "
                   "launches, best grid"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mla_prefill",
                    choices=["mla_prefill", "mla_decode", "mla_mixed", "mla_tiny",
                             "mla_prefill_inplace", "mla_decode_planned", "mla_mixed_planned",
                             "mla_prefill_f16", "qk_generic", "qk_generic_f16", "kv_norm",
                             "kv_norm_planned", "gather"])
    ap.add_argument("--no-siblings", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--no-references", action="store_true",
                    help="skip the streaming-copy and matched-stream reference measurements "
                         "(for profiler runs that only need the workload's own launches)")
    ap.add_argument("--source-hash", action="store_true",
                    help="print the hash of the workload's kernel sources and exit")
    args = ap.parse_args()
    if args.source_hash:
        print(kernel_source_hash(args.workload))
        return
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path needs no inter-GPU exchange and is measured on a single MI355X.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no ROCm GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.steps, args.warmup)
        return
    log(f"[bench] workload {args.workload}; timing {args.steps} steps")
    r, label, case = run_workload(args.workload, args.steps, args.warmup)
    main_sum = summarize(label, r, args.steps)
    gbps = main_sum["effective_GBps"]
    siblings = None if args.no_siblings else measure_siblings(
        args.workload, max(20, args.steps // 2), args.warmup)
    cpu = parity = None
    if (not args.no_cpu_baseline and args.workload.startswith("mla_")
            and not args.workload.endswith("_planned")):
        log("[bench] cpu baseline (oracle)")
        cpu, oracle_out = cpu_baseline(case)
        if args.workload != "mla_prefill_inplace":
            parity = parity_stats(case, oracle_out)
    copy_ref = refs = None
    if not args.no_references:
        copy_ref = measured_copy(args.steps, args.warmup)
        refs = with_references(args.workload, r, case, args.steps, args.warmup, use_graph=False)
    traffic = profiled_traffic(args.workload)
    is_mla = args.workload.startswith("mla_")
    if is_mla:
        config = {"workload": args.workload, "tokens": case.T, "requests": case.B,
                  "q_heads": case.H, "rope_dim": case.R, "kv_norm_dim": case.Dn,
                  "page_size": case.meta["page_size"], "scale_mode": case.scale_mode,
                  "parallelism": "single GPU"}
    elif args.workload == "gather":
        config = {"workload": args.workload, "rows": r["T"], "requests": case.B,
                  "row": "576 fp8 -> 576 bf16", "page_size": case.meta["page_size"],
                  "parallelism": "single GPU"}
    else:
        config = {"workload": args.workload, "tokens": case.T, "requests": case.B,
                  "q_heads": int(case.q.shape[1]), "kv_heads": int(case.k_cache.shape[3]),
                  "head_dim": int(case.q.shape[2]), "page_size": case.meta["page_size"],
                  "parallelism": "single GPU"}
    line = {
        "metric": METRIC if is_mla else f"{label}: tokens/s and effective HBM GB/s",
        "value": round(r["T"] * args.steps / r["wall"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtypes": io_dtypes(args.workload, case),
        "data": "synthetic (seeded; DeepSeek-V3-shaped random tensors, no weights)",
        "config": config,
        "effective_GBps": gbps,
        "pct_of_hbm_peak": main_sum["pct_of_hbm_peak"],
        "buffer_rotation": main_sum["buffer_rotation"],
        "measured_copy": copy_ref,
        "pct_of_measured_copy": round(100.0 * gbps / copy_ref["GBps"], 1) if copy_ref else None,
        **(refs or {}),
        "kernel_us": {k: main_sum[k] for k in ("kernel_us_avg", "eager_us_p10_p50_p90",
                                               "cold_us_p10_p50_p90", "graph_us_avg")},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": r["bytes"]},
        "cpu_baseline": cpu,
        "parity": parity,
        "siblings": siblings,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
