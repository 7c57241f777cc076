"""Benchmark: NSA selected-attention forward (FSA order) on one MI355X.

One step = the whole path on one batch of synthetic input already resident in
HBM: index build (fsa_build_index), softmax statistics (fsa_softmax_stats),
main kernel (fsa_selected_attn_main) and reduction (fsa_selected_attn_reduce).
Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--partial input|fp32] [--no-cpu-baseline] [--no-variants]
                    [--no-query-outer] [--no-backward] [--no-selection]
                    [--onepass] [--graph] [--cold-reps R]

With the default workload (the 64K-token, 4 KV-head, g = 4 latency shape) the
line also carries every other workload of the benchmark set under `variants`:
the 1K and 8K shapes, the 64K fp16 g = 1 shape, the two packed 32K-token
sequences with d = 256 and g = 8, the 64K bf16 shape at g = 2 and g = 1, and
the 64K shape with 128-key blocks and the 32K shape with 128-key blocks at
d = 256, each with its stage times, TFLOP/s and the
main stage's fractions of the MFMA and HBM peaks.

The query-outer forward (fsa_nsa_selected_attn_fwd, the vanilla NSA loop
order) is timed on the same inputs and reported beside the step, with the
FSA-order speedup over it; so is the backward (fsa_selected_attn_bwd) from the
step's O and lse, with its algorithmic TFLOP/s (10 g d flops per visible key),
and block selection (fsa_select_blocks, the step that produces Sel) on
synthetic scores of the same shape, with its HBM rate on the causal scores read.

Besides the mean over back-to-back steps (`value`, `stages_ms`), the line
carries the median and minimum step time, the same step timed R more times
each after a 1 GiB fill that evicts the L2s and the MALL (`cold_cache`), and
what this GPU reaches on a plain device copy and a large GEMM
(`measured_peaks`), with the main kernel's fractions of both.

Throughput is algorithmic TFLOP/s: 4 * g * d * (sum over (token, KV head) of
the number of keys the token attends to), i.e. QK^T and PV over the visible
keys only, divided by the step time.
"""

from __future__ import annotations

import argparse
import json
import re
import math
import os
import sys
import time

import numpy as np

METRIC = "selected-attn fwd latency (ms) + TFLOP/s at 64K tokens, g=1/2/4; % MFMA peak"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, GB/s
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}  # dense MFMA
DEFAULT_WORKLOAD = "n64k_h4_g4_d128_t16_bf16"
VARIANTS = [
    "n1k_h1_g1_d64_t4_bf16",
    "n8k_h4_g2_d128_t16_bf16",
    "n64k_h4_g1_d128_t16_fp16",
    "b2_n32k_h8_g8_d256_t16_bf16",
    "n64k_h4_g2_d128_t16_bf16",
    "n64k_h4_g1_d128_t16_bf16",
    "n64k_h4_g4_d128_b128_t8_bf16",
    "n32k_h4_g4_d256_b128_t8_bf16",
]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--partial", default="input", choices=["input", "fp32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-query-outer", action="store_true",
                    help="skip timing the query-outer (vanilla NSA order) forward")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward pass")
    ap.add_argument("--no-selection", action="store_true", help="skip timing block selection")
    ap.add_argument("--onepass", action="store_true",
                    help="also time the one-pass forward (statistics fused into main and reduction)")
    ap.add_argument("--graph", action="store_true", help="also time the step captured in a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target wall time of the CPU baseline")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="extra steps timed after a 1 GiB cache-evicting fill each (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of 1 GiB (5 times): the known-size kernel "
                         "against which HBM byte counters are scaled")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Work accounting (host bookkeeping for the FLOP and byte counts)
# ---------------------------------------------------------------------------
def work_counts(sel, cu, block_size):
    """Number of selecting entries P, the local ones among them (entries of
    the token's own, previous or first block, which the forward computes per
    query block) and total visible keys over all (KV head, token) rows.  An
    entry selects block e of the token's sequence iff 0 <= e <= own block and
    e did not occur earlier in the row; it sees the whole block, or only keys
    <= t in the own block."""
    cu = np.asarray(cu, dtype=np.int64)
    n = int(cu[-1])
    tok = np.arange(n)
    seq = np.searchsorted(cu, tok, side="right") - 1
    local = tok - cu[seq]
    own = local // block_size
    H, _, T = sel.shape
    pairs = 0
    local_pairs = 0
    keys = 0
    for h in range(H):
        s = sel[h]
        ok = (s >= 0) & (s <= own[:, None])
        for j in range(1, T):
            ok[:, j] &= ~np.any(s[:, :j] == s[:, j : j + 1], axis=1)
        pairs += int(ok.sum())
        local_pairs += int((ok & ((s == own[:, None]) | (s == own[:, None] - 1) | (s == 0))).sum())
        full = ok & (s < own[:, None])
        mine = ok & (s == own[:, None])
        keys += int(full.sum()) * block_size + int(((local % block_size + 1)[:, None] * mine).sum())
    return pairs, local_pairs, keys


KERNEL_SOURCES = ("fsa_attn.hip", "fsa_internal.h", "fsa_index.hip", "fsa_api.hip")


def measured_traffic(workload):
    """HBM bytes per launch of the main kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE record of this workload, or None when there is no
    record or the kernel sources changed since it was taken."""
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash(root):
        return None
    return rec


def kernel_source_hash(root):
    """SHA-256 of the forward kernels' sources with comments and blank lines
    removed, so that the traffic record follows changes of the code only."""
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(root, "sparse_attention_sel_amd", "csrc", name)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            line = re.sub(r"//.*", "", line).strip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def main_stage_kernels(w):
    """The three-pass main stage's kernels as the library launches them: with
    local entries (B_K = 64, g >= 2), k_main_mixed (k_main_mixed16 at d = 256)
    where the per-query-block items (KV head, block, 128-row group; in units of
    four blocks, a whole number per XCD) fill four rounds of its persistent
    grid (256 CUs times two workgroups per CU, one at d = 256), unless
    FSA_MAIN_MIXED says otherwise."""
    B, g, d = w.block_size, w.gqa_group, w.head_dim
    if B != 64 or g < 2:
        return "k_main16" if d == 256 or B == 128 and d == 128 else "k_main"
    nb = sum(-(-int(w.cu_seqlens[i + 1] - w.cu_seqlens[i]) // B) for i in range(len(w.cu_seqlens) - 1))
    units = -(-w.num_kv_heads * nb // 4)
    items = -(-units // 8) * 8 * 4 * -(-B * g // 128)
    env = os.environ.get("FSA_MAIN_MIXED")
    mixed = env == "1" or (env != "0" and items >= 4 * (1 if d == 256 else 2) * 256)
    if d == 256:
        return "k_main_mixed16" if mixed else "k_main_local16+k_main16"
    return "k_main_mixed" if mixed else "k_main_local+k_main"


def kernel_bytes(w, P, P_loc, s_in, s_p):
    """Compulsory HBM bytes of each stage (each input read once, each output
    written once).  Block-outer kernels take the P - P_loc non-local pairs;
    the local entries of a (KV head, token) give one partial row group and one
    (max, sum) pair per query head (P_loc = 0 where the local path does not
    run: then the local rows, pairs and words drop out)."""
    N, H, g, d, T = int(w.cu_seqlens[-1]), w.num_kv_heads, w.gqa_group, w.head_dim, w.topk
    HQ = H * g
    Pn = P - P_loc
    has_local = 1 if P_loc else 0
    q_bytes = N * HQ * d * s_in
    kv_bytes = 2 * N * H * d * s_in
    loc = 4 * H * N * has_local
    local_rows = N * HQ * d * s_p * has_local
    main = q_bytes + kv_bytes + N * HQ * 4 + Pn * 4 + Pn * g * d * s_p + local_rows + loc
    reduce = Pn * g * d * s_p + local_rows + H * N * T * 4 + loc + N * HQ * d * s_in
    stats = (q_bytes + kv_bytes // 2 + Pn * 4 + 2 * Pn * g * 8 + 2 * N * HQ * 8 * has_local + H * N * T * 4 + loc
             + 2 * N * HQ * 4)
    index = 3 * H * N * T * 4 + P * 4 + loc
    return {"index": index, "stats": stats, "main": main, "reduce": reduce}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, on a bounded sample of query tokens
# ---------------------------------------------------------------------------
_G = {}


def _oracle_shard(tokens):
    from threadpoolctl import threadpool_limits

    import oracle

    with threadpool_limits(1):
        oracle.selected_attention(_G["q"], _G["k"], _G["v"], _G["sel"], _G["cu"], _G["B"], _G["scale"], tokens)
    return len(tokens)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cgroup_cpus():
    """CPU quota of this process's cgroup (cgroup v2 cpu.max), or None."""
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        return None if quota == "max" else round(int(quota) / int(period), 2)
    except (OSError, ValueError):
        return None


def cpu_baseline(w, target_s):
    """The float64 oracle on a bounded sample of the workload's query tokens,
    in worker processes (one per core of this process's CPU share: the
    affinity set, at most 16, the share of a one-GPU machine), each with one BLAS
    thread; plus the index oracle (a stable sort over every entry) on the
    whole workload in this process.  Runs before the GPU is touched (the pool
    forks)."""
    import multiprocessing as mp

    import oracle

    q, k, v = (x.float().numpy() for x in (w.q, w.k, w.v))
    _G.update(q=q, k=k, v=v, sel=w.sel, cu=w.cu_seqlens, B=w.block_size, scale=w.scale)
    n = int(w.cu_seqlens[-1])
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(16, affinity))
    t0 = time.perf_counter()
    oracle.build_index(w.sel, w.cu_seqlens, w.block_size)
    index_s = time.perf_counter() - t0
    rng = np.random.default_rng(12345)
    # calibrate on one core
    probe = np.sort(rng.choice(n, size=min(32, n), replace=False))
    t0 = time.perf_counter()
    _oracle_shard(probe)
    per_tok = (time.perf_counter() - t0) / probe.size
    m = int(min(n, max(cores, target_s * cores / max(per_tok, 1e-9))))
    sample = np.sort(rng.choice(n, size=m, replace=False))
    shards = np.array_split(sample, cores * 4)
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_shard, shards)
    wall = time.perf_counter() - t0
    # algorithmic FLOPs of the sampled rows
    sub = w.sel[:, sample, :]
    cu = w.cu_seqlens.astype(np.int64)
    seq = np.searchsorted(cu, sample, side="right") - 1
    local = sample - cu[seq]
    own = local // w.block_size
    keys = 0
    for h in range(w.num_kv_heads):
        s = sub[h]
        ok = (s >= 0) & (s <= own[:, None])
        for j in range(1, s.shape[1]):
            ok[:, j] &= ~np.any(s[:, :j] == s[:, j : j + 1], axis=1)
        keys += int((ok & (s < own[:, None])).sum()) * w.block_size
        keys += int(((local % w.block_size + 1)[:, None] * (ok & (s == own[:, None]))).sum())
    flops = 4.0 * w.gqa_group * w.head_dim * keys
    return {
        "value": flops / wall / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{m} of {n} query tokens (all KV heads), uniform without replacement, seed 12345; "
                  f"{wall:.1f} s wall on {cores} worker processes, 1 BLAS thread each",
        "wall_s": round(wall, 3),
        "cpu_model": cpu_model(),
        "affinity_cpus": affinity,
        "cgroup_cpus": cgroup_cpus(),
        "index_oracle_s": round(index_s, 3),
        "index_oracle_sample": f"all {n} tokens, one process (numpy stable sort)",
    }


# ---------------------------------------------------------------------------
# GPU run
# ---------------------------------------------------------------------------
class _Skip(Exception):
    pass


def run_gpu(w, partial, steps, warmup, query_outer=False, backward=False, selection=False, cold_reps=0,
            onepass=False, graph=False):
    import torch

    import sparse_attention_sel_amd as fsa

    dev = torch.device("cuda:0")
    prob = fsa.Problem(
        w.cu_seqlens, w.num_kv_heads, w.gqa_group, w.head_dim, w.block_size, w.topk,
        dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float16,
        partial_dtype=partial, softmax_scale=w.scale, device=dev,
    )
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    sel = torch.from_numpy(w.sel).to(dev)
    index = fsa.allocate_index(prob, dev)
    ws = fsa.Workspaces(prob, dev, index.sizes)
    n, hq = prob.total_tokens, prob.num_q_heads
    lse = torch.empty((n, hq), dtype=torch.float32, device=dev)
    row_max = torch.empty((n, hq), dtype=torch.float32, device=dev)
    out = torch.empty((n, hq, prob.head_dim), dtype=prob.dtype, device=dev)
    stream = torch.cuda.current_stream()
    names = ["index", "stats", "main", "reduce"]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fsa.build_index(prob, sel, index, ws.build, stream)
        if ev is not None:
            ev[1].record(stream)
        fsa.softmax_stats(prob, q, k, index, row_max, lse, ws.stats, stream)
        if ev is not None:
            ev[2].record(stream)
        fsa.selected_attn_main(prob, q, k, v, index, lse, ws.partial, stream)
        if ev is not None:
            ev[3].record(stream)
        fsa.selected_attn_reduce(prob, index, ws.partial, out, stream)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = {nm: 0.0 for nm in names}
    for ev in events:
        for i, nm in enumerate(names):
            stage[nm] += ev[i].elapsed_time(ev[i + 1])
    stage = {nm: v_ / steps for nm, v_ in stage.items()}
    warm_steps = sorted(ev[0].elapsed_time(ev[4]) for ev in events)
    # cold caches: before each rep a 1 GiB fill evicts the L2s and the MALL,
    # so every input of the step comes from HBM
    cold = None
    if cold_reps:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(cold_reps)]
        for i in range(cold_reps):
            scratch.fill_(float(i))
            step(cev[i])
        torch.cuda.synchronize()
        per = {nm: sorted(ev[j].elapsed_time(ev[j + 1]) for ev in cev) for j, nm in enumerate(names)}
        tot = sorted(ev[0].elapsed_time(ev[4]) for ev in cev)
        cold = {
            "reps": cold_reps,
            "flush_bytes": scratch.numel() * 4,
            "step_ms_median": round(float(np.median(tot)), 4),
            "step_ms_min": round(tot[0], 4),
            "stages_ms_median": {nm: round(float(np.median(v_)), 4) for nm, v_ in per.items()},
            "stages_ms_min": {nm: round(v_[0], 4) for nm, v_ in per.items()},
        }
        del scratch
    # the query-outer (vanilla NSA loop order) forward on the same inputs,
    # timed the same way, for the loop-order comparison
    qo_ms = None
    if query_outer:
        try:
            fsa.nsa_selected_attn_fwd(prob, q, k, v, sel, lse, out, stream)
        except fsa.FsaError as e:  # no query-outer kernel for this shape
            log(f"query-outer leg skipped: {e}")
            query_outer = False
    if query_outer:
        for _ in range(2):
            fsa.nsa_selected_attn_fwd(prob, q, k, v, sel, lse, out, stream)
        qev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3)]
        for a, b in qev:
            a.record(stream)
            fsa.nsa_selected_attn_fwd(prob, q, k, v, sel, lse, out, stream)
            b.record(stream)
        torch.cuda.synchronize()
        qo_ms = sum(a.elapsed_time(b) for a, b in qev) / len(qev)
    # the same step captured once in a HIP graph and replayed (the library
    # allocates nothing and clears its counters with kernels, so the calls
    # capture as they are): what launch overhead costs at this size
    graph_ms = None
    try:
        if not graph:
            raise _Skip()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fsa.build_index(prob, sel, index, ws.build)
            fsa.softmax_stats(prob, q, k, index, row_max, lse, ws.stats)
            fsa.selected_attn_main(prob, q, k, v, index, lse, ws.partial)
            fsa.selected_attn_reduce(prob, index, ws.partial, out)
        graph.replay()
        torch.cuda.synchronize()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record(stream)
        for _ in range(steps):
            graph.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        graph_ms = ga.elapsed_time(gb) / steps
        del graph
    except _Skip:
        pass
    except RuntimeError as e:  # capture unsupported in this runtime: report none
        log(f"graph capture skipped: {e}")
    # the one-pass forward (fsa_selected_attn_fwd_onepass: the statistics fused
    # into the main kernel and the reduction) on the same inputs: index build
    # plus the fused call per step, timed like the step above
    op = None
    if onepass and w.block_size == 128 and w.head_dim == 256:
        log("one-pass leg skipped: no one-pass kernels for 128-key blocks at d = 256")
        onepass = False
    if onepass:
        o_lse, o_rm, o_out = torch.empty_like(lse), torch.empty_like(row_max), torch.empty_like(out)

        def ostep(ev):
            ev[0].record(stream)
            fsa.build_index(prob, sel, index, ws.build, stream)
            ev[1].record(stream)
            fsa.selected_attn_fwd_onepass(prob, q, k, v, index, o_rm, o_lse, o_out, ws.stats, ws.partial, stream)
            ev[2].record(stream)

        for _ in range(max(2, warmup)):
            ostep([torch.cuda.Event(enable_timing=True) for _ in range(3)])
        oev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for ev in oev:
            ostep(ev)
        torch.cuda.synchronize()
        owall = time.perf_counter() - t1
        op = {
            "ms_per_step": owall * 1e3 / steps,
            "index_ms": sum(ev[0].elapsed_time(ev[1]) for ev in oev) / steps,
            "fused_ms": sum(ev[1].elapsed_time(ev[2]) for ev in oev) / steps,
        }
        del o_lse, o_rm, o_out
    # the backward (fsa_selected_attn_bwd) from this forward's O and lse, for
    # a seeded output gradient, timed the same way
    bwd_ms = None
    if backward and index.sizes["bwd_ws_bytes"] > 0:
        from sparse_attention_sel_amd.inputs import make_dout

        do = make_dout(n, hq, prob.head_dim, w.dtype, 7).to(dev)
        wsb = fsa.Workspaces(prob, dev, index.sizes, backward=True)
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        for _ in range(2):
            fsa.selected_attn_bwd(prob, q, k, v, out, do, lse, index, dq, dk, dv, wsb.bwd, stream)
        bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in bev:
            a.record(stream)
            fsa.selected_attn_bwd(prob, q, k, v, out, do, lse, index, dq, dk, dv, wsb.bwd, stream)
            b.record(stream)
        torch.cuda.synchronize()
        bwd_ms = sum(a.elapsed_time(b) for a, b in bev) / len(bev)
        del wsb, dq, dk, dv, do
    # block selection (fsa_select_blocks) on synthetic recency-weighted scores
    # of this shape, init_blocks = 1, local_blocks = 2
    sel_ms = sel_bytes = None
    if selection:
        from sparse_attention_sel_amd.inputs import make_block_scores

        scores = torch.from_numpy(make_block_scores(w.seqlens, w.num_kv_heads, w.block_size, 17)).to(dev)
        sel_out = torch.empty_like(sel)
        fsa.select_blocks(prob, scores, 1, 2, sel_out, stream)
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in sev:
            a.record(stream)
            fsa.select_blocks(prob, scores, 1, 2, sel_out, stream)
            b.record(stream)
        torch.cuda.synchronize()
        sel_ms = sum(a.elapsed_time(b) for a, b in sev) / len(sev)
        own_blocks = sum(int(((np.arange(L) // w.block_size) + 1).sum()) for L in w.seqlens)
        sel_bytes = w.num_kv_heads * (4 * own_blocks + 4 * int(w.cu_seqlens[-1]) * w.topk)
        del scores, sel_out
    counts = index.counts.cpu().numpy()
    return {
        "ms_per_step": wall * 1e3 / steps,
        "step_ms_median": float(np.median(warm_steps)),
        "step_ms_min": warm_steps[0],
        "cold": cold,
        "selection_ms": sel_ms,
        "selection_bytes": sel_bytes,
        "query_outer_ms": qo_ms,
        "graph_ms_per_step": graph_ms,
        "onepass": op,
        "backward_ms": bwd_ms,
        "stage_ms": stage,
        "pairs": index.num_pairs(),
        "partial_ws_bytes": int(index.sizes["partial_ws_bytes"]),
        "n_valid": {"min": int(counts.min()), "median": float(np.median(counts)), "max": int(counts.max())},
    }


def measured_peaks(dtype):
    """What this GPU reaches on plain work: a 1 GiB device copy (bytes read +
    written per second), an 8192^3 GEMM in the workload's dtype through torch
    (hipBLASLt) and the library's MFMA loop (independent 32x32x16 MFMAs, eight
    four-wave workgroups per CU), each the median of 10 timed runs."""
    import torch

    import sparse_attention_sel_amd as fsa

    dev = torch.device("cuda:0")
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    n = 8192
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    a = torch.randn((n, n), device=dev, dtype=tdt)
    b = torch.randn((n, n), device=dev, dtype=tdt)

    def timed(fn):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for s, e in ev:
            s.record()
            fn()
            e.record()
        torch.cuda.synchronize()
        return float(np.median([s.elapsed_time(e) for s, e in ev])) * 1e-3

    t_copy = timed(lambda: dst.copy_(src))
    t_gemm = timed(lambda: torch.matmul(a, b))
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    mfma_dtype = torch.bfloat16 if dtype == "bf16" else torch.float16
    wgs, iters = 8 * torch.cuda.get_device_properties(dev).multi_processor_count, 2000
    loop_flops = fsa.mfma_loop(mfma_dtype, wgs, iters, sink)
    t_loop = timed(lambda: fsa.mfma_loop(mfma_dtype, wgs, iters, sink))
    out = {
        "copy_gbs": round(2 * src.numel() * 4 / t_copy / 1e9, 1),
        "gemm_tflops": round(2.0 * n ** 3 / t_gemm / 1e12, 1),
        "gemm_dtype": dtype,
        "mfma_loop_tflops": round(loop_flops / t_loop / 1e12, 1),
    }
    del src, dst, a, b, sink
    return out


def measure(w, partial, steps, warmup, query_outer=False, backward=False, selection=False, cold_reps=0,
            onepass=False, graph=False):
    P_host, P_loc, keys = work_counts(w.sel, w.cu_seqlens, w.block_size)
    if w.block_size != 64 or w.gqa_group < 2:
        P_loc = 0  # the library computes local entries per query block only with B_K = 64 and g >= 2
    r = run_gpu(w, partial, steps, warmup, query_outer, backward, selection, cold_reps, onepass, graph)
    assert r["pairs"] == P_host, (r["pairs"], P_host)
    f_alg = 4.0 * w.gqa_group * w.head_dim * keys
    f_main = 4.0 * w.gqa_group * w.block_size * w.head_dim * P_host
    s_in, s_p = 2, (2 if partial == "input" else 4)
    byts = kernel_bytes(w, P_host, P_loc, s_in, s_p)
    N, HQ = int(w.cu_seqlens[-1]), w.num_kv_heads * w.gqa_group
    # partial rows the main stage writes: one per non-local (block, query) pair
    # and head (two with 128-key blocks at d = 256, one per 64-key half), plus
    # one local row per (token, query head) where the local path runs
    halves = 2 if (w.block_size == 128 and w.head_dim == 256) else 1
    rows_written = (P_host - P_loc) * w.gqa_group * halves + (N * HQ if P_loc else 0)
    r.update(f_alg=f_alg, f_main=f_main, bytes=byts, local_pairs=P_loc,
             partial_bytes_written=rows_written * w.head_dim * s_p)
    return r


def stage_fractions(r, w):
    """Main stage against the MFMA (algorithmic FLOPs) and HBM (algorithmic
    bytes) peaks, and the reduction against HBM."""
    st = r["stage_ms"]
    main_tf = r["f_alg"] / (st["main"] * 1e-3) / 1e12
    return {
        "main_tflops_alg": round(main_tf, 2),
        "main_mfma_frac": round(main_tf / PEAK_MFMA_TFLOPS[w.dtype], 4),
        "main_hbm_frac": round(r["bytes"]["main"] / (st["main"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "reduce_hbm_frac": round(r["bytes"]["reduce"] / (st["reduce"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); "
              "the selected-attention path shards over KV heads without communication, "
              "so each GPU's throughput is the single-GPU figure.", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    if args.copy_calibration:
        import torch

        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "launches": 5}))
        return
    from sparse_attention_sel_amd.inputs import make_workload

    log(f"generating {args.workload}")
    w = make_workload(args.workload)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(w, args.cpu_seconds)  # before the GPU is touched (fork pool)
        log(f"cpu baseline done: {cpu['value']:.4g} TFLOP/s on {cpu['cores']} cores")
    log("gpu run")
    r = measure(w, args.partial, args.steps, args.warmup, not args.no_query_outer, not args.no_backward,
                not args.no_selection, cold_reps=args.cold_reps, onepass=args.onepass, graph=args.graph)
    peaks = measured_peaks(w.dtype)
    log(f"gpu run done: {r['ms_per_step']:.3f} ms/step")
    ms = r["ms_per_step"]
    value = r["f_alg"] / (ms * 1e-3) / 1e12
    st = r["stage_ms"]
    dominant = max(("main", "reduce"), key=lambda s: st[s])
    ach = r["bytes"][dominant] / (st[dominant] * 1e-3) / 1e9
    traffic = None
    if dominant == "main" and args.partial == "input":
        rec = measured_traffic(w.name)
        if rec is not None:
            traffic = int(round(rec["fetch_bytes"] + rec["write_bytes"]))
    main_tflops = r["f_alg"] / (st["main"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "tokens": int(w.cu_seqlens[-1]),
            "kv_heads": w.num_kv_heads,
            "gqa_group": w.gqa_group,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "topk": w.topk,
            "partial_dtype": w.dtype if args.partial == "input" else "fp32",
            "pairs": r["pairs"],
            "local_pairs": r["local_pairs"],
            "seed": w.meta.get("seed"),
        },
        "partial_buffer": {
            "bytes_written": int(r["partial_bytes_written"]),
            "workspace_bytes": r["partial_ws_bytes"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_reduce" if dominant == "reduce" else main_stage_kernels(w),
            "achieved": round(ach, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": int(r["bytes"][dominant]),
        },
        "stages_ms": {k_: round(v_, 4) for k_, v_ in st.items()},
        "main_kernel": {
            "tflops_alg": round(main_tflops, 2),
            "mfma_frac": round(main_tflops / PEAK_MFMA_TFLOPS[w.dtype], 4),
            "tflops_issued": round(r["f_main"] / (st["main"] * 1e-3) / 1e12, 2),
            "hbm_gbs": round(r["bytes"]["main"] / (st["main"] * 1e-3) / 1e9, 1),
            "hbm_frac_of_measured_copy": round(r["bytes"]["main"] / (st["main"] * 1e-3) / 1e9 / peaks["copy_gbs"], 4),
            "mfma_frac_of_measured_gemm": round(main_tflops / peaks["gemm_tflops"], 4),
            "mfma_frac_of_measured_loop": round(main_tflops / peaks["mfma_loop_tflops"], 4),
        },
        "measured_peaks": peaks,
        "step_ms_median": round(r["step_ms_median"], 4),
        "step_ms_min": round(r["step_ms_min"], 4),
        "cold_cache": r["cold"],
        "reduce_kernel_hbm_gbs": round(r["bytes"]["reduce"] / (st["reduce"] * 1e-3) / 1e9, 1),
        "index_hbm_gbs": round(r["bytes"]["index"] / (st["index"] * 1e-3) / 1e9, 1),
        "n_valid": r["n_valid"],
        "cpu_baseline": cpu,
    }
    if r["selection_ms"] is not None:
        gbs = r["selection_bytes"] / (r["selection_ms"] * 1e-3) / 1e9
        line["selection"] = {
            "ms": round(r["selection_ms"], 4),
            "hbm_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": int(r["selection_bytes"]),
        }
    if r["backward_ms"] is not None:
        # algorithmic backward work: S, dP, dV, dK, dQ over the visible keys
        f_bwd = r["f_alg"] * 10.0 / 4.0
        line["backward"] = {
            "ms": round(r["backward_ms"], 4),
            "tflops_alg": round(f_bwd / (r["backward_ms"] * 1e-3) / 1e12, 2),
            "ratio_to_forward": round(r["backward_ms"] / ms, 3),
        }
    if r["graph_ms_per_step"] is not None:
        line["graph_replay_ms_per_step"] = round(r["graph_ms_per_step"], 4)
    if r["onepass"] is not None:
        # not the pages' three-kernel split: a measured alternative, same outputs
        opm = r["onepass"]["ms_per_step"]
        line["onepass"] = {
            "ms_per_step": round(opm, 4),
            "tflops": round(r["f_alg"] / (opm * 1e-3) / 1e12, 2),
            "fused_ms": round(r["onepass"]["fused_ms"], 4),
            "speedup_vs_three_pass": round(ms / opm, 3),
        }
    if r["query_outer_ms"] is not None:
        line["query_outer"] = {
            "ms": round(r["query_outer_ms"], 4),
            "fsa_speedup": round(r["query_outer_ms"] / ms, 3),
        }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    if not args.no_variants and args.workload == DEFAULT_WORKLOAD:
        var = {}
        for name in VARIANTS:
            log(f"variant {name}")
            wv = make_workload(name)
            rv = measure(wv, args.partial, max(3, args.steps // 2), 2, not args.no_query_outer, not args.no_backward,
                         onepass=args.onepass)
            stv = rv["stage_ms"]
            var[name] = {
                "ms_per_step": round(rv["ms_per_step"], 4),
                "tflops": round(rv["f_alg"] / (rv["ms_per_step"] * 1e-3) / 1e12, 2),
                "dtype": wv.dtype,
                "stages_ms": {k_: round(v_, 4) for k_, v_ in stv.items()},
                **stage_fractions(rv, wv),
                "backward_ms": None if rv["backward_ms"] is None else round(rv["backward_ms"], 4),
                "query_outer_ms": None if rv["query_outer_ms"] is None else round(rv["query_outer_ms"], 4),
                "onepass_ms": None if rv["onepass"] is None else round(rv["onepass"]["ms_per_step"], 4),
                "pairs": rv["pairs"],
                "partial_bytes_written": int(rv["partial_bytes_written"]),
                "n_valid": rv["n_valid"],
                "seed": wv.meta.get("seed"),
            }
            del wv
        line["variants"] = var
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
