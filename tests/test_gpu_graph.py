"""The forward captured in a HIP graph (torch.cuda.CUDAGraph over the C-ABI
calls): the library allocates nothing and clears its own work-queue counters
with kernels, so a captured index build + statistics + forward (with the main
stage in one or two launches, and the one-pass forward) replays to the eager
result, bit for bit, on every replay, with other eager work between
replays."""

import numpy as np
import pytest
import torch

import sparse_attention_sel_amd as fsa
from gpu_helpers import log, problem_for
from sparse_attention_sel_amd.inputs import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["three_pass", "three_pass_mixed", "one_pass"])
def test_forward_graph_replays_match_eager(mode, monkeypatch):
    # the second mode forces the main stage's mixed launch (per-query-block
    # and block-outer items in one persistent kernel), whose two counter sets
    # a captured clear kernel zeroes before every replay
    onepass = mode == "one_pass"
    monkeypatch.setenv("FSA_MAIN_MIXED", "1" if mode == "three_pass_mixed" else "0")
    w = make_workload("n8k_h4_g2_d128_t16_bf16")
    dev = torch.device("cuda:0")
    prob = problem_for(w, "input")
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    sel = torch.from_numpy(w.sel).to(dev)
    index = fsa.allocate_index(prob, dev)
    ws = fsa.Workspaces(prob, dev, index.sizes)
    n, hq, d = prob.total_tokens, prob.num_q_heads, prob.head_dim
    lse = torch.empty((n, hq), dtype=torch.float32, device=dev)
    row_max = torch.empty_like(lse)
    out = torch.empty((n, hq, d), dtype=prob.dtype, device=dev)

    def forward():
        fsa.build_index(prob, sel, index, ws.build)
        if onepass:
            fsa.selected_attn_fwd_onepass(prob, q, k, v, index, row_max, lse, out, ws.stats, ws.partial)
        else:
            fsa.softmax_stats(prob, q, k, index, row_max, lse, ws.stats)
            fsa.selected_attn_fwd(prob, q, k, v, index, lse, out, ws.partial)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), row_max.clone())

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        forward()
    a = torch.randn(512, 512, device=dev)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        row_max.fill_(float("nan"))
        _ = a @ a  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        log(f"    replay {rep}")
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]) and torch.equal(row_max, ref[2])
    assert np.isfinite(out.float().cpu().numpy()).all()
