"""fsa_build_index_noalloc (the index build for callers that cannot allocate:
its scratch is the library's static per-GPU array) against fsa_build_index
with a caller workspace, through the C ABI: bit-exact index tensors and the
same forward outputs from either index, on consecutive calls that share the
static scratch, the later ones on smaller inputs."""

import numpy as np
import pytest
import torch

import sparse_attention_sel_amd as fsa
from gpu_helpers import log, problem_for
from sparse_attention_sel_amd.inputs import make_workload

pytestmark = pytest.mark.gpu

# largest first: every later call runs on scratch that still holds the
# previous (larger) call's contents
SEQUENCE = ["n64k_h4_g4_d128_t16_bf16", "n8k_h4_g2_d128_t16_bf16", "n1k_h1_g1_d64_t4_bf16"]


def index_and_forward(w, prob, sel, q, k, v, noalloc):
    dev = sel.device
    index = fsa.allocate_index(prob, dev)
    ws = fsa.Workspaces(prob, dev, index.sizes)
    for t in (index.counts, index.offsets, index.qidx, index.slot):
        t.fill_(-7)
    if noalloc:
        fsa.build_index_noalloc(prob, sel, index)
    else:
        fsa.build_index(prob, sel, index, ws.build)
    n, hq = prob.total_tokens, prob.num_q_heads
    lse = torch.empty((n, hq), dtype=torch.float32, device=dev)
    row_max = torch.empty_like(lse)
    out = torch.empty((n, hq, prob.head_dim), dtype=prob.dtype, device=dev)
    fsa.softmax_stats(prob, q, k, index, row_max, lse, ws.stats)
    fsa.selected_attn_fwd(prob, q, k, v, index, lse, out, ws.partial)
    torch.cuda.synchronize()
    P = index.num_pairs()
    res = {
        "pairs": P,
        "counts": index.counts.cpu().numpy(),
        "offsets": index.offsets.cpu().numpy(),
        "qidx": index.qidx[:P].cpu().numpy(),
        "slot": index.slot.cpu().numpy(),
        "out": out.view(torch.int16).cpu().numpy(),
        "lse": lse.cpu().numpy(),
        "row_max": row_max.cpu().numpy(),
    }
    del index, ws, lse, row_max, out
    return res


@pytest.mark.timeout(600)
def test_noalloc_build_matches_workspace_build_on_consecutive_calls():
    dev = torch.device("cuda:0")
    for name in SEQUENCE:
        w = make_workload(name)
        prob = problem_for(w, "input")
        ws_bytes = fsa.get_sizes(prob)["build_ws_bytes"]
        assert ws_bytes <= fsa.NOALLOC_BUILD_SCRATCH_BYTES
        sel = torch.from_numpy(w.sel).to(dev)
        q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
        log(f"[run] noalloc build {name} (build scratch {ws_bytes} bytes)")
        a = index_and_forward(w, prob, sel, q, k, v, noalloc=True)
        b = index_and_forward(w, prob, sel, q, k, v, noalloc=False)
        assert a["pairs"] == b["pairs"] > 0
        for key in ("counts", "offsets", "qidx", "slot", "out", "lse", "row_max"):
            assert np.array_equal(a[key], b[key]), (name, key)
        del w, sel, q, k, v
