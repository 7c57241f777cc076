"""Shared plumbing for the GPU parity tests: run the HIP path through the
C-ABI binding and bring results back to the host for comparison with the
oracle.  Holds no attention arithmetic."""

import os
import sys
import tempfile

import numpy as np
import torch

import sparse_attention_sel_amd as fsa
from sparse_attention_sel_amd.inputs import Workload, cu_seqlens_of, make_qkv

TOL_O = {"bf16": 2e-2, "fp16": 5e-3}
TOL_LSE = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def problem_for(w: Workload, partial: str = "fp32", device="cuda") -> fsa.Problem:
    return fsa.Problem(
        w.cu_seqlens, w.num_kv_heads, w.gqa_group, w.head_dim, w.block_size, w.topk,
        dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float16,
        partial_dtype=partial, softmax_scale=w.scale, device=device,
    )


def bits16(x: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a 16-bit device tensor (its exact storage bits)."""
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


def run_gpu(w: Workload, partial: str = "fp32", keep_partial: bool = False, onepass: bool = False,
            float_out: bool = True):
    """Whole forward on cuda:0 (onepass: fsa_selected_attn_fwd_onepass in
    place of the statistics and forward calls).  Returns a dict of host numpy
    arrays: the index tensors, out (float32, unless float_out is False),
    out_bits (the output's 16-bit storage), lse and row_max."""
    prob = problem_for(w, partial)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    sel = torch.from_numpy(w.sel).to(dev)
    index = fsa.allocate_index(prob, dev)
    ws = fsa.Workspaces(prob, dev, index.sizes)
    n, hq = prob.total_tokens, prob.num_q_heads
    lse = torch.full((n, hq), float("nan"), dtype=torch.float32, device=dev)
    row_max = torch.full((n, hq), float("nan"), dtype=torch.float32, device=dev)
    out = torch.full((n, hq, prob.head_dim), float("nan"), dtype=prob.dtype, device=dev)
    fsa.build_index(prob, sel, index, ws.build)
    if onepass:
        fsa.selected_attn_fwd_onepass(prob, q, k, v, index, row_max, lse, out, ws.stats, ws.partial)
    else:
        fsa.softmax_stats(prob, q, k, index, row_max, lse, ws.stats)
        fsa.selected_attn_fwd(prob, q, k, v, index, lse, out, ws.partial)
    torch.cuda.synchronize()
    P = index.num_pairs()
    res = {
        "counts": index.counts.cpu().numpy(),
        "offsets": index.offsets[: index.counts.numel() + 1].cpu().numpy(),
        "qidx": index.qidx[:P].cpu().numpy(),
        "slot": index.slot.cpu().numpy(),
        "pairs": P,
        "out_bits": bits16(out),
        "lse": lse.cpu().numpy(),
        "row_max": row_max.cpu().numpy(),
    }
    if float_out:
        res["out"] = out.float().cpu().numpy()
    if keep_partial:
        res["partial"] = ws.partial
        res["index"] = index
        res["out_dev"] = out
    return res


def run_gpu_bwd(w: Workload, dout, partial: str = "fp32", float_out: bool = True):
    """FSA forward then backward on cuda:0 for the output gradient ``dout``
    (torch CPU tensor, input dtype).  Returns host float32 numpy arrays
    dq, dk, dv and out of the forward (None unless float_out), their 16-bit
    storage bits (dq_bits, ...) and the forward's lse."""
    prob = problem_for(w, partial)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    do = dout.to(dev)
    sel = torch.from_numpy(w.sel).to(dev)
    index = fsa.allocate_index(prob, dev)
    ws = fsa.Workspaces(prob, dev, index.sizes, backward=True)
    n, hq, d = prob.total_tokens, prob.num_q_heads, prob.head_dim
    lse = torch.empty((n, hq), dtype=torch.float32, device=dev)
    row_max = torch.empty((n, hq), dtype=torch.float32, device=dev)
    out = torch.empty((n, hq, d), dtype=prob.dtype, device=dev)
    fsa.build_index(prob, sel, index, ws.build)
    fsa.softmax_stats(prob, q, k, index, row_max, lse, ws.stats)
    fsa.selected_attn_fwd(prob, q, k, v, index, lse, out, ws.partial)
    dq = torch.full((n, hq, d), float("nan"), dtype=prob.dtype, device=dev)
    dk = torch.full((n, prob.num_kv_heads, d), float("nan"), dtype=prob.dtype, device=dev)
    dv = torch.full_like(dk, float("nan"))
    fsa.selected_attn_bwd(prob, q, k, v, out, do, lse, index, dq, dk, dv, ws.bwd)
    torch.cuda.synchronize()
    res = {"lse": lse.cpu().numpy()}
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv), ("out", out)):
        res[name + "_bits"] = bits16(x)
        res[name] = x.float().cpu().numpy() if float_out else None
    return res


def run_gpu_nsa(w: Workload):
    """Query-outer forward on cuda:0 straight from Sel.  Returns host numpy
    arrays out [N, h_q, d] (float32) and lse [N, h_q]."""
    prob = problem_for(w)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    sel = torch.from_numpy(w.sel).to(dev)
    n, hq = prob.total_tokens, prob.num_q_heads
    lse = torch.full((n, hq), float("nan"), dtype=torch.float32, device=dev)
    out = torch.full((n, hq, prob.head_dim), float("nan"), dtype=prob.dtype, device=dev)
    fsa.nsa_selected_attn_fwd(prob, q, k, v, sel, lse, out)
    torch.cuda.synchronize()
    return {"out": out.float().cpu().numpy(), "out_bits": bits16(out), "lse": lse.cpu().numpy()}


def sample_tokens(cu, block_size, n_random=96, seed=0):
    """Tokens that exercise the edges (first tokens of each sequence, block
    boundaries, last tokens) plus a seeded random spread."""
    rng = np.random.default_rng(seed)
    toks = set()
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        if c1 == c0:
            continue
        for off in (0, 1, 2, block_size - 1, block_size, block_size + 1, 2 * block_size + 5):
            if c0 + off < c1:
                toks.add(c0 + off)
        for off in (1, 2, block_size + 1):
            if c1 - off >= c0:
                toks.add(c1 - off)
    n = int(cu[-1])
    toks.update(int(x) for x in rng.integers(0, n, size=min(n_random, n)))
    return np.array(sorted(toks), dtype=np.int64)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().numpy().astype(np.float64)


def custom_workload(seqlens, H, g, d, B, T, dtype, sel, seed, scale=None):
    cu = cu_seqlens_of(seqlens)
    q, k, v = make_qkv(int(cu[-1]), H, g, d, dtype, seed)
    return Workload(
        name="custom", seqlens=list(seqlens), cu_seqlens=cu, num_kv_heads=H, gqa_group=g, head_dim=d,
        block_size=B, topk=T, dtype=dtype, scale=scale if scale is not None else 1.0 / np.sqrt(d),
        q=q, k=k, v=v, sel=np.ascontiguousarray(sel.astype(np.int32)), meta={},
    )


class ResultFiles:
    """A temporary directory for GPU results handed to the oracle service as
    .npy files; removed on exit."""

    def __enter__(self):
        self._dir = tempfile.TemporaryDirectory(prefix="fsa_parity_")
        return self

    def save(self, name: str, arr) -> str:
        path = os.path.join(self._dir.name, name + ".npy")
        np.save(path, np.ascontiguousarray(arr), allow_pickle=False)
        return path

    def __exit__(self, *exc):
        self._dir.cleanup()
        return False


def check_full_forward(svc, w: Workload, res: dict, with_row_max: bool = True):
    """Every token's O, lse (and row max) against the float64 oracle, through
    the oracle service: O within TOL_O, lse and row max within TOL_LSE, and
    rows with no keys giving lse = row max = -inf and a zero output."""
    with ResultFiles() as f:
        r = svc.forward(w.name, f.save("out", res["out_bits"]), f.save("lse", res["lse"]),
                        f.save("row_max", res["row_max"]) if with_row_max else None)
    log(f"    all {r['tokens']} tokens: max|dO|={r['err_o']:.3e} at {r['err_o_at']} "
        f"max|dlse|={r['err_lse']:.3e} at {r['err_lse_at']} max|dm|={r['err_m']:.3e} "
        f"(empty rows {r['empty_rows']}; oracle {r['oracle_s']:.1f} s on {r['workers']} processes)")
    assert r["empty_mismatch"] == 0, "empty key sets must give lse = row max = -inf, and only they"
    assert r["nonzero_empty_out"] == 0, "rows with no keys must output zero"
    assert r["nonfinite"] == 0, "non-finite outputs"
    assert r["err_o"] <= TOL_O[w.dtype], f"O error {r['err_o']} at {r['err_o_at']}"
    assert r["err_lse"] <= TOL_LSE, f"lse error {r['err_lse']} at {r['err_lse_at']}"
    assert r["err_m"] <= TOL_LSE, f"row max error {r['err_m']} at {r['err_m_at']}"
    return r
