"""GPU parity of the one-pass forward (fsa_selected_attn_fwd_onepass, through
the C ABI): statistics fused into the main kernel and the reduction.

Same bar as the three-pass path: O within max-abs 2e-2 (bf16) / 5e-3 (fp16)
and lse, row max within 1e-3 of the float64 oracle, on every token (the
full-size workloads through the oracle service).  The merged (max, sum)
of a row is computed exactly as the statistics kernels compute it, so lse and
row max must equal those of fsa_softmax_stats bit for bit.
"""

import numpy as np
import pytest

from gpu_helpers import check_full_forward, custom_workload, log, run_gpu
from sparse_attention_sel_amd.inputs import cu_seqlens_of
from test_gpu_parity import CASES, adversarial_sel, check_attention, check_index, oracle_index, workload

import oracle.fsa_oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("partial", ["fp32", "input"])
@pytest.mark.parametrize("name", ["n1k_h1_g1_d64_t4_bf16", "n8k_h4_g2_d128_t16_bf16"])
def test_onepass_all_tokens(name, partial):
    w = workload(name)
    log(f"[run] one-pass {name} partial={partial}")
    res = run_gpu(w, partial, onepass=True)
    check_index(res, oracle_index(name))
    check_attention(res, w)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_onepass_adversarial_selection(case):
    seqlens, H, g, d, B, T, dtype = CASES[case]
    rng = np.random.default_rng(700 + case)
    cu = cu_seqlens_of(seqlens)
    sel = adversarial_sel(rng, H, cu, B, T)
    sel[:, ::37, :] = -1  # some rows select nothing
    w = custom_workload(seqlens, H, g, d, B, T, dtype, sel, seed=900 + case)
    log(f"[run] one-pass adversarial case {case} {CASES[case]}")
    res = run_gpu(w, "input", onepass=True)
    check_index(res, O.build_index(w.sel, w.cu_seqlens, B))
    check_attention(res, w)


@pytest.mark.timeout(900)
@pytest.mark.parametrize(
    "name,partial",
    [
        ("n64k_h4_g4_d128_t16_bf16", "input"),
        ("n64k_h4_g1_d128_t16_fp16", "fp32"),
        ("b2_n32k_h8_g8_d256_t16_bf16", "input"),
        ("n64k_h4_g4_d128_b128_t8_bf16", "input"),
    ],
)
def test_onepass_large_all_tokens_and_stats_bitwise(name, partial, oracle_service):
    oracle_service.prepare(name)
    w = workload(name)
    log(f"[run] one-pass {name} partial={partial}")
    one = run_gpu(w, partial, onepass=True, float_out=False)
    check_full_forward(oracle_service, w, one)
    log("    three-pass statistics for comparison")
    three = run_gpu(w, partial, float_out=False)
    for key in ("lse", "row_max"):
        assert np.array_equal(one[key], three[key]), key


def test_onepass_deterministic_bitwise():
    w = workload("n8k_h4_g2_d128_t16_bf16")
    a = run_gpu(w, "input", onepass=True)
    b = run_gpu(w, "input", onepass=True)
    for key in ("out", "lse", "row_max"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_onepass_repeated_and_interleaved_on_one_index():
    # the one-pass call claims work items through the same index counters as
    # the three-pass calls: alternating them on one index gives every call
    # the result of a fresh index
    import torch

    import sparse_attention_sel_amd as fsa

    w = workload("n8k_h4_g2_d128_t16_bf16")
    ref1 = run_gpu(w, "input", onepass=True)
    ref3 = run_gpu(w, "input")
    dev = torch.device("cuda:0")
    prob = fsa.Problem(w.cu_seqlens, w.num_kv_heads, w.gqa_group, w.head_dim, w.block_size, w.topk,
                       dtype=torch.bfloat16, partial_dtype="input", softmax_scale=w.scale, device=dev)
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    index = fsa.allocate_index(prob, dev)
    ws = fsa.Workspaces(prob, dev, index.sizes)
    fsa.build_index(prob, torch.from_numpy(w.sel).to(dev), index, ws.build)
    n, hq = prob.total_tokens, prob.num_q_heads
    for rnd, onepass in enumerate((True, False, True, False)):
        log(f"    call {rnd} onepass={onepass}")
        lse = torch.full((n, hq), float("nan"), dtype=torch.float32, device=dev)
        row_max = torch.full_like(lse, float("nan"))
        out = torch.full((n, hq, prob.head_dim), float("nan"), dtype=prob.dtype, device=dev)
        if onepass:
            fsa.selected_attn_fwd_onepass(prob, q, k, v, index, row_max, lse, out, ws.stats, ws.partial)
        else:
            fsa.softmax_stats(prob, q, k, index, row_max, lse, ws.stats)
            fsa.selected_attn_fwd(prob, q, k, v, index, lse, out, ws.partial)
        torch.cuda.synchronize()
        ref = ref1 if onepass else ref3
        assert np.array_equal(out.float().cpu().numpy(), ref["out"])
        assert np.array_equal(lse.cpu().numpy(), ref["lse"])
        assert np.array_equal(row_max.cpu().numpy(), ref["row_max"])


def test_backward_from_onepass_forward():
    # training flow: the one-pass forward's O and lse feed the backward
    import torch

    import sparse_attention_sel_amd as fsa
    from sparse_attention_sel_amd.inputs import make_dout
    from test_gpu_backward import check_all, oracle_grads

    w = workload("n8k_h4_g2_d128_t16_bf16")
    dev = torch.device("cuda:0")
    prob = fsa.Problem(w.cu_seqlens, w.num_kv_heads, w.gqa_group, w.head_dim, w.block_size, w.topk,
                       dtype=torch.bfloat16, partial_dtype="input", softmax_scale=w.scale, device=dev)
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    out, lse, _, index = fsa.selected_attention(prob, q, k, v, torch.from_numpy(w.sel).to(dev), onepass=True)
    do_cpu = make_dout(prob.total_tokens, prob.num_q_heads, prob.head_dim, w.dtype, 21)
    dq, dk, dv = fsa.selected_attention_backward(prob, q, k, v, out, do_cpu.to(dev), lse, index)
    torch.cuda.synchronize()
    log("[run] backward from the one-pass forward")
    res = {"dq": dq.float().cpu().numpy(), "dk": dk.float().cpu().numpy(), "dv": dv.float().cpu().numpy()}
    check_all(res, oracle_grads(w, do_cpu), w.dtype)
