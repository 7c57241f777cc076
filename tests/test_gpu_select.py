"""GPU parity of block selection (fsa_select_blocks, through the C ABI)
against the oracle: bit-exact Sel rows.  Scores mix ties, NaN, +-inf, -0 and
denormals; rows longer than the register-resident limit take the memory path;
the 64K shape is compared on sampled tokens; and a selection -> attention run
checks the whole path against the oracle."""

import numpy as np
import pytest
import torch

import oracle.fsa_oracle as O
import sparse_attention_sel_amd as fsa
from gpu_helpers import TOL_LSE, TOL_O, ResultFiles, custom_workload, log, run_gpu
from sparse_attention_sel_amd.inputs import cu_seqlens_of, make_block_scores

pytestmark = pytest.mark.gpu


def run_select(scores, cu, H, B, T, init_blocks, local_blocks):
    dev = torch.device("cuda:0")
    prob = fsa.Problem(cu, H, 1, 64, B, T, device=dev)
    sc = torch.from_numpy(np.ascontiguousarray(scores)).to(dev)
    sel = torch.full((H, int(cu[-1]), T), -7, dtype=torch.int32, device=dev)
    fsa.select_blocks(prob, sc, init_blocks, local_blocks, sel)
    torch.cuda.synchronize()
    return sel.cpu().numpy()


def nasty_scores(rng, H, N, S):
    sc = rng.standard_normal((H, N, S)).astype(np.float32)
    special = np.array([0.5, -0.0, 0.0, 1e-40, -1e-40, np.nan, np.inf, -np.inf], dtype=np.float32)
    mask = rng.random(sc.shape) < 0.3
    sc[mask] = rng.choice(special, size=int(mask.sum()))
    return sc


CASES = [
    # seqlens, H, B, T, init, local
    ((300, 0, 129, 64), 2, 64, 16, 1, 2),
    ((1000,), 1, 64, 5, 0, 0),
    ((700, 333), 3, 64, 8, 2, 1),
    ((513,), 2, 128, 8, 1, 2),
    ((200, 40), 1, 64, 2, 1, 2),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_select_bitexact(case):
    seqlens, H, B, T, ib, lb = CASES[case]
    rng = np.random.default_rng(600 + case)
    cu = cu_seqlens_of(seqlens)
    S = max([-(-L // B) for L in seqlens] + [1]) + 3  # a stride wider than needed
    sc = nasty_scores(rng, H, int(cu[-1]), S)
    log(f"[run] select case {case} {CASES[case]}")
    got = run_select(sc, cu, H, B, T, ib, lb)
    np.testing.assert_array_equal(got, O.select_blocks(sc, cu, B, T, ib, lb))


@pytest.mark.timeout(900)
def test_select_long_rows_memory_path(oracle_service):
    # 90 000 tokens in blocks of 64 = 1407 blocks > 1024: the rows past block
    # 1023 rescan their candidates from memory; every token is compared
    seqlens, H, B, T = (90000,), 1, 64, 16
    cu = cu_seqlens_of(seqlens)
    sc = make_block_scores(seqlens, H, B, 41)
    got = run_select(sc, cu, H, B, T, 1, 2)
    del sc
    check_select_all_tokens(oracle_service, got, seqlens, H, B, T, 41)


def check_select_all_tokens(svc, got, seqlens, H, B, T, seed):
    with ResultFiles() as f:
        r = svc.select(seqlens, H, B, T, 1, 2, seed, f.save("sel", got))
    log(f"    all {r['tokens']} tokens: {r['mismatch']} mismatching rows "
        f"(oracle {r['oracle_s']:.1f} s on {r['workers']} processes)")
    assert r["mismatch"] == 0, r["first_mismatch"]


@pytest.mark.timeout(900)
def test_select_64k_all_tokens(oracle_service):
    seqlens, H, B, T = (65536,), 4, 64, 16
    cu = cu_seqlens_of(seqlens)
    sc = make_block_scores(seqlens, H, B, 42)
    log("[run] select 64K")
    got = run_select(sc, cu, H, B, T, 1, 2)
    del sc
    assert np.all((got >= -1) & (got < 1024))
    check_select_all_tokens(oracle_service, got, seqlens, H, B, T, 42)


def test_selection_then_attention():
    # scores -> Sel on the GPU -> index, statistics, output on the GPU,
    # against oracle selection -> oracle attention
    seqlens, H, g, d, B, T = (3000, 1200), 2, 4, 128, 64, 16
    cu = cu_seqlens_of(seqlens)
    sc = make_block_scores(seqlens, H, B, 43)
    sel_gpu = run_select(sc, cu, H, B, T, 1, 2)
    sel_ref = O.select_blocks(sc, cu, B, T, 1, 2)
    np.testing.assert_array_equal(sel_gpu, sel_ref)
    w = custom_workload(seqlens, H, g, d, B, T, "bf16", sel_gpu, seed=44)
    res = run_gpu(w, "fp32")
    q, k, v = (x.float().numpy() for x in (w.q, w.k, w.v))
    o_ref, _, lse_ref = O.selected_attention(q, k, v, sel_ref, cu, B, w.scale)
    assert float(np.max(np.abs(res["out"] - o_ref))) <= TOL_O["bf16"]
    assert float(np.max(np.abs(res["lse"] - lse_ref))) <= TOL_LSE
