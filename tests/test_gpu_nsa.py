"""GPU parity of the query-outer (vanilla NSA loop order) forward against the
float64 oracle: O within max-abs 2e-2 (bf16) or 5e-3 (fp16), lse within 1e-3,
lse = -inf and a zero row where a row selects nothing.  The same workloads
and adversarial selections as the KV-block-outer path."""

import functools

import numpy as np
import pytest

import oracle.fsa_oracle as O
from gpu_helpers import TOL_LSE, TOL_O, check_full_forward, custom_workload, log, run_gpu, run_gpu_nsa
from sparse_attention_sel_amd.inputs import cu_seqlens_of, make_workload
from test_gpu_parity import CASES, adversarial_sel

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def workload(name):
    log(f"[gen] {name}")
    return make_workload(name)


def check(res, w, tokens=None):
    q, k, v = (x.float().numpy() for x in (w.q, w.k, w.v))
    o_ref, _, lse_ref = O.selected_attention(q, k, v, w.sel, w.cu_seqlens, w.block_size, w.scale, tokens)
    rows = slice(None) if tokens is None else tokens
    o, lse = res["out"][rows], res["lse"][rows]
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), "empty key sets must give lse = -inf"
    assert np.all(o[empty] == 0)
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    fin = ~empty
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    log(f"    max|dO|={err_o:.3e} max|dlse|={err_l:.3e}")
    assert err_o <= TOL_O[w.dtype], f"O error {err_o}"
    assert err_l <= TOL_LSE, f"lse error {err_l}"


@pytest.mark.parametrize("name", ["n1k_h1_g1_d64_t4_bf16", "n8k_h4_g2_d128_t16_bf16"])
def test_nsa_all_tokens(name):
    w = workload(name)
    log(f"[run] nsa {name}")
    check(run_gpu_nsa(w), w)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["n64k_h4_g4_d128_t16_bf16", "n64k_h4_g1_d128_t16_fp16", "b2_n32k_h8_g8_d256_t16_bf16"])
def test_nsa_large_all_tokens(name, oracle_service):
    oracle_service.prepare(name)
    w = workload(name)
    log(f"[run] nsa {name}")
    check_full_forward(oracle_service, w, run_gpu_nsa(w), with_row_max=False)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_nsa_adversarial_selection(case):
    seqlens, H, g, d, B, T, dtype = CASES[case]
    rng = np.random.default_rng(700 + case)
    cu = cu_seqlens_of(seqlens)
    sel = adversarial_sel(rng, H, cu, B, T)
    sel[:, ::37, :] = -1
    w = custom_workload(seqlens, H, g, d, B, T, dtype, sel, seed=900 + case)
    log(f"[run] nsa adversarial case {case} {CASES[case]}")
    check(run_gpu_nsa(w), w)


def test_nsa_long_topk_rows():
    # T > 64: the first-occurrence test spans several 64-entry groups.
    seqlens, H, g, d, B, T = (4000, 1500), 2, 4, 128, 64, 80
    rng = np.random.default_rng(4242)
    cu = cu_seqlens_of(seqlens)
    sel = adversarial_sel(rng, H, cu, B, T)
    sel[:, :, 70:] = sel[:, :, 3:13]  # repeats across the group boundary
    w = custom_workload(seqlens, H, g, d, B, T, "bf16", sel, seed=4243)
    log("[run] nsa long topk rows")
    check(run_gpu_nsa(w), w)


def test_nsa_matches_kv_block_outer_path():
    # The two GPU paths compute the same function; each is within tolerance of
    # the oracle, so they agree within twice that.
    w = workload("n8k_h4_g2_d128_t16_bf16")
    a = run_gpu_nsa(w)
    b = run_gpu(w, "fp32")
    assert np.array_equal(np.isneginf(a["lse"]), np.isneginf(b["lse"]))
    assert float(np.max(np.abs(a["out"] - b["out"]))) <= 2 * TOL_O["bf16"]
    fin = np.isfinite(b["lse"])
    assert float(np.max(np.abs(a["lse"][fin] - b["lse"][fin]))) <= 2 * TOL_LSE
