"""GPU parity of the backward (fsa_selected_attn_bwd, through the C ABI)
against the float64 oracle's gradient: the GPU runs its own forward (index,
statistics, output) and then the backward from that O and lse.

Small shapes compare dQ, dK, dV element by element on every token.  The
full-size shapes (through the oracle service, the oracle run in CPU worker
processes started before the first GPU call) compare dQ on every token and
dK / dV element by element on the keys of whole blocks: block 0 (every token
selects it), the last block and the hottest and some random blocks; the dV
column-sum identity covers every key.
"""

import functools

import numpy as np
import pytest
import torch

import oracle.fsa_oracle as O
from gpu_helpers import ResultFiles, custom_workload, log, run_gpu_bwd
from oracle_service import decode_out
from sparse_attention_sel_amd.inputs import cu_seqlens_of, make_dout, make_sel, make_workload
from test_gpu_parity import adversarial_sel

pytestmark = pytest.mark.gpu

# Elementwise tolerance |gpu - ref| <= ATOL + RTOL |ref| on dQ, dK, dV.  The
# gradients are rounded once to the input dtype (half an ulp: 2^-9 relative for
# bf16, 2^-12 for fp16), P and dS enter the MFMAs as 16-bit values (the same
# relative size per term) and D comes from the 16-bit forward output; RTOL =
# 2^-7 covers the relative part, ATOL (the forward's bound on O) the small
# gradients whose error is set by their larger neighbours.
ATOL = {"bf16": 2e-2, "fp16": 5e-3}
RTOL = 2.0**-7


@functools.lru_cache(maxsize=1)
def workload(name):
    log(f"[gen] {name}")
    return make_workload(name)


def dout_for(w, seed):
    return make_dout(int(w.cu_seqlens[-1]), w.num_kv_heads * w.gqa_group, w.head_dim, w.dtype, seed)


def oracle_grads(w, do, tokens=None):
    q, k, v = (x.float().numpy() for x in (w.q, w.k, w.v))
    return O.selected_attention_backward(q, k, v, w.sel, w.cu_seqlens, w.block_size, do.float().numpy(), w.scale,
                                         tokens)


def check_all(res, ref, dtype, what=("dq", "dk", "dv")):
    for name, r in zip(("dq", "dk", "dv"), ref):
        if name not in what:
            continue
        g = res[name]
        assert np.all(np.isfinite(g)), f"{name} not finite"
        err = np.abs(g - r)
        ratio = float(np.max(err / (ATOL[dtype] + RTOL * np.abs(r)))) if g.size else 0.0
        log(f"    {name}: max|err|={float(err.max()) if g.size else 0.0:.3e} "
            f"max|ref|={float(np.max(np.abs(r))) if r.size else 0.0:.3e} err/tol={ratio:.3f}")
        assert ratio <= 1.0, f"{name} exceeds tolerance ({ratio:.3f})"


@pytest.mark.parametrize("partial", ["fp32", "input"])
@pytest.mark.parametrize("name", ["n1k_h1_g1_d64_t4_bf16", "n8k_h4_g2_d128_t16_bf16"])
def test_backward_all_tokens(name, partial):
    w = workload(name)
    do = dout_for(w, 11)
    log(f"[run] bwd {name} partial={partial}")
    res = run_gpu_bwd(w, do, partial)
    check_all(res, oracle_grads(w, do), w.dtype)


CASES = [
    # seqlens, H, g, d, B, T, dtype
    ((300, 0, 129, 64), 2, 3, 64, 64, 5, "bf16"),
    ((513, 77), 1, 16, 128, 64, 3, "fp16"),
    ((1000,), 2, 1, 128, 64, 8, "bf16"),
    ((64, 1, 65), 1, 2, 64, 64, 1, "fp16"),
    ((700, 300), 2, 5, 128, 64, 12, "bf16"),
    ((640, 384), 2, 8, 256, 64, 6, "bf16"),
    ((200, 57), 1, 3, 256, 64, 4, "fp16"),
    ((700, 300), 2, 4, 128, 128, 6, "bf16"),
    ((257, 130, 1), 1, 3, 64, 128, 4, "fp16"),
    ((900, 500), 2, 2, 64, 64, 40, "bf16"),
    ((300, 100), 1, 16, 256, 64, 6, "bf16"),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_adversarial_selection(case):
    seqlens, H, g, d, B, T, dtype = CASES[case]
    rng = np.random.default_rng(800 + case)
    cu = cu_seqlens_of(seqlens)
    sel = adversarial_sel(rng, H, cu, B, T)
    sel[:, ::37, :] = -1  # some rows select nothing
    w = custom_workload(seqlens, H, g, d, B, T, dtype, sel, seed=950 + case)
    do = dout_for(w, 960 + case)
    log(f"[run] bwd adversarial case {case} {CASES[case]}")
    check_all(run_gpu_bwd(w, do, "fp32"), oracle_grads(w, do), dtype)


@pytest.mark.parametrize("partial", ["fp32", "input"])
def test_backward_d256_hot_selection_all_tokens(partial):
    # the large-head shape (two packed sequences, g = 8, d = 256, hot-block
    # selection) at a size the oracle covers on every token; sequences this
    # short reach a 30% hot share with hot sets of 20% of the blocks
    seqlens, H, g, d, B, T = (2048, 1024), 2, 8, 256, 64, 16
    sel, _ = make_sel("init_local_hot", seqlens, H, B, T, seed=5150, hot_fraction=0.2, hot_share=0.3)
    w = custom_workload(seqlens, H, g, d, B, T, "bf16", sel, seed=5160)
    do = dout_for(w, 5170)
    log(f"[run] bwd d=256 hot selection partial={partial}")
    check_all(run_gpu_bwd(w, do, partial), oracle_grads(w, do), w.dtype)


@pytest.mark.parametrize("partial", ["fp32", "input"])
def test_backward_b128_zipf_all_tokens(partial):
    # 128-key blocks (eight waves per block in the backward), 8 selected blocks
    seqlens, H, g, d, B, T = (4096,), 2, 4, 128, 128, 8
    sel, _ = make_sel("init_local_zipf", seqlens, H, B, T, seed=3350)
    w = custom_workload(seqlens, H, g, d, B, T, "bf16", sel, seed=3360)
    do = dout_for(w, 3370)
    log(f"[run] bwd B_K=128 partial={partial}")
    check_all(run_gpu_bwd(w, do, partial), oracle_grads(w, do), w.dtype)


def test_backward_full_selection_matches_torch_autograd():
    # Sel holding every block is causal attention: compare with torch float32
    # autograd of the dense causal softmax on the CPU (an independent route)
    seqlens, H, g, d, B = (300, 200), 2, 2, 64, 64
    cu = cu_seqlens_of(seqlens)
    nb = max(-(-L // B) for L in seqlens)
    sel = np.broadcast_to(np.arange(nb, dtype=np.int32), (H, int(cu[-1]), nb)).copy()
    w = custom_workload(seqlens, H, g, d, B, nb, "bf16", sel, seed=71)
    do = dout_for(w, 72)
    res = run_gpu_bwd(w, do, "fp32")
    qf, kf, vf = (x.float().clone().requires_grad_(True) for x in (w.q, w.k, w.v))
    outs = []
    for s in range(len(seqlens)):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        qt = qf[c0:c1].permute(1, 0, 2)
        kt = kf[c0:c1].permute(1, 0, 2).repeat_interleave(g, dim=0)
        vt = vf[c0:c1].permute(1, 0, 2).repeat_interleave(g, dim=0)
        sc = (qt @ kt.transpose(1, 2)) * w.scale
        L = c1 - c0
        sc = sc.masked_fill(~torch.tril(torch.ones(L, L, dtype=torch.bool)), float("-inf"))
        outs.append((torch.softmax(sc, dim=-1) @ vt).permute(1, 0, 2))
    (torch.cat(outs) * do.float()).sum().backward()
    for name, ref in (("dq", qf.grad), ("dk", kf.grad), ("dv", vf.grad)):
        err = np.abs(res[name] - ref.numpy())
        ratio = float(np.max(err / (ATOL["bf16"] + RTOL * np.abs(ref.numpy()))))
        log(f"    {name} vs torch autograd: max|err|={float(err.max()):.3e} err/tol={ratio:.3f}")
        assert ratio <= 1.0


def test_backward_deterministic_bitwise():
    w = workload("n8k_h4_g2_d128_t16_bf16")
    do = dout_for(w, 12)
    a = run_gpu_bwd(w, do, "input")
    b = run_gpu_bwd(w, do, "input")
    for key in ("dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key]), key


def hot_key_blocks(w, n_hot=3, n_random=2, seed=0):
    """(sequence, local block) pairs whose keys get an elementwise dK / dV
    check: every sequence's block 0 (selected by every token: the longest
    accumulation), its last block, the n_hot blocks selected most often in any
    KV head, and n_random seeded others."""
    idx = O.build_index(w.sel, w.cu_seqlens, w.block_size)
    H = w.num_kv_heads
    NB = idx["num_blocks"]
    cnt = idx["counts"].reshape(H, NB).max(axis=0)
    B = w.block_size
    gboff = np.concatenate([[0], np.cumsum([-(-L // B) for L in w.seqlens])])
    rng = np.random.default_rng(seed)
    out = set()
    for s_, L in enumerate(w.seqlens):
        nb = -(-L // B)
        if nb == 0:
            continue
        out.update({(s_, 0), (s_, nb - 1)})
        c = cnt[gboff[s_] : gboff[s_] + nb].copy()
        c[0] = -1
        out.update((s_, int(e)) for e in np.argsort(-c, kind="stable")[:n_hot])
        out.update((s_, int(e)) for e in rng.integers(0, nb, size=n_random))
    return sorted(out)


def check_large_backward(svc, w, seed, partial="input"):
    svc.prepare(w.name)
    do = dout_for(w, seed)
    log(f"[run] bwd {w.name} (partials: {partial})")
    res = run_gpu_bwd(w, do, partial, float_out=False)
    blocks = hot_key_blocks(w)
    with ResultFiles() as f:
        r = svc.backward(w.name, seed, f.save("dq", res["dq_bits"]), f.save("dk", res["dk_bits"]),
                         f.save("dv", res["dv_bits"]), blocks)
    log(f"    dQ on all {r['tokens']} tokens: max|err|={r['dq_err']:.3e} err/tol={r['dq_ratio']:.3f} at {r['dq_at']}")
    for nm in ("dk", "dv"):
        log(f"    {nm} on {r['keys']} keys of blocks {blocks}: max|err|={r[nm + '_err']:.3e} "
            f"max|ref|={r[nm + '_max_ref']:.3e} err/tol={r[nm + '_ratio']:.3f} at {r[nm + '_at']}")
    log(f"    (oracle {r['oracle_s']:.1f} s on {r['workers']} processes)")
    assert r["dq_nonfinite"] == 0 and r["dk_nonfinite"] == 0 and r["dv_nonfinite"] == 0
    assert r["dq_ratio"] <= 1.0, f"dQ exceeds tolerance at {r['dq_at']}"
    assert r["dk_ratio"] <= 1.0, f"dK exceeds tolerance at {r['dk_at']}"
    assert r["dv_ratio"] <= 1.0, f"dV exceeds tolerance at {r['dv_at']}"
    return res, do


def check_dv_column_sums(w, res, do):
    # every softmax row sums to one: sum over keys of dV[:, h] = sum of dO over
    # the rows of head h (every row attends to its own block here), on all keys
    H, g = w.num_kv_heads, w.gqa_group
    dof = do.float().numpy()
    dv = res["dv_bits"]
    for h in range(H):
        want = dof[:, h * g : (h + 1) * g, :].astype(np.float64).sum(axis=(0, 1))
        dvh = decode_out(dv[:, h, :], w.dtype)
        got = dvh.sum(axis=0)
        # each 16-bit dV element is off by at most half an ulp (2^-9 relative):
        # the column sum by at most 2^-9 sum|dV|; 2^-8 leaves room for fp32 order
        tol = 2.0**-8 * np.abs(dvh).sum(axis=0) + 1e-3
        log(f"    dV column sums head {h}: max|diff|={float(np.max(np.abs(got - want))):.3e}")
        assert np.all(np.abs(got - want) <= tol)


@pytest.mark.timeout(900)
def test_backward_64k_all_dq_hot_block_dk_dv(oracle_service):
    w = workload("n64k_h4_g4_d128_t16_bf16")
    res, do = check_large_backward(oracle_service, w, 13)
    check_dv_column_sums(w, res, do)


@pytest.mark.timeout(900)
def test_backward_large_head_shape_all_dq_hot_block_dk_dv(oracle_service):
    # two packed 32K sequences, h_K = 8, g = 8, d = 256 with 16-bit partials
    w = workload("b2_n32k_h8_g8_d256_t16_bf16")
    res, do = check_large_backward(oracle_service, w, 14)
    check_dv_column_sums(w, res, do)
