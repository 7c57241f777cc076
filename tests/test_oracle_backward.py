"""Pins of the oracle's backward (selected_attention_backward) to things other
than its own code: central finite differences of the forward oracle, torch
float64 autograd through a dense block-masked softmax built straight from Sel,
closed forms (zero output gradient, constant values, column sums of dV) and
invariance under shuffled Sel rows.

The pages define the forward only and state that the module trains and that
its tests compare backward outputs (README, Usage and Evaluation), so the
backward's reference is the derivative of the forward definition.
"""

import math

import numpy as np
import pytest
import torch

import oracle.fsa_oracle as O
from sparse_attention_sel_amd.inputs import cu_seqlens_of, shuffle_rows
from test_oracle_attention import rand_qkv, random_sel


def small_problem(seed, seqlens=(13, 0, 17), H=2, g=2, d=4, B=4, T=3):
    rng = np.random.default_rng(seed)
    cu = cu_seqlens_of(seqlens)
    n = int(cu[-1])
    q, k, v = rand_qkv(rng, n, H, g, d)
    sel = random_sel(rng, H, cu, B, T)
    do = rng.standard_normal(q.shape)
    return q, k, v, sel, cu, B, do


def loss(q, k, v, sel, cu, B, do, scale):
    o, _, _ = O.selected_attention(q, k, v, sel, cu, B, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("seed", range(2))
def test_finite_differences(seed):
    # dL/dx for L = sum(O * dO) by central differences of the forward oracle
    q, k, v, sel, cu, B, do = small_problem(seed)
    scale = 1.0 / math.sqrt(q.shape[2])
    dq, dk, dv = O.selected_attention_backward(q, k, v, sel, cu, B, do, scale)
    rng = np.random.default_rng(100 + seed)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = x.reshape(-1)
        picks = rng.choice(flat.size, size=min(60, flat.size), replace=False)
        for i in picks:
            old = flat[i]
            flat[i] = old + eps
            lp = loss(q, k, v, sel, cu, B, do, scale)
            flat[i] = old - eps
            lm = loss(q, k, v, sel, cu, B, do, scale)
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.reshape(-1)[i]) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, grad.reshape(-1)[i])


def dense_masked_torch(q, k, v, sel, cu, B, scale):
    """O from a dense masked softmax over all keys (mask M[t, k]: the block of
    k in t's sequence is listed in Sel[h, t] and k <= t), differentiable."""
    N, HQ, D = q.shape
    H = k.shape[1]
    g = HQ // H
    seq = np.searchsorted(cu, np.arange(N), side="right") - 1
    outs = []
    for h in range(H):
        M = np.zeros((N, N), dtype=bool)
        for t in range(N):
            c0, c1 = int(cu[seq[t]]), int(cu[seq[t] + 1])
            for e in sel[h, t]:
                if e >= 0:
                    M[t, c0 + e * B : min(c0 + (e + 1) * B, c1)] = True
        M &= np.tril(np.ones((N, N), dtype=bool))
        Mt = torch.from_numpy(M)
        rows = Mt.any(dim=1, keepdim=True)
        for j in range(g):
            S = scale * (q[:, h * g + j, :] @ k[:, h, :].T)
            S = S.masked_fill(~Mt, float("-inf"))
            P = torch.softmax(torch.where(rows, S, torch.zeros_like(S)), dim=1)
            P = torch.where(Mt, P, torch.zeros_like(P))  # rows with no key: all zero
            outs.append(P @ v[:, h, :])
    return torch.stack(outs, dim=1)  # [N, HQ, D] (head order h*g + j)


@pytest.mark.parametrize("seed", range(3))
def test_torch_autograd_dense_mask(seed):
    q, k, v, sel, cu, B, do = small_problem(seed + 10, seqlens=(21, 30), H=2, g=3, d=8, B=8, T=3)
    scale = 1.0 / math.sqrt(8)
    dq, dk, dv = O.selected_attention_backward(q, k, v, sel, cu, B, do, scale)
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = dense_masked_torch(qt, kt, vt, sel, cu, B, scale)
    (o * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(qt.grad.numpy(), dq, atol=1e-10)
    np.testing.assert_allclose(kt.grad.numpy(), dk, atol=1e-10)
    np.testing.assert_allclose(vt.grad.numpy(), dv, atol=1e-10)


def test_zero_output_gradient():
    q, k, v, sel, cu, B, do = small_problem(3)
    for x in O.selected_attention_backward(q, k, v, sel, cu, B, np.zeros_like(do)):
        assert np.all(x == 0)


def test_constant_values_give_no_score_gradient():
    # V identical for every key: O does not depend on the scores, so dQ = dK = 0
    q, k, v, sel, cu, B, do = small_problem(4)
    v[:] = np.array([0.3, -1.2, 0.7, 2.0])
    dq, dk, dv = O.selected_attention_backward(q, k, v, sel, cu, B, do)
    assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
    assert np.abs(dv).max() > 0.1


def test_value_gradient_column_sums():
    # every softmax row sums to 1, so summing dV over the keys of head h gives
    # the sum of dO over the rows of head h that attend to at least one key
    q, k, v, sel, cu, B, do = small_problem(5, seqlens=(40,), H=2, g=2, d=4, B=4, T=4)
    sel[:, ::7, :] = -1  # some rows select nothing
    _, _, dv = O.selected_attention_backward(q, k, v, sel, cu, B, do)
    _, _, lse = O.selected_attention(q, k, v, sel, cu, B)
    H, g = k.shape[1], q.shape[1] // k.shape[1]
    for h in range(H):
        rows = np.isfinite(lse[:, h * g : (h + 1) * g])  # [N, g]
        want = (do[:, h * g : (h + 1) * g, :] * rows[:, :, None]).sum(axis=(0, 1))
        np.testing.assert_allclose(dv[:, h, :].sum(axis=0), want, atol=1e-10)


def test_shuffled_rows_bitwise():
    q, k, v, sel, cu, B, do = small_problem(6)
    a = O.selected_attention_backward(q, k, v, sel, cu, B, do)
    b = O.selected_attention_backward(q, k, v, shuffle_rows(sel, 7), cu, B, do)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_sums_of_squared_terms_match_autograd():
    # with_sq: the sums of squares of the terms each gradient element adds
    # up, pinned to torch autograd through the dense block-masked softmax:
    # a row's loss L_r = O_r . dO_r has dL_r/dK_k = scale dS_rk Q_r and
    # dL_r/dV_k = P_rk dO_r (one term per row), and dL/dS_tk times scale K_k
    # is the key-k term of dQ_t
    q, k, v, sel, cu, B, do = small_problem(12, seqlens=(11, 14), H=2, g=2, d=4, B=4, T=3)
    scale = 1.0 / math.sqrt(4)
    res = O.selected_attention_backward(q, k, v, sel, cu, B, do, scale, with_sq=True)
    dq, dk, dv, dq_sq, dk_sq, dv_sq = res
    base = O.selected_attention_backward(q, k, v, sel, cu, B, do, scale)
    for a, b in zip(base, (dq, dk, dv)):
        assert np.array_equal(a, b)  # the gradients themselves are unchanged
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    dot = torch.from_numpy(do)

    def row_losses(kk, vv):
        return (dense_masked_torch(qt, kk, vv, sel, cu, B, scale) * dot).sum(-1).reshape(-1)

    jk, jv = torch.autograd.functional.jacobian(row_losses, (kt, vt))  # [rows, N, H, D] each
    np.testing.assert_allclose((jk**2).sum(0).numpy(), dk_sq, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose((jv**2).sum(0).numpy(), dv_sq, atol=1e-12, rtol=1e-10)
    # dQ terms: gradient of L with respect to each head's score matrix
    N, HQ, D = q.shape
    H = k.shape[1]
    g = HQ // H
    seq = np.searchsorted(cu, np.arange(N), side="right") - 1
    want = np.zeros_like(dq_sq)
    for h in range(H):
        M = np.zeros((N, N), dtype=bool)
        for t in range(N):
            c0, c1 = int(cu[seq[t]]), int(cu[seq[t] + 1])
            for e in sel[h, t]:
                if e >= 0:
                    M[t, c0 + e * B : min(c0 + (e + 1) * B, c1)] = True
        M &= np.tril(np.ones((N, N), dtype=bool))
        Mt = torch.from_numpy(M)
        rows = Mt.any(dim=1, keepdim=True)
        for j in range(g):
            S = (scale * (qt[:, h * g + j, :] @ kt[:, h, :].T)).requires_grad_(True)
            Sm = S.masked_fill(~Mt, float("-inf"))
            P = torch.softmax(torch.where(rows, Sm, torch.zeros_like(Sm)), dim=1)
            P = torch.where(Mt, P, torch.zeros_like(P))
            ((P @ vt[:, h, :]) * dot[:, h * g + j, :]).sum().backward()
            G = S.grad.numpy()  # dL/dS [N, N]
            want[:, h * g + j, :] = (G**2) @ ((scale * k[:, h, :]) ** 2)
    np.testing.assert_allclose(want, dq_sq, atol=1e-12, rtol=1e-10)
