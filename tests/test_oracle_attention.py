"""Pins for the attention oracle (CPU only).

Each test checks ``oracle.selected_attention`` against something other than
itself: a hand-worked example, a dense masked-softmax formulation built
straight from the block mask, torch's float64 scaled-dot-product attention
when the selection covers every block, closed forms (zero queries, constant
values, single-key queries) and invariances (order of Sel entries, duplicated
entries, identical query heads).
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from conftest import GOLDEN
import oracle.fsa_oracle as O
from sparse_attention_sel_amd.inputs import cu_seqlens_of, make_sel, shuffle_rows


def rand_qkv(rng, n, H, g, d):
    q = rng.standard_normal((n, H * g, d))
    k = rng.standard_normal((n, H, d))
    v = rng.standard_normal((n, H, d))
    return q, k, v


def random_sel(rng, H, cu, B, T):
    n = int(cu[-1])
    sel = np.empty((H, n, T), dtype=np.int32)
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        nb = (c1 - c0 + B - 1) // B
        sel[:, c0:c1, :] = rng.integers(-2, nb + 2, size=(H, c1 - c0, T))
    dup = rng.random(sel.shape) < 0.2
    sel[dup] = np.roll(sel, 1, axis=2)[dup]
    return sel


def dense_block_mask_attention(q, k, v, sel, cu, B, scale):
    """Masked softmax over all N keys with M[t, k] = (block of k in t's
    sequence is listed in Sel[h, t]) and (k <= t)."""
    N, HQ, D = q.shape
    H = k.shape[1]
    g = HQ // H
    o = np.zeros((N, HQ, D))
    lse = np.full((N, HQ), -np.inf)
    mx = np.full((N, HQ), -np.inf)
    seq = np.searchsorted(cu, np.arange(N), side="right") - 1
    causal = np.tril(np.ones((N, N), dtype=bool))
    for h in range(H):
        M = np.zeros((N, N), dtype=bool)
        for t in range(N):
            c0, c1 = int(cu[seq[t]]), int(cu[seq[t] + 1])
            for e in sel[h, t]:
                if e >= 0:
                    M[t, c0 + e * B : min(c0 + (e + 1) * B, c1)] = True
        M &= causal
        for j in range(g):
            S = scale * (q[:, h * g + j, :] @ k[:, h, :].T)
            S = np.where(M, S, -np.inf)
            rows = M.any(axis=1)
            m = np.where(rows, S.max(axis=1), -np.inf)
            P = np.where(M, np.exp(S - np.where(rows, m, 0.0)[:, None]), 0.0)
            l = P.sum(axis=1)
            o[rows, h * g + j] = (P[rows] @ v[:, h, :]) / l[rows, None]
            lse[rows, h * g + j] = m[rows] + np.log(l[rows])
            mx[rows, h * g + j] = m[rows]
    return o, mx, lse


def test_handworked_example():
    with open(os.path.join(GOLDEN, "attention_handworked.json")) as f:
        g = json.load(f)
    o, m, lse = O.selected_attention(
        np.asarray(g["q"]), np.asarray(g["k"]), np.asarray(g["v"]), np.asarray(g["sel"]),
        g["cu_seqlens"], g["block_size"], scale=g["scale"],
    )
    np.testing.assert_allclose(o, np.asarray(g["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(m, np.asarray(g["row_max"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.asarray(g["lse"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", range(5))
def test_dense_block_mask_equivalence(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 90, size=int(rng.integers(1, 4)))
    cu = cu_seqlens_of(lens)
    B = int(rng.choice([4, 8, 16]))
    T = int(rng.integers(1, 6))
    H, g, d = int(rng.integers(1, 3)), int(rng.integers(1, 4)), 8
    q, k, v = rand_qkv(rng, int(cu[-1]), H, g, d)
    sel = random_sel(rng, H, cu, B, T)
    scale = 1.0 / math.sqrt(d)
    o, m, lse = O.selected_attention(q, k, v, sel, cu, B, scale)
    o2, m2, lse2 = dense_block_mask_attention(q, k, v, sel, cu, B, scale)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lse2))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], lse2[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(m[fin], m2[fin], rtol=0, atol=1e-12)


def sdpa_causal(q, k, v, cu, scale, mask_fn=None):
    """torch float64 scaled-dot-product attention per packed sequence, GQA by
    repeating each KV head over its consecutive query heads."""
    N, HQ, D = q.shape
    H = k.shape[1]
    g = HQ // H
    o = np.zeros((N, HQ, D))
    lse = np.zeros((N, HQ))
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        if c1 == c0:
            continue
        qt = torch.from_numpy(q[c0:c1]).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k[c0:c1]).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        vt = torch.from_numpy(v[c0:c1]).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        L = c1 - c0
        allowed = torch.tril(torch.ones(L, L, dtype=torch.bool))
        if mask_fn is not None:
            allowed &= mask_fn(L)
        out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed, scale=scale)
        o[c0:c1] = out[0].permute(1, 0, 2).numpy()
        scores = (qt @ kt.transpose(-1, -2)) * scale
        scores = scores.masked_fill(~allowed, float("-inf"))
        lse[c0:c1] = torch.logsumexp(scores, dim=-1)[0].permute(1, 0).numpy()
    return o, lse


@pytest.mark.parametrize("seed", range(3))
def test_full_selection_is_causal_attention(seed):
    rng = np.random.default_rng(50 + seed)
    lens = [int(x) for x in rng.integers(5, 120, size=2)]
    cu = cu_seqlens_of(lens)
    B, H, g, d = 16, 2, 3, 16
    nbmax = max(-(-L // B) for L in lens)
    sel = np.broadcast_to(np.arange(nbmax, dtype=np.int32), (H, int(cu[-1]), nbmax)).copy()
    q, k, v = rand_qkv(rng, int(cu[-1]), H, g, d)
    scale = 0.3
    o, _, lse = O.selected_attention(q, k, v, sel, cu, B, scale)
    o2, lse2 = sdpa_causal(q, k, v, cu, scale)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def test_own_block_only_is_block_diagonal_causal():
    rng = np.random.default_rng(3)
    lens = [100, 37]
    cu = cu_seqlens_of(lens)
    B, H, g, d = 8, 2, 2, 16
    n = int(cu[-1])
    own = np.concatenate([np.arange(L) // B for L in lens]).astype(np.int32)
    sel = np.broadcast_to(own[None, :, None], (H, n, 1)).copy()
    q, k, v = rand_qkv(rng, n, H, g, d)
    o, _, lse = O.selected_attention(q, k, v, sel, cu, B, 0.25)

    def same_block(L):
        b = torch.arange(L) // B
        return b[:, None] == b[None, :]

    o2, lse2 = sdpa_causal(q, k, v, cu, 0.25, same_block)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def test_order_invariance_bitwise():
    rng = np.random.default_rng(9)
    cu = cu_seqlens_of([200, 90])
    B, H, g, d = 16, 2, 2, 8
    sel = random_sel(rng, H, cu, B, 5)
    q, k, v = rand_qkv(rng, int(cu[-1]), H, g, d)
    a = O.selected_attention(q, k, v, sel, cu, B)
    b = O.selected_attention(q, k, v, shuffle_rows(sel, 10), cu, B)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_duplicates_equal_deduplicated():
    rng = np.random.default_rng(11)
    cu = cu_seqlens_of([150])
    B, H, g, d = 16, 1, 2, 8
    q, k, v = rand_qkv(rng, 150, H, g, d)
    base = random_sel(rng, H, cu, B, 3)
    dup = np.concatenate([base, base[:, :, :2]], axis=2)
    a = O.selected_attention(q, k, v, base, cu, B)
    b = O.selected_attention(q, k, v, dup, cu, B)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_zero_queries_give_key_mean():
    # With q = 0 all scores vanish: lse = ln |K_t| and o = mean of V over K_t.
    rng = np.random.default_rng(12)
    lens = [70, 45]
    cu = cu_seqlens_of(lens)
    B, H, g, d = 16, 2, 2, 4
    n = int(cu[-1])
    q = np.zeros((n, H * g, d))
    _, k, v = rand_qkv(rng, n, H, g, d)
    sel = np.zeros((H, n, 1), dtype=np.int32)  # block 0 only: K_t = [c_s, min(c_s + B, t + 1))
    o, m, lse = O.selected_attention(q, k, v, sel, cu, B)
    for s, L in enumerate(lens):
        c0 = int(cu[s])
        for t in range(c0, c0 + L):
            nk = min(B, t - c0 + 1)
            for h in range(H):
                want = v[c0 : c0 + nk, h].mean(axis=0)
                for j in range(g):
                    np.testing.assert_allclose(o[t, h * g + j], want, rtol=0, atol=1e-13)
                    assert abs(lse[t, h * g + j] - math.log(nk)) < 1e-13
                    assert m[t, h * g + j] == 0.0


def test_constant_values_and_first_token():
    rng = np.random.default_rng(13)
    lens = [64, 33, 1]
    cu = cu_seqlens_of(lens)
    B, H, g, d = 16, 2, 3, 8
    n = int(cu[-1])
    q, k, _ = rand_qkv(rng, n, H, g, d)
    v = np.broadcast_to(np.arange(d, dtype=np.float64) - 2.5, (n, H, d)).copy()
    sel = random_sel(rng, H, cu, B, 4)
    sel[:, :, 0] = 0  # every row keeps block 0, so no key set is empty
    o, m, lse = O.selected_attention(q, k, v, sel, cu, B, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, :1, :], o.shape), rtol=0, atol=1e-13)
    # first token of each sequence sees only itself
    _, _, v2 = rand_qkv(rng, n, H, g, d)
    o2, m2, lse2 = O.selected_attention(q, k, v2, sel, cu, B, 0.5)
    for s in range(len(lens)):
        c0 = int(cu[s])
        for h in range(H):
            for j in range(g):
                sc = 0.5 * float(q[c0, h * g + j] @ k[c0, h])
                np.testing.assert_allclose(o2[c0, h * g + j], v2[c0, h], rtol=0, atol=1e-15)
                assert abs(lse2[c0, h * g + j] - sc) < 1e-14 and abs(m2[c0, h * g + j] - sc) < 1e-14


def test_identical_heads_identical_outputs_and_empty_rows():
    rng = np.random.default_rng(14)
    cu = cu_seqlens_of([90])
    B, H, g, d = 16, 1, 3, 8
    q1, k, v = rand_qkv(rng, 90, H, 1, d)
    q = np.repeat(q1, g, axis=1)
    sel = random_sel(rng, H, cu, B, 3)
    sel[:, 10] = -1  # a row that selects nothing
    o, m, lse = O.selected_attention(q, k, v, sel, cu, B)
    for j in range(1, g):
        assert np.array_equal(o[:, j], o[:, 0]) and np.array_equal(lse[:, j], lse[:, 0])
    assert np.all(o[10] == 0) and np.all(np.isneginf(lse[10])) and np.all(np.isneginf(m[10]))


def test_generated_selection_matches_dense_mask():
    # the synthetic generators' rows through both formulations
    rng = np.random.default_rng(15)
    lens = [300, 200]
    cu = cu_seqlens_of(lens)
    sel, _ = make_sel("init_local_zipf", lens, 2, 16, 6, 16)
    q, k, v = rand_qkv(rng, int(cu[-1]), 2, 2, 8)
    a = O.selected_attention(q, k, v, sel, cu, 16)
    b = dense_block_mask_attention(q, k, v, sel, cu, 16, 1.0 / math.sqrt(8))
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a[2], b[2], rtol=0, atol=1e-12)
