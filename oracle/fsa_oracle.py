"""CPU float64 oracle for the NSA selected-attention forward (FSA order).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path
and imports nothing from it.

What it computes
----------------
Sources: "FSA: An Alternative Efficient Implementation of Native Sparse
Attention Kernel" paper notes (papernotes.org, ICLR 2026), sections
"Overall framework" (整体框架) and "Key design 2" (关键设计 2: the index
tensors I_i, N_valid, O_i built from the selection tensor of shape
h_K x N x T), and the Flash-Sparse-Attention README (Method and Usage
sections: GQA groups share one KV head, packed sequences with cu_seqlens).
FSA only reorders the loops of NSA's selected attention and leaves its result
unchanged (README, Features; paper notes, Overall framework), so the oracle is
the plain definition of that attention:

* every query token t of sequence s (tokens [c_s, c_{s+1})) and KV head h has a
  selected block set S = {e in Sel[h, t, :] : 0 <= e <= own block}; the set
  semantics make duplicates count once;
* its keys are the union of those blocks, restricted causally to k <= t;
* each of the g query heads h*g + j of the group attends to those keys with a
  softmax scaled by ``scale``; the outputs are the softmax-weighted values, the
  row maximum m and the log-sum-exp lse (natural log) of the scaled scores;
* an empty key set gives O = 0 and m = lse = -inf.

``selected_attention_backward`` is the derivative of that forward for a given
output gradient (dQ, dK, dV), Sel held constant.  ``select_blocks`` produces
the Sel rows from per-block scores (top-k with forced initial / local blocks).

The index oracle produces the canonical layout: segment f = h*NB + global
block, counts[f] = N_valid (number of queries that select the block), offsets =
exclusive prefix of counts (the compact output offsets O_i), qidx = the query
tokens of each segment in ascending order (I_i) and slot[h, t, j] = position of
entry (h, t, j) in qidx, or -1 for entries that select nothing.

Where the pages are silent this module takes the plainest reading: a Sel row
is a set (a repeated block counts once, at its first position), negative
entries and entries past the token's own block select nothing, key k is
visible to token t iff k <= t, query head h*g + j belongs to KV head h, and
lse is in natural-log units with the softmax scale applied.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

__all__ = [
    "sequence_layout",
    "valid_entries",
    "build_index",
    "key_indices",
    "selected_attention",
    "selected_attention_backward",
    "select_blocks",
]


def sequence_layout(cu_seqlens, block_size: int):
    """Per-token sequence id and own local block; per-sequence block counts and
    the global-block offset of each sequence (blocks numbered sequence by
    sequence)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = int(cu[-1])
    tok = np.arange(n, dtype=np.int64)
    seq = np.searchsorted(cu, tok, side="right") - 1
    own = (tok - cu[seq]) // block_size
    nb = -(-(cu[1:] - cu[:-1]) // block_size)
    gboff = np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)
    return seq, own, nb, gboff


def valid_entries(sel, cu_seqlens, block_size: int) -> np.ndarray:
    """Boolean [h_K, N, T]: entry (h, t, j) contributes a block iff
    0 <= Sel[h,t,j] <= own block of t and no earlier entry of the row holds the
    same block (the set is a union, so a repeated block is counted once)."""
    sel = np.asarray(sel)
    _, own, _, _ = sequence_layout(cu_seqlens, block_size)
    in_range = (sel >= 0) & (sel <= own[None, :, None])
    first = np.ones(sel.shape, dtype=bool)
    T = sel.shape[2]
    for j in range(1, T):
        for jj in range(j):
            first[:, :, j] &= sel[:, :, j] != sel[:, :, jj]
    return in_range & first


def build_index(sel, cu_seqlens, block_size: int):
    """Invert Sel into per-(KV head, block) query lists (paper notes, Key
    design 2).

    Entries are enumerated in (h, t, j) order and stably sorted by their
    segment key f = h*NB + global block (a counting sort), so each segment
    lists its query tokens in ascending order.
    """
    sel = np.asarray(sel, dtype=np.int64)
    H, N, T = sel.shape
    seq, _, _, gboff = sequence_layout(cu_seqlens, block_size)
    NB = int(gboff[-1])
    valid = valid_entries(sel, cu_seqlens, block_size)
    hh, tt, jj = np.nonzero(valid)  # C order: h, then t, then j
    gb = gboff[seq[tt]] + sel[hh, tt, jj]
    key = hh * NB + gb
    order = np.argsort(key, kind="stable")
    counts = np.bincount(key, minlength=H * NB).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    qidx = tt[order].astype(np.int64)
    slot = np.full((H, N, T), -1, dtype=np.int64)
    slot[hh[order], tt[order], jj[order]] = np.arange(order.size, dtype=np.int64)
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "qidx": qidx.astype(np.int32),
        "slot": slot.astype(np.int32),
        "num_blocks": NB,
        "pairs": int(order.size),
    }


def key_indices(sel_row, t: int, seq_start: int, seq_end: int, block_size: int) -> np.ndarray:
    """Sorted global key indices that query t attends to: the union of its
    selected blocks within its own sequence, causally restricted to k <= t."""
    own = (t - seq_start) // block_size
    blocks = sorted({int(e) for e in np.asarray(sel_row).tolist() if 0 <= e <= own})
    keys = []
    for e in blocks:
        lo = seq_start + e * block_size
        hi = min(seq_start + (e + 1) * block_size, seq_end, t + 1)
        keys.extend(range(lo, hi))
    return np.asarray(keys, dtype=np.int64)


def selected_attention(
    q,
    k,
    v,
    sel,
    cu_seqlens,
    block_size: int,
    scale: Optional[float] = None,
    tokens: Optional[Iterable[int]] = None,
):
    """NSA selected attention, one (token, KV head) at a time, in float64.

    q: [N, h_K*g, d]; k, v: [N, h_K, d]; sel: [h_K, N, T].  Query head
    h*g + j belongs to KV head h.  ``tokens`` restricts the evaluation to a
    subset of query tokens (all by default).

    Returns (o [n, h_q, d], row_max [n, h_q], lse [n, h_q]) for the evaluated
    tokens, in float64; lse is the natural-log log-sum-exp of the scaled scores.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    sel = np.asarray(sel)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N, HQ, D = q.shape
    H = k.shape[1]
    g = HQ // H
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    toks = np.arange(N) if tokens is None else np.asarray(list(tokens), dtype=np.int64)
    o = np.zeros((toks.size, HQ, v.shape[2]), dtype=np.float64)
    row_max = np.full((toks.size, HQ), -np.inf, dtype=np.float64)
    lse = np.full((toks.size, HQ), -np.inf, dtype=np.float64)
    for i, t in enumerate(toks.tolist()):
        s = int(np.searchsorted(cu, t, side="right") - 1)
        c0, c1 = int(cu[s]), int(cu[s + 1])
        for h in range(H):
            keys = key_indices(sel[h, t], t, c0, c1, block_size)
            if keys.size == 0:
                continue
            qh = np.asarray(q[t, h * g : (h + 1) * g, :], dtype=np.float64)  # [g, d]
            kh = np.asarray(k[keys, h, :], dtype=np.float64)  # [nk, d]
            vh = np.asarray(v[keys, h, :], dtype=np.float64)  # [nk, d]
            scores = scale * (qh @ kh.T)  # [g, nk]
            m = scores.max(axis=1)
            l = np.exp(scores - m[:, None]).sum(axis=1)
            ls = m + np.log(l)
            p = np.exp(scores - ls[:, None])
            o[i, h * g : (h + 1) * g, :] = p @ vh
            row_max[i, h * g : (h + 1) * g] = m
            lse[i, h * g : (h + 1) * g] = ls
    return o, row_max, lse


def selected_attention_backward(
    q,
    k,
    v,
    sel,
    cu_seqlens,
    block_size: int,
    dout,
    scale: Optional[float] = None,
    tokens: Optional[Iterable[int]] = None,
    with_sq: bool = False,
):
    """Gradients of ``selected_attention`` for an output gradient ``dout``, in
    float64, one (token, KV head) at a time.

    ``tokens`` restricts the loop to those query tokens: dq then holds their
    rows only (in the given order; a row's dQ depends on that row alone), while
    dk and dv, full size, hold only those tokens' contributions.

    The pages give the forward only and state that the module trains (README,
    Usage: ``loss.backward()``; Evaluation: the unit tests compare forward and
    backward outputs).  The gradient is therefore the plain derivative of the
    forward definition above, with Sel a constant.  For the g query rows of
    (t, h) with key set K_t: P = softmax(scale * Q K^T), O = P V, and for an
    output gradient dO:

        dP = dO V^T,   D = rowsum(dO * O),   dS = P * (dP - D),
        dQ = scale * dS K,   dK += scale * dS^T Q,   dV += P^T dO,

    dK and dV summed over every (t, h) whose key set holds the key.  Rows with
    an empty key set contribute nothing.

    Returns (dq [n, h_q, d] for the n evaluated tokens, dk [N, h_K, d],
    dv [N, h_K, d]) in float64.

    ``with_sq`` also returns, for bounding the rounding error of an
    implementation that rounds each term's operands, the sum of the squares of
    the terms every gradient element adds up: dq_sq over the keys k of
    (scale dS[:, k] K[k])^2, dk_sq over the rows of (scale dS Q)^2 and dv_sq over
    the rows of (P dO)^2 (same shapes as dq, dk, dv).  These are not part of
    the gradient.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    sel = np.asarray(sel)
    dout = np.asarray(dout)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N, HQ, D = q.shape
    H = k.shape[1]
    g = HQ // H
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    toks = list(range(N)) if tokens is None else [int(x) for x in tokens]
    dq = np.zeros((len(toks), HQ, D), dtype=np.float64)
    dk = np.zeros((N, H, D), dtype=np.float64)
    dv = np.zeros((N, H, v.shape[2]), dtype=np.float64)
    if with_sq:
        dq_sq, dk_sq, dv_sq = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for i, t in enumerate(toks):
        s = int(np.searchsorted(cu, t, side="right") - 1)
        c0, c1 = int(cu[s]), int(cu[s + 1])
        for h in range(H):
            keys = key_indices(sel[h, t], t, c0, c1, block_size)
            if keys.size == 0:
                continue
            qh = np.asarray(q[t, h * g : (h + 1) * g, :], dtype=np.float64)  # [g, d]
            kh = np.asarray(k[keys, h, :], dtype=np.float64)  # [nk, d]
            vh = np.asarray(v[keys, h, :], dtype=np.float64)  # [nk, d]
            doh = np.asarray(dout[t, h * g : (h + 1) * g, :], dtype=np.float64)  # [g, d]
            scores = scale * (qh @ kh.T)  # [g, nk]
            m = scores.max(axis=1)
            p = np.exp(scores - m[:, None])
            p /= p.sum(axis=1, keepdims=True)
            o = p @ vh
            dp = doh @ vh.T
            delta = (doh * o).sum(axis=1)
            ds = p * (dp - delta[:, None])
            dq[i, h * g : (h + 1) * g, :] = scale * (ds @ kh)
            dk[keys, h, :] += scale * (ds.T @ qh)
            dv[keys, h, :] += p.T @ doh
            if with_sq:
                dq_sq[i, h * g : (h + 1) * g, :] = scale**2 * ((ds**2) @ (kh**2))
                dk_sq[keys, h, :] += scale**2 * ((ds**2).T @ (qh**2))
                dv_sq[keys, h, :] += (p**2).T @ (doh**2)
    if with_sq:
        return dq, dk, dv, dq_sq, dk_sq, dv_sq
    return dq, dk, dv


def select_blocks(scores, cu_seqlens, block_size: int, topk: int, init_blocks: int, local_blocks: int,
                  tokens: Optional[Iterable[int]] = None):
    """NSA block selection: the Sel rows the attention consumes, from per-block
    importance scores, in int32 [h_K, N, T].

    The pages give the selection's hyper-parameters (README, Usage:
    ``topk=16, init_blocks=1, local_blocks=2``) and say that each query token
    picks T KV blocks per KV head (paper notes, Background and motivation);
    the scores themselves (NSA's compressed attention) are not described and
    are an input here: ``scores[h, t, e]`` for the local blocks e of t's
    sequence (entries e > own block are ignored).  For query token t (own
    block b) and KV head h the row is

      * the forced blocks: initial blocks 0 .. init_blocks-1, then the local
        blocks b, b-1, .. b-local_blocks+1, each kept once and only if
        0 <= e <= b, truncated to T entries;
      * then the remaining candidates e in [0, b] ranked by score, highest
        first, ties to the smaller e (NaN counts as -inf), as many as fit;
      * then -1 padding.

    ``tokens`` restricts the evaluation to those query tokens (the other rows
    stay -1).
    """
    scores = np.asarray(scores)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    H, N = scores.shape[0], scores.shape[1]
    sel = np.full((H, N, topk), -1, dtype=np.int32)
    for t in range(N) if tokens is None else [int(x) for x in tokens]:
        s = int(np.searchsorted(cu, t, side="right") - 1)
        own = (t - int(cu[s])) // block_size
        forced = []
        for e in list(range(init_blocks)) + [own - i for i in range(local_blocks)]:
            if 0 <= e <= own and e not in forced:
                forced.append(e)
        forced = forced[:topk]
        free = [e for e in range(own + 1) if e not in forced]
        for h in range(H):
            sc = np.asarray(scores[h, t, : own + 1], dtype=np.float64)
            sc = np.where(np.isnan(sc), -np.inf, sc)
            # rank by (score descending, block ascending)
            order = sorted(free, key=lambda e: (-sc[e], e))
            row = forced + order[: topk - len(forced)]
            sel[h, t, : len(row)] = row
    return sel
