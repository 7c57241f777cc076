"""Pins of the block-selection oracle (select_blocks): a hand-derived example,
a brute force that counts ranks instead of sorting, and invariants (no
duplicates, causal bounds, forced blocks present, every unselected candidate
scores no higher than every selected free block, invariance to per-row shifts
and positive scaling of the scores, NaN = -inf)."""

import json
import os

import numpy as np
import pytest

import oracle.fsa_oracle as O
from conftest import GOLDEN
from sparse_attention_sel_amd.inputs import cu_seqlens_of


def test_handworked_example():
    g = json.load(open(os.path.join(GOLDEN, "select_handworked.json")))
    B = g["block_size"]
    cu = cu_seqlens_of(g["seqlens"])
    N = int(cu[-1])
    by_block = np.array([[float(x) for x in row] for row in g["scores_by_block"]], dtype=np.float32)
    scores = np.broadcast_to(by_block[:, None, :], (by_block.shape[0], N, by_block.shape[1])).copy()
    own = np.concatenate([np.arange(L) // B for L in g["seqlens"]])
    for case in g["cases"]:
        sel = O.select_blocks(scores, cu, B, case["topk"], case["init_blocks"], case["local_blocks"])
        for t in range(N):
            want = case["rows_by_own_block"][str(int(own[t]))]
            for h in range(2):
                assert sel[h, t].tolist() == want[h], (case["topk"], t, h)


def brute_force(scores, cu, B, T, init_blocks, local_blocks):
    H, N = scores.shape[:2]
    out = np.full((H, N, T), -1, dtype=np.int64)
    for t in range(N):
        s = max(i for i in range(len(cu) - 1) if cu[i] <= t)
        b = (t - cu[s]) // B
        want_forced = list(range(init_blocks)) + [b - i for i in range(local_blocks)]
        forced = []
        for e in want_forced:
            if e < 0 or e > b or e in forced:
                continue
            forced.append(e)
        forced = forced[:T]
        for h in range(H):
            sc = [(-np.inf if np.isnan(x) else float(x)) for x in scores[h, t, : b + 1]]
            free = [e for e in range(b + 1) if e not in forced]
            # rank of e = number of free candidates strictly ahead of it
            rank = {e: sum(1 for f in free if (sc[f] > sc[e]) or (sc[f] == sc[e] and f < e)) for e in free}
            k = T - len(forced)
            picks = [e for r in range(min(k, len(free))) for e in free if rank[e] == r]
            row = forced + picks
            out[h, t, : len(row)] = row
    return out


def random_scores(rng, H, cu, B, S):
    N = int(cu[-1])
    sc = rng.standard_normal((H, N, S)).astype(np.float32)
    sc[rng.random(sc.shape) < 0.15] = 0.5  # ties
    sc[rng.random(sc.shape) < 0.05] = np.nan
    sc[rng.random(sc.shape) < 0.05] = -np.inf
    return sc


@pytest.mark.parametrize("seed", range(6))
def test_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    seqlens = rng.integers(0, 40, size=3).tolist()
    if sum(seqlens) == 0:
        seqlens[0] = 7
    cu = cu_seqlens_of(seqlens)
    B = int(rng.choice([2, 4, 8]))
    S = max(1, -(-max(seqlens) // B))
    T = int(rng.integers(1, 8))
    ib, lb = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    sc = random_scores(rng, 2, cu, B, S)
    np.testing.assert_array_equal(O.select_blocks(sc, cu, B, T, ib, lb), brute_force(sc, cu, B, T, ib, lb))


@pytest.mark.parametrize("seed", range(3))
def test_invariants(seed):
    rng = np.random.default_rng(50 + seed)
    seqlens = [300, 77, 128]
    cu = cu_seqlens_of(seqlens)
    B, T, ib, lb = 16, 6, 1, 2
    S = -(-max(seqlens) // B)
    sc = random_scores(rng, 3, cu, B, S)
    sel = O.select_blocks(sc, cu, B, T, ib, lb)
    scn = np.where(np.isnan(sc), -np.inf, sc)
    for t in range(int(cu[-1])):
        s = int(np.searchsorted(cu, t, side="right") - 1)
        b = (t - int(cu[s])) // B
        forced = {e for e in [0, b, b - 1] if 0 <= e <= b}
        for h in range(3):
            row = sel[h, t].tolist()
            kept = [e for e in row if e >= 0]
            assert row == kept + [-1] * (T - len(kept))  # padding only at the end
            assert len(set(kept)) == len(kept) and all(0 <= e <= b for e in kept)
            assert forced <= set(kept)
            assert len(kept) == min(T, b + 1)
            free_sel = [e for e in kept if e not in forced]
            unsel = [e for e in range(b + 1) if e not in kept]
            if free_sel and unsel:
                assert min(scn[h, t, e] for e in free_sel) >= max(scn[h, t, e] for e in unsel)
    # exact order-preserving transforms of a row's scores change nothing: a
    # per-row shift in float64 (exact for float32 inputs), scaling by 4
    shift = rng.standard_normal((3, int(cu[-1]), 1)).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(O.select_blocks(sc.astype(np.float64) + shift, cu, B, T, ib, lb), sel)
    np.testing.assert_array_equal(O.select_blocks(sc * np.float32(4.0), cu, B, T, ib, lb), sel)
    nan_as_inf = np.where(np.isnan(sc), -np.inf, sc)
    np.testing.assert_array_equal(O.select_blocks(nan_as_inf, cu, B, T, ib, lb), sel)
