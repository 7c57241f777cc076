"""Seeded synthetic inputs for NSA selected attention.

This module produces inputs only: Q/K/V tensors, an output gradient dO for the
backward, and the per-KV-head block selection tensor Sel[h_K, N, T].  It holds none of the attention arithmetic and
is shared by the oracle tests, the GPU tests and the benchmark, so that both
sides of every parity check see the same bytes.

Selection structure follows the NSA hyper-parameters printed on the FSA README
mirror ("Usage" section: ``init_blocks=1``, ``local_blocks=2``, ``topk=16``,
``block_size=64``): every query keeps the first block of its sequence and the
local blocks, and the remaining picks come from earlier blocks.  The pick
distributions (uniform, recency-skewed Zipf, hot-block) are synthetic stand-ins
for the learned block scores that the pages do not describe.

Sel entries are block indices local to the query's own sequence; ``-1`` pads
rows that have fewer than T candidates.  Rows carry no duplicates and no
future blocks, but the attention path accepts both (see the index builder).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "WORKLOADS",
    "Workload",
    "make_workload",
    "make_qkv",
    "make_dout",
    "make_block_scores",
    "make_sel",
    "shuffle_rows",
    "cu_seqlens_of",
]


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    seqlens: tuple
    num_kv_heads: int
    gqa_group: int
    head_dim: int
    block_size: int
    topk: int
    dtype: str  # "bf16" or "fp16"
    sel_kind: str  # see make_sel
    seed: int


# Workloads, named by shape.  The three 64K-token bf16 shapes at g = 4, 2, 1 are
# the latency shape of the README's "Advantages" chart (64K tokens, 4 KV heads,
# B_K = 64, T = 16, varied GQA group size).
WORKLOADS: Dict[str, WorkloadSpec] = {
    "n1k_h1_g1_d64_t4_bf16": WorkloadSpec((1024,), 1, 1, 64, 64, 4, "bf16", "init_own_uniform", 1000),
    "n8k_h4_g2_d128_t16_bf16": WorkloadSpec((8192,), 4, 2, 128, 64, 16, "bf16", "init_local_zipf", 2000),
    "n64k_h4_g4_d128_t16_bf16": WorkloadSpec((65536,), 4, 4, 128, 64, 16, "bf16", "init_local_zipf", 3000),
    "n64k_h4_g1_d128_t16_fp16": WorkloadSpec((65536,), 4, 1, 128, 64, 16, "fp16", "init_local_uniform", 4000),
    "b2_n32k_h8_g8_d256_t16_bf16": WorkloadSpec((32768, 32768), 8, 8, 256, 64, 16, "bf16", "init_local_hot", 5000),
    # 64K-token bf16 latency shape at the two smaller group sizes.
    "n64k_h4_g2_d128_t16_bf16": WorkloadSpec((65536,), 4, 2, 128, 64, 16, "bf16", "init_local_zipf", 3200),
    "n64k_h4_g1_d128_t16_bf16": WorkloadSpec((65536,), 4, 1, 128, 64, 16, "bf16", "init_local_zipf", 3100),
    # the same 64K g = 4 shape with 128-key blocks and 8 selected blocks (the
    # same 1024 selected keys per token; the README's Performance section
    # benchmarks both (B_K, T) = (64, 16) and (128, 8))
    "n64k_h4_g4_d128_b128_t8_bf16": WorkloadSpec((65536,), 4, 4, 128, 128, 8, "bf16", "init_local_zipf", 3300),
    # 128-key blocks at head dim 256 (8 selected blocks: the same 1024 keys per token)
    "n32k_h4_g4_d256_b128_t8_bf16": WorkloadSpec((32768,), 4, 4, 256, 128, 8, "bf16", "init_local_zipf", 3400),
    # two short packed sequences: a quick case for the checking harness
    "b2_n1k_h2_g4_d64_t8_bf16": WorkloadSpec((640, 384), 2, 4, 64, 64, 8, "bf16", "init_local_zipf", 6000),
}


@dataclasses.dataclass
class Workload:
    name: str
    seqlens: List[int]
    cu_seqlens: np.ndarray  # int32 [B+1]
    num_kv_heads: int
    gqa_group: int
    head_dim: int
    block_size: int
    topk: int
    dtype: str
    scale: float
    q: "object"  # torch.Tensor [N, h_K*g, d] on CPU, dtype bf16/fp16
    k: "object"  # torch.Tensor [N, h_K, d]
    v: "object"  # torch.Tensor [N, h_K, d]
    sel: np.ndarray  # int32 [h_K, N, T]
    meta: dict


def cu_seqlens_of(seqlens: Sequence[int]) -> np.ndarray:
    """Exclusive prefix of the sequence lengths, the packed-varlen convention
    of the README's usage example (int32, length B+1)."""
    cu = np.zeros(len(seqlens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(seqlens, dtype=np.int64))
    if cu[-1] >= 2**31:
        raise ValueError("total token count must fit in int32")
    return cu.astype(np.int32)


def _torch_dtype(name: str):
    import torch

    return {"bf16": torch.bfloat16, "fp16": torch.float16}[name]


def make_qkv(num_tokens: int, num_kv_heads: int, gqa_group: int, head_dim: int, dtype: str, seed: int):
    """Q, K, V ~ N(0, 1) drawn in float32 from seeded CPU generators, then cast
    to the storage dtype with round-to-nearest-even."""
    import torch

    td = _torch_dtype(dtype)
    out = []
    for i, heads in enumerate((num_kv_heads * gqa_group, num_kv_heads, num_kv_heads)):
        g = torch.Generator(device="cpu").manual_seed(int(seed) * 8 + i)
        x = torch.randn((num_tokens, heads, head_dim), generator=g, dtype=torch.float32)
        out.append(x.to(td))
    return tuple(out)


def make_dout(num_tokens: int, num_q_heads: int, head_dim: int, dtype: str, seed: int):
    """An output gradient dO ~ N(0, 1) of shape [N, h_q, d] for the backward,
    from its own seeded CPU generator (stream 3 of the workload's seed), cast
    to the storage dtype with round-to-nearest-even."""
    import torch

    g = torch.Generator(device="cpu").manual_seed(int(seed) * 8 + 3)
    x = torch.randn((num_tokens, num_q_heads, head_dim), generator=g, dtype=torch.float32)
    return x.to(_torch_dtype(dtype))


def make_block_scores(seqlens: Sequence[int], num_kv_heads: int, block_size: int, seed: int) -> np.ndarray:
    """Synthetic block-importance scores for the selection step, float32
    [h_K, N, S] with S = blocks of the longest sequence: a recency term
    -log(b - e + 1) for query token t of local block b and block e, plus
    standard Gumbel noise (PCG64, seeded).  Entries e > b are noise only (the
    selection ignores them).  A stand-in for NSA's compressed-attention
    scores, which the pages do not describe."""
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    seqlens = [int(x) for x in seqlens]
    S = max([-(-L // block_size) for L in seqlens] + [1])
    N = sum(seqlens)
    out = np.empty((num_kv_heads, N, S), dtype=np.float32)
    e = np.arange(S, dtype=np.float64)
    t0 = 0
    for L in seqlens:
        b = np.arange(L) // block_size
        rec = -np.log(np.maximum(b[:, None] - e[None, :], 0.0) + 1.0)
        for h in range(num_kv_heads):
            g = rng.gumbel(size=(L, S))
            out[h, t0 : t0 + L] = (rec + g).astype(np.float32)
        t0 += L
    return out


def _forced_blocks(kind: str, b: int) -> List[int]:
    """The blocks every query in local block ``b`` keeps: the first block of the
    sequence and its own block, plus the previous block for the two-local-block
    kinds.  Duplicates (b <= 1) are dropped."""
    if kind == "init_own_uniform":
        want = [0, b]
    else:
        want = [0, b, b - 1]
    out: List[int] = []
    for x in want:
        if x >= 0 and x not in out:
            out.append(x)
    return out


def _first_free(kind: str, b: int) -> int:
    """Largest candidate for the free picks is b-1 (one local block) or b-2
    (two local blocks); candidates start at block 1."""
    return b - 1 if kind == "init_own_uniform" else b - 2


def _smallest_k(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k smallest keys along the last axis, ordered by key."""
    m = keys.shape[-1]
    if k <= 0:
        return np.zeros(keys.shape[:-1] + (0,), dtype=np.int64)
    if k < m:
        part = np.argpartition(keys, k - 1, axis=-1)[..., :k]
    else:
        part = np.broadcast_to(np.arange(m), keys.shape).copy()
    pk = np.take_along_axis(keys, part, axis=-1)
    order = np.argsort(pk, axis=-1, kind="stable")
    return np.take_along_axis(part, order, axis=-1)


def make_sel(
    kind: str,
    seqlens: Sequence[int],
    num_kv_heads: int,
    block_size: int,
    topk: int,
    seed: int,
    hot_fraction: float = 0.05,
    hot_share: float = 0.50,
):
    """Selection tensor Sel[h_K, N, T] (int32, local block indices, -1 padding).

    kinds
      ``init_own_uniform``   keep {0, b}; the rest uniform without replacement
                             from {1..b-1}.
      ``init_local_uniform`` keep {0, b, b-1}; the rest uniform from {1..b-2}.
      ``init_local_zipf``    keep {0, b, b-1}; the rest from {1..b-2} with
                             weight 1/r on recency rank r = b-1-j (Zipf s=1),
                             without replacement (Gumbel top-k).
      ``init_local_hot``     keep {0, b, b-1}; each sequence/head has a hot set
                             of ceil(hot_fraction * nb) blocks (block 0 plus
                             uniform picks).  Each free pick is hot with
                             probability pi, else cold, uniform within its
                             class; pi is set by bisection so that the share of
                             all kept entries that land in hot blocks equals
                             ``hot_share``.

    Returns (sel, meta) where meta holds generator diagnostics.
    """
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    seqlens = [int(x) for x in seqlens]
    n_total = int(sum(seqlens))
    H, B, T = int(num_kv_heads), int(block_size), int(topk)
    sel = np.full((H, n_total, T), -1, dtype=np.int32)
    meta: dict = {}

    if kind == "init_local_hot":
        return _make_sel_hot(rng, seqlens, H, B, T, hot_fraction, hot_share, sel)

    c0 = 0
    for L in seqlens:
        nb = -(-L // B)
        for b in range(nb):
            t0 = c0 + b * B
            t1 = min(c0 + L, t0 + B)
            n = t1 - t0
            forced = _forced_blocks(kind, b)[:T]
            sel[:, t0:t1, : len(forced)] = np.asarray(forced, dtype=np.int32)
            hi = _first_free(kind, b)
            cand = np.arange(1, hi + 1, dtype=np.int32)  # may be empty
            k = min(T - len(forced), cand.size)
            if k <= 0:
                continue
            if kind in ("init_own_uniform", "init_local_uniform"):
                keys = rng.random((H, n, cand.size))
            elif kind == "init_local_zipf":
                rank = (b - 1 - cand).astype(np.float64)  # 1 .. b-2
                logw = -np.log(rank)
                u = rng.random((H, n, cand.size))
                gumbel = -np.log(-np.log(np.maximum(u, 1e-300)))
                keys = -(logw + gumbel)  # smallest keys = largest perturbed log-weight
            else:
                raise ValueError(f"unknown selection kind {kind!r}")
            pick = _smallest_k(keys, k)
            sel[:, t0:t1, len(forced) : len(forced) + k] = cand[pick]
        c0 += L
    return sel, meta


def _make_sel_hot(rng, seqlens, H, B, T, hot_fraction, hot_share, sel):
    # Pass 1: hot sets and the hot/cold coin for every free pick.
    seq_info = []
    c0 = 0
    for L in seqlens:
        nb = -(-L // B)
        nh = max(1, int(math.ceil(hot_fraction * nb)))
        hot = np.zeros((H, nb), dtype=bool)
        hot[:, 0] = True
        for h in range(H):
            if nb > 1 and nh > 1:
                extra = rng.choice(nb - 1, size=min(nh - 1, nb - 1), replace=False) + 1
                hot[h, extra] = True
        seq_info.append((c0, L, nb, hot))
        c0 += L
    n_total = sel.shape[1]
    coins = rng.random((H, n_total, T))

    # Per token: number of free picks, hot/cold candidate counts, forced-hot count.
    n_free = np.zeros((H, n_total), dtype=np.int64)
    n_hot_c = np.zeros((H, n_total), dtype=np.int64)
    n_cold_c = np.zeros((H, n_total), dtype=np.int64)
    forced_hot = np.zeros((H, n_total), dtype=np.int64)
    n_forced = np.zeros((H, n_total), dtype=np.int64)
    for c0, L, nb, hot in seq_info:
        hot_prefix = np.concatenate([np.zeros((H, 1), np.int64), np.cumsum(hot, axis=1)], axis=1)
        for b in range(nb):
            t0, t1 = c0 + b * B, min(c0 + L, c0 + (b + 1) * B)
            forced = _forced_blocks("init_local_hot", b)[:T]
            hi = b - 2
            ncand = max(0, hi)
            nh = (hot_prefix[:, hi + 1] - hot_prefix[:, 1]) if hi >= 1 else np.zeros(H, np.int64)
            n_forced[:, t0:t1] = len(forced)
            forced_hot[:, t0:t1] = hot[:, forced].sum(axis=1)[:, None]
            n_free[:, t0:t1] = min(T - len(forced), ncand)
            n_hot_c[:, t0:t1] = nh[:, None]
            n_cold_c[:, t0:t1] = (ncand - nh)[:, None]

    jidx = np.arange(T)[None, None, :]
    usable = jidx < n_free[:, :, None]

    def hot_counts(pi):
        want = ((coins < pi) & usable).sum(axis=2)
        k_hot = np.minimum(want, n_hot_c)
        k_cold = np.minimum(n_free - k_hot, n_cold_c)
        return n_free - k_cold

    total = float((n_forced + n_free).sum())

    def share(pi):
        return float((forced_hot + hot_counts(pi)).sum()) / total

    lo, hi_ = 0.0, 1.0
    if not (share(lo) <= hot_share <= share(hi_)):
        raise ValueError("hot share out of reach for this shape")
    for _ in range(60):
        mid = 0.5 * (lo + hi_)
        if share(mid) < hot_share:
            lo = mid
        else:
            hi_ = mid
    pi = hi_
    k_hot_all = hot_counts(pi)

    # Pass 2: materialise the rows.
    for c0, L, nb, hot in seq_info:
        for b in range(nb):
            t0, t1 = c0 + b * B, min(c0 + L, c0 + (b + 1) * B)
            n = t1 - t0
            forced = _forced_blocks("init_local_hot", b)[:T]
            sel[:, t0:t1, : len(forced)] = np.asarray(forced, dtype=np.int32)
            nf = len(forced)
            if b - 2 < 1 or T - nf <= 0:
                continue
            cand = np.arange(1, b - 1, dtype=np.int32)
            for h in range(H):
                is_hot = hot[h, cand]
                ch, cc = cand[is_hot], cand[~is_hot]
                kh = k_hot_all[h, t0:t1]
                kc = n_free[h, t0:t1] - kh
                col = np.full((n, T - nf), -1, dtype=np.int32)
                if ch.size and kh.max() > 0:
                    ph = _smallest_k(rng.random((n, ch.size)), int(kh.max()))
                    vals = ch[ph]
                    m = np.arange(ph.shape[1])[None, :] < kh[:, None]
                    col[:, : ph.shape[1]] = np.where(m, vals, -1)
                if cc.size and kc.max() > 0:
                    pc = _smallest_k(rng.random((n, cc.size)), int(kc.max()))
                    vals = cc[pc]
                    # append cold picks after each row's hot picks
                    for r in range(n):
                        a, z = int(kh[r]), int(kc[r])
                        col[r, a : a + z] = vals[r, :z]
                sel[h, t0:t1, nf:] = col
    meta = {"hot_pick_probability": pi, "hot_share_target": hot_share}
    return sel, meta


def shuffle_rows(sel: np.ndarray, seed: int) -> np.ndarray:
    """Permute the entries inside every Sel row (the selection is a set, so the
    attention result must not change)."""
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    keys = rng.random(sel.shape)
    perm = np.argsort(keys, axis=-1)
    return np.take_along_axis(sel, perm, axis=-1)


def make_workload(name: str, seed: Optional[int] = None, with_qkv: bool = True) -> Workload:
    spec = WORKLOADS[name]
    s = spec.seed if seed is None else int(seed)
    cu = cu_seqlens_of(spec.seqlens)
    n = int(cu[-1])
    sel, meta = make_sel(spec.sel_kind, spec.seqlens, spec.num_kv_heads, spec.block_size, spec.topk, s * 10 + 3)
    meta = dict(meta, seed=s)  # Q, K, V from seed s (make_qkv), Sel from seed 10 s + 3
    if with_qkv:
        q, k, v = make_qkv(n, spec.num_kv_heads, spec.gqa_group, spec.head_dim, spec.dtype, s)
    else:
        q = k = v = None
    return Workload(
        name=name,
        seqlens=list(spec.seqlens),
        cu_seqlens=cu,
        num_kv_heads=spec.num_kv_heads,
        gqa_group=spec.gqa_group,
        head_dim=spec.head_dim,
        block_size=spec.block_size,
        topk=spec.topk,
        dtype=spec.dtype,
        scale=1.0 / math.sqrt(spec.head_dim),
        q=q,
        k=k,
        v=v,
        sel=sel,
        meta=meta,
    )
