"""CPU oracle service for the full-size GPU parity tests.

Test infrastructure: nothing here touches the GPU.  `OracleService` forks one
server process when the test session starts, before the test process makes
its first GPU call.  The server regenerates the seeded workloads itself (the
same generators the tests use) and, per request, evaluates the float64 oracle
on every query token in a pool of worker processes forked from it, so the
workers share the inputs copy-on-write.  The GPU results reach it as .npy files
written by the test; only comparison statistics come back.

Forward requests compare O, lse and row max on every token.  Backward requests
compare dQ on every token and dK / dV on the keys of chosen blocks: the
oracle's backward runs per token shard, each shard's dK / dV contributions at
those keys are summed in shard order (float64) and compared once complete.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import time
import traceback

import numpy as np

__all__ = ["OracleService", "n_workers", "encode_out", "decode_out"]

# Server-side state: the current workloads, inherited by the forked workers.
_S: dict = {}


def n_workers() -> int:
    """Worker processes: every core this process may run on, at most 16 (the
    CPU share of a one-GPU machine)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def encode_out(x_u16: np.ndarray) -> np.ndarray:
    """GPU output bits (uint16 view of bf16 / fp16) as stored on disk."""
    return np.ascontiguousarray(x_u16.view(np.uint16))


def decode_out(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit storage bits -> float64 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# client
# ---------------------------------------------------------------------------
class OracleService:
    def __init__(self):
        ctx = mp.get_context("fork")
        self._conn, child = ctx.Pipe()
        self._proc = ctx.Process(target=_serve, args=(child, os.getpid()), name="oracle-service")
        self._proc.start()
        child.close()
        self._pending = 0

    def _drain(self):
        while self._pending:
            status, payload = self._conn.recv()
            self._pending -= 1
            if status != "ok":
                raise RuntimeError(f"oracle service: {payload}")

    def _call(self, *msg):
        self._drain()
        self._conn.send(msg)
        status, payload = self._conn.recv()
        if status != "ok":
            raise RuntimeError(f"oracle service: {payload}")
        return payload

    def prepare(self, name: str):
        """Start generating workload `name` on the server; returns at once."""
        self._conn.send(("prepare", name))
        self._pending += 1

    def forward(self, name: str, out_path: str, lse_path: str, row_max_path: str | None = None) -> dict:
        """Compare a forward's O (16-bit bits, [N, h_q, d]), lse and row max
        (fp32 [N, h_q]) with the oracle on every token of workload `name`."""
        return self._call("forward", name, out_path, lse_path, row_max_path)

    def backward(self, name: str, dout_seed: int, dq_path: str, dk_path: str, dv_path: str, key_blocks) -> dict:
        """Compare dQ on every token and dK / dV at the keys of `key_blocks`
        ((sequence, local block) pairs) with the oracle's gradient for the
        output gradient make_dout(..., dout_seed)."""
        return self._call("backward", name, int(dout_seed), dq_path, dk_path, dv_path, list(key_blocks))

    def select(self, seqlens, H: int, B: int, T: int, init_blocks: int, local_blocks: int, score_seed: int,
               sel_path: str) -> dict:
        """Compare a GPU Sel (int32 [H, N, T] file) with the oracle's block
        selection on every token, for the scores
        make_block_scores(seqlens, H, B, score_seed)."""
        return self._call("select", [int(x) for x in seqlens], int(H), int(B), int(T), int(init_blocks),
                          int(local_blocks), int(score_seed), sel_path)

    def close(self):
        try:
            self._drain()
            self._conn.send(("quit",))
            self._conn.recv()
        except Exception:
            pass
        self._proc.join(10)
        if self._proc.is_alive():
            self._proc.terminate()
            self._proc.join(5)


# ---------------------------------------------------------------------------
# server
# ---------------------------------------------------------------------------
def _serve(conn, parent_pid):
    handlers = {"prepare": _load, "forward": _forward, "backward": _backward, "select": _select}
    while True:
        if not conn.poll(5.0):
            if os.getppid() != parent_pid:  # the test process is gone
                return
            continue
        try:
            msg = conn.recv()
        except EOFError:
            return
        if msg[0] == "quit":
            conn.send(("ok", None))
            return
        try:
            conn.send(("ok", handlers[msg[0]](*msg[1:])))
        except Exception:
            conn.send(("err", traceback.format_exc()))


def _load(name: str):
    """Workload `name` as float32 numpy arrays (exact upcasts of the 16-bit
    inputs); the two most recent are kept."""
    cache = _S.setdefault("cache", {})
    if name in cache:
        _S["cur"] = cache[name]
        return None
    from sparse_attention_sel_amd.inputs import make_workload

    w = make_workload(name)
    st = {
        "name": name,
        "q": w.q.float().numpy(),
        "k": w.k.float().numpy(),
        "v": w.v.float().numpy(),
        "sel": w.sel,
        "cu": np.asarray(w.cu_seqlens, dtype=np.int64),
        "B": w.block_size,
        "scale": w.scale,
        "dtype": w.dtype,
        "H": w.num_kv_heads,
        "g": w.gqa_group,
        "d": w.head_dim,
        "dout": {},
    }
    del w
    while len(cache) >= 2:
        cache.pop(next(iter(cache)))
    cache[name] = st
    _S["cur"] = st
    return None


def _init_worker():
    from threadpoolctl import threadpool_limits

    _S["limits"] = threadpool_limits(1)


def _pool():
    return mp.get_context("fork").Pool(n_workers(), initializer=_init_worker)


def _forward(name, out_path, lse_path, row_max_path):
    _load(name)
    st = _S["cur"]
    n = int(st["cu"][-1])
    shards = [(int(a[0]), int(a[-1]) + 1) for a in np.array_split(np.arange(n), max(1, 4 * n_workers())) if a.size]
    t0 = time.perf_counter()
    with _pool() as pool:
        res = pool.map(_forward_shard, [(a, b, out_path, lse_path, row_max_path) for a, b in shards])
    agg = {"tokens": n, "shards": len(shards), "workers": n_workers(), "oracle_s": time.perf_counter() - t0}
    for key in ("err_o", "err_lse", "err_m"):
        best = max(res, key=lambda r: r[key])
        agg[key] = best[key]
        agg[key + "_at"] = best[key + "_at"]
    agg["empty_rows"] = sum(r["empty_rows"] for r in res)
    agg["empty_mismatch"] = sum(r["empty_mismatch"] for r in res)
    agg["nonzero_empty_out"] = sum(r["nonzero_empty_out"] for r in res)
    agg["nonfinite"] = sum(r["nonfinite"] for r in res)
    return agg


def _forward_shard(args):
    import oracle.fsa_oracle as O

    a, b, out_path, lse_path, row_max_path = args
    st = _S["cur"]
    o_ref, m_ref, lse_ref = O.selected_attention(st["q"], st["k"], st["v"], st["sel"], st["cu"], st["B"],
                                                 st["scale"], range(a, b))
    o = decode_out(np.load(out_path, mmap_mode="r")[a:b], st["dtype"])
    lse = np.asarray(np.load(lse_path, mmap_mode="r")[a:b], dtype=np.float64)
    m = None if row_max_path is None else np.asarray(np.load(row_max_path, mmap_mode="r")[a:b], dtype=np.float64)
    empty = np.isneginf(lse_ref)
    r = {"empty_rows": int(empty.sum())}
    mism = np.isneginf(lse) != empty
    if m is not None:
        mism |= np.isneginf(m) != empty
    r["empty_mismatch"] = int(mism.sum())
    r["nonzero_empty_out"] = int(np.count_nonzero(o[empty]))
    fin = ~empty
    r["nonfinite"] = int((~np.isfinite(o)).sum() + (~np.isfinite(lse[fin])).sum())
    err_o = np.abs(o - o_ref)
    i = int(np.argmax(err_o)) if err_o.size else 0
    r["err_o"] = float(err_o.reshape(-1)[i]) if err_o.size else 0.0
    r["err_o_at"] = [int(x) for x in np.unravel_index(i, err_o.shape)] if err_o.size else []
    if r["err_o_at"]:
        r["err_o_at"][0] += a
    for key, got, ref in (("err_lse", lse, lse_ref), ("err_m", m, m_ref)):
        if got is None or not fin.any():
            r[key], r[key + "_at"] = 0.0, []
            continue
        e = np.where(fin, np.abs(got - np.where(fin, ref, 0.0)), 0.0)
        j = int(np.argmax(e))
        r[key] = float(e.reshape(-1)[j])
        at = [int(x) for x in np.unravel_index(j, e.shape)]
        at[0] += a
        r[key + "_at"] = at
    return r


def _key_rows(st, key_blocks):
    """Global key tokens of the (sequence, local block) pairs, ascending."""
    cu, B = st["cu"], st["B"]
    rows = []
    for s, e in sorted(set((int(s), int(e)) for s, e in key_blocks)):
        lo = int(cu[s]) + e * B
        hi = min(lo + B, int(cu[s + 1]))
        rows.extend(range(lo, hi))
    return np.asarray(rows, dtype=np.int64)


def _backward(name, dout_seed, dq_path, dk_path, dv_path, key_blocks):
    _load(name)
    st = _S["cur"]
    if dout_seed not in st["dout"]:
        from sparse_attention_sel_amd.inputs import make_dout

        n = int(st["cu"][-1])
        st["dout"] = {dout_seed: make_dout(n, st["H"] * st["g"], st["d"], st["dtype"], dout_seed).float().numpy()}
    _S["dout"] = st["dout"][dout_seed]
    keys = _key_rows(st, key_blocks)
    _S["keys"] = keys
    cu = st["cu"]
    shards = []
    per = max(1, 2 * n_workers() // max(1, len(cu) - 1))
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        if c1 > c0:
            for a in np.array_split(np.arange(c0, c1), per):
                if a.size:
                    shards.append((c0, int(a[0]), int(a[-1]) + 1))
    t0 = time.perf_counter()
    with _pool() as pool:
        res = pool.map(_backward_shard, [(c0, a, b, dq_path) for c0, a, b in shards])
    H, d = st["H"], st["d"]
    dk_ref, dv_ref, dk_sq, dv_sq = (np.zeros((keys.size, H, d), dtype=np.float64) for _ in range(4))
    for r in res:  # shard order
        dk_ref[r["key_pos"]] += r["dk"]
        dv_ref[r["key_pos"]] += r["dv"]
        dk_sq[r["key_pos"]] += r["dk_sq"]
        dv_sq[r["key_pos"]] += r["dv_sq"]
    agg = {"tokens": int(cu[-1]), "shards": len(shards), "workers": n_workers(), "keys": int(keys.size),
           "oracle_s": time.perf_counter() - t0}
    best = max(res, key=lambda r: r["dq_ratio"])
    agg.update(dq_ratio=best["dq_ratio"], dq_err=max(r["dq_err"] for r in res), dq_at=best["dq_at"],
               dq_nonfinite=sum(r["dq_nonfinite"] for r in res))
    for nm, path, ref, sq in (("dk", dk_path, dk_ref, dk_sq), ("dv", dv_path, dv_ref, dv_sq)):
        got = decode_out(np.load(path, mmap_mode="r")[keys], st["dtype"])
        err = np.abs(got - ref)
        ratio = err / grad_tol(ref, sq, st["dtype"])
        j = int(np.argmax(ratio)) if ratio.size else 0
        agg[nm + "_ratio"] = float(ratio.reshape(-1)[j]) if ratio.size else 0.0
        agg[nm + "_err"] = float(err.max()) if err.size else 0.0
        agg[nm + "_max_ref"] = float(np.abs(ref).max()) if ref.size else 0.0
        at = [int(x) for x in np.unravel_index(j, ratio.shape)] if ratio.size else []
        if at:
            at[0] = int(keys[at[0]])
        agg[nm + "_at"] = at
        agg[nm + "_nonfinite"] = int((~np.isfinite(got)).sum())
    return agg


# Elementwise gradient tolerance for sums over many rows or keys:
#   |gpu - ref| <= ATOL + RTOL |ref| + LAMBDA u sqrt(sum of squared terms).
# ATOL + RTOL |ref| is the GPU backward tests' bound for short sums (the final
# rounding to 16 bits and the error of D from the 16-bit forward output).  The
# GPU rounds each term's P or dS operand to 16 bits (unit roundoff u = 2^-8
# for bf16, 2^-11 for fp16): term i is off by at most u |t_i|, and with these
# errors independent and zero-mean their sum has standard deviation at most
# u sqrt(sum t_i^2 / 3) (uniform on [-u |t_i|, u |t_i|]); LAMBDA = 4 puts the
# bound at 6.9 standard deviations.
_RTOL = 2.0**-7
_LAMBDA = 4.0
_UNIT_ROUNDOFF = {"bf16": 2.0**-8, "fp16": 2.0**-11}


def _atol(dtype):
    return {"bf16": 2e-2, "fp16": 5e-3}[dtype]


def grad_tol(ref, sq, dtype):
    return _atol(dtype) + _RTOL * np.abs(ref) + _LAMBDA * _UNIT_ROUNDOFF[dtype] * np.sqrt(sq)


def _backward_shard(args):
    import oracle.fsa_oracle as O

    c0, a, b, dq_path = args
    st = _S["cur"]
    sl = slice(c0, b)  # the sequence up to the shard's last token: all the keys its rows see
    dq, dk, dv, dq_sq, dk_sq, dv_sq = O.selected_attention_backward(
        st["q"][sl], st["k"][sl], st["v"][sl], st["sel"][:, sl], [0, b - c0], st["B"], _S["dout"][sl], st["scale"],
        range(a - c0, b - c0), with_sq=True)
    got = decode_out(np.load(dq_path, mmap_mode="r")[a:b], st["dtype"])
    err = np.abs(got - dq)
    ratio = err / grad_tol(dq, dq_sq, st["dtype"])
    j = int(np.argmax(ratio))
    at = [int(x) for x in np.unravel_index(j, ratio.shape)]
    at[0] += a
    keys = _S["keys"]
    pos = np.nonzero((keys >= c0) & (keys < b))[0]
    return {
        "dq_ratio": float(ratio.reshape(-1)[j]),
        "dq_err": float(err.max()),
        "dq_at": at,
        "dq_nonfinite": int((~np.isfinite(got)).sum()),
        "key_pos": pos,
        "dk": dk[keys[pos] - c0],
        "dv": dv[keys[pos] - c0],
        "dk_sq": dk_sq[keys[pos] - c0],
        "dv_sq": dv_sq[keys[pos] - c0],
    }


def _select(seqlens, H, B, T, init_blocks, local_blocks, score_seed, sel_path):
    from sparse_attention_sel_amd.inputs import cu_seqlens_of, make_block_scores

    _S["scores"] = make_block_scores(seqlens, H, B, score_seed)
    _S["sel_cfg"] = (np.asarray(cu_seqlens_of(seqlens), dtype=np.int64), B, T, init_blocks, local_blocks)
    n = int(sum(seqlens))
    shards = [(int(a[0]), int(a[-1]) + 1) for a in np.array_split(np.arange(n), max(1, 4 * n_workers())) if a.size]
    t0 = time.perf_counter()
    with _pool() as pool:
        res = pool.map(_select_shard, [(a, b, sel_path) for a, b in shards])
    del _S["scores"]
    bad = [r for r in res if r["mismatch"]]
    return {"tokens": n, "workers": n_workers(), "oracle_s": time.perf_counter() - t0,
            "mismatch": sum(r["mismatch"] for r in res), "first_mismatch": bad[0]["first"] if bad else None}


def _select_shard(args):
    import oracle.fsa_oracle as O

    a, b, sel_path = args
    cu, B, T, init_blocks, local_blocks = _S["sel_cfg"]
    ref = O.select_blocks(_S["scores"], cu, B, T, init_blocks, local_blocks, tokens=range(a, b))[:, a:b]
    got = np.asarray(np.load(sel_path, mmap_mode="r")[:, a:b])
    diff = np.nonzero(np.any(got != ref, axis=2))
    first = None
    if diff[0].size:
        h, t = int(diff[0][0]), int(diff[1][0])
        first = {"head": h, "token": a + t, "got": got[h, t].tolist(), "want": ref[h, t].tolist()}
    return {"mismatch": int(diff[0].size), "first": first}
