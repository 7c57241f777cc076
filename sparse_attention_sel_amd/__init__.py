"""MI355X (gfx950) NSA selected-attention forward in FSA's KV-block-outer order.

Thin ctypes binding over ``libfsa.so`` (C ABI declared in ``include/fsa.h``).
The functions here only marshal arguments: they check tensor shapes, dtypes
and devices, pass raw pointers and the current torch stream, and turn status
codes into exceptions.  Every step of the computation runs in the library's
HIP kernels; there is no fallback path.  PyTorch supplies device memory and
the stream.

Typical use::

    import sparse_attention_sel_amd as fsa
    prob = fsa.Problem(cu_seqlens, num_kv_heads=4, gqa_group=4, head_dim=128,
                       block_size=64, topk=16, dtype=torch.bfloat16)
    out, lse, row_max, index = fsa.selected_attention(prob, q, k, v, sel)
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

__all__ = [
    "FsaError",
    "Problem",
    "Index",
    "library_path",
    "load_library",
    "get_sizes",
    "allocate_index",
    "build_index",
    "build_index_noalloc",
    "softmax_stats",
    "selected_attn_fwd",
    "selected_attn_fwd_onepass",
    "selected_attn_main",
    "selected_attn_reduce",
    "nsa_selected_attn_fwd",
    "mfma_loop",
    "selected_attn_bwd",
    "selected_attention_backward",
    "select_blocks",
    "selected_attention",
    "status_string",
]

FSA_OK = 0
DTYPE_CODES = {torch.bfloat16: 0, torch.float16: 1}
PARTIAL_CODES = {"fp32": 0, "input": 1}


class FsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class _Problem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("cu_seqlens_dev", ctypes.c_void_p),
        ("num_kv_heads", ctypes.c_int32),
        ("gqa_group", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("partial_dtype", ctypes.c_int32),
    ]


class _Sizes(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int64),
        ("num_blocks", ctypes.c_int64),
        ("max_pairs", ctypes.c_int64),
        ("max_work_items", ctypes.c_int64),
        ("counts_bytes", ctypes.c_size_t),
        ("offsets_bytes", ctypes.c_size_t),
        ("qidx_bytes", ctypes.c_size_t),
        ("slot_bytes", ctypes.c_size_t),
        ("aux_bytes", ctypes.c_size_t),
        ("build_ws_bytes", ctypes.c_size_t),
        ("stats_ws_bytes", ctypes.c_size_t),
        ("partial_ws_bytes", ctypes.c_size_t),
        ("bwd_ws_bytes", ctypes.c_size_t),
    ]

    def as_dict(self):
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


class _Index(ctypes.Structure):
    _fields_ = [
        ("counts", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p),
        ("qidx", ctypes.c_void_p),
        ("slot", ctypes.c_void_p),
        ("aux", ctypes.c_void_p),
    ]


_LIB = None
ABI_VERSION = 2  # FSA_ABI_VERSION of include/fsa.h


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfsa.so")


def load_library():
    """Load libfsa.so once.  torch is imported first so that the process's
    HIP runtime is torch's and streams/pointers are shared with it."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the gfx950 library first (python -m sparse_attention_sel_amd.build)"
        )
    lib = ctypes.CDLL(path)
    P, S, I = ctypes.POINTER(_Problem), ctypes.POINTER(_Sizes), ctypes.POINTER(_Index)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    lib.fsa_abi_version.restype = i32
    lib.fsa_abi_version.argtypes = []
    lib.fsa_status_string.restype = ctypes.c_char_p
    lib.fsa_status_string.argtypes = [i32]
    lib.fsa_get_sizes.restype = i32
    lib.fsa_get_sizes.argtypes = [P, S]
    lib.fsa_build_index.restype = i32
    lib.fsa_build_index.argtypes = [P, vp, I, vp, sz, vp]
    lib.fsa_build_index_noalloc.restype = i32
    lib.fsa_build_index_noalloc.argtypes = [P, vp, I, vp]
    lib.fsa_softmax_stats.restype = i32
    lib.fsa_softmax_stats.argtypes = [P, vp, vp, I, vp, vp, vp, sz, vp]
    lib.fsa_selected_attn_fwd.restype = i32
    lib.fsa_selected_attn_fwd.argtypes = [P, vp, vp, vp, I, vp, vp, vp, sz, vp]
    lib.fsa_selected_attn_fwd_onepass.restype = i32
    lib.fsa_selected_attn_fwd_onepass.argtypes = [P, vp, vp, vp, I, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.fsa_selected_attn_main.restype = i32
    lib.fsa_selected_attn_main.argtypes = [P, vp, vp, vp, I, vp, vp, sz, vp]
    lib.fsa_selected_attn_reduce.restype = i32
    lib.fsa_selected_attn_reduce.argtypes = [P, I, vp, sz, vp, vp]
    lib.fsa_selected_attn_bwd.restype = i32
    lib.fsa_selected_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, I, vp, vp, vp, vp, sz, vp]
    lib.fsa_select_blocks.restype = i32
    lib.fsa_select_blocks.argtypes = [P, vp, ctypes.c_int64, i32, i32, vp, vp]
    lib.fsa_mfma_loop.restype = i32
    lib.fsa_mfma_loop.argtypes = [i32, i32, i32, vp, vp]
    lib.fsa_nsa_selected_attn_fwd.restype = i32
    lib.fsa_nsa_selected_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    if lib.fsa_abi_version() != ABI_VERSION:
        raise RuntimeError("libfsa.so ABI version mismatch")
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fsa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != FSA_OK:
        raise FsaError(status, where)


class Problem:
    """Problem description (fsa_problem).  Keeps the host copy of cu_seqlens
    alive and a device copy on ``device`` for the kernels."""

    def __init__(
        self,
        cu_seqlens,
        num_kv_heads: int,
        gqa_group: int,
        head_dim: int,
        block_size: int,
        topk: int,
        dtype: torch.dtype = torch.bfloat16,
        partial_dtype: str = "fp32",
        softmax_scale: Optional[float] = None,
        device=None,
    ):
        if dtype not in DTYPE_CODES:
            raise ValueError(f"dtype must be bfloat16 or float16, got {dtype}")
        if partial_dtype not in PARTIAL_CODES:
            raise ValueError(f"partial_dtype must be one of {sorted(PARTIAL_CODES)}")
        if isinstance(cu_seqlens, torch.Tensor):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
        self.cu_host = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        self.num_seqs = int(self.cu_host.size - 1)
        self.total_tokens = int(self.cu_host[-1])
        self.num_kv_heads, self.gqa_group, self.head_dim = int(num_kv_heads), int(gqa_group), int(head_dim)
        self.block_size, self.topk = int(block_size), int(topk)
        self.dtype = dtype
        self.partial_dtype = partial_dtype
        self.softmax_scale = softmax_scale
        self.cu_dev = None
        if device is not None:
            self.cu_dev = torch.from_numpy(self.cu_host).to(device)
        self._c = _Problem(
            num_seqs=self.num_seqs,
            cu_seqlens_host=self.cu_host.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            cu_seqlens_dev=self.cu_dev.data_ptr() if self.cu_dev is not None else None,
            num_kv_heads=self.num_kv_heads,
            gqa_group=self.gqa_group,
            head_dim=self.head_dim,
            block_size=self.block_size,
            topk=self.topk,
            softmax_scale=float(softmax_scale) if softmax_scale is not None else 0.0,
            dtype=DTYPE_CODES[dtype],
            partial_dtype=PARTIAL_CODES[partial_dtype],
        )

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.gqa_group

    def c(self):
        return ctypes.byref(self._c)


def get_sizes(prob: Problem) -> dict:
    out = _Sizes()
    _check(load_library().fsa_get_sizes(prob.c(), ctypes.byref(out)), "fsa_get_sizes")
    return out.as_dict()


class Index:
    """Device buffers of the index tensors (fsa_index): counts, offsets, qidx,
    slot and the library-private aux blob that travels with them."""

    def __init__(self, counts, offsets, qidx, slot, aux, sizes, buffers=None):
        """``counts`` and ``slot`` may be shaped views; ``buffers`` (the five
        underlying allocations, in the same order) supplies the addresses
        handed to the library, which stay valid when a view is empty."""
        self.counts, self.offsets, self.qidx, self.slot, self.aux = counts, offsets, qidx, slot, aux
        self.sizes = sizes
        self._bufs = buffers if buffers is not None else (counts, offsets, qidx, slot, aux)
        self._c = _Index(*(b.data_ptr() for b in self._bufs))

    def c(self):
        return ctypes.byref(self._c)

    def num_pairs(self) -> int:
        return int(self.offsets[-1].item())


def allocate_index(prob: Problem, device) -> Index:
    s = get_sizes(prob)
    i32 = dict(dtype=torch.int32, device=device)
    bufs = (
        torch.empty(s["counts_bytes"] // 4, **i32),
        torch.empty(s["offsets_bytes"] // 4, **i32),
        torch.empty(s["qidx_bytes"] // 4, **i32),
        torch.empty(s["slot_bytes"] // 4, **i32),
        torch.empty(s["aux_bytes"], dtype=torch.uint8, device=device),
    )
    counts = bufs[0][: prob.num_kv_heads * s["num_blocks"]]
    slot = bufs[3][: prob.num_kv_heads * prob.total_tokens * prob.topk].view(
        prob.num_kv_heads, prob.total_tokens, prob.topk)
    return Index(counts, bufs[1], bufs[2], slot, bufs[4], s, buffers=bufs)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _ws(t: torch.Tensor, name: str, need: int):
    if t.numel() * t.element_size() < need:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {need}")
    return _ptr(t, name), t.numel() * t.element_size()


def build_index(prob: Problem, sel: torch.Tensor, index: Index, ws: torch.Tensor, stream=None):
    """fsa_build_index: Sel [h_K, N, T] int32 -> index tensors."""
    p = _ptr(sel, "sel", torch.int32, (prob.num_kv_heads, prob.total_tokens, prob.topk))
    w, wb = _ws(ws, "build workspace", index.sizes["build_ws_bytes"])
    _check(load_library().fsa_build_index(prob.c(), p, index.c(), w, wb, _stream(stream)), "fsa_build_index")


# Build scratch that fsa_build_index_noalloc holds per GPU (FSA_NOALLOC_BUILD_SCRATCH_BYTES).
NOALLOC_BUILD_SCRATCH_BYTES = 16 << 20


def build_index_noalloc(prob: Problem, sel: torch.Tensor, index: Index, stream=None):
    """fsa_build_index_noalloc: fsa_build_index without a workspace (the
    library's static per-GPU scratch); allocates nothing."""
    p = _ptr(sel, "sel", torch.int32, (prob.num_kv_heads, prob.total_tokens, prob.topk))
    _check(load_library().fsa_build_index_noalloc(prob.c(), p, index.c(), _stream(stream)), "fsa_build_index_noalloc")


def _qkv_shapes(prob: Problem):
    n, hk, d = prob.total_tokens, prob.num_kv_heads, prob.head_dim
    return (n, prob.num_q_heads, d), (n, hk, d)


def softmax_stats(prob, q, k, index: Index, row_max, lse, ws, stream=None):
    """fsa_softmax_stats: row max and log-sum-exp, fp32 [N, h_q]."""
    qs, ks = _qkv_shapes(prob)
    st = (prob.total_tokens, prob.num_q_heads)
    args = (
        _ptr(q, "q", prob.dtype, qs),
        _ptr(k, "k", prob.dtype, ks),
        index.c(),
        _ptr(row_max, "row_max", torch.float32, st),
        _ptr(lse, "lse", torch.float32, st),
        *_ws(ws, "stats workspace", index.sizes["stats_ws_bytes"]),
    )
    _check(load_library().fsa_softmax_stats(prob.c(), *args, _stream(stream)), "fsa_softmax_stats")


def selected_attn_fwd(prob, q, k, v, index: Index, lse, out, partial_ws, stream=None):
    """fsa_selected_attn_fwd: main kernel then reduction into out [N, h_q, d]."""
    qs, ks = _qkv_shapes(prob)
    w, wb = _ws(partial_ws, "partial workspace", index.sizes["partial_ws_bytes"])
    args = (
        _ptr(q, "q", prob.dtype, qs),
        _ptr(k, "k", prob.dtype, ks),
        _ptr(v, "v", prob.dtype, ks),
        index.c(),
        _ptr(lse, "lse", torch.float32, (prob.total_tokens, prob.num_q_heads)),
        _ptr(out, "out", prob.dtype, qs),
        w,
        wb,
    )
    _check(load_library().fsa_selected_attn_fwd(prob.c(), *args, _stream(stream)), "fsa_selected_attn_fwd")


def selected_attn_fwd_onepass(prob, q, k, v, index: Index, row_max, lse, out, stats_ws, partial_ws, stream=None):
    """fsa_selected_attn_fwd_onepass: row max, lse [N, h_q] and out [N, h_q, d]
    with the statistics fused into the main kernel and the reduction."""
    qs, ks = _qkv_shapes(prob)
    st = (prob.total_tokens, prob.num_q_heads)
    args = (
        _ptr(q, "q", prob.dtype, qs),
        _ptr(k, "k", prob.dtype, ks),
        _ptr(v, "v", prob.dtype, ks),
        index.c(),
        _ptr(row_max, "row_max", torch.float32, st),
        _ptr(lse, "lse", torch.float32, st),
        _ptr(out, "out", prob.dtype, qs),
        *_ws(stats_ws, "stats workspace", index.sizes["stats_ws_bytes"]),
        *_ws(partial_ws, "partial workspace", index.sizes["partial_ws_bytes"]),
    )
    _check(load_library().fsa_selected_attn_fwd_onepass(prob.c(), *args, _stream(stream)),
           "fsa_selected_attn_fwd_onepass")


def selected_attn_main(prob, q, k, v, index: Index, lse, partial_ws, stream=None):
    """fsa_selected_attn_main: the token-selection kernel alone (partials)."""
    qs, ks = _qkv_shapes(prob)
    w, wb = _ws(partial_ws, "partial workspace", index.sizes["partial_ws_bytes"])
    args = (
        _ptr(q, "q", prob.dtype, qs),
        _ptr(k, "k", prob.dtype, ks),
        _ptr(v, "v", prob.dtype, ks),
        index.c(),
        _ptr(lse, "lse", torch.float32, (prob.total_tokens, prob.num_q_heads)),
        w,
        wb,
    )
    _check(load_library().fsa_selected_attn_main(prob.c(), *args, _stream(stream)), "fsa_selected_attn_main")


def selected_attn_reduce(prob, index: Index, partial_ws, out, stream=None):
    """fsa_selected_attn_reduce: the reduction kernel alone."""
    qs, _ = _qkv_shapes(prob)
    w, wb = _ws(partial_ws, "partial workspace", index.sizes["partial_ws_bytes"])
    _check(
        load_library().fsa_selected_attn_reduce(prob.c(), index.c(), w, wb, _ptr(out, "out", prob.dtype, qs),
                                                _stream(stream)),
        "fsa_selected_attn_reduce",
    )


class Workspaces:
    """Scratch buffers for one problem (plumbing: plain torch allocations).
    The backward workspace is allocated only with ``backward=True``."""

    def __init__(self, prob: Problem, device, sizes: dict, backward: bool = False):
        u8 = dict(dtype=torch.uint8, device=device)
        self.build = torch.empty(sizes["build_ws_bytes"], **u8)
        self.stats = torch.empty(sizes["stats_ws_bytes"], **u8)
        self.partial = torch.empty(sizes["partial_ws_bytes"], **u8)
        self.bwd = None
        if backward:
            if sizes["bwd_ws_bytes"] == 0:
                raise FsaError(4, "Workspaces(backward=True)")
            self.bwd = torch.empty(sizes["bwd_ws_bytes"], **u8)


def selected_attn_bwd(prob: Problem, q, k, v, out, dout, lse, index: Index, dq, dk, dv, ws, stream=None):
    """fsa_selected_attn_bwd: dq [N, h_q, d], dk and dv [N, h_K, d] from the
    output gradient dout, the forward's out and lse, and the same index."""
    qs, ks = _qkv_shapes(prob)
    w, wb = _ws(ws, "backward workspace", index.sizes["bwd_ws_bytes"])
    args = (
        _ptr(q, "q", prob.dtype, qs),
        _ptr(k, "k", prob.dtype, ks),
        _ptr(v, "v", prob.dtype, ks),
        _ptr(out, "out", prob.dtype, qs),
        _ptr(dout, "dout", prob.dtype, qs),
        _ptr(lse, "lse", torch.float32, (prob.total_tokens, prob.num_q_heads)),
        index.c(),
        _ptr(dq, "dq", prob.dtype, qs),
        _ptr(dk, "dk", prob.dtype, ks),
        _ptr(dv, "dv", prob.dtype, ks),
        w,
        wb,
    )
    _check(load_library().fsa_selected_attn_bwd(prob.c(), *args, _stream(stream)), "fsa_selected_attn_bwd")


def selected_attention_backward(prob: Problem, q, k, v, out, dout, lse, index: Index, stream=None):
    """Gradients with torch-allocated outputs and workspace; returns (dq, dk, dv)."""
    dev = q.device
    ws = Workspaces(prob, dev, index.sizes, backward=True)
    qs, ks = _qkv_shapes(prob)
    dq = torch.empty(qs, dtype=prob.dtype, device=dev)
    dk = torch.empty(ks, dtype=prob.dtype, device=dev)
    dv = torch.empty(ks, dtype=prob.dtype, device=dev)
    selected_attn_bwd(prob, q, k, v, out, dout, lse, index, dq, dk, dv, ws.bwd, stream)
    return dq, dk, dv


def select_blocks(prob: Problem, scores, init_blocks: int, local_blocks: int, sel, stream=None):
    """fsa_select_blocks: scores fp32 [h_K, N, S] (S >= blocks of the longest
    sequence) -> sel int32 [h_K, N, T]."""
    if scores.dim() != 3:
        raise ValueError("scores must be [h_K, N, S]")
    S = int(scores.shape[2])
    p = _ptr(scores, "scores", torch.float32, (prob.num_kv_heads, prob.total_tokens, S))
    o = _ptr(sel, "sel", torch.int32, (prob.num_kv_heads, prob.total_tokens, prob.topk))
    _check(load_library().fsa_select_blocks(prob.c(), p, S, int(init_blocks), int(local_blocks), o, _stream(stream)),
           "fsa_select_blocks")


def mfma_loop(dtype, workgroups: int, iters: int, sink, stream=None) -> float:
    """fsa_mfma_loop: launch the matrix-core throughput loop; returns the
    flops it executes.  sink: fp32 device tensor of at least 256 elements."""
    if sink.dtype != torch.float32 or sink.numel() < 256 or not sink.is_cuda:
        raise ValueError("sink must be a float32 device tensor of at least 256 elements")
    _check(load_library().fsa_mfma_loop(DTYPE_CODES[dtype], int(workgroups), int(iters), sink.data_ptr(),
                                        _stream(stream)), "fsa_mfma_loop")
    return 2.0 * 32 * 32 * 16 * 8 * iters * 4 * workgroups


def nsa_selected_attn_fwd(prob: Problem, q, k, v, sel, lse, out, stream=None):
    """fsa_nsa_selected_attn_fwd: query-outer forward straight from Sel
    [h_K, N, T] into out [N, h_q, d] and lse [N, h_q]; no index or workspace."""
    qs, ks = _qkv_shapes(prob)
    args = (
        _ptr(q, "q", prob.dtype, qs),
        _ptr(k, "k", prob.dtype, ks),
        _ptr(v, "v", prob.dtype, ks),
        _ptr(sel, "sel", torch.int32, (prob.num_kv_heads, prob.total_tokens, prob.topk)),
        _ptr(lse, "lse", torch.float32, (prob.total_tokens, prob.num_q_heads)),
        _ptr(out, "out", prob.dtype, qs),
    )
    _check(load_library().fsa_nsa_selected_attn_fwd(prob.c(), *args, _stream(stream)), "fsa_nsa_selected_attn_fwd")


def selected_attention(prob: Problem, q, k, v, sel, stream=None, onepass: bool = False):
    """Whole forward: index, statistics and output, with torch-allocated
    buffers (onepass: the statistics fused into the main kernel and the
    reduction).  Returns (out, lse, row_max, index)."""
    dev = q.device
    if prob.cu_dev is None or prob.cu_dev.device != dev:
        raise ValueError("Problem must be created with device= the tensors' device")
    index = allocate_index(prob, dev)
    ws = Workspaces(prob, dev, index.sizes)
    n, hq = prob.total_tokens, prob.num_q_heads
    lse = torch.empty((n, hq), dtype=torch.float32, device=dev)
    row_max = torch.empty((n, hq), dtype=torch.float32, device=dev)
    out = torch.empty((n, hq, prob.head_dim), dtype=prob.dtype, device=dev)
    build_index(prob, sel, index, ws.build, stream)
    if onepass:
        selected_attn_fwd_onepass(prob, q, k, v, index, row_max, lse, out, ws.stats, ws.partial, stream)
    else:
        softmax_stats(prob, q, k, index, row_max, lse, ws.stats, stream)
        selected_attn_fwd(prob, q, k, v, index, lse, out, ws.partial, stream)
    return out, lse, row_max, index
