"""C-ABI checks that need no GPU: the library loads, exports every function
include/fsa.h declares, sizes match closed forms, and every argument error
returns its documented status before anything is launched (device pointers
here are never dereferenced: validation fails first)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import sparse_attention_sel_amd as fsa
from sparse_attention_sel_amd.inputs import WORKLOADS, cu_seqlens_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsa.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS, HIP, ALIGN, SCRATCH = range(9)
FAKE = 1 << 40  # 256-byte aligned fake device address, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|const char\*)\s+(fsa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = fsa.load_library()
    names = declared_functions()
    assert "fsa_build_index" in names and "fsa_softmax_stats" in names and "fsa_selected_attn_fwd" in names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fsa.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (fsa_\w+)", out))
    assert set(names) <= exported


def test_library_is_gfx950():
    # the offload bundle of our own build names its only device target
    blob = open(fsa.library_path(), "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob
    for other in (b"--gfx942", b"--gfx90a", b"--gfx1100"):
        assert other not in blob


def test_version_and_status_strings():
    lib = fsa.load_library()
    assert lib.fsa_abi_version() == fsa.ABI_VERSION == 2
    for s in range(9):
        assert len(fsa.status_string(s)) > 0 and fsa.status_string(s) != "unknown status"
    assert fsa.status_string(99) == "unknown status"
    m = re.search(r"#define FSA_NOALLOC_BUILD_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == fsa.NOALLOC_BUILD_SCRATCH_BYTES


def prob(cu=(0, 1000), H=2, g=2, d=128, B=64, T=16, dtype=0, partial=0, scale=0.0, num_seqs=None, dev=True):
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    p = fsa._Problem(
        num_seqs=len(cu) - 1 if num_seqs is None else num_seqs,
        cu_seqlens_host=cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        cu_seqlens_dev=FAKE if dev else None,
        num_kv_heads=H, gqa_group=g, head_dim=d, block_size=B, topk=T,
        softmax_scale=scale, dtype=dtype, partial_dtype=partial,
    )
    p._keep = cu
    return p


def sizes(p):
    s = fsa._Sizes()
    st = fsa.load_library().fsa_get_sizes(ctypes.byref(p), ctypes.byref(s))
    return st, s


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_sizes_closed_form(name):
    sp = WORKLOADS[name]
    p = prob(cu_seqlens_of(sp.seqlens), sp.num_kv_heads, sp.gqa_group, sp.head_dim, sp.block_size, sp.topk)
    st, s = sizes(p)
    assert st == OK
    N = sum(sp.seqlens)
    B, T, H = sp.block_size, sp.topk, sp.num_kv_heads
    nb = [-(-L // B) for L in sp.seqlens]
    assert s.total_tokens == N and s.num_blocks == sum(nb)
    pmax = H * sum(min(B, L - e * B) * min(T, e + 1) for L in sp.seqlens for e in range(-(-L // B)))
    assert s.max_pairs == pmax
    assert s.counts_bytes == 4 * H * sum(nb) and s.offsets_bytes == 4 * (H * sum(nb) + 1)
    assert s.slot_bytes == 4 * H * N * T and s.qidx_bytes == 4 * pmax
    # one partial row per (pair, group head) + 32 dump rows, and the work-queue
    # counters (8 of them, 128 bytes apart); no region beyond that (a query's
    # local row sits at the rows of one of its local entries)
    g, d = sp.gqa_group, sp.head_dim
    halves = 2 if (B, d) == (128, 256) else 1  # two 64-key halves per 128-key block at d = 256
    rows = halves * pmax * g + 32
    queue = 8 * 128

    def r256(x):
        return -(-x // 256) * 256

    assert s.partial_ws_bytes == r256(r256(rows * d * 4) + queue)
    assert s.stats_ws_bytes == r256(r256(rows * 8) + queue)
    # backward: delta [N, h_q] fp32 + dQ partial rows (no local rows) + fp32 dK/dV slots of [2][B_K][d]
    CT = -(-1024 // g)
    slots = pmax // CT + H * sum(nb) + 2
    if halves == 1:
        assert s.bwd_ws_bytes >= 4 * N * H * g + rows * d * 4 + slots * 2 * B * d * 4 + queue
    else:
        assert s.bwd_ws_bytes == 0  # no backward kernel for this shape


def test_max_pairs_bounds_real_pairs():
    # the forced-block generators reach the bound exactly (every token keeps
    # min(T, own block + 1) distinct blocks)
    from oracle import build_index
    from sparse_attention_sel_amd.inputs import make_workload

    w = make_workload("n8k_h4_g2_d128_t16_bf16", with_qkv=False)
    ref = build_index(w.sel, w.cu_seqlens, w.block_size)
    st, s = sizes(prob(w.cu_seqlens, 4, 2, 128, 64, 16))
    assert st == OK and s.max_pairs == ref["pairs"]
    counts = ref["counts"]
    assert s.max_work_items >= int(np.sum((counts + 1023 // 2) // (1024 // 2)))


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(g=0), SHAPE), (dict(g=17), SHAPE), (dict(H=0), SHAPE),
        (dict(d=48), UNSUP), (dict(d=100), SHAPE), (dict(d=512), SHAPE),
        (dict(B=32), UNSUP), (dict(B=0), SHAPE),
        (dict(T=0), SHAPE), (dict(T=257), SHAPE),
        (dict(dtype=2), DTYPE), (dict(partial=5), DTYPE),
        (dict(cu=(1, 100)), SHAPE), (dict(cu=(0, 100, 50)), SHAPE), (dict(num_seqs=0), SHAPE),
        (dict(scale=float("nan")), SHAPE), (dict(scale=float("inf")), SHAPE),
        (dict(cu=(0, 2**29), H=8, T=16), SHAPE),
        (dict(cu=(0, 600000)), UNSUP),
        (dict(cu=(0, 6912 * 64 + 1)), UNSUP),  # a tile's block window beyond 6912 blocks
    ],
)
def test_sizes_rejects(kw, status):
    assert sizes(prob(**kw))[0] == status


def test_sizes_accepts_edge_shapes():
    for kw in (dict(cu=(0, 0)), dict(cu=(0, 0, 5, 5)), dict(T=256), dict(g=16, d=256), dict(B=128, d=64),
               dict(scale=-1.0), dict(cu=(0, 1)), dict(cu=(0, 6912 * 64)), dict(B=128, d=256)):
        assert sizes(prob(**kw))[0] == OK, kw
    # 128-key blocks at d = 256: forward only (two partial rows per pair, no backward)
    st, s = sizes(prob(B=128, d=256, g=2))
    st64, s64 = sizes(prob(B=64, d=256, g=2))
    assert st == OK and s.bwd_ws_bytes == 0 and s.partial_ws_bytes >= 2 * s.max_pairs * 2 * 256 * 4
    assert sizes(prob(cu=(0, 0)))[1].max_pairs == 0


def fake_index():
    return fsa._Index(FAKE, FAKE, FAKE, FAKE, FAKE)


def test_entry_points_reject_before_launch():
    lib = fsa.load_library()
    p = prob()
    st, s = sizes(p)
    assert st == OK
    P, I = ctypes.byref(p), ctypes.byref(fake_index())
    null_idx = fsa._Index(FAKE, None, FAKE, FAKE, FAKE)
    bad_aux = fsa._Index(FAKE, FAKE, FAKE, FAKE, FAKE + 4)
    # build_index
    assert lib.fsa_build_index(None, FAKE, I, FAKE, s.build_ws_bytes, None) == NULL
    assert lib.fsa_build_index(P, None, I, FAKE, s.build_ws_bytes, None) == NULL
    assert lib.fsa_build_index(P, FAKE, ctypes.byref(null_idx), FAKE, s.build_ws_bytes, None) == NULL
    assert lib.fsa_build_index(P, FAKE, ctypes.byref(bad_aux), FAKE, s.build_ws_bytes, None) == ALIGN
    assert lib.fsa_build_index(P, FAKE + 2, I, FAKE, s.build_ws_bytes, None) == ALIGN
    assert lib.fsa_build_index(P, FAKE, I, FAKE, s.build_ws_bytes - 1, None) == WS
    assert lib.fsa_build_index(ctypes.byref(prob(dev=False)), FAKE, I, FAKE, s.build_ws_bytes, None) == NULL
    assert lib.fsa_build_index(ctypes.byref(prob(g=0)), FAKE, I, FAKE, s.build_ws_bytes, None) == SHAPE
    # build_index_noalloc: the same checks, no workspace argument, and problems
    # whose build scratch exceeds the static array are refused
    assert lib.fsa_build_index_noalloc(None, FAKE, I, None) == NULL
    assert lib.fsa_build_index_noalloc(P, None, I, None) == NULL
    assert lib.fsa_build_index_noalloc(P, FAKE, ctypes.byref(null_idx), None) == NULL
    assert lib.fsa_build_index_noalloc(P, FAKE, ctypes.byref(bad_aux), None) == ALIGN
    assert lib.fsa_build_index_noalloc(P, FAKE + 2, I, None) == ALIGN
    assert lib.fsa_build_index_noalloc(ctypes.byref(prob(dev=False)), FAKE, I, None) == NULL
    assert lib.fsa_build_index_noalloc(ctypes.byref(prob(g=0)), FAKE, I, None) == SHAPE
    big = prob(cu=(0, 65536), H=16, T=16)
    st_big, s_big = sizes(big)
    assert st_big == OK and s_big.build_ws_bytes > fsa.NOALLOC_BUILD_SCRATCH_BYTES
    assert lib.fsa_build_index_noalloc(ctypes.byref(big), FAKE, I, None) == SCRATCH
    fits = prob(cu=(0, 32768, 65536), H=8, g=8, d=256)  # the largest workload's shape
    assert sizes(fits)[1].build_ws_bytes <= fsa.NOALLOC_BUILD_SCRATCH_BYTES
    # softmax_stats
    f = FAKE
    assert lib.fsa_softmax_stats(P, None, f, I, f, f, f, s.stats_ws_bytes, None) == NULL
    assert lib.fsa_softmax_stats(P, f, f, I, f, None, f, s.stats_ws_bytes, None) == NULL
    assert lib.fsa_softmax_stats(P, f + 8, f, I, f, f, f, s.stats_ws_bytes, None) == ALIGN
    assert lib.fsa_softmax_stats(P, f, f, I, f, f, f, s.stats_ws_bytes - 1, None) == WS
    assert lib.fsa_softmax_stats(ctypes.byref(prob(dtype=7)), f, f, I, f, f, f, s.stats_ws_bytes, None) == DTYPE
    # forward / main / reduce
    pw = s.partial_ws_bytes
    assert lib.fsa_selected_attn_fwd(P, f, f, None, I, f, f, f, pw, None) == NULL
    assert lib.fsa_selected_attn_fwd(P, f, f, f, I, f, None, f, pw, None) == NULL
    assert lib.fsa_selected_attn_fwd(P, f, f, f, I, f, f + 4, f, pw, None) == ALIGN
    assert lib.fsa_selected_attn_fwd(P, f, f, f, I, f, f, f, pw - 1, None) == WS
    sw = s.stats_ws_bytes
    assert lib.fsa_selected_attn_fwd_onepass(P, f, f, f, I, None, f, f, f, sw, f, pw, None) == NULL
    assert lib.fsa_selected_attn_fwd_onepass(P, f, f, f, I, f, f, f, None, sw, f, pw, None) == NULL
    assert lib.fsa_selected_attn_fwd_onepass(P, f, f, f, I, f, f, f, f, sw, None, pw, None) == NULL
    assert lib.fsa_selected_attn_fwd_onepass(P, f, f, f, I, f + 2, f, f, f, sw, f, pw, None) == ALIGN
    assert lib.fsa_selected_attn_fwd_onepass(P, f, f, f, I, f, f, f, f + 8, sw, f, pw, None) == ALIGN
    assert lib.fsa_selected_attn_fwd_onepass(P, f, f, f, I, f, f, f, f, sw - 1, f, pw, None) == WS
    assert lib.fsa_selected_attn_fwd_onepass(P, f, f, f, I, f, f, f, f, sw, f, pw - 1, None) == WS
    assert lib.fsa_selected_attn_main(P, f, f, f, I, None, f, pw, None) == NULL
    assert lib.fsa_selected_attn_main(P, f, f, f, I, f, f, pw - 256, None) == WS
    assert lib.fsa_selected_attn_reduce(P, I, f, pw, None, None) == NULL
    assert lib.fsa_selected_attn_reduce(P, I, f, pw - 1, f, None) == WS
    assert lib.fsa_selected_attn_reduce(P, ctypes.byref(null_idx), f, pw, f, None) == NULL
    # backward
    bw = s.bwd_ws_bytes
    assert bw > 0
    assert lib.fsa_selected_attn_bwd(P, f, f, f, None, f, f, I, f, f, f, f, bw, None) == NULL
    assert lib.fsa_selected_attn_bwd(P, f, f, f, f, None, f, I, f, f, f, f, bw, None) == NULL
    assert lib.fsa_selected_attn_bwd(P, f, f, f, f, f, f, I, f, f, None, f, bw, None) == NULL
    assert lib.fsa_selected_attn_bwd(P, f, f, f, f, f, f, ctypes.byref(null_idx), f, f, f, f, bw, None) == NULL
    assert lib.fsa_selected_attn_bwd(P, f, f, f, f, f + 8, f, I, f, f, f, f, bw, None) == ALIGN
    assert lib.fsa_selected_attn_bwd(P, f, f, f, f, f, f, I, f, f, f, f + 16, bw, None) == ALIGN
    assert lib.fsa_selected_attn_bwd(P, f, f, f, f, f, f, I, f, f, f, f, bw - 1, None) == WS
    # measurement loop
    assert lib.fsa_mfma_loop(0, 8, 10, None, None) == NULL
    assert lib.fsa_mfma_loop(0, 0, 10, f, None) == SHAPE
    assert lib.fsa_mfma_loop(0, 8, 0, f, None) == SHAPE
    assert lib.fsa_mfma_loop(5, 8, 10, f, None) == DTYPE
    # block selection
    assert lib.fsa_select_blocks(P, None, 16, 1, 2, f, None) == NULL
    assert lib.fsa_select_blocks(P, f, 16, 1, 2, None, None) == NULL
    assert lib.fsa_select_blocks(P, f, 15, 1, 2, f, None) == SHAPE  # 1000 tokens / 64 = 16 blocks
    assert lib.fsa_select_blocks(P, f, 16, -1, 2, f, None) == SHAPE
    assert lib.fsa_select_blocks(P, f, 16, 1, -2, f, None) == SHAPE
    assert lib.fsa_select_blocks(P, f + 2, 16, 1, 2, f, None) == ALIGN
    assert lib.fsa_select_blocks(ctypes.byref(prob(dev=False)), f, 16, 1, 2, f, None) == NULL
    # query-outer forward (no index, no workspace)
    assert lib.fsa_nsa_selected_attn_fwd(None, f, f, f, f, f, f, None) == NULL
    assert lib.fsa_nsa_selected_attn_fwd(P, f, f, f, None, f, f, None) == NULL
    assert lib.fsa_nsa_selected_attn_fwd(P, f, f, f, f, None, f, None) == NULL
    assert lib.fsa_nsa_selected_attn_fwd(P, f, f, f, f, f, None, None) == NULL
    assert lib.fsa_nsa_selected_attn_fwd(P, f, f + 8, f, f, f, f, None) == ALIGN
    assert lib.fsa_nsa_selected_attn_fwd(P, f, f, f, f + 2, f, f, None) == ALIGN
    assert lib.fsa_nsa_selected_attn_fwd(P, f, f, f, f, f, f + 4, None) == ALIGN
    assert lib.fsa_nsa_selected_attn_fwd(ctypes.byref(prob(dev=False)), f, f, f, f, f, f, None) == NULL
    assert lib.fsa_nsa_selected_attn_fwd(ctypes.byref(prob(d=48)), f, f, f, f, f, f, None) == UNSUP


def test_python_binding_checks_tensors():
    import torch

    p = fsa.Problem([0, 128], 1, 1, 64, 64, 4)
    s = fsa.get_sizes(p)
    assert s["max_pairs"] == 64 * 1 + 64 * 2
    with pytest.raises(ValueError):
        fsa.Problem([0, 128], 1, 1, 64, 64, 4, dtype=torch.float32)
    with pytest.raises(fsa.FsaError) as e:
        fsa.get_sizes(fsa.Problem([0, 128], 1, 1, 48, 64, 4))
    assert e.value.status == UNSUP
    # CPU tensors are refused by the binding before reaching the library
    idx = fsa.Index(*(torch.zeros(8, dtype=torch.int32) for _ in range(4)), torch.zeros(256, dtype=torch.uint8), s)
    with pytest.raises(ValueError):
        fsa.build_index(p, torch.zeros((1, 128, 4), dtype=torch.int32), idx, torch.zeros(s["build_ws_bytes"], dtype=torch.uint8))


def test_empty_problem_accepts_null_data_pointers():
    # N = 0: the per-token buffers may be NULL; calls that launch nothing
    # for an empty problem succeed without a GPU (the index build launches
    # its offsets kernel and is exercised by the GPU tests instead)
    lib = fsa.load_library()
    p = prob(cu=(0, 0))
    st, s = sizes(p)
    assert st == OK and s.total_tokens == 0 and s.max_pairs == 0
    P, I = ctypes.byref(p), ctypes.byref(fake_index())
    f = FAKE
    assert lib.fsa_softmax_stats(P, None, None, I, None, None, f, s.stats_ws_bytes, None) == OK
    assert lib.fsa_selected_attn_main(P, None, None, None, I, None, f, s.partial_ws_bytes, None) == OK
    assert lib.fsa_selected_attn_reduce(P, I, f, s.partial_ws_bytes, None, None) == OK
    assert lib.fsa_selected_attn_fwd(P, None, None, None, I, None, None, f, s.partial_ws_bytes, None) == OK
    assert lib.fsa_selected_attn_fwd_onepass(P, None, None, None, I, None, None, None, f, s.stats_ws_bytes, f,
                                             s.partial_ws_bytes, None) == OK
    assert lib.fsa_selected_attn_bwd(P, None, None, None, None, None, None, I, None, None, None, f, s.bwd_ws_bytes,
                                     None) == OK
    assert lib.fsa_nsa_selected_attn_fwd(P, None, None, None, None, None, None, None) == OK
    assert lib.fsa_select_blocks(P, None, 1, 1, 2, None, None) == OK
    # workspaces stay required
    assert lib.fsa_selected_attn_main(P, None, None, None, I, None, None, s.partial_ws_bytes, None) == NULL


def test_header_is_plain_c_and_links(tmp_path):
    # the ABI is C: the header compiles as strict C99 and a C program links
    # against every declared entry point of libfsa.so (no GPU call is made)
    src = tmp_path / "use_fsa.c"
    names = declared_functions()
    body = "\n".join(f"  (void)&{n};" for n in names)
    src.write_text('#include "fsa.h"\nint main(void) {\n  fsa_problem p; fsa_sizes s; fsa_index i;\n'
                   '  (void)p; (void)s; (void)i;\n' + body + '\n  return 0;\n}\n')
    exe = tmp_path / "use_fsa"
    lib = fsa.library_path()
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{os.path.dirname(HEADER)}", str(src),
           f"-L{os.path.dirname(lib)}", "-l:" + os.path.basename(lib), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no CPU or PyTorch fallback: without libfsa.so every call raises
    monkeypatch.setattr(fsa, "_LIB", None)
    monkeypatch.setattr(fsa, "library_path", lambda: str(tmp_path / "absent" / "libfsa.so"))
    with pytest.raises(RuntimeError, match="missing"):
        fsa.load_library()
    with pytest.raises(RuntimeError):
        fsa.get_sizes(prob())
