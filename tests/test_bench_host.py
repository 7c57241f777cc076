"""Host-side logic of bench.py (no GPU): the traffic record's source key and
the algorithmic byte counts it divides by."""

import os
import shutil

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _copy_sources(tmp_path):
    dst = tmp_path / "sparse_attention_sel_amd" / "csrc"
    dst.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(ROOT, "sparse_attention_sel_amd", "csrc", name), dst / name)
    return dst


def test_kernel_source_hash_ignores_comments_but_not_code(tmp_path):
    dst = _copy_sources(tmp_path)
    h0 = bench.kernel_source_hash(str(tmp_path))
    assert h0 == bench.kernel_source_hash(ROOT)
    f = dst / bench.KERNEL_SOURCES[0]
    text = f.read_text()
    f.write_text("// a new comment line\n" + text.replace("\n", "\n\n", 3) + "/* block\ncomment */\n")
    assert bench.kernel_source_hash(str(tmp_path)) == h0
    f.write_text(text + "\nstatic int unused_marker = 1;\n")
    assert bench.kernel_source_hash(str(tmp_path)) != h0


def test_kernel_bytes_counts_each_compulsory_access_once():
    class W:
        cu_seqlens = np.array([0, 1024], dtype=np.int32)
        num_kv_heads, gqa_group, head_dim, topk = 2, 4, 128, 16

    P, P_loc = 10000, 3000
    b = bench.kernel_bytes(W, P, P_loc, 2, 2)
    N, H, g, d, T = 1024, 2, 4, 128, 16
    q = N * H * g * d * 2
    main = q + 2 * N * H * d * 2 + N * H * g * 4 + (P - P_loc) * 4 + (P - P_loc) * g * d * 2 + N * H * g * d * 2 + 4 * H * N
    assert b["main"] == main
    assert b["reduce"] == (P - P_loc) * g * d * 2 + N * H * g * d * 2 + H * N * T * 4 + 4 * H * N + q
