"""Host-side logic of bench.py (no GPU): the traffic record's source key and
the algorithmic byte counts it divides by."""

import json
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
    # without the local path every entry is block-outer: no local rows, pairs or words
    b0 = bench.kernel_bytes(W, P, 0, 2, 2)
    assert b0["main"] == q + 2 * N * H * d * 2 + N * H * g * 4 + P * 4 + P * g * d * 2
    assert b0["reduce"] == P * g * d * 2 + H * N * T * 4 + q


def test_profile_summary_on_rocprof_csv(tmp_path):
    # the summariser reads rocprofv3's CSV (mangled names of the library's
    # template kernels) and scales FETCH_SIZE / WRITE_SIZE by a copy's bytes
    import csv

    from sparse_attention_sel_amd import profile_summary as ps

    mangled = "_ZN3fsa12_GLOBAL__N_16k_mainIDF16bLi128ELi64EDF16bLb0EEEvPKT_S4_S4_PKiS6_S6_Pf"
    assert ps.demangle(mangled) == "fsa::(anonymous namespace)::k_main<__bf16, 128, 64, __bf16, false>"
    assert ps.pretty(mangled) == "`k_main<bf16, d=128, B_K=64, partial=bf16>`"
    assert ps.pretty("_ZN3fsa12_GLOBAL__N_18k_reduceIDF16_fLb1ELb1EEEvPKi") == \
        "`k_reduce<fp16, partial=fp32, local, one-pass>`"
    assert ps.pretty("fsa::(anonymous namespace)::k_hist(int const*)") == "`k_hist`"
    # the current kernels carry a split-halves flag after the one-pass flag
    assert ps.pretty("_ZN3fsa12_GLOBAL__N_16k_mainIDF16bLi128ELi64EDF16bLb0ELb0EEEvPKT_S4_S4_PKi") == \
        "`k_main<bf16, d=128, B_K=64, partial=bf16>`"
    assert ps.pretty("_ZN3fsa12_GLOBAL__N_16k_mainIDF16bLi256ELi64EDF16bLb0ELb1EEEvPKT_S4_S4_PKi") == \
        "`k_main<bf16, d=256, B_K=64, partial=bf16, two 64-key halves>`"
    assert ps.pretty("_ZN3fsa12_GLOBAL__N_18k_reduceIDF16bDF16bLb1ELb0ELb0EEEvPKi") == \
        "`k_reduce<bf16, partial=bf16, local>`"
    assert ps.pretty("_ZN3fsa12_GLOBAL__N_18k_main16IDF16bLi256ELi64EDF16bLb1EEEvPKT_S4_S4_PKi") == \
        "`k_main16<bf16, d=256, B_K=64, partial=bf16, two 64-key halves>`"
    assert ps.pretty("_ZN3fsa12_GLOBAL__N_18k_main16IDF16_Li128ELi128EfLb0EEEvPKT_S4_S4_PKi") == \
        "`k_main16<fp16, d=128, B_K=128, partial=fp32>`"
    assert ps.pretty("_ZN3fsa12_GLOBAL__N_114k_main_local16IDF16_fEEvPKT_S4_S4_PKiS6_i") == \
        "`k_main_local16<fp16, d=256, B_K=64, partial=fp32>`"
    assert ps.pretty("_ZN3fsa12_GLOBAL__N_112k_main_mixedIDF16bLi128ELi64EDF16bEEvPKT_S4_S4_PKi") == \
        "`k_main_mixed<bf16, d=128, B_K=64, partial=bf16>`"
    assert ps.pretty("_ZN3fsa12_GLOBAL__N_114k_main_mixed16IDF16bDF16bEEvPKT_S4_S4_PKiS6_S6_PK4int4S6_PiPKfPS3_m") == \
        "`k_main_mixed16<bf16, d=256, B_K=64, partial=bf16>`"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]

    def pmc(d, counter, rows):
        os.makedirs(d)
        with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(hdr)
            for i, (k, v) in enumerate(rows):
                w.writerow([i, k, counter, v, 0, 1000])

    pmc(tmp_path / "f", "FETCH_SIZE", [(mangled, 100.0), (mangled, 300.0)])
    pmc(tmp_path / "w", "WRITE_SIZE", [(mangled, 400.0), (mangled, 400.0)])
    pmc(tmp_path / "cf", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 524288.0)])
    pmc(tmp_path / "cw", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1048576.0)])
    os.makedirs(tmp_path / "t")
    with open(tmp_path / "t" / "x_kernel_stats.csv", "w") as f:
        f.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        f.write(f'"{mangled}",2,2000,1000,100,900,1100,1\n')
    out, js = tmp_path / "t.md", tmp_path / "t.json"
    ps.main(["traffic", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"), "--copy-fetch",
             str(tmp_path / "cf"), "--copy-write", str(tmp_path / "cw"), "--trace", str(tmp_path / "t"),
             "--workload", "W", "--command", "c", "--out", str(out), "--json", str(js), "--source-sha256", "h"])
    rec = json.load(open(js))
    # copy: 1 GiB read as 524288 KiB of FETCH_SIZE -> x2; average fetch 200 KiB
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes"] == 200 * 1024 * 2 and rec["write_bytes"] == 400 * 1024
    assert "k_main<bf16, d=128, B_K=64, partial=bf16>" in open(out).read()


def test_main_stage_kernel_names(monkeypatch):
    # the roofline's kernel label follows the library's choice of launches
    class W:
        num_kv_heads, head_dim, block_size = 4, 128, 64

    big, small = W(), W()
    big.cu_seqlens, big.gqa_group = np.array([0, 65536], dtype=np.int32), 4
    small.cu_seqlens, small.gqa_group = np.array([0, 8192], dtype=np.int32), 2
    monkeypatch.delenv("FSA_MAIN_MIXED", raising=False)
    assert bench.main_stage_kernels(big) == "k_main_mixed"  # 8192 local items
    assert bench.main_stage_kernels(small) == "k_main_local+k_main"  # 512
    monkeypatch.setenv("FSA_MAIN_MIXED", "1")
    assert bench.main_stage_kernels(small) == "k_main_mixed"
    monkeypatch.setenv("FSA_MAIN_MIXED", "0")
    assert bench.main_stage_kernels(big) == "k_main_local+k_main"
    small.gqa_group = 1
    assert bench.main_stage_kernels(small) == "k_main"
    monkeypatch.delenv("FSA_MAIN_MIXED")
    big.head_dim = 256
    assert bench.main_stage_kernels(big) == "k_main_mixed16"
    big.num_kv_heads = 1  # 2048 local items: at least four rounds of 256 workgroups
    assert bench.main_stage_kernels(big) == "k_main_mixed16"
    big.cu_seqlens = np.array([0, 8192], dtype=np.int32)  # 128 blocks, 4 groups: 512 items
    assert bench.main_stage_kernels(big) == "k_main_local16+k_main16"
