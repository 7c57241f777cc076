"""GPU parity: the HIP path (through the C-ABI) against the float64 oracle.

Index tensors must match bit-exactly; O within max-abs 2e-2 (bf16) or 5e-3
(fp16); lse (and row max) within 1e-3.  Every shape is compared on every
token: the small ones here, the full-size workloads through the oracle
service (the oracle evaluated in CPU worker processes started before the
first GPU call).
"""

import functools

import numpy as np
import pytest
import torch

import oracle.fsa_oracle as O
from gpu_helpers import TOL_LSE, TOL_O, check_full_forward, custom_workload, log, run_gpu, sample_tokens
from sparse_attention_sel_amd.inputs import WORKLOADS, make_workload

pytestmark = pytest.mark.gpu

# (workload, partial dtype).  The 64K g=4 case runs in both partial dtypes:
# "input" (16-bit partials) is the configuration the benchmark times.
LARGE = [
    ("n64k_h4_g4_d128_t16_bf16", "fp32"),
    ("n64k_h4_g4_d128_t16_bf16", "input"),
    ("n64k_h4_g1_d128_t16_fp16", "fp32"),
    ("b2_n32k_h8_g8_d256_t16_bf16", "input"),
    ("n64k_h4_g2_d128_t16_bf16", "fp32"),
    ("n64k_h4_g1_d128_t16_bf16", "fp32"),
    ("n64k_h4_g4_d128_b128_t8_bf16", "input"),
    ("n32k_h4_g4_d256_b128_t8_bf16", "input"),
]


@functools.lru_cache(maxsize=2)
def workload(name):
    log(f"[gen] {name}")
    return make_workload(name)


@functools.lru_cache(maxsize=8)
def oracle_index(name):
    w = workload(name)
    return O.build_index(w.sel, w.cu_seqlens, w.block_size)


def check_index(res, ref):
    assert res["pairs"] == ref["pairs"]
    np.testing.assert_array_equal(res["counts"], ref["counts"])
    np.testing.assert_array_equal(res["offsets"], ref["offsets"])
    np.testing.assert_array_equal(res["qidx"], ref["qidx"])
    np.testing.assert_array_equal(res["slot"], ref["slot"])


def check_attention(res, w, tokens=None):
    q = w.q.float().numpy()
    k = w.k.float().numpy()
    v = w.v.float().numpy()
    o_ref, m_ref, lse_ref = O.selected_attention(q, k, v, w.sel, w.cu_seqlens, w.block_size, w.scale, tokens)
    sel = slice(None) if tokens is None else tokens
    o, lse, m = res["out"][sel], res["lse"][sel], res["row_max"][sel]
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), "empty key sets must give lse = -inf"
    assert np.array_equal(np.isneginf(m), empty)
    assert np.all(o[empty] == 0)
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    fin = ~empty
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    err_m = float(np.max(np.abs(m[fin] - m_ref[fin]))) if fin.any() else 0.0
    log(f"    max|dO|={err_o:.3e} max|dlse|={err_l:.3e} max|dm|={err_m:.3e}")
    assert err_o <= TOL_O[w.dtype], f"O error {err_o}"
    assert err_l <= TOL_LSE and err_m <= TOL_LSE


@pytest.mark.parametrize("partial", ["fp32", "input"])
def test_small_all_tokens(partial):
    w = workload("n1k_h1_g1_d64_t4_bf16")
    log(f"[run] n1k partial={partial}")
    res = run_gpu(w, partial)
    check_index(res, oracle_index(w.name))
    check_attention(res, w)


@pytest.mark.parametrize("partial", ["fp32", "input"])
def test_n8k_all_tokens(partial):
    w = workload("n8k_h4_g2_d128_t16_bf16")
    log(f"[run] n8k partial={partial}")
    res = run_gpu(w, partial)
    check_index(res, oracle_index(w.name))
    check_attention(res, w)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,partial", LARGE)
def test_large_index_and_all_tokens(name, partial, oracle_service):
    oracle_service.prepare(name)  # the service generates its copy meanwhile
    w = workload(name)
    log(f"[run] {name} partial={partial}")
    res = run_gpu(w, partial, float_out=False)
    log("    index")
    check_index(res, oracle_index(name))
    check_full_forward(oracle_service, w, res)


def adversarial_sel(rng, H, cu, B, T):
    n = int(cu[-1])
    sel = np.empty((H, n, T), dtype=np.int32)
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        nb = (c1 - c0 + B - 1) // B
        sel[:, c0:c1, :] = rng.integers(-2, nb + 2, size=(H, c1 - c0, T))
    dup = rng.random(sel.shape) < 0.2
    sel[dup] = np.roll(sel, 1, axis=2)[dup]
    return sel


CASES = [
    # seqlens, H, g, d, B, T, dtype
    ((300, 0, 129, 64), 2, 3, 64, 64, 5, "bf16"),
    ((513, 77), 1, 16, 128, 64, 3, "fp16"),
    ((1000,), 2, 1, 128, 128, 8, "bf16"),
    ((200, 333), 3, 5, 256, 64, 7, "bf16"),
    ((64, 1, 65), 1, 2, 64, 64, 1, "fp16"),
    ((3000, 1100), 2, 4, 128, 64, 48, "bf16"),  # long rows: most blocks, duplicates, out-of-range
    ((700,), 1, 2, 64, 64, 256, "fp16"),  # the largest T: one token per scatter step
    ((300, 100), 1, 16, 256, 64, 6, "bf16"),  # g * d = 4096: two output vectors per reduction thread
    ((257,), 2, 3, 256, 64, 5, "fp16"),
    ((600, 200), 1, 2, 64, 128, 4, "fp16"),
    ((500, 77, 300), 2, 1, 128, 64, 6, "bf16"),  # g = 1 with 64-key blocks: every entry block-outer
    ((300, 129), 1, 1, 256, 64, 4, "fp16"),
]


def adversarial_workload(case):
    seqlens, H, g, d, B, T, dtype = CASES[case]
    rng = np.random.default_rng(700 + case)
    from sparse_attention_sel_amd.inputs import cu_seqlens_of

    cu = cu_seqlens_of(seqlens)
    sel = adversarial_sel(rng, H, cu, B, T)
    sel[:, ::37, :] = -1  # some rows select nothing
    return custom_workload(seqlens, H, g, d, B, T, dtype, sel, seed=900 + case)


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("partial", ["fp32", "input"])
def test_adversarial_selection(case, partial):
    w = adversarial_workload(case)
    log(f"[run] adversarial case {case} {CASES[case]} partial={partial}")
    res = run_gpu(w, partial)
    check_index(res, O.build_index(w.sel, w.cu_seqlens, CASES[case][4]))
    check_attention(res, w)


# the cases with per-query-block (local) entries
MIXED_CASES = [i for i, c in enumerate(CASES) if c[4] == 64 and c[2] >= 2]


def _same_bits(a, b):
    for key in ("out_bits", "lse", "row_max"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key


@pytest.mark.parametrize("case", MIXED_CASES)
def test_mixed_main_launch(case, monkeypatch):
    # The local and block-outer items of the forward in one persistent launch,
    # forced (these sizes take two launches by default): the oracle's outputs
    # on every token, and the bits of the two-launch path.
    w = adversarial_workload(case)
    log(f"[run] mixed main launch, adversarial case {case} {CASES[case]}")
    monkeypatch.setenv("FSA_MAIN_MIXED", "1")
    a = run_gpu(w, "input")
    check_attention(a, w)
    monkeypatch.setenv("FSA_MAIN_MIXED", "0")
    _same_bits(a, run_gpu(w, "input"))


@pytest.mark.parametrize("name", ["n8k_h4_g2_d128_t16_bf16", "n64k_h4_g4_d128_t16_bf16"])
def test_mixed_and_split_main_launch_bitwise(name, monkeypatch):
    # 8K tokens take two launches by default and 64K one: both ways agree bit
    # for bit (each item runs the same code).
    w = workload(name)
    log(f"[run] mixed against split main launch: {name}")
    monkeypatch.setenv("FSA_MAIN_MIXED", "1")
    a = run_gpu(w, "input")
    monkeypatch.setenv("FSA_MAIN_MIXED", "0")
    _same_bits(a, run_gpu(w, "input"))


def test_largest_block_window():
    # One sequence of 6912 blocks of 64 tokens: the last token tiles can select
    # any of the 6912 blocks, the largest window the index builder takes (one
    # more block is FSA_ERR_UNSUPPORTED), which sizes k_scatter's LDS.  Rows keep
    # their own block and block 0 and add one pick uniform over every earlier
    # block and one recent block; every 41st row is padding only.  The index is
    # compared bit for bit; outputs on sampled tokens, and lse / row max of
    # every token against bounds that hold at any size.
    nb, B, T = 6912, 64, 4
    n = nb * B
    rng = np.random.default_rng(8800)
    own = np.arange(n, dtype=np.int64) // B
    sel = np.empty((1, n, T), dtype=np.int32)
    sel[0, :, 0] = own
    sel[0, :, 1] = 0
    sel[0, :, 2] = (rng.random(n) * (own + 1)).astype(np.int64)
    sel[0, :, 3] = own - rng.geometric(0.2, size=n)  # -1 and below: padding
    sel[:, ::41, :] = -1
    w = custom_workload((n,), 1, 2, 64, B, T, "bf16", sel, seed=8801)
    log(f"[run] largest block window: {n} tokens, {nb} blocks")
    res = run_gpu(w, "input")
    ref = O.build_index(w.sel, w.cu_seqlens, B)
    log(f"    index: {ref['pairs']} pairs")
    check_index(res, ref)
    lse, m = res["lse"], res["row_max"]
    empty = np.zeros(n, dtype=bool)
    empty[::41] = True
    assert np.all(np.isneginf(lse[empty])) and np.all(np.isneginf(m[empty]))
    assert np.all(res["out"][empty] == 0)
    # lse - row max = ln(sum exp(s - max)) lies in [0, ln(visible keys)]
    nkeys = np.zeros(n, dtype=np.float64)
    for t0 in range(0, n, 1 << 16):
        toks = np.arange(t0, min(n, t0 + (1 << 16)))
        rows = w.sel[0, toks]
        e = np.where(_valid_rows(rows, toks, B), rows, -1)
        ownb = (toks // B)[:, None]
        full = ((e >= 0) & (e < ownb)).sum(axis=1) * B
        nkeys[toks] = full + np.where((e == ownb).any(axis=1), toks % B + 1, 0)
    fin = ~empty
    d = lse[fin] - m[fin]
    bound = np.log(nkeys[fin])[:, None]
    assert np.all(d >= -1e-3) and np.all(d <= bound + 1e-3), "lse outside [row max, row max + ln(keys)]"
    check_attention(res, w, sample_tokens(w.cu_seqlens, B, n_random=160, seed=8802))


def _valid_rows(rows, toks, B):
    # first occurrences of the entries 0 <= e <= own block of each row
    own = (toks // B)[:, None]
    ok = (rows >= 0) & (rows <= own)
    for j in range(1, rows.shape[1]):
        ok[:, j] &= ~np.any(rows[:, :j] == rows[:, j : j + 1], axis=1)
    return ok


BLOCK128_D256 = [
    # seqlens, H, g, T, dtype: last blocks of 44, 1, 64 and 65 tokens leave the
    # second 64-key half of the block empty or one key long
    ((300, 129, 64, 1000), 2, 3, 5, "fp16"),
    ((4096, 700), 2, 4, 8, "bf16"),
]


@pytest.mark.parametrize("case", range(len(BLOCK128_D256)))
@pytest.mark.parametrize("partial", ["fp32", "input"])
def test_block128_d256_all_tokens(case, partial):
    # 128-key blocks at head dim 256: the main kernel runs each block as two
    # 64-key halves with a partial row each; the reduction adds both
    seqlens, H, g, T, dtype = BLOCK128_D256[case]
    rng = np.random.default_rng(7100 + case)
    from sparse_attention_sel_amd.inputs import cu_seqlens_of

    cu = cu_seqlens_of(seqlens)
    sel = adversarial_sel(rng, H, cu, 128, T)
    sel[:, ::37, :] = -1
    w = custom_workload(seqlens, H, g, 256, 128, T, dtype, sel, seed=7200 + case)
    log(f"[run] B_K=128 d=256 case {case} partial={partial}")
    res = run_gpu(w, partial)
    check_index(res, O.build_index(w.sel, w.cu_seqlens, 128))
    check_attention(res, w)


def test_block128_d256_unsupported_paths():
    # no query-outer, one-pass or backward kernels exist for this shape
    import sparse_attention_sel_amd as fsa

    w = custom_workload((300,), 1, 2, 256, 128, 3, "bf16", np.zeros((1, 300, 3), np.int32), seed=1)
    dev = torch.device("cuda:0")
    prob = fsa.Problem(w.cu_seqlens, 1, 2, 256, 128, 3, device=dev)
    assert fsa.get_sizes(prob)["bwd_ws_bytes"] == 0
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    sel = torch.zeros((1, 300, 3), dtype=torch.int32, device=dev)
    lse = torch.empty((300, 2), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    with pytest.raises(fsa.FsaError) as e:
        fsa.nsa_selected_attn_fwd(prob, q, k, v, sel, lse, out)
    assert e.value.status == 4
    index = fsa.allocate_index(prob, dev)
    ws = fsa.Workspaces(prob, dev, index.sizes)
    fsa.build_index(prob, sel, index, ws.build)
    with pytest.raises(fsa.FsaError) as e:
        fsa.selected_attn_fwd_onepass(prob, q, k, v, index, torch.empty_like(lse), lse, out, ws.stats, ws.partial)
    assert e.value.status == 4
    torch.cuda.synchronize()


def test_full_selection_equals_causal_attention():
    # Sel holding every block (future ones included) is plain causal attention;
    # compare with torch's float32 SDPA on the CPU as an independent reference.
    seqlens, H, g, d, B = (700, 300), 2, 2, 64, 64
    from sparse_attention_sel_amd.inputs import cu_seqlens_of

    cu = cu_seqlens_of(seqlens)
    nb = max(-(-L // B) for L in seqlens)
    sel = np.broadcast_to(np.arange(nb, dtype=np.int32), (H, int(cu[-1]), nb)).copy()
    w = custom_workload(seqlens, H, g, d, B, nb, "bf16", sel, seed=77)
    res = run_gpu(w, "fp32")
    for s in range(len(seqlens)):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        qt = w.q[c0:c1].float().permute(1, 0, 2)[None]
        kt = w.k[c0:c1].float().permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        vt = w.v[c0:c1].float().permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=w.scale)
        ref = ref[0].permute(1, 0, 2).numpy()
        assert np.max(np.abs(res["out"][c0:c1] - ref)) <= TOL_O["bf16"]


def test_deterministic_bitwise():
    w = workload("n8k_h4_g2_d128_t16_bf16")
    a = run_gpu(w, "input")
    b = run_gpu(w, "input")
    for key in ("counts", "offsets", "qidx", "slot", "out", "lse", "row_max"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_repeated_calls_on_one_index():
    # The compute calls claim their work items through counters kept with the
    # index.  Calls that reuse one index without rebuilding it must each cover
    # every item: three rounds of stats + forward and two backward calls on one
    # index give bitwise the results of a freshly built index.
    import sparse_attention_sel_amd as fsa
    from sparse_attention_sel_amd.inputs import make_dout

    w = workload("n8k_h4_g2_d128_t16_bf16")
    ref = run_gpu(w, "input")
    prob = fsa.Problem(w.cu_seqlens, w.num_kv_heads, w.gqa_group, w.head_dim, w.block_size, w.topk,
                       dtype=torch.bfloat16, partial_dtype="input", softmax_scale=w.scale, device="cuda:0")
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    sel = torch.from_numpy(w.sel).to(dev)
    index = fsa.allocate_index(prob, dev)
    ws = fsa.Workspaces(prob, dev, index.sizes, backward=True)
    fsa.build_index(prob, sel, index, ws.build)
    n, hq = prob.total_tokens, prob.num_q_heads
    for rnd in range(3):
        log(f"    round {rnd}")
        lse = torch.full((n, hq), float("nan"), dtype=torch.float32, device=dev)
        row_max = torch.full_like(lse, float("nan"))
        out = torch.full((n, hq, prob.head_dim), float("nan"), dtype=prob.dtype, device=dev)
        fsa.softmax_stats(prob, q, k, index, row_max, lse, ws.stats)
        fsa.selected_attn_fwd(prob, q, k, v, index, lse, out, ws.partial)
        torch.cuda.synchronize()
        assert np.array_equal(out.float().cpu().numpy(), ref["out"])
        assert np.array_equal(lse.cpu().numpy(), ref["lse"])
        assert np.array_equal(row_max.cpu().numpy(), ref["row_max"])
    do = make_dout(n, hq, prob.head_dim, "bf16", 11).to(dev)
    grads = []
    for _ in range(2):
        dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
        fsa.selected_attn_bwd(prob, q, k, v, out, do, lse, index, dq, dk, dv, ws.bwd)
        torch.cuda.synchronize()
        grads.append([x.float().cpu() for x in (dq, dk, dv)])
    for a, b in zip(*grads):
        assert torch.isfinite(a).all()
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["n8k_h4_g2_d128_t16_bf16", "n1k_h1_g1_d64_t4_bf16"])
def test_concurrent_calls_on_one_index(name):
    # After the build the index is read-only (the work-queue counters live in
    # each call's workspace): two streams that share the index but not their
    # workspaces run the statistics, forward and backward at the same time and
    # each gets bitwise the single-stream results.  (g = 1 takes the path
    # without local kernels, where a clear kernel zeroes the counters.)
    import sparse_attention_sel_amd as fsa
    from sparse_attention_sel_amd.inputs import make_dout

    w = workload(name)
    ref = run_gpu(w, "input")
    dev = torch.device("cuda:0")
    prob = fsa.Problem(w.cu_seqlens, w.num_kv_heads, w.gqa_group, w.head_dim, w.block_size, w.topk,
                       dtype=torch.bfloat16, partial_dtype="input", softmax_scale=w.scale, device=dev)
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    sel = torch.from_numpy(w.sel).to(dev)
    index = fsa.allocate_index(prob, dev)
    ws0 = fsa.Workspaces(prob, dev, index.sizes, backward=True)
    fsa.build_index(prob, sel, index, ws0.build)
    n, hq = prob.total_tokens, prob.num_q_heads
    do = make_dout(n, hq, prob.head_dim, "bf16", 17).to(dev)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for s_ in streams:
        ws = fsa.Workspaces(prob, dev, index.sizes, backward=True)
        lse = torch.full((n, hq), float("nan"), dtype=torch.float32, device=dev)
        row_max = torch.full_like(lse, float("nan"))
        out = torch.full((n, hq, prob.head_dim), float("nan"), dtype=prob.dtype, device=dev)
        grads = [torch.full_like(x, float("nan")) for x in (q, k, v)]
        runs.append((s_, ws, lse, row_max, out, grads))
    for rep in range(3):
        for s_, ws, lse, row_max, out, grads in runs:
            with torch.cuda.stream(s_):
                fsa.softmax_stats(prob, q, k, index, row_max, lse, ws.stats)
                fsa.selected_attn_fwd(prob, q, k, v, index, lse, out, ws.partial)
                fsa.selected_attn_bwd(prob, q, k, v, out, do, lse, index, *grads, ws.bwd)
    torch.cuda.synchronize()
    dq_ref = None
    for s_, ws, lse, row_max, out, grads in runs:
        assert np.array_equal(out.float().cpu().numpy(), ref["out"])
        assert np.array_equal(lse.cpu().numpy(), ref["lse"])
        assert np.array_equal(row_max.cpu().numpy(), ref["row_max"])
        g_host = [x.float().cpu() for x in grads]
        assert all(bool(torch.isfinite(x).all()) for x in g_host)
        if dq_ref is None:
            dq_ref = g_host
        else:
            assert all(torch.equal(a, b) for a, b in zip(g_host, dq_ref))


def test_partial_rows_sum_to_output():
    # fp32 partials: each query's local row (its own, previous and first
    # block, computed per query block and stored at the partial rows of its
    # designated local entry: the own-block entry, else the previous-block
    # one, else the first-block one) plus the partial rows of its other
    # selecting entries, summed in slot order, give the output before its
    # final rounding.  Locality is derived here from Sel itself.
    w = workload("n8k_h4_g2_d128_t16_bf16")
    res = run_gpu(w, "fp32", keep_partial=True)
    idx = res["index"]
    g, d, H, B = w.gqa_group, w.head_dim, w.num_kv_heads, w.block_size
    P = res["pairs"]
    part = res["partial"].view(torch.float32)
    dev = part.device
    slot = idx.slot.long()  # [H, N, T]
    N = slot.shape[1]
    pairs = part[: P * g * d].view(P, g, d)
    sel = torch.from_numpy(w.sel).to(dev).long()
    tok = torch.arange(N, device=dev)
    cu = torch.from_numpy(np.asarray(w.cu_seqlens, dtype=np.int64)).to(dev)
    seq = torch.searchsorted(cu, tok, right=True) - 1
    own = ((tok - cu[seq]) // B).view(1, N, 1)
    # the library takes this path for B_K = 64 and g >= 2 (this workload)
    assert B == 64 and g >= 2
    valid = slot >= 0
    kinds = [valid & (sel == own), valid & (sel == own - 1), valid & (sel == 0) & (own >= 2)]
    is_local = kinds[0] | kinds[1] | kinds[2]
    has_local = is_local.any(dim=2)  # [H, N]
    # designated entry: the first kind present, its (unique) position
    des = torch.full((H, N), -1, dtype=torch.long, device=dev)
    for kd in reversed(kinds):
        pos = torch.argmax(kd.long(), dim=2)
        des = torch.where(kd.any(dim=2), torch.gather(slot, 2, pos.unsqueeze(2)).squeeze(2), des)
    assert bool(torch.all((des >= 0) == has_local))
    local = pairs[des.clamp(min=0)].permute(1, 0, 2, 3)  # [N, H, g, d]
    acc = torch.where(has_local.permute(1, 0).view(N, H, 1, 1), local, torch.zeros((), device=dev))
    for j in range(slot.shape[2]):
        s_ = slot[:, :, j].permute(1, 0)  # [N, H]
        ok = ((s_ >= 0) & ~is_local[:, :, j].permute(1, 0)).unsqueeze(-1).unsqueeze(-1)
        acc += torch.where(ok, pairs[s_.clamp(min=0)], torch.zeros((), device=dev))
    out = res["out_dev"].float().view(N, H, g, d)
    ulp = torch.clamp(out.abs(), min=2.0**-126)
    half_ulp = torch.pow(2.0, torch.floor(torch.log2(ulp)) - 8)
    assert bool(torch.all((acc - out).abs() <= half_ulp * 1.001 + 1e-30))


def test_empty_problem_through_every_entry_point():
    # no tokens at all: every call succeeds, writes nothing per token, and the
    # index reports zero pairs
    import sparse_attention_sel_amd as fsa

    dev = torch.device("cuda:0")
    H, g, d, B, T = 2, 2, 128, 64, 4
    prob = fsa.Problem([0, 0], H, g, d, B, T, device=dev)
    index = fsa.allocate_index(prob, dev)
    ws = fsa.Workspaces(prob, dev, index.sizes, backward=True)
    q = torch.empty((0, H * g, d), dtype=torch.bfloat16, device=dev)
    k = torch.empty((0, H, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    sel = torch.empty((H, 0, T), dtype=torch.int32, device=dev)
    lse = torch.empty((0, H * g), dtype=torch.float32, device=dev)
    row_max = torch.empty_like(lse)
    out = torch.empty_like(q)
    fsa.build_index(prob, sel, index, ws.build)
    fsa.softmax_stats(prob, q, k, index, row_max, lse, ws.stats)
    fsa.selected_attn_fwd(prob, q, k, v, index, lse, out, ws.partial)
    fsa.selected_attn_fwd_onepass(prob, q, k, v, index, row_max, lse, out, ws.stats, ws.partial)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fsa.selected_attn_bwd(prob, q, k, v, out, q, lse, index, dq, dk, dv, ws.bwd)
    fsa.nsa_selected_attn_fwd(prob, q, k, v, sel, lse, out)
    fsa.select_blocks(prob, torch.empty((H, 0, 1), dtype=torch.float32, device=dev), 1, 2, sel)
    torch.cuda.synchronize()
    assert index.num_pairs() == 0
    assert int(index.offsets[0].item()) == 0
