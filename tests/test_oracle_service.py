"""The checking harness itself: the oracle service that runs the full-size
GPU comparisons (tests/oracle_service.py), fed here with results the oracle
made on the CPU.  Its per-shard evaluation must reproduce the oracle's
one-call result (only the 16-bit rounding of the fed results remains), and a
single planted error must be found at its place."""

import numpy as np
import pytest
import torch

import oracle.fsa_oracle as O
from gpu_helpers import ResultFiles
from oracle_service import decode_out
from sparse_attention_sel_amd.inputs import cu_seqlens_of, make_block_scores, make_dout, make_workload

NAME = "b2_n1k_h2_g4_d64_t8_bf16"  # two packed sequences


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(scope="module")
def work():
    w = make_workload(NAME)
    q, k, v = (x.float().numpy() for x in (w.q, w.k, w.v))
    return w, q, k, v


def test_decode_is_exact():
    x = np.array([1.0, -2.5, 3.140625, 0.0, -0.0, 65504.0, 1e-20], dtype=np.float32)
    b = bf16_bits(x)
    np.testing.assert_array_equal(decode_out(b, "bf16"), torch.from_numpy(x).to(torch.bfloat16).double().numpy())
    h = x.astype(np.float16)
    np.testing.assert_array_equal(decode_out(h.view(np.uint16), "fp16"), h.astype(np.float64))


def test_forward_all_tokens_and_planted_error(oracle_service, work):
    w, q, k, v = work
    oracle_service.prepare(NAME)
    o, m, lse = O.selected_attention(q, k, v, w.sel, w.cu_seqlens, w.block_size, w.scale)
    bits = bf16_bits(o)
    with ResultFiles() as f:
        r = oracle_service.forward(NAME, f.save("out", bits), f.save("lse", lse.astype(np.float32)),
                                   f.save("row_max", m.astype(np.float32)))
    assert r["tokens"] == 1024
    # only the bf16 rounding of O (half an ulp) and the fp32 rounding of lse remain
    assert 0 < r["err_o"] <= 2.0**-8 * np.abs(o).max()
    assert r["err_lse"] <= 1e-6 and r["err_m"] <= 1e-6
    assert r["empty_mismatch"] == 0 and r["nonzero_empty_out"] == 0 and r["nonfinite"] == 0
    bad = bits.copy()
    bad[700, 5, 33] ^= 0x0400  # the second sequence, a middle head
    lse_bad = lse.astype(np.float32)
    lse_bad[100, 2] += 0.01
    with ResultFiles() as f:
        r = oracle_service.forward(NAME, f.save("out", bad), f.save("lse", lse_bad),
                                   f.save("row_max", m.astype(np.float32)))
    assert r["err_o_at"] == [700, 5, 33] and r["err_o"] > 0.02
    assert r["err_lse_at"] == [100, 2] and r["err_lse"] > 0.009


def test_backward_shards_reproduce_one_call(oracle_service, work):
    w, q, k, v = work
    oracle_service.prepare(NAME)
    do = make_dout(1024, 8, 64, "bf16", 21)
    dq, dk, dv = O.selected_attention_backward(q, k, v, w.sel, w.cu_seqlens, w.block_size, do.float().numpy(), w.scale)
    blocks = [(0, 0), (0, 4), (0, 9), (1, 0), (1, 3), (1, 5)]
    with ResultFiles() as f:
        r = oracle_service.backward(NAME, 21, f.save("dq", bf16_bits(dq)), f.save("dk", bf16_bits(dk)),
                                    f.save("dv", bf16_bits(dv)), blocks)
    assert r["tokens"] == 1024 and r["keys"] == 6 * 64
    # bf16 rounding of the fed gradients is at most 2^-9 relative: ratio < 0.5
    for nm in ("dq", "dk", "dv"):
        assert r[nm + "_ratio"] < 0.5, (nm, r)
    dk_bad = bf16_bits(dk)
    dk_bad[640 + 3 * 64 + 7, 1, 9] ^= 0x0200  # a key of sequence 1, block 3
    with ResultFiles() as f:
        r = oracle_service.backward(NAME, 21, f.save("dq", bf16_bits(dq)), f.save("dk", dk_bad),
                                    f.save("dv", bf16_bits(dv)), blocks)
    assert r["dk_ratio"] > 1.0 and r["dk_at"] == [640 + 3 * 64 + 7, 1, 9]


def test_select_all_tokens_and_planted_error(oracle_service):
    seqlens, H, B, T = (700, 300), 2, 64, 6
    cu = cu_seqlens_of(seqlens)
    sc = make_block_scores(seqlens, H, B, 31)
    ref = O.select_blocks(sc, cu, B, T, 1, 2)
    with ResultFiles() as f:
        r = oracle_service.select(seqlens, H, B, T, 1, 2, 31, f.save("sel", ref))
    assert r["tokens"] == 1000 and r["mismatch"] == 0
    bad = ref.copy()
    bad[1, 905, 2] = 7 - bad[1, 905, 2]  # a different block
    with ResultFiles() as f:
        r = oracle_service.select(seqlens, H, B, T, 1, 2, 31, f.save("sel", bad))
    assert r["mismatch"] == 1 and r["first_mismatch"]["head"] == 1 and r["first_mismatch"]["token"] == 905
