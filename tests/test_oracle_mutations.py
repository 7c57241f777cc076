"""Plant plausible mistakes in a copy of the oracle and check the pins see them.

Each mutation rewrites one expression of the oracle's source (a dropped term,
an off-by-one, a wrong sign, index or operand), loads the result as a separate
module on the CPU and swaps it in for the real oracle.  The fast pins of
test_oracle_index.py and test_oracle_attention.py then run against the mutant;
at least one must fail, otherwise the pins do not constrain that expression.
"""

import os
import types

import pytest

import oracle.fsa_oracle as O
import test_oracle_attention as A
import test_oracle_backward as BW
import test_oracle_index as I
import test_oracle_select as SEL

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fsa_oracle.py")
with open(SRC_PATH) as f:
    SRC = f.read()

MUTATIONS = [
    # attention: key set
    ("if 0 <= e <= own})", "if 0 <= e < own})"),
    ("min(seq_start + (e + 1) * block_size, seq_end, t + 1)", "min(seq_start + (e + 1) * block_size, seq_end, t)"),
    ("lo = seq_start + e * block_size", "lo = e * block_size"),
    ("sorted({int(e) for e in np.asarray(sel_row).tolist() if 0 <= e <= own})",
     "sorted([int(e) for e in np.asarray(sel_row).tolist() if 0 <= e <= own])"),
    # attention: arithmetic
    ("scores = scale * (qh @ kh.T)", "scores = (qh @ kh.T)"),
    ("qh = np.asarray(q[t, h * g : (h + 1) * g, :]", "qh = np.asarray(q[t, h : HQ : H, :]"),
    ("ls = m + np.log(l)", "ls = m + np.log2(l)"),
    ("p = np.exp(scores - ls[:, None])", "p = np.exp(scores - m[:, None])"),
    ("o[i, h * g : (h + 1) * g, :] = p @ vh", "o[i, h * g : (h + 1) * g, :] = p @ kh"),
    ("row_max[i, h * g : (h + 1) * g] = m", "row_max[i, h * g : (h + 1) * g] = ls"),
    ("l = np.exp(scores - m[:, None]).sum(axis=1)", "l = np.exp(m[:, None] - scores).sum(axis=1)"),
    # index
    ("in_range = (sel >= 0) & (sel <= own[None, :, None])", "in_range = (sel >= 0) & (sel < own[None, :, None])"),
    ("in_range = (sel >= 0) & (sel <= own[None, :, None])", "in_range = (sel > 0) & (sel <= own[None, :, None])"),
    ("first[:, :, j] &= sel[:, :, j] != sel[:, :, jj]", "first[:, :, j] &= True"),
    ("key = hh * NB + gb", "key = gb * H + hh"),
    ("gb = gboff[seq[tt]] + sel[hh, tt, jj]", "gb = sel[hh, tt, jj]"),
    ('order = np.argsort(key, kind="stable")', 'order = np.lexsort((-tt, key))'),
    ("offsets = np.concatenate([[0], np.cumsum(counts)])", "offsets = np.concatenate([np.cumsum(counts), [counts.sum()]])"),
    ("qidx = tt[order].astype(np.int64)", "qidx = tt.astype(np.int64)"),
]


def fast_pins():
    pins = [I.test_handworked_example, I.test_row_permutation_moves_slot_with_entry, I.test_shuffled_rows_same_lists]
    pins += [lambda s=s: I.test_against_brute_force(s) for s in range(6)]
    pins += [lambda s=s: I.test_invariants(s) for s in range(2)]
    pins += [lambda n=n: I.test_closed_form_pair_counts(n) for n in ("n1k_h1_g1_d64_t4_bf16", "n8k_h4_g2_d128_t16_bf16")]
    pins += [A.test_handworked_example, A.test_own_block_only_is_block_diagonal_causal, A.test_order_invariance_bitwise,
             A.test_duplicates_equal_deduplicated, A.test_zero_queries_give_key_mean, A.test_constant_values_and_first_token,
             A.test_identical_heads_identical_outputs_and_empty_rows]
    pins += [lambda s=s: A.test_dense_block_mask_equivalence(s) for s in range(5)]
    pins += [lambda s=s: A.test_full_selection_is_causal_attention(s) for s in range(3)]
    return pins


# backward: dropped term, wrong scale / operand / axis / head grouping,
# overwrite instead of accumulate
BWD_MUTATIONS = [
    ("ds = p * (dp - delta[:, None])", "ds = p * dp"),
    ("dq[i, h * g : (h + 1) * g, :] = scale * (ds @ kh)", "dq[i, h * g : (h + 1) * g, :] = ds @ kh"),
    ("dk[keys, h, :] += scale * (ds.T @ qh)", "dk[keys, h, :] += scale * (ds.T @ doh)"),
    ("dk[keys, h, :] += scale * (ds.T @ qh)", "dk[keys, h, :] = scale * (ds.T @ qh)"),
    ("dv[keys, h, :] += p.T @ doh", "dv[keys, h, :] += ds.T @ doh"),
    ("dp = doh @ vh.T", "dp = doh @ kh.T"),
    ("p /= p.sum(axis=1, keepdims=True)", "p /= p.sum(axis=0, keepdims=True)"),
    ("doh = np.asarray(dout[t, h * g : (h + 1) * g, :]", "doh = np.asarray(dout[t, h : HQ : H, :]"),
    ("delta = (doh * o).sum(axis=1)", "delta = (doh * vh[:1]).sum(axis=1)"),
]


# block selection: ranking direction, tie order, forced set, truncation, NaN
SEL_MUTATIONS = [
    ("order = sorted(free, key=lambda e: (-sc[e], e))", "order = sorted(free, key=lambda e: (sc[e], e))"),
    ("order = sorted(free, key=lambda e: (-sc[e], e))", "order = sorted(free, key=lambda e: (-sc[e], -e))"),
    ("[own - i for i in range(local_blocks)]", "[own - i - 1 for i in range(local_blocks)]"),
    ("if 0 <= e <= own and e not in forced:", "if 0 <= e <= own:"),
    ("forced = forced[:topk]", "forced = forced"),
    ("sc = np.where(np.isnan(sc), -np.inf, sc)", "sc = np.where(np.isnan(sc), np.inf, sc)"),
    ("own = (t - int(cu[s])) // block_size", "own = t // block_size"),
    ("free = [e for e in range(own + 1) if e not in forced]", "free = [e for e in range(own) if e not in forced]"),
]


def fast_pins_sel():
    return [SEL.test_handworked_example] + [lambda s=s: SEL.test_against_brute_force(s) for s in range(3)] + [
        lambda: SEL.test_invariants(0)]


def fast_pins_bwd():
    return [lambda: BW.test_finite_differences(0), lambda: BW.test_torch_autograd_dense_mask(0),
            BW.test_zero_output_gradient, BW.test_constant_values_give_no_score_gradient,
            BW.test_value_gradient_column_sums]


def load_mutant(old, new):
    # an expression shared by the forward and the backward is mutated in both
    assert SRC.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_unmutated_oracle_passes_fast_pins():
    for pin in fast_pins() + fast_pins_bwd() + fast_pins_sel():
        pin()


@pytest.mark.parametrize("old,new", MUTATIONS, ids=[f"m{i}" for i in range(len(MUTATIONS))])
def test_mutant_is_caught(old, new, monkeypatch):
    mut = load_mutant(old, new)
    for name in O.__all__:
        monkeypatch.setattr(O, name, getattr(mut, name))
    failures = 0
    for pin in fast_pins():
        try:
            pin()
        except Exception:  # an assertion, or a crash the mutant causes
            failures += 1
            break
    assert failures, f"no pin fails when {old!r} becomes {new!r}"


@pytest.mark.parametrize("old,new", BWD_MUTATIONS, ids=[f"b{i}" for i in range(len(BWD_MUTATIONS))])
def test_backward_mutant_is_caught(old, new, monkeypatch):
    mut = load_mutant(old, new)
    for name in O.__all__:
        monkeypatch.setattr(O, name, getattr(mut, name))
    failures = 0
    for pin in fast_pins_bwd():
        try:
            pin()
        except Exception:  # an assertion, or a crash the mutant causes
            failures += 1
            break
    assert failures, f"no backward pin fails when {old!r} becomes {new!r}"


@pytest.mark.parametrize("old,new", SEL_MUTATIONS, ids=[f"s{i}" for i in range(len(SEL_MUTATIONS))])
def test_selection_mutant_is_caught(old, new, monkeypatch):
    mut = load_mutant(old, new)
    for name in O.__all__:
        monkeypatch.setattr(O, name, getattr(mut, name))
    failures = 0
    for pin in fast_pins_sel():
        try:
            pin()
        except Exception:  # an assertion, or a crash the mutant causes
            failures += 1
            break
    assert failures, f"no selection pin fails when {old!r} becomes {new!r}"
