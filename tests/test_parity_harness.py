"""CPU checks of the parity harness itself (tests/parity.py): the near-tie
exemption accepts a selection only when it is a valid Top-K of the oracle's
fp64 scores, and compare() replays such rows instead of dropping them.

The "GPU" results here are built from the oracle on the CPU, with planted
differences, so the harness's accept and reject paths both run."""
import numpy as np
import pytest
import torch

from hierarchical_kv_pruning_amd import synth
from oracle import oracle
from tests import parity


def test_valid_topk_accepts_the_oracle_set_and_swaps_within_the_gap():
    cand = np.array([10, 11, 12, 13, 14])
    score = np.array([5.0, 4.0, 3.0, 3.0 * (1 - 1e-7), 1.0])
    assert parity.valid_topk(cand, score, 3, [10, 11, 12]) is None
    assert parity.valid_topk(cand, score, 3, [12, 11, 10]) is None          # order is free
    assert parity.valid_topk(cand, score, 3, [10, 11, 13]) is None          # 1e-7 from the K-th
    assert parity.valid_topk(cand, score, 9, [10, 11, 12, 13, 14]) is None  # K clamps to n
    assert parity.valid_topk(cand, score, 0, []) is None


@pytest.mark.parametrize("chosen", [[10, 11, 14], [10, 11], [10, 11, 12, 13], [10, 10, 11], [10, 11, 99]])
def test_valid_topk_rejects(chosen):
    cand = np.array([10, 11, 12, 13, 14])
    score = np.array([5.0, 4.0, 3.0, 3.0 * (1 - 1e-7), 1.0])
    assert parity.valid_topk(cand, score, 3, chosen) is not None


def test_valid_topk_gap_is_relative_to_the_kth_score():
    cand = np.array([0, 1, 2])
    score = np.array([2.0, -1.0, -1.0 * (1 + 2e-6)])
    assert parity.valid_topk(cand, score, 2, [0, 2]) is not None
    score = np.array([2.0, -1.0, -1.0 * (1 + 5e-7)])
    assert parity.valid_topk(cand, score, 2, [0, 2]) is None


def _case():
    return synth.make_case("harness", device="cpu", seed=3, ragged=False, dtype="f32", B=1, N=6, S_kv=8,
                           Hq=4, Hkv=2, d=64, M_R=6, M_I=36, M=360, K=(2, 3, 5))


def _fake_gpu(case, ora):
    R = case.rows
    return dict(out=ora["out"].copy(), sel=[ora[k].astype(np.int32).copy() for k in ("sel_R", "sel_I", "sel_L")],
                lse_kg=ora["lse_kg"].astype(np.float32), lse_seq=ora["lse_seq"].astype(np.float32))


def _ranked_leaves(case, P, row, sel_I):
    b, n, h = row
    cand = parity._children(case.mid_off.numpy(), sel_I)
    score = oracle.candidate_scores(P, b, n, h, parity.leaf_keys(case, h, cand))
    order = sorted(range(len(cand)), key=lambda i: (-score[i], cand[i]))
    return cand[order], score[order]


def _replay(case):
    def replay(rws, selI, selL):
        return parity.oracle_rows(case, rws, forced_sel_L=selL, sel_I=selI)
    return replay


def test_compare_accepts_a_tie_swap_and_replays_it():
    case = _case()
    rows = oracle.all_rows(case.B, case.N, case.Hq)
    P = parity.oracle_problem(case)
    ora0 = parity.oracle_rows(case, rows)
    i = 5
    K = case.K[2]
    ranked, _ = _ranked_leaves(case, P, rows[i], ora0["sel_I"][i])
    kth, nxt = int(ranked[K - 1]), int(ranked[K])
    g = (rows[i][2]) // (case.Hq // case.Hkv)
    # plant an exact tie at the row's leaf boundary: the (K+1)-th key becomes the K-th's copy
    case.leaf_k[g, nxt] = case.leaf_k[g, kth]
    P = parity.oracle_problem(case)
    ora = parity.oracle_rows(case, rows)
    assert ora["gap"][i][2] == 0.0
    lo, hi = min(kth, nxt), max(kth, nxt)
    assert lo in ora["sel_L"][i] and hi not in ora["sel_L"][i]
    gpu = _fake_gpu(case, ora)
    row = gpu["sel"][2][i]
    row[row == lo] = hi                       # the other member of the tie
    rep = parity.oracle_rows(case, rows[i:i + 1], forced_sel_L=gpu["sel"][2][i:i + 1].astype(np.int64),
                             sel_I=gpu["sel"][1][i:i + 1].astype(np.int64))
    gpu["out"][i] = rep["out"][0]
    gpu["lse_kg"][i] = rep["lse_kg"][0]
    res = parity.compare(case, rows, gpu, ora, replay=_replay(case), problem=P)
    assert res["exempt"] == 1
    # the replayed output is what is compared: the oracle's own output for
    # that row (other value row) is not what the GPU row holds
    assert not np.allclose(ora["out"][i], gpu["out"][i])


def test_compare_rejects_a_swap_across_a_real_gap():
    case = _case()
    rows = oracle.all_rows(case.B, case.N, case.Hq)
    P = parity.oracle_problem(case)
    ora = parity.oracle_rows(case, rows)
    i = 7
    K = case.K[2]
    ranked, score = _ranked_leaves(case, P, rows[i], ora["sel_I"][i])
    assert parity.rel_gap(score[K - 1], score[K + 1]) > 1e-3
    gpu = _fake_gpu(case, ora)
    row = gpu["sel"][2][i]
    row[row == int(ranked[K - 1])] = int(ranked[K + 1])
    with pytest.raises(AssertionError, match="not exempt"):
        parity.compare(case, rows, gpu, ora, replay=_replay(case), problem=P)


def test_compare_checks_levels_below_an_exempt_one():
    """An exempt mid-level swap is accepted only if the leaf selection under
    the GPU's mids is itself a valid Top-K: a leaf planted from outside them
    is rejected."""
    case = _case()
    rows = oracle.all_rows(case.B, case.N, case.Hq)
    ora = parity.oracle_rows(case, rows)
    gpu = _fake_gpu(case, ora)
    i = 3
    ora["gap"][i][1] = 0.0                     # pretend the mid boundary is a near tie
    P = parity.oracle_problem(case)
    # a mid selection the oracle would accept (its own), but a leaf that is not a child of it
    mids = set(int(x) for x in gpu["sel"][1][i] if x >= 0)
    mo = case.mid_off.numpy()
    alien = next(int(l) for m in range(case.M_I) if m not in mids for l in range(mo[m], mo[m + 1]))
    gpu["sel"][1][i][0], gpu["sel"][1][i][1] = gpu["sel"][1][i][1], gpu["sel"][1][i][0]
    first = parity.first_mismatch([gpu["sel"][lev][i] for lev in range(3)], ora, i)
    assert first == -1                         # a permutation is the same set
    gpu["sel"][2][i][0] = alien
    ora["gap"][i][2] = 0.0
    with pytest.raises(AssertionError, match="not a valid Top-K"):
        parity.compare(case, rows, gpu, ora, replay=_replay(case), problem=P)


def test_compare_checks_both_log_sum_exps():
    case = _case()
    rows = oracle.all_rows(case.B, case.N, case.Hq)
    ora = parity.oracle_rows(case, rows)
    gpu = _fake_gpu(case, ora)
    assert parity.compare(case, rows, gpu, ora)["exempt"] == 0
    gpu["lse_seq"][4] += 5e-5
    with pytest.raises(AssertionError, match="lse_seq"):
        parity.compare(case, rows, gpu, ora)
    gpu = _fake_gpu(case, ora)
    gpu["lse_kg"][2] += 5e-5
    with pytest.raises(AssertionError, match="lse_kg"):
        parity.compare(case, rows, gpu, ora)


def test_two_phase_oracle_over_chunks_equals_the_full_oracle():
    """The harness's chunked, concurrent two-phase run equals one full call."""
    case = synth.make_case("chunks", device="cpu", seed=4, ragged=True, dtype="bf16", B=2, N=40, S_kv=41,
                           Hq=8, Hkv=2, d=64, M_R=20, M_I=400, M=40000, K=(3, 4, 9))
    rows = oracle.all_rows(case.B, case.N, case.Hq)
    assert len(parity._row_chunks(case, len(rows), case.K)) > 1
    full = oracle.hikvp_rows(parity.oracle_problem(case), rows)
    two = parity.oracle_rows(case, rows, two_phase=True)
    for k in ("sel_R", "sel_I", "sel_L", "out", "lse_kg", "lse_seq", "gap"):
        assert np.array_equal(full[k], two[k]), k
