"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself:
the hand-worked 2x2x2 tree, the rectangular (KBLaM) attention formula at full
K, textbook causal attention when the KG half is empty, the level-size
definitions, brute-force top-K, and algebraic invariants of the merge.

Page cited: "AtlasKV: Augmenting LLMs with Billion-Scale Knowledge Graphs in
20GB VRAM" (digest of arXiv 2510.17934).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from hierarchical_kv_pruning_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        neg = x.startswith("-")
        v = math.log(float(x.lstrip("-")[2:]))
        return -v if neg else v
    return float(x)


def _small_case(seed, B=1, N=5, S=7, Hq=4, Hkv=2, d=8, MR=3, MI=7, M=23, K=(2, 2, 3), ragged=True):
    return synth.make_case("custom", seed=seed, ragged=ragged, dtype="f32", B=B, N=N, S_kv=S,
                           Hq=Hq, Hkv=Hkv, d=d, M_R=MR, M_I=MI, M=M, K=K)


def _problem(oracle, c, K=None, f64=True, drop_seq=False, **kw):
    cv = (lambda t: None if t is None else t.double()) if f64 else (lambda t: t)
    return oracle.Problem(cv(c.q), cv(c.root_k), cv(c.mid_k), cv(c.leaf_k), cv(c.leaf_v),
                          c.root_off, c.mid_off, None if drop_seq else cv(c.seq_k),
                          None if drop_seq else cv(c.seq_v), K if K is not None else c.K, **kw)


# ---------------------------------------------------------------------------
# hand-worked example (tests/golden/hand_2x2x2.json)
# ---------------------------------------------------------------------------

def _hand_problem(oracle, fx, K):
    d = fx["d"]

    def keys(xs):
        a = np.zeros((1, len(xs), d))
        a[0, :, 0] = [_num(x) for x in xs]
        return a

    q = np.zeros((1, 2, 1, d))
    q[0, :, 0, 0] = fx["q_x"]
    seq_k = np.zeros((1, 2, 1, d))
    seq_k[0, :, 0, 0] = [_num(x) for x in fx["seq_x"]]
    seq_v = np.array(fx["seq_v"], dtype=np.float64).reshape(1, 2, 1, d)
    leaf_v = np.array(fx["leaf_v"], dtype=np.float64).reshape(1, 8, d)
    return oracle.Problem(q, keys(fx["root_x"]), keys(fx["mid_x"]), keys(fx["leaf_x"]), leaf_v,
                          fx["root_off"], fx["mid_off"], seq_k, seq_v, K, scale=fx["scale"])


def test_hand_worked_tree(oracle_mod):
    fx = json.load(open(os.path.join(GOLDEN, "hand_2x2x2.json")))
    for case in fx["cases"]:
        P = _hand_problem(oracle_mod, fx, case["K"])
        o = oracle_mod.hikvp_rows(P, oracle_mod.all_rows(1, 2, 1))
        for i, exp in enumerate(case["rows"]):
            tol = 1e-12 if "sel_L" in exp else 5e-8
            for key in ("sel_R", "sel_I", "sel_L"):
                if key in exp:
                    assert o[key][i].tolist() == exp[key], (i, key)
            if "logit_L" in exp:
                np.testing.assert_allclose(o["logit_L"][i], [_num(x) for x in exp["logit_L"]], atol=1e-14)
            for key in ("lam_kg", "lam_seq"):
                if key in exp:
                    assert abs(o[key][i] - exp[key]) < 1e-11, (i, key)
            for key in ("o_kg", "o_seq", "out"):
                if key in exp:
                    np.testing.assert_allclose(o[key][i], exp[key], rtol=tol, atol=tol)


# ---------------------------------------------------------------------------
# full K == the rectangular (KBLaM) joint softmax over all M leaves
# ---------------------------------------------------------------------------

def _rectangular(q, leaf_k, leaf_v, seq_k, seq_v, scale, q_kg=None):
    """KBLaM中的矩形注意力: one softmax over every KB logit plus the causal
    sequence logits (bottom-right aligned when S_kv > N); numpy fp64.  The KB
    logits use q_kg when given (the KB query of the projection heads)."""
    B, N, Hq, d = q.shape
    Hkv = leaf_k.shape[0]
    S = 0 if seq_k is None else seq_k.shape[1]
    qk = q if q_kg is None else q_kg
    out = np.zeros((B, N, Hq, d))
    for b in range(B):
        for n in range(N):
            for h in range(Hq):
                g = h * Hkv // Hq
                kg = scale * (leaf_k[g] @ qk[b, n, h])
                vis = S - N + n + 1 if S else 0
                sq = scale * (seq_k[b, :vis, g] @ q[b, n, h]) if vis else np.zeros(0)
                allx = np.concatenate([kg, sq])
                w = np.exp(allx - allx.max())
                num = w[:len(kg)] @ leaf_v[g]
                if vis:
                    num = num + w[len(kg):] @ seq_v[b, :vis, g]
                out[b, n, h] = num / w.sum()
    return out


@pytest.mark.parametrize("seed", range(6))
def test_full_k_equals_rectangular_attention(oracle_mod, seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 4))
    N = int(rng.integers(1, 6))
    S = N + int(rng.integers(0, 4))
    MR = int(rng.integers(1, 5))
    MI = MR + int(rng.integers(0, 8))
    M = MI + int(rng.integers(0, 200))
    c = _small_case(seed, B=2, N=N, S=S, Hq=Hq, Hkv=Hkv, d=int(rng.integers(1, 9)), MR=MR, MI=MI, M=M)
    K = (MR, MI, M)  # at least every fanout sum: nothing is pruned
    P = _problem(oracle_mod, c, K)
    o = oracle_mod.hikvp_rows(P, oracle_mod.all_rows(c.B, c.N, c.Hq))
    ref = _rectangular(c.q.double().numpy(), c.leaf_k.double().numpy(), c.leaf_v.double().numpy(),
                       c.seq_k.double().numpy(), c.seq_v.double().numpy(), P.scale)
    np.testing.assert_allclose(o["out"], ref.reshape(-1, c.d), rtol=1e-12, atol=1e-12)
    # every leaf selected exactly once
    for r in range(o["sel_L"].shape[0]):
        assert sorted(o["sel_L"][r].tolist()) == list(range(M))


# ---------------------------------------------------------------------------
# unpruned equivalent attention (the flat KG softmax over every leaf)
# ---------------------------------------------------------------------------

def _random_shape(rng):
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 4))
    N = int(rng.integers(1, 6))
    S = N + int(rng.integers(0, 4))
    MR = int(rng.integers(1, 5))
    MI = MR + int(rng.integers(0, 8))
    M = MI + int(rng.integers(0, 300))
    return dict(B=2, N=N, S=S, Hq=Hq, Hkv=Hkv, d=int(rng.integers(1, 9)), MR=MR, MI=MI, M=M)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("use_qkg", [False, True])
def test_flat_equals_rectangular_attention(oracle_mod, seed, use_qkg):
    """The oracle's unpruned path against the rectangular formula written
    out in numpy, with and without a separate KB query."""
    rng = np.random.default_rng(100 + seed)
    c = _small_case(100 + seed, **_random_shape(rng))
    qkg = torch.randn(c.q.shape, generator=torch.Generator().manual_seed(seed)).double() if use_qkg else None
    P = _problem(oracle_mod, c, q_kg=qkg)
    o = oracle_mod.flat_rows(P, oracle_mod.all_rows(c.B, c.N, c.Hq))
    ref = _rectangular(c.q.double().numpy(), c.leaf_k.double().numpy(), c.leaf_v.double().numpy(),
                       c.seq_k.double().numpy(), c.seq_v.double().numpy(), P.scale,
                       None if qkg is None else qkg.numpy())
    np.testing.assert_allclose(o["out"], ref.reshape(-1, c.d), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o["lam_kg"] + o["lam_seq"], 1.0, rtol=0, atol=1e-15)
    merged = o["lam_kg"][:, None] * o["o_kg"] + o["lam_seq"][:, None] * o["o_seq"]
    np.testing.assert_allclose(merged, o["out"], rtol=1e-13, atol=1e-13)


def test_flat_equals_descent_at_full_k(oracle_mod):
    """With K at least every fanout sum nothing is pruned, so the descent's
    KG half (its own candidate order) equals the flat one."""
    c = _small_case(120, B=2, N=4, S=6, Hq=6, Hkv=2, d=7, MR=4, MI=13, M=157)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    a = oracle_mod.flat_rows(_problem(oracle_mod, c), rows)
    b = oracle_mod.hikvp_rows(_problem(oracle_mod, c, (c.M_R, c.M_I, c.M)), rows)
    for k in ("out", "o_kg", "lse_kg", "lse_seq", "lam_kg"):
        np.testing.assert_allclose(a[k], b[k], rtol=1e-12, atol=1e-12)
    # the flat call leaves the selection outputs untouched
    assert (a["sel_L"] == -1).all() and (a["sel_R"] == -1).all()


def test_flat_single_leaf_without_sequence_returns_its_value(oracle_mod):
    c = _small_case(121, N=3, S=3, MR=1, MI=1, M=1)
    o = oracle_mod.flat_rows(_problem(oracle_mod, c, drop_seq=True), oracle_mod.all_rows(c.B, c.N, c.Hq))
    G = c.Hq // c.Hkv
    for r, (b, n, h) in enumerate(oracle_mod.all_rows(c.B, c.N, c.Hq)):
        np.testing.assert_array_equal(o["out"][r], c.leaf_v[h // G, 0].double().numpy())
    assert (o["lam_kg"] == 1.0).all() and (o["lam_seq"] == 0.0).all()


def test_flat_logit_shift_by_value_shift(oracle_mod):
    """Adding a constant vector to every value (leaves and sequence) adds it
    to the output: the joint weights sum to one."""
    c = _small_case(122, M=60)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    o = oracle_mod.flat_rows(_problem(oracle_mod, c), rows)
    shift = torch.linspace(-2.0, 3.0, c.d, dtype=torch.float64)
    c2 = _small_case(122, M=60)
    c2.leaf_v = c2.leaf_v.double() + shift
    c2.seq_v = c2.seq_v.double() + shift
    o2 = oracle_mod.flat_rows(_problem(oracle_mod, c2), rows)
    np.testing.assert_allclose(o2["out"], o["out"] + shift.numpy(), rtol=1e-12, atol=1e-12)


def test_full_k_without_sequence(oracle_mod):
    c = _small_case(11, N=3, S=3)
    P = _problem(oracle_mod, c, (c.M_R, c.M_I, c.M), drop_seq=True)
    o = oracle_mod.hikvp_rows(P, oracle_mod.all_rows(c.B, c.N, c.Hq))
    ref = _rectangular(c.q.double().numpy(), c.leaf_k.double().numpy(), c.leaf_v.double().numpy(),
                       None, None, P.scale)
    np.testing.assert_allclose(o["out"], ref.reshape(-1, c.d), rtol=1e-12, atol=1e-12)
    assert np.all(o["lam_kg"] == 1.0) and np.all(o["lam_seq"] == 0.0)


# ---------------------------------------------------------------------------
# empty KG half == textbook causal self-attention (自注意力层机制)
# ---------------------------------------------------------------------------

def _causal_textbook(q, seq_k, seq_v, scale, b, n, h, N, Hq, Hkv):
    S = seq_k.shape[1]
    g = h * Hkv // Hq
    num = np.zeros(q.shape[-1])
    den = 0.0
    for i in range(S - N + n + 1):
        e = math.exp(scale * float(np.dot(q[b, n, h], seq_k[b, i, g])))
        num += e * seq_v[b, i, g]
        den += e
    return num / den


@pytest.mark.parametrize("K", [(2, 2, 0), (0, 3, 3), (3, 0, 5)])
def test_empty_kg_is_causal_attention(oracle_mod, K):
    c = _small_case(3, B=2, N=4, S=9)
    P = _problem(oracle_mod, c, K)
    o = oracle_mod.hikvp_rows(P, oracle_mod.all_rows(c.B, c.N, c.Hq))
    q, sk, sv = (t.double().numpy() for t in (c.q, c.seq_k, c.seq_v))
    for r, (b, n, h) in enumerate(oracle_mod.all_rows(c.B, c.N, c.Hq)):
        ref = _causal_textbook(q, sk, sv, P.scale, b, n, h, c.N, c.Hq, c.Hkv)
        np.testing.assert_allclose(o["out"][r], ref, rtol=1e-13, atol=1e-13)
    assert np.all(o["lam_kg"] == 0.0) and np.all(o["lse_kg"] == -np.inf)


def test_both_halves_empty_is_an_error(oracle_mod):
    c = _small_case(4)
    P = _problem(oracle_mod, c, (2, 2, 0), drop_seq=True)
    with pytest.raises(RuntimeError):
        oracle_mod.hikvp_rows(P, oracle_mod.all_rows(1, 1, 1))


# ---------------------------------------------------------------------------
# λ merge == joint softmax; λ weights sum to one
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny"])
def test_lambda_merge_identities(oracle_mod, name):
    c = synth.make_case(name)
    P = _problem(oracle_mod, c)
    o = oracle_mod.hikvp_rows(P, oracle_mod.all_rows(c.B, c.N, c.Hq))
    lam = o["lam_kg"][:, None]
    merged = lam * o["o_kg"] + o["lam_seq"][:, None] * o["o_seq"]
    np.testing.assert_allclose(merged, o["out"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o["lam_kg"] + o["lam_seq"], 1.0, rtol=0, atol=1e-15)
    sig = 1.0 / (1.0 + np.exp(o["lse_seq"] - o["lse_kg"]))
    np.testing.assert_allclose(o["lam_kg"], sig, rtol=1e-14, atol=1e-15)
    # both halves really contribute in this workload
    assert 0.05 < o["lam_kg"].min() and o["lam_kg"].max() < 0.999


def test_kg_half_is_softmax_over_selected_leaves(oracle_mod):
    c = _small_case(5)
    P = _problem(oracle_mod, c)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    o = oracle_mod.hikvp_rows(P, rows)
    lv = c.leaf_v.double().numpy()
    for r, (b, n, h) in enumerate(rows):
        g = h * c.Hkv // c.Hq
        sel = o["sel_L"][r][o["sel_L"][r] >= 0]
        lg = o["logit_L"][r][:len(sel)]
        w = np.exp(lg - lg.max())
        np.testing.assert_allclose(o["o_kg"][r], (w / w.sum()) @ lv[g, sel], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(o["lse_kg"][r], lg.max() + math.log(w.sum()), rtol=1e-14)


# ---------------------------------------------------------------------------
# descent and Top-K against brute force
# ---------------------------------------------------------------------------

def _brute_topk(score, idx, K):
    """Every selected element outranks every unselected one; count min(K, n)."""
    n = len(score)
    order = []
    remaining = list(range(n))
    for _ in range(min(K, n)):
        best = remaining[0]
        for j in remaining[1:]:
            if score[j] > score[best] or (score[j] == score[best] and idx[j] < idx[best]):
                best = j
        order.append(best)
        remaining.remove(best)
    return order


@pytest.mark.parametrize("seed", range(20))
def test_topk_brute_force_with_ties(oracle_mod, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 40))
    score = rng.choice([-1.5, -0.0, 0.0, 0.25, 0.25, 2.0, 3.0], size=n).astype(np.float64)
    idx = rng.permutation(1000)[:n].astype(np.int64)
    K = int(rng.integers(0, 45))
    got = oracle_mod.topk(score, idx, K).tolist()
    assert got == _brute_topk(score, idx, K)


def test_signed_zero_ties_break_by_index(oracle_mod):
    got = oracle_mod.topk(np.array([0.0, -0.0, 0.0]), np.array([5, 2, 9]), 2).tolist()
    assert got == [1, 0]


@pytest.mark.parametrize("seed,use_qkg", [(s, s % 2 == 1) for s in range(6)])
def test_descent_matches_level_by_level_brute_force(oracle_mod, seed, use_qkg):
    """The tree is scored with the KG query (q_kg when given, else q)."""
    c = _small_case(20 + seed, B=1, N=4, S=4, Hq=2, Hkv=1, d=6, MR=5, MI=17, M=120, K=(2, 3, 4))
    qkg = torch.randn(c.q.shape, generator=torch.Generator().manual_seed(seed), dtype=torch.float64)
    P = _problem(oracle_mod, c, q_kg=qkg if use_qkg else None)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    o = oracle_mod.hikvp_rows(P, rows)
    q = qkg.numpy() if use_qkg else c.q.double().numpy()
    rk, mk, lk = (t.double().numpy() for t in (c.root_k, c.mid_k, c.leaf_k))
    ro, mo = c.root_off.numpy(), c.mid_off.numpy()
    for r, (b, n, h) in enumerate(rows):
        g = h * c.Hkv // c.Hq
        qq = q[b, n, h]
        s = rk[g] @ qq
        selR = [int(j) for j in _brute_topk(s, np.arange(c.M_R), c.K[0])]
        assert o["sel_R"][r].tolist()[:len(selR)] == selR
        cand = np.concatenate([np.arange(ro[j], ro[j + 1]) for j in selR])
        s = mk[g, cand] @ qq
        selI = [int(cand[j]) for j in _brute_topk(s, cand, c.K[1])]
        assert o["sel_I"][r].tolist()[:len(selI)] == selI
        cand = np.concatenate([np.arange(mo[m], mo[m + 1]) for m in selI] + [np.zeros(0, np.int64)])
        s = lk[g, cand] @ qq
        selL = [int(cand[j]) for j in _brute_topk(s, cand, c.K[2])]
        assert o["sel_L"][r].tolist()[:len(selL)] == selL
        # complexity invariant: roots + children of chosen roots + children of chosen mids
        assert o["n_cand"][r].tolist() == [c.M_R, int(sum(ro[j + 1] - ro[j] for j in selR)),
                                           int(sum(mo[m + 1] - mo[m] for m in selI))]


def test_pruning_differs_from_flat_in_hand_example(oracle_mod):
    """The hand tree's token 0 loses leaf 4 (logit 5), which sits under the
    unselected root: pruned attention is not flat attention in general."""
    fx = json.load(open(os.path.join(GOLDEN, "hand_2x2x2.json")))
    P = _hand_problem(oracle_mod, fx, (1, 2, 2))
    o = oracle_mod.hikvp_rows(P, oracle_mod.all_rows(1, 2, 1))
    assert 4 not in o["sel_L"][0].tolist()


def test_gap_reporting(oracle_mod):
    fx = json.load(open(os.path.join(GOLDEN, "hand_2x2x2.json")))
    P = _hand_problem(oracle_mod, fx, (1, 2, 2))
    o = oracle_mod.hikvp_rows(P, oracle_mod.all_rows(1, 2, 1))
    # token 0: roots 1 vs 0.5 -> 0.5; mids: all selected -> inf; leaves ln2 vs 0 -> 1
    np.testing.assert_allclose(o["gap"][0], [0.5, np.inf, 1.0])


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_permuting_nodes_permutes_indices_only(oracle_mod):
    c = _small_case(31, N=3, S=4, MR=4, MI=11, M=60, K=(2, 2, 5))
    P = _problem(oracle_mod, c)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    o = oracle_mod.hikvp_rows(P, rows)
    rng = np.random.default_rng(0)
    ro, mo = c.root_off.numpy(), c.mid_off.numpy()
    # permute roots (and with them the order of their mid blocks), then leaves within mids
    rperm = rng.permutation(c.M_R)
    mid_order = np.concatenate([np.arange(ro[j], ro[j + 1]) for j in rperm])
    leaf_order = np.concatenate([rng.permutation(np.arange(mo[m], mo[m + 1])) for m in mid_order])
    new_ro = np.concatenate([[0], np.cumsum([ro[j + 1] - ro[j] for j in rperm])])
    new_mo = np.concatenate([[0], np.cumsum([mo[m + 1] - mo[m] for m in mid_order])])
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    P2 = oracle_mod.Problem(c.q.double(), t(c.root_k.double().numpy()[:, rperm]),
                            t(c.mid_k.double().numpy()[:, mid_order]),
                            t(c.leaf_k.double().numpy()[:, leaf_order]),
                            t(c.leaf_v.double().numpy()[:, leaf_order]), new_ro, new_mo,
                            c.seq_k.double(), c.seq_v.double(), c.K)
    o2 = oracle_mod.hikvp_rows(P2, rows)
    np.testing.assert_allclose(o2["out"], o["out"], rtol=1e-13, atol=1e-13)
    for r in range(len(rows)):
        mapped = {int(leaf_order[i]) for i in o2["sel_L"][r] if i >= 0}
        assert mapped == {int(i) for i in o["sel_L"][r] if i >= 0}


def test_values_shift_and_scale(oracle_mod):
    c = _small_case(41)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    o = oracle_mod.hikvp_rows(_problem(oracle_mod, c), rows)
    shift = torch.linspace(-3, 3, c.d, dtype=torch.float64)
    P2 = oracle_mod.Problem(c.q.double(), c.root_k.double(), c.mid_k.double(), c.leaf_k.double(),
                            2.0 * c.leaf_v.double() + shift, c.root_off, c.mid_off,
                            c.seq_k.double(), 2.0 * c.seq_v.double() + shift, c.K)
    o2 = oracle_mod.hikvp_rows(P2, rows)
    np.testing.assert_allclose(o2["out"], 2.0 * o["out"] + shift.numpy(), rtol=1e-12, atol=1e-12)


def test_single_candidate_gets_weight_one(oracle_mod):
    c = _small_case(51, N=2, S=2, MR=1, MI=1, M=1, K=(4, 4, 4), ragged=False)
    P = _problem(oracle_mod, c, drop_seq=True)
    o = oracle_mod.hikvp_rows(P, oracle_mod.all_rows(c.B, c.N, c.Hq))
    for r in range(o["out"].shape[0]):
        g = (r % c.Hq) * c.Hkv // c.Hq
        np.testing.assert_array_equal(o["out"][r], c.leaf_v.double().numpy()[g, 0])
        assert o["sel_L"][r].tolist() == [0, -1, -1, -1]


def test_bf16_storage_reads_exactly(oracle_mod):
    c = synth.make_case("tiny", dtype="bf16")
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    o_bf = oracle_mod.hikvp_rows(_problem(oracle_mod, c, f64=False), rows)
    o_64 = oracle_mod.hikvp_rows(_problem(oracle_mod, c, f64=True), rows)
    for k in ("sel_L", "out", "lse_kg", "lse_seq"):
        np.testing.assert_array_equal(o_bf[k], o_64[k])


def test_q_kg_scores_the_tree(oracle_mod):
    """A separate KG query changes the selection and KG logits, not the
    sequence half."""
    c = _small_case(61)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    qkg = -c.q.double()
    o = oracle_mod.hikvp_rows(_problem(oracle_mod, c), rows)
    o2 = oracle_mod.hikvp_rows(_problem(oracle_mod, c, q_kg=qkg), rows)
    np.testing.assert_array_equal(o["lse_seq"], o2["lse_seq"])
    # with q_kg = -q the best root becomes the worst one
    ro = oracle_mod.level_scores(_problem(oracle_mod, c), 0, 0, 0, 0)[1]
    assert o2["sel_R"][0][0] == int(np.argmin(ro))


# ---------------------------------------------------------------------------
# level sizes (方法细节 › KGKVs的层次化聚类)
# ---------------------------------------------------------------------------

SIZE_TABLE = {1_000: (10, 100, 10), 10_000: (22, 465, 22), 1_000_000: (100, 10_000, 100),
              10_000_000: (216, 46_416, 216), 100_000_000: (465, 215_444, 465),
              1_000_000_000: (1000, 1_000_000, 1000)}


@pytest.mark.parametrize("M", sorted(SIZE_TABLE))
def test_tree_sizes_table(oracle_mod, M):
    assert oracle_mod.tree_sizes(M) == SIZE_TABLE[M]


@pytest.mark.parametrize("M", [1, 2, 7, 8, 9, 26, 27, 28, 999, 1001, 12345, 999_999, 10**12 + 3])
def test_tree_sizes_are_the_defining_ceilings(oracle_mod, M):
    S, MI, MR = oracle_mod.tree_sizes(M)
    assert S ** 3 >= M > (S - 1) ** 3                       # S = ceil(M^(1/3))
    assert MI ** 3 >= M ** 2 > (MI - 1) ** 3                # M_I = ceil(M^(2/3))
    assert MR ** 3 * M >= MI ** 3 > (MR - 1) ** 3 * M       # M_R = ceil(M_I * M^(-1/3))
    x = M ** (2.0 / 3.0)
    if abs(x - round(x)) > 1e-6:
        assert MI == math.ceil(x)


def test_configs_follow_the_level_sizes(oracle_mod):
    for name, cfg in synth.CONFIGS.items():
        S, MI, MR = oracle_mod.tree_sizes(cfg["M"])
        assert (cfg["M_R"], cfg["M_I"]) == (MR, MI), name


# ---------------------------------------------------------------------------
# two-phase and replay modes agree with the full mode
# ---------------------------------------------------------------------------

def _gather_candidates(c, rows, selI):
    mo = c.mid_off.numpy()
    lk, lv = c.leaf_k.double().numpy(), c.leaf_v.double().numpy()
    off, idx, ks, vs = [0], [], [], []
    for r, (b, n, h) in enumerate(rows):
        g = h * c.Hkv // c.Hq
        cand = [lf for m in selI[r] if m >= 0 for lf in range(mo[m], mo[m + 1])]
        idx += cand
        ks.append(lk[g, cand].reshape(-1, c.d))
        vs.append(lv[g, cand].reshape(-1, c.d))
        off.append(off[-1] + len(cand))
    return np.array(off), np.array(idx, np.int64), np.concatenate(ks), np.concatenate(vs)


def test_two_phase_equals_full(oracle_mod):
    c = _small_case(71, B=2, N=3, S=5)
    P = _problem(oracle_mod, c)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)[::2]
    full = oracle_mod.hikvp_rows(P, rows)
    ph1 = oracle_mod.select_mids_rows(P, rows)
    np.testing.assert_array_equal(ph1["sel_I"], full["sel_I"])
    off, idx, ks, vs = _gather_candidates(c, rows, ph1["sel_I"])
    ph2 = oracle_mod.finish_rows(P, rows, off, idx, ks, vs)
    for k in ("sel_L", "out", "lam_kg", "gap"):
        np.testing.assert_array_equal(ph2[k][:, -1] if k == "gap" else ph2[k],
                                      full[k][:, -1] if k == "gap" else full[k])


def test_replay_with_forced_selection(oracle_mod):
    c = _small_case(81, N=3, S=5)
    P = _problem(oracle_mod, c)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    full = oracle_mod.hikvp_rows(P, rows)
    off, idx, ks, vs = _gather_candidates(c, rows, full["sel_I"])
    same = oracle_mod.finish_rows(P, rows, off, idx, ks, vs, forced_sel_L=full["sel_L"])
    np.testing.assert_array_equal(same["out"], full["out"])
    # forcing the worst candidates instead changes the result to their softmax
    forced = np.full_like(full["sel_L"], -1)
    for r in range(len(rows)):
        cand = idx[off[r]:off[r + 1]]
        forced[r, 0] = cand[-1]
    alt = oracle_mod.finish_rows(P, rows, off, idx, ks, vs, forced_sel_L=forced)
    np.testing.assert_allclose(alt["o_kg"], c.leaf_v.double().numpy()[
        [h * c.Hkv // c.Hq for (_, _, h) in rows], forced[:, 0]], rtol=0, atol=0)


# ---------------------------------------------------------------------------
# shared selections (one descent per KV group or per sequence)
# ---------------------------------------------------------------------------

def test_shared_kv_group_of_one_is_per_row(oracle_mod):
    """Hq == Hkv: a KV group is one row, its summed query is the row's own,
    so the shared variant equals the per-row descent."""
    c = _small_case(130, B=2, N=4, S=6, Hq=3, Hkv=3, d=8, MR=4, MI=15, M=90, K=(2, 3, 5))
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    a = oracle_mod.shared_rows(_problem(oracle_mod, c, f64=False), rows, oracle_mod.SHARE_KV_GROUP)
    b = oracle_mod.hikvp_rows(_problem(oracle_mod, c, f64=False), rows)
    for k in ("sel_R", "sel_I", "sel_L", "out", "lse_kg", "lse_seq"):
        np.testing.assert_array_equal(a[k], b[k])


def test_shared_sequence_with_one_token_is_kv_group(oracle_mod):
    c = _small_case(131, B=3, N=1, S=5, Hq=4, Hkv=2, d=8, MR=4, MI=15, M=90, K=(2, 3, 5))
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    P = _problem(oracle_mod, c, f64=False)
    a = oracle_mod.shared_rows(P, rows, oracle_mod.SHARE_SEQUENCE)
    b = oracle_mod.shared_rows(P, rows, oracle_mod.SHARE_KV_GROUP)
    for k in ("sel_L", "out"):
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("share", [1, 2])
def test_shared_selection_is_top_k_of_summed_logits(oracle_mod, share):
    """fp64 storage (the group query needs no rounding): every level's shared
    selection is the brute-force Top-K of the members' summed logits, and each
    row's output is its own softmax over the group's leaves plus its causal
    sequence half, written out in numpy."""
    c = _small_case(132, B=2, N=3, S=4, Hq=4, Hkv=2, d=6, MR=5, MI=17, M=120, K=(2, 3, 4))
    P = _problem(oracle_mod, c)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    o = oracle_mod.shared_rows(P, rows, share)
    q = c.q.double().numpy()
    G = c.Hq // c.Hkv
    ro, mo = c.root_off.numpy(), c.mid_off.numpy()
    keys = [c.root_k.double().numpy(), c.mid_k.double().numpy(), c.leaf_k.double().numpy()]
    for i, (b, n, h) in enumerate(rows):
        g = h // G
        toks = [n] if share == 1 else list(range(c.N))
        members = [(b, t, hh) for t in toks for hh in range(g * G, (g + 1) * G)]
        parents = None
        for lev, (key, Kl) in enumerate(zip(("sel_R", "sel_I", "sel_L"), c.K)):
            if lev == 0:
                cand = np.arange(c.M_R)
            else:
                off = ro if lev == 1 else mo
                cand = np.concatenate([np.arange(off[p], off[p + 1]) for p in parents])
            score = np.zeros(len(cand))
            for (mb, mn, mh) in members:        # sum of the members' fp64 logits
                score += P.scale * (keys[lev][g, cand] @ q[mb, mn, mh])
            order = sorted(range(len(cand)), key=lambda j: (-score[j], cand[j]))
            want = sorted(cand[j] for j in order[:Kl])
            assert sorted(x for x in o[key][i] if x >= 0) == want, (i, key)
            parents = want
        # the row's own softmax over the group's leaves and its causal half
        lv = c.leaf_v.double().numpy()[g, parents]
        kg = P.scale * (keys[2][g, parents] @ q[b, n, h])
        vis = c.S_kv - c.N + n + 1
        sq = P.scale * (c.seq_k.double().numpy()[b, :vis, g] @ q[b, n, h])
        allx = np.concatenate([kg, sq])
        w = np.exp(allx - allx.max())
        ref = (w[:len(kg)] @ lv + w[len(kg):] @ c.seq_v.double().numpy()[b, :vis, g]) / w.sum()
        np.testing.assert_allclose(o["out"][i], ref, rtol=1e-12, atol=1e-12)


def test_shared_group_query_is_the_exact_member_sum(oracle_mod):
    """bf16 storage: the group query is the members' sum itself (fp64, not
    rounded to bf16); two bf16 values always add exactly in fp64."""
    c = synth.make_case("custom", seed=133, ragged=True, dtype="bf16", B=1, N=3, S_kv=3, Hq=4,
                        Hkv=2, d=8, M_R=3, M_I=7, M=23, K=(2, 2, 3))
    P = _problem(oracle_mod, c, f64=False)
    gq = oracle_mod.group_queries(P, oracle_mod.SHARE_KV_GROUP)
    assert gq.dtype == torch.float64
    q = c.q.double().numpy()
    want = q.reshape(1, 3, 2, 2, 8).sum(axis=3)
    for b, n, h in oracle_mod.all_rows(1, 3, 4):
        np.testing.assert_array_equal(gq.numpy()[b, n, h], want[b, n, h // 2])


@pytest.mark.parametrize("share", [1, 2])
def test_shared_bf16_selection_is_top_k_of_summed_logits(oracle_mod, share):
    """bf16 storage: each level's shared selection is the brute-force Top-K
    of the sum of the members' fp64 logits (the sum of G logits, each a
    sequential fp64 dot product of stored values), with no rounding of the
    group query in between.  (At these seeds, rounding the group query to
    bf16 first changes the selected leaf set of some rows.)"""
    c = synth.make_case("custom", seed={1: 140, 2: 149}[share], ragged=True, dtype="bf16", B=2, N=3, S_kv=4, Hq=8,
                        Hkv=2, d=32, M_R=7, M_I=40, M=400, K=(3, 5, 8))
    P = _problem(oracle_mod, c, f64=False)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    o = oracle_mod.shared_rows(P, rows, share)
    q = c.q.double().numpy()
    G = c.Hq // c.Hkv
    ro, mo = c.root_off.numpy(), c.mid_off.numpy()
    keys = [c.root_k.double().numpy(), c.mid_k.double().numpy(), c.leaf_k.double().numpy()]
    for i, (b, n, h) in enumerate(rows):
        g = h // G
        toks = [n] if share == 1 else list(range(c.N))
        members = [(b, t, hh) for t in toks for hh in range(g * G, (g + 1) * G)]
        parents = None
        for lev, (key, Kl) in enumerate(zip(("sel_R", "sel_I", "sel_L"), c.K)):
            if lev == 0:
                cand = np.arange(c.M_R)
            else:
                off = ro if lev == 1 else mo
                cand = np.concatenate([np.arange(off[p], off[p + 1]) for p in parents])
            score = np.zeros(len(cand))
            for (mb, mn, mh) in members:
                score += keys[lev][g, cand] @ q[mb, mn, mh]
            order = sorted(range(len(cand)), key=lambda j: (-score[j], cand[j]))
            if len(cand) > Kl:   # a near-tie at the boundary could flip on fp64 rounding
                s0, s1 = score[order[Kl - 1]], score[order[Kl]]
                assert abs(s0 - s1) > 1e-9 * max(abs(s0), abs(s1)), (i, key)
            want = sorted(cand[j] for j in order[:Kl])
            assert sorted(x for x in o[key][i] if x >= 0) == want, (i, key)
            parents = want


# ---------------------------------------------------------------------------
# folded projections (one base-embedding tree for every head)
# ---------------------------------------------------------------------------

def _base_tree(seed, DE, MR, MI, M, dtype=torch.float64):
    c = synth.make_case("custom", seed=seed, ragged=True, dtype="f32", B=1, N=1, S_kv=1, Hq=1, Hkv=1,
                        d=DE, M_R=MR, M_I=MI, M=M, K=(1, 1, 1))
    return (c.root_k.to(dtype), c.mid_k.to(dtype), c.leaf_k.to(dtype), c.leaf_v.to(dtype),
            c.root_off, c.mid_off)


def test_folded_with_identity_projections_is_the_per_row_path(oracle_mod):
    """One KV head, W_K = W_V = I (D_E = d): folding changes nothing, so the
    result is the per-row descent over the base tree itself."""
    d = 8
    tree = _base_tree(140, d, 4, 15, 90)
    c = _small_case(140, B=2, N=3, S=5, Hq=3, Hkv=1, d=d, MR=4, MI=15, M=90)
    q, sk, sv = c.q.double(), c.seq_k.double(), c.seq_v.double()
    eye = torch.eye(d, dtype=torch.float64)[None]
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    K = (2, 3, 5)
    a = oracle_mod.folded_rows(tree, q, eye, eye, sk, sv, K, rows)
    b = oracle_mod.hikvp_rows(oracle_mod.Problem(q, *tree[:4], tree[4], tree[5], sk, sv, K), rows)
    for k in ("sel_R", "sel_I", "sel_L"):
        np.testing.assert_array_equal(a[k], b[k])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_folded_equals_projected_per_head_trees(oracle_mod, seed):
    """fp64 storage: scoring the base tree with W_K^T q equals scoring the
    per-head projected tree W_K k with q, and W_V applied after the weighted
    sum equals weighting the projected values W_V v: the folded variant must
    equal the per-row descent over explicitly projected per-head trees."""
    rng = np.random.default_rng(seed)
    d, DE, Hkv, Hq = 6, 9, 2, 4
    tree = _base_tree(150 + seed, DE, 4, 13, 110)
    c = _small_case(150 + seed, B=2, N=3, S=4, Hq=Hq, Hkv=Hkv, d=d, MR=4, MI=13, M=110)
    q, sk, sv = c.q.double(), c.seq_k.double(), c.seq_v.double()
    wk = torch.from_numpy(rng.standard_normal((Hkv, d, DE)) / 3.0)
    wv = torch.from_numpy(rng.standard_normal((Hkv, d, DE)) / 3.0)
    proj = lambda t, w: torch.stack([t[0] @ w[g].T for g in range(Hkv)])   # [Hkv, M_x, d]
    rk, mk, lk, lv, ro, mo = tree
    K = (2, 4, 6)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    a = oracle_mod.folded_rows(tree, q, wk, wv, sk, sv, K, rows)
    b = oracle_mod.hikvp_rows(oracle_mod.Problem(q, proj(rk, wk), proj(mk, wk), proj(lk, wk), proj(lv, wv),
                                                 ro, mo, sk, sv, K), rows)
    for k in ("sel_R", "sel_I", "sel_L"):
        np.testing.assert_array_equal(a[k], b[k])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["lse_kg"], b["lse_kg"], rtol=1e-12, atol=1e-12)


def test_folded_query_is_the_exact_product_sum(oracle_mod):
    """bf16 inputs: q' = W_K^T q_kg is formed exactly (products of two bf16
    values are exact in fp64, and so is their sum here) and not rounded."""
    rng = np.random.default_rng(7)
    q = torch.from_numpy(rng.standard_normal((1, 2, 2, 8))).to(torch.bfloat16)
    wk = torch.from_numpy(rng.standard_normal((1, 8, 5))).to(torch.bfloat16)
    got = oracle_mod.folded_query(q, wk)
    assert got.dtype == torch.float64
    exact = np.einsum("bnht,td->bnhd", q.double().numpy(), wk.double().numpy()[0])
    np.testing.assert_array_equal(got.numpy(), exact)


@pytest.mark.parametrize("seed", range(2))
def test_folded_bf16_equals_projected_per_head_trees(oracle_mod, seed):
    """bf16 storage of the base tree, W_K, W_V and the queries: the folded
    variant (the base tree ranked by <W_K^T q, k> with the exact folded
    query) selects and outputs what the per-row descent selects over the
    per-head trees projected in fp64 (W_K k, W_V v) with the stored q, since
    both score the same exact sum of products."""
    rng = np.random.default_rng(10 + seed)
    d, DE, Hkv, Hq = 8, 24, 2, 4
    tree = _base_tree(160 + seed, DE, 5, 17, 140, dtype=torch.bfloat16)
    c = _small_case(160 + seed, B=2, N=3, S=4, Hq=Hq, Hkv=Hkv, d=d, MR=5, MI=17, M=140)
    bf = lambda x: x.to(torch.bfloat16)
    q, sk, sv = bf(c.q), bf(c.seq_k), bf(c.seq_v)
    wk = bf(torch.from_numpy(rng.standard_normal((Hkv, d, DE)) / 3.0))
    wv = bf(torch.from_numpy(rng.standard_normal((Hkv, d, DE)) / 3.0))
    proj = lambda t, w: torch.stack([t[0].double() @ w[g].double().T for g in range(Hkv)])
    rk, mk, lk, lv, ro, mo = tree
    K = (2, 4, 6)
    rows = oracle_mod.all_rows(c.B, c.N, c.Hq)
    a = oracle_mod.folded_rows(tree, q, wk, wv, sk, sv, K, rows)
    b = oracle_mod.hikvp_rows(oracle_mod.Problem(q.double(), proj(rk, wk), proj(mk, wk), proj(lk, wk),
                                                 proj(lv, wv), ro, mo, sk.double(), sv.double(), K), rows)
    assert np.all(b["gap"] > 1e-9)          # no boundary that fp64 rounding could flip
    for k in ("sel_R", "sel_I", "sel_L"):
        np.testing.assert_array_equal(a[k], b[k])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["lse_kg"], b["lse_kg"], rtol=1e-12, atol=1e-12)
