"""GPU parity of the shared-selection variant (one descent per KV group or per
sequence on the group's summed query) against the fp64 oracle, through the C
ABI.  Group selections are compared as sets (the same 1e-6 boundary-gap
exemption as the per-row path: an exempt group's selections must be valid
Top-Ks of the oracle's scores under the GPU's own parents, and its rows are
compared in replay mode with the GPU's leaves); outputs to the same bar: fp32 max-abs <= 1e-5, bf16 max-abs
<= 2e-2 x RMS and cosine >= 0.9999.

For bf16 inputs the bar is applied to an fp32 output (the API's other output
type), which carries the kernels' arithmetic alone: a bf16 output adds its own
rounding, up to 2^-9 of each value, which exceeds 2e-2 x RMS wherever a row's
output is above ~5x the RMS (rows dominated by one leaf).  The bf16 output is
then required to be exactly that fp32 output rounded to nearest even."""
import gc
import sys

import numpy as np
import pytest
import torch

from hierarchical_kv_pruning_amd import atlaskv, synth
from oracle import oracle
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KVG, SEQ = atlaskv.SHARE_KV_GROUP, atlaskv.SHARE_SEQUENCE


def say(msg):
    print(f"[gpu-shared] {msg}", flush=True)
    sys.stdout.flush()


def shared_run(case, share, K=None, out_dtype=None, with_seq=True, q_kg=None):
    K = tuple(case.K if K is None else K)
    seq_k = case.seq_k if with_seq else None
    seq_v = case.seq_v if with_seq else None
    tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, case.mid_off)
    ws = atlaskv.alloc_shared_workspace(tree, case.q, seq_k, K, share)
    ng = case.B * (case.N if share == KVG else 1) * case.Hkv
    out = torch.full(case.q.shape, float("nan"), dtype=out_dtype or case.q.dtype, device=DEV)
    sels = [torch.full((ng, k), -7, dtype=torch.int32, device=DEV) for k in K]
    lse_kg = torch.full((case.rows,), 7.0, dtype=torch.float32, device=DEV)
    atlaskv.shared_attend_ex(case.q, tree, seq_k, seq_v, K, share, out, workspace=ws, q_kg=q_kg,
                             sel_root=sels[0], sel_mid=sels[1], sel_leaf=sels[2], lse_kg=lse_kg)
    torch.cuda.synchronize()
    tree.close()
    return dict(out=out.float().reshape(case.rows, -1).cpu().numpy().astype(np.float64),
                sel=[s.cpu().numpy() for s in sels], lse_kg=lse_kg.cpu().numpy())


def bf16_rne(x):
    """fp32 values (held as fp64) rounded to bf16, nearest with ties to even."""
    u = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).view(torch.int32).to(torch.int64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & ~0xFFFF
    return u.to(torch.int32).view(torch.float32).numpy().astype(np.float64)


def group_of(case, rows, share):
    rows = np.asarray(rows)
    G = case.Hq // case.Hkv
    b, n, g = rows[:, 0], rows[:, 1], rows[:, 2] // G
    return (b * case.N + n) * case.Hkv + g if share == KVG else b * case.Hkv + g


def check(case, share, rows=None, **kw):
    rows = oracle.all_rows(case.B, case.N, case.Hq) if rows is None else rows
    okw = {k: v for k, v in kw.items() if k in ("K", "q_kg", "with_seq")}
    say(f"{case.name}: share={share} B={case.B} N={case.N} Hq={case.Hq} Hkv={case.Hkv} d={case.d} "
        f"tree={case.M_R}/{case.M_I}/{case.M} K={kw.get('K', case.K)} dtype={case.dtype} rows={len(rows)}")
    gkw = dict(kw)
    if case.dtype == "bf16" and "out_dtype" not in kw:
        gkw["out_dtype"] = torch.float32
    gpu = shared_run(case, share, **gkw)
    if case.dtype == "bf16" and "out_dtype" not in kw:
        b16 = shared_run(case, share, **kw)
        np.testing.assert_array_equal(b16["out"], bf16_rne(gpu["out"]))
        for a, b in zip(b16["sel"], gpu["sel"]):
            np.testing.assert_array_equal(a, b)
    P = parity.oracle_problem(case, **okw)
    ora = oracle.shared_rows(P, rows, share)
    grp = group_of(case, rows, share)
    exempt = []
    Pg = None
    for i, gi in enumerate(grp):
        g = [gpu["sel"][lev][gi] for lev in range(3)]
        lev = parity.first_mismatch(g, ora, i)
        if lev < 0:
            continue
        assert ora["gap"][i][lev] < parity.GAP_EXEMPT, (tuple(rows[i]), lev, ora["gap"][i][lev])
        if Pg is None:  # the descent's problem: the group queries as KG queries
            Pg = oracle.Problem(*P._args, scale=P._kw["scale"], q_kg=oracle.group_queries(P, share))
        parity.check_selection_chain(case, Pg, rows[i], g)
        exempt.append(i)
    out_o = ora["out"].copy()
    if exempt:  # replay: the oracle finishes those rows over the GPU's group leaves
        rr = np.asarray(rows)[exempt]
        G = case.Hq // case.Hkv
        lk, lv = P._args[3], P._args[4]
        off, idx, ks, vs = [0], [], [], []
        for (b, n, h), gi in zip(rr, grp[exempt]):
            leaves = [int(x) for x in gpu["sel"][2][gi] if x >= 0]
            idx += leaves
            ks.append(lk[h // G, leaves])
            vs.append(lv[h // G, leaves])
            off.append(off[-1] + len(leaves))
        rep = oracle.finish_rows(P, rr, off, idx, torch.cat(ks), torch.cat(vs),
                                 forced_sel_L=gpu["sel"][2][grp[exempt]].astype(np.int64))
        out_o[exempt] = rep["out"]
        rep_lse = rep["lse_kg"]
    ridx = parity.row_index(case, rows)
    g, o = gpu["out"][ridx], out_o
    err = float(np.abs(g - o).max(initial=0.0))
    rep = dict(rows=len(rows), exempt=len(exempt), max_abs=err)
    if case.dtype == "f32":
        assert err <= 1e-5, rep
    else:
        rms = float(np.sqrt(np.mean(o ** 2)))
        cos = float(np.sum(g * o) / (np.linalg.norm(g) * np.linalg.norm(o)))
        rep.update(rms=rms, cos=cos)
        assert err <= 2e-2 * rms, rep
        assert cos >= 0.9999, rep
    lk_o = ora["lse_kg"].copy()
    if exempt:
        lk_o[exempt] = rep_lse
    rep["lse_kg_err"] = parity.check_lse("lse_kg", gpu["lse_kg"][ridx], lk_o, parity.LSE_TOL[case.dtype])
    say(f"{case.name}: {rep}")
    return gpu, ora


def _small(seed, **kw):
    cfg = dict(dtype="bf16", B=2, N=9, S_kv=13, Hq=8, Hkv=2, d=128, M_R=37, M_I=411, M=5003, K=(5, 7, 19))
    cfg.update(kw)
    return synth.make_case("shared", device=DEV, seed=seed, ragged=True, **cfg)


@pytest.mark.parametrize("share", [KVG, SEQ])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_shared_ragged_dtypes_and_head_dims(share, dtype, d):
    check(_small(1, dtype=dtype, d=d), share)


@pytest.mark.parametrize("share", [KVG, SEQ])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_shared_filtered_leaf_stream(share, dtype, d):
    """Mids with at least four times K_L children (ragged spans of 15 to 728
    leaves): the group descent runs the filtered leaf stream; in bf16 with
    the summed query's residual pass and its rounding bound in the margin."""
    check(_small(31, dtype=dtype, d=d, M_I=40, M=6000), share)


@pytest.mark.parametrize("share", [KVG, SEQ])
@pytest.mark.parametrize("Hq,dtype,d", [(6, "bf16", 128), (12, "f32", 64), (16, "bf16", 64)])
def test_shared_group_sizes(share, Hq, dtype, d):
    """KV groups of 3, 6 and 8 query heads: the KG kernel takes a group's
    heads four at a time, so these cover a partial set of four, a full set
    plus a partial one, and two full sets."""
    check(_small(6, Hq=Hq, Hkv=2, dtype=dtype, d=d), share)


@pytest.mark.parametrize("share", [KVG, SEQ])
def test_shared_k_edges_and_no_sequence(share):
    case = _small(2, M=3001)
    check(case, share, K=(1, 1, 1))
    check(case, share, K=(37, 256, 256))
    check(case, share, with_seq=False)


def test_shared_separate_kg_query():
    case = _small(3)
    q_kg = torch.randn(case.q.shape, generator=torch.Generator(device=DEV).manual_seed(5),
                       device=DEV).to(case.q.dtype)
    check(case, KVG, q_kg=q_kg)


def test_shared_groups_of_one_select_like_the_per_row_path():
    """Hq == Hkv: each group is one row, so the shared descent selects exactly
    what the per-row path selects."""
    case = _small(4, Hq=2, Hkv=2)
    gpu, _ = check(case, KVG)
    per_row = parity.gpu_run(case)
    for lev in range(3):
        a = [sorted(x for x in r if x >= 0) for r in gpu["sel"][lev]]
        b = [sorted(x for x in r if x >= 0) for r in per_row["sel"][lev]]
        assert a == b, lev


def test_shared_m1e4_all_rows():
    case = synth.make_case("m1e4", device=DEV)
    check(case, KVG)
    check(case, SEQ)


@pytest.mark.parametrize("share", [KVG, SEQ])
def test_shared_m1e6_sampled_rows(share):
    case = synth.make_case("m1e6", device=DEV)
    check(case, share, rows=parity.sample_rows(case, 256, seed=8))
    del case
    gc.collect()
    torch.cuda.empty_cache()
