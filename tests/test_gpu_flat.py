"""GPU parity of the unpruned equivalent attention (every leaf in the KG
softmax) against the fp64 oracle's flat path, through the C ABI.

Acceptance as for the pruned path: fp32 inputs max-abs <= 1e-5; bf16 inputs
max-abs <= 2e-2 x the oracle output RMS and cosine >= 0.9999; log-sum-exp of
the KG half within 1e-3 (bf16 matrix-core operands) of the oracle's.  For bf16
inputs the bar is applied to an fp32 output, which carries the kernels'
arithmetic alone (a bf16 output's own rounding, 2^-9 of each value, exceeds
2e-2 x RMS wherever an output is above ~5x the RMS); the bf16 output must
then be exactly that fp32 output rounded to nearest even."""
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


def say(msg):
    print(f"[gpu-flat] {msg}", flush=True)
    sys.stdout.flush()


def _release():
    gc.collect()
    torch.cuda.empty_cache()


def flat_run(case, q=None, q_kg=None, scale=None, out_dtype=None, with_seq=True, tree=None):
    q = case.q if q is None else q
    seq_k = case.seq_k if with_seq else None
    seq_v = case.seq_v if with_seq else None
    own = tree is None
    if own:
        tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off,
                                case.mid_off)
    ws = atlaskv.alloc_flat_workspace(tree, q, seq_k)
    R = q.shape[0] * q.shape[1] * q.shape[2]
    out = torch.full(q.shape, float("nan"), dtype=out_dtype or q.dtype, device=DEV)
    lse_kg = torch.full((R,), 7.0, dtype=torch.float32, device=DEV)
    lse_seq = torch.full((R,), 7.0, dtype=torch.float32, device=DEV)
    atlaskv.flat_attend_ex(q, tree, seq_k, seq_v, out, q_kg=q_kg, scale=scale, workspace=ws,
                           lse_kg=lse_kg, lse_seq=lse_seq)
    torch.cuda.synchronize()
    if own:
        tree.close()
    return dict(out=out.float().reshape(R, -1).cpu().numpy().astype(np.float64),
                lse_kg=lse_kg.cpu().numpy(), lse_seq=lse_seq.cpu().numpy())


def _bf16_rne(x):
    u = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).view(torch.int32).to(torch.int64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & ~0xFFFF
    return u.to(torch.int32).view(torch.float32).numpy().astype(np.float64)


def check(case, rows=None, fp32_tol=1e-5, **kw):
    rows = oracle.all_rows(case.B, case.N, case.Hq) if rows is None else rows
    gkw = {k: v for k, v in kw.items() if k in ("q", "q_kg", "scale", "with_seq", "out_dtype")}
    okw = {k: v for k, v in kw.items() if k in ("q", "q_kg", "scale", "with_seq")}
    say(f"{case.name}: flat B={case.B} N={case.N} S={case.S_kv} Hq={case.Hq} Hkv={case.Hkv} d={case.d} "
        f"M={case.M} dtype={case.dtype} rows={len(rows)}")
    bf16_out = case.dtype == "bf16" and "out_dtype" not in kw
    if bf16_out:
        gkw["out_dtype"] = torch.float32
    gpu = flat_run(case, **gkw)
    if bf16_out:
        b16 = flat_run(case, **{k: v for k, v in gkw.items() if k != "out_dtype"})
        np.testing.assert_array_equal(b16["out"], _bf16_rne(gpu["out"]))
    ora = oracle.flat_rows(parity.oracle_problem(case, **okw), rows)
    ridx = parity.row_index(case, rows)
    g, o = gpu["out"][ridx], ora["out"]
    err = float(np.abs(g - o).max(initial=0.0))
    rep = dict(rows=len(rows), max_abs=err)
    if case.dtype == "f32":
        assert err <= fp32_tol, rep
    else:
        rms = float(np.sqrt(np.mean(o ** 2)))
        cos = float(np.sum(g * o) / (np.linalg.norm(g) * np.linalg.norm(o)))
        rep.update(rms=rms, cos=cos)
        assert err <= 2e-2 * rms, rep
        assert cos >= 0.9999, rep
    for key in ("lse_kg", "lse_seq"):
        ref = ora[key]
        fin = np.isfinite(ref)
        assert np.array_equal(np.isfinite(gpu[key][ridx]), fin), key
        if fin.any():
            d = float(np.max(np.abs(gpu[key][ridx][fin] - ref[fin])))
            rep[key] = d
            assert d <= 1e-3 + 1e-5 * float(np.abs(ref[fin]).max()), (key, rep)
    say(f"{case.name}: {rep}")
    return gpu, ora, rep


def _small(seed, **kw):
    cfg = dict(dtype="bf16", B=2, N=33, S_kv=45, Hq=8, Hkv=2, d=128, M_R=37, M_I=411, M=5003,
               K=(5, 7, 19))
    cfg.update(kw)
    return synth.make_case("flat", device=DEV, seed=seed, ragged=True, **cfg)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_flat_ragged_dtypes_and_head_dims(dtype, d):
    """M = 5003 (a ragged last key block), 2*33*4 = 264 rows per KV head (a
    ragged last row tile)."""
    check(_small(1, dtype=dtype, d=d))


def test_flat_tiny_all_rows():
    check(synth.make_case("tiny", device=DEV))


def test_flat_single_kv_head_many_groups():
    """Hkv = 1: the split count is rounded to a multiple of the 8 XCDs."""
    check(_small(2, Hq=6, Hkv=1, M=20011))


def test_flat_no_sequence_half():
    check(_small(3, M=777), with_seq=False)


def test_flat_separate_kg_query_scale_and_fp32_output():
    case = _small(4, M=3001)
    q_kg = torch.randn(case.q.shape, generator=torch.Generator(device=DEV).manual_seed(9),
                       device=DEV).to(case.q.dtype)
    check(case, q_kg=q_kg, scale=0.05, out_dtype=torch.float32)


def test_flat_strided_query():
    case = _small(5, M=2500)
    big = torch.zeros(case.B, case.N, case.Hq, 2 * case.d, dtype=case.q.dtype, device=DEV)
    big[..., :case.d] = case.q
    check(case, q=big[..., :case.d])


@pytest.mark.parametrize("M", [1, 40, 63, 64, 65])
def test_flat_fewer_keys_than_one_block(M):
    """Fewer leaves than one 64-key block, and the block edge.  With so few
    leaves one leaf can dominate a row, so single outputs reach ~10x the output
    RMS and a bf16 output's own rounding (2^-9 of the value) can exceed
    2e-2 x RMS: the arithmetic is checked on an fp32 output, and the bf16
    output must be exactly that fp32 result rounded to nearest even."""
    check(_small(6 + M, M_R=1, M_I=1, M=M))


def test_flat_equals_pruned_path_at_full_k():
    """With K at least every fanout sum nothing is pruned: the flat kernels and
    the descent agree (both against the oracle, and with each other)."""
    case = _small(8, B=1, N=20, S_kv=24, Hq=4, Hkv=2, M_R=4, M_I=16, M=200)
    K = (case.M_R, case.M_I, case.M)  # every node of every level
    flat = flat_run(case)
    pr = parity.gpu_run(case, K=K)
    rms = float(np.sqrt(np.mean(flat["out"] ** 2)))
    assert float(np.abs(flat["out"] - pr["out"]).max()) <= 2e-2 * rms
    np.testing.assert_allclose(flat["lse_kg"], pr["lse_kg"], rtol=0, atol=2e-3)


def test_flat_deterministic_reruns():
    case = _small(10, M=9000)
    a = flat_run(case)
    b = flat_run(case)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse_kg"], b["lse_kg"])


def test_flat_m1e4_sampled_rows():
    case = synth.make_case("m1e4", device=DEV)
    check(case, rows=parity.sample_rows(case, 256, seed=5))


def test_flat_m1e6_sampled_rows():
    case = synth.make_case("m1e6", device=DEV)
    check(case, rows=parity.sample_rows(case, 12, seed=6))
    del case
    _release()


def test_flat_m1e7_decode_sampled_rows():
    case = synth.make_case("m1e7_decode", device=DEV)
    check(case, rows=parity.sample_rows(case, 6, seed=7))
    del case
    _release()
