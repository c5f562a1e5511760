"""GPU test of atlaskv_hikvp_attend_noalloc (the entry point that allocates
nothing: its workspace is a fixed device array inside the library), through
the C ABI: two calls in a row, the second smaller, each bit for bit equal to
atlaskv_hikvp_attend_ex with a caller workspace; oversized calls and a given
workspace are refused before anything is enqueued."""
import sys

import numpy as np
import pytest
import torch

from hierarchical_kv_pruning_amd import atlaskv, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-noalloc] {msg}", flush=True)
    sys.stdout.flush()


def _outputs(case, q, seq_k, seq_v, K, call, **kw):
    R = q.shape[0] * q.shape[1] * q.shape[2]
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    sels = [torch.full((R, k), -7, dtype=torch.int32, device=DEV) for k in K]
    lk = torch.full((R,), 7.0, dtype=torch.float32, device=DEV)
    ls = torch.full((R,), 7.0, dtype=torch.float32, device=DEV)
    call(q, case.tree, seq_k, seq_v, K, out, sel_root=sels[0], sel_mid=sels[1], sel_leaf=sels[2],
         lse_kg=lk, lse_seq=ls, **kw)
    torch.cuda.synchronize()
    return [out.cpu().numpy()] + [s.cpu().numpy() for s in sels] + [lk.cpu().numpy(), ls.cpu().numpy()]


def test_noalloc_equals_attend_ex_on_two_calls_second_smaller():
    case = synth.make_case("m1e4", device=DEV)
    case.tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, case.mid_off)
    calls = [(case.q, case.seq_k, case.seq_v),                       # 128 tokens, 4096 rows
             (case.q[:, 100:].contiguous(), case.seq_k[:, :40].contiguous(), case.seq_v[:, :40].contiguous())]
    assert calls[1][0].shape[1] < calls[0][0].shape[1]
    for i, (q, sk, sv) in enumerate(calls):
        say(f"call {i}: N={q.shape[1]} S={sk.shape[1]} K={case.K}")
        ws = atlaskv.alloc_workspace(case.tree, q, sk, case.K)
        ref = _outputs(case, q, sk, sv, case.K, atlaskv.hikvp_attend_ex, workspace=ws)
        got = _outputs(case, q, sk, sv, case.K, atlaskv.hikvp_attend_noalloc)
        assert np.isfinite(got[0]).all()
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)
    case.tree.close()


def test_noalloc_refuses_a_workspace_and_oversized_calls():
    case = synth.make_case("m1e4", device=DEV)
    tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, case.mid_off)
    out = torch.empty_like(case.q)
    ws = atlaskv.alloc_workspace(tree, case.q, case.seq_k, case.K)
    with pytest.raises(atlaskv.AtlasKVError) as e:
        atlaskv.hikvp_attend_noalloc(case.q, tree, case.seq_k, case.seq_v, case.K, out, workspace=ws)
    assert e.value.status == atlaskv.ERR_WORKSPACE
    # enough tokens that the workspace exceeds the fixed array
    cap = atlaskv.noalloc_scratch_bytes()
    N = 128
    while atlaskv.hikvp_workspace_size(tree, torch.empty(1, N, case.Hq, case.d, dtype=case.q.dtype, device=DEV),
                                       None, case.K) <= cap:
        N *= 2
    q = torch.zeros(1, N, case.Hq, case.d, dtype=case.q.dtype, device=DEV)
    big_out = torch.full(q.shape, 3.0, dtype=q.dtype, device=DEV)
    say(f"oversized call: N={N}")
    with pytest.raises(atlaskv.AtlasKVError) as e:
        atlaskv.hikvp_attend_noalloc(q, tree, None, None, case.K, big_out)
    assert e.value.status == atlaskv.ERR_WORKSPACE and "fixed scratch" in atlaskv.last_error()
    torch.cuda.synchronize()
    assert bool((big_out == 3.0).all())          # nothing was enqueued
    # the next call still works
    got = _outputs(type("C", (), {"tree": tree})(), case.q, case.seq_k, case.seq_v, case.K,
                   atlaskv.hikvp_attend_noalloc)
    assert np.isfinite(got[0]).all()
    tree.close()
