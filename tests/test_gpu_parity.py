"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Every workload compares every row; the full workloads
(1e6 prefill, 1e7 decode, 1e8 slice) use the oracle's two-phase mode (roots
and mids on the host, each row's leaf candidates copied from the device) in
the launch configuration the benchmark times."""
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
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def _check(case, rows=None, two_phase=False, **kw):
    rows = oracle.all_rows(case.B, case.N, case.Hq) if rows is None else rows
    gkw = {k: v for k, v in kw.items() if k in ("K", "q", "q_kg", "scale", "with_seq", "out_dtype")}
    okw = {k: v for k, v in kw.items() if k in ("K", "q", "q_kg", "scale", "with_seq")}
    say(f"{case.name}: attend B={case.B} N={case.N} S={case.S_kv} Hq={case.Hq} Hkv={case.Hkv} "
        f"d={case.d} tree={case.M_R}/{case.M_I}/{case.M} K={gkw.get('K', case.K)} rows={len(rows)}")
    gpu = parity.gpu_run(case, **gkw)
    ora = parity.oracle_rows(case, rows, two_phase=two_phase, **okw)

    def replay(rws, selI, selL):
        return parity.oracle_rows(case, np.array(rws), forced_sel_L=np.array(selL, np.int64),
                                  sel_I=np.array(selI, np.int64), **okw)

    P = parity.oracle_problem(case, leaves=False, **okw)
    rep = parity.compare(case, rows, gpu, ora, replay=replay, problem=P)
    say(f"{case.name}: {rep}")
    return gpu, ora, rep


def _release():
    gc.collect()
    torch.cuda.empty_cache()


def _small(name="edge", seed=0, **kw):
    cfg = dict(dtype="f32", B=2, N=33, S_kv=45, Hq=8, Hkv=2, d=128, M_R=37, M_I=411, M=5003,
               K=(5, 7, 19))
    cfg.update(kw)
    ragged = cfg.pop("ragged", True)
    return synth.make_case(name, device=DEV, seed=seed, ragged=ragged, **cfg)


# ---------------------------------------------------------------------------
# small workloads, every row
# ---------------------------------------------------------------------------

def test_tiny_all_rows():
    _check(synth.make_case("tiny", device=DEV))


@pytest.mark.parametrize("dtype,d", [("f32", 128), ("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_ragged_tree_dtypes_and_head_dims(dtype, d):
    _check(_small(seed=3, dtype=dtype, d=d))


@pytest.mark.parametrize("K", [(3, 256, 256), (37, 256, 256), (1, 1, 1), (0, 4, 4), (4, 0, 4),
                               (4, 4, 0), (200, 2, 3)])
def test_k_edge_cases(K):
    """K above the candidate count clamps; K = 0 at any level gives plain causal
    attention; K = 1 everywhere."""
    _check(_small(seed=5, M=2000), K=K)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wide_candidate_lists(dtype):
    """More than 2048 candidates per row at the mid and the leaf level: the
    select kernels then use a whole workgroup per row."""
    _check(_small(seed=21, dtype=dtype, N=5, S_kv=9, M_R=3, M_I=6000, M=30000, K=(2, 3, 40)))


def test_full_k_selects_every_leaf():
    case = _small(seed=6, M_R=4, M_I=20, M=200, K=(4, 20, 200))
    gpu, _, _ = _check(case)
    assert all(sorted(s[s >= 0].tolist()) == list(range(200)) for s in gpu["sel"][2])


def test_k_above_every_candidate_count_equals_full_k():
    """K = 1000 at every level (above 256) clamps to each level's candidates:
    the same selections and bits as K = (M_R, M_I, M) on a 4/20/200 tree, the
    caller's selection rows (stride 1000) -1 padded past them."""
    case = _small(seed=61, M_R=4, M_I=20, M=200, K=(4, 20, 200))
    full = parity.gpu_run(case, K=(4, 20, 200))
    big = parity.gpu_run(case, K=(1000, 1000, 1000))
    assert np.array_equal(full["out"], big["out"]) and np.array_equal(full["lse_kg"], big["lse_kg"])
    for a, b in zip(full["sel"], big["sel"]):
        assert b.shape[1] == 1000
        assert np.array_equal(a, b[:, :a.shape[1]]) and np.all(b[:, a.shape[1]:] == -1)
    _check(case, K=(1000, 1000, 1000))


def test_no_sequence_half():
    _check(_small(seed=7), with_seq=False)


def test_sequence_longer_than_queries_and_gqa_8():
    _check(_small(seed=8, N=17, S_kv=200, Hq=16, Hkv=2, dtype="bf16"))


@pytest.mark.parametrize("N,S_kv,Hq,Hkv", [
    (1, 300, 16, 2),     # decode, 8 query heads per KV head: two groups of 4 per wave
    (3, 50, 6, 2),       # 3 tokens, 3 heads per KV head: a partial group
    (2, 9, 10, 2),       # 5 heads per KV head (4 + 1), keys shorter than one chunk
    (15, 700, 8, 1),     # the longest query block on the decode path, keys split
])
def test_decode_head_groups(N, S_kv, Hq, Hkv):
    """Query blocks below 16 tokens take the decode kernel, which handles a KV
    head's query heads in groups of four per wave."""
    _check(_small(seed=40 + N, dtype="bf16", N=N, S_kv=S_kv, Hq=Hq, Hkv=Hkv, B=3))


def test_single_head_group():
    _check(_small(seed=9, Hq=3, Hkv=3, dtype="bf16"))


def test_separate_kg_query_and_scale():
    case = _small(seed=10, dtype="bf16")
    qkg = torch.randn(case.q.shape, generator=torch.Generator(device=DEV).manual_seed(1),
                      device=DEV).to(case.q.dtype)
    _check(case, q_kg=qkg, scale=0.0625)


def test_fp32_output_of_bf16_inputs():
    case = _small(seed=11, dtype="bf16")
    gpu, ora, _ = _check(case, out_dtype=torch.float32)
    # no bf16 rounding on the output: much tighter than the bf16 bar
    ridx = parity.row_index(case, oracle.all_rows(case.B, case.N, case.Hq))
    assert np.max(np.abs(gpu["out"][ridx] - ora["out"])) < 1e-4


def test_strided_query():
    case = _small(seed=12)
    big = torch.randn(case.B, case.N, case.Hq * 3, case.d, device=DEV, dtype=case.q.dtype)
    q = big[:, :, 1::3, :]          # not contiguous over heads
    q.copy_(case.q)
    _check(case, q=q)


def test_exact_ties_break_to_lower_index():
    """Duplicate keys give bit-equal scores; the lower node index must win."""
    case = _small(seed=13, M_R=6, M_I=30, M=600, ragged=False, K=(3, 4, 9))
    with torch.no_grad():
        case.root_k[:, 3] = case.root_k[:, 1].clone()
        case.mid_k[:, 5::5] = case.mid_k[:, 0:25:5].clone()
        case.leaf_k[:, 1::2] = case.leaf_k[:, 0::2].clone()
    _check(case)


def test_deterministic_reruns():
    case = _small(seed=14, dtype="bf16")
    a = parity.gpu_run(case)
    b = parity.gpu_run(case)
    assert np.array_equal(a["out"], b["out"])
    for x, y in zip(a["sel"], b["sel"]):
        assert np.array_equal(x, y)


def test_deterministic_with_overflowing_buckets():
    """Buckets of far more than 32 rows (eight query heads on one KV head, most
    mids selected): members past the fixed slots are scored from their lists
    at the end of the leaf stream with the same arithmetic, so reruns agree
    bit for bit although which members overflow depends on atomic order."""
    case = _small(seed=19, dtype="bf16", B=2, N=9, S_kv=13, Hq=8, Hkv=1, M_R=37, M_I=411, M=3001)
    K = (37, 256, 256)
    a = parity.gpu_run(case, K=K, out_dtype=torch.float32)
    b = parity.gpu_run(case, K=K, out_dtype=torch.float32)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse_kg"], b["lse_kg"])
    for x, y in zip(a["sel"], b["sel"]):
        assert np.array_equal(x, y)
    _check(case, K=K)


@pytest.mark.parametrize("dtype,d", [("f32", 128), ("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_filtered_leaf_stream(dtype, d):
    """Mids with at least four times K_L children (ragged spans of 15 to 728
    leaves): the leaf stream writes only the candidates that can still be
    among a row's K_L best, and the select over them takes the same leaves."""
    _check(_small(seed=31, dtype=dtype, d=d, M_I=40, M=6000, K=(5, 7, 19)))


@pytest.mark.parametrize("K", [(6, 30, 1), (3, 5, 64), (6, 12, 200)])
def test_filtered_leaf_stream_overflow_and_k(K):
    """The filtered leaf stream with buckets of up to 144 rows (most past the
    fixed slots, scored from their lists), K_L = 1, K_L = 64 over spans of
    18 to 454 leaves, and K_L = 200 (filter off: spans too short for it);
    reruns agree bit for bit."""
    case = _small(seed=33, dtype="bf16", B=2, N=9, S_kv=13, Hq=8, Hkv=1, M_R=6, M_I=30, M=6000)
    gpu, _, _ = _check(case, K=K)
    again = parity.gpu_run(case, K=K)
    assert np.array_equal(gpu["out"], again["out"]) and np.array_equal(gpu["sel"][2], again["sel"][2])


@pytest.mark.parametrize("N,S_kv", [(33, 45), (1, 300)])
def test_overlapped_and_serial_sequence_half_agree(N, S_kv):
    """Without phase events a decode block's sequence half runs on the view's
    second stream beside the KG half and k_seq_combine merges; with phase
    events (and for prefill blocks) it runs after the KG half.  Both write the
    same bits."""
    case = _small(seed=23, dtype="bf16", B=2, N=N, S_kv=S_kv, Hq=8, Hkv=2)
    tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, case.mid_off)
    ws = atlaskv.alloc_workspace(tree, case.q, case.seq_k, case.K)
    outs = []
    for timed in (False, True, False):
        out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((case.rows,), 7.0, dtype=torch.float32, device=DEV)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(atlaskv.phase_names()) + 1)] if timed else None
        atlaskv.hikvp_attend_ex(case.q, tree, case.seq_k, case.seq_v, case.K, out, workspace=ws, lse_seq=lse,
                                phase_events=evs)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    tree.close()
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])
    assert np.isfinite(outs[0][0]).all()


@pytest.mark.parametrize("Hq,Hkv,N", [(32, 8, 256), (12, 3, 683)])
def test_split_descent_matches_serial_and_oracle(Hq, Hkv, N):
    """With 16384 rows or more the KG descent runs as two concurrent parts (the
    halves of the KV heads, uneven for Hkv = 3) on two streams; with phase
    events it runs as one part.  Selections, KG log-sum-exps and outputs agree
    bit for bit, and sampled rows match the oracle."""
    case = _small(seed=29, dtype="bf16", B=2, N=N, S_kv=N + 7, Hq=Hq, Hkv=Hkv, M_R=61, M_I=907, M=20011,
                  K=(6, 9, 24))
    assert case.rows >= 16384
    tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, case.mid_off)
    ws = atlaskv.alloc_workspace(tree, case.q, case.seq_k, case.K)
    runs = []
    for timed in (False, True, False):
        out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((case.rows,), 7.0, dtype=torch.float32, device=DEV)
        sels = [torch.full((case.rows, k), -7, dtype=torch.int32, device=DEV) for k in case.K]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(atlaskv.phase_names()) + 1)] if timed else None
        say(f"split descent: Hq={Hq} Hkv={Hkv} rows={case.rows} timed={timed}")
        atlaskv.hikvp_attend_ex(case.q, tree, case.seq_k, case.seq_v, case.K, out, workspace=ws, lse_kg=lse,
                                sel_root=sels[0], sel_mid=sels[1], sel_leaf=sels[2], phase_events=evs)
        torch.cuda.synchronize()
        runs.append([out.cpu().numpy(), lse.cpu().numpy()] + [x.cpu().numpy() for x in sels])
    tree.close()
    for r in runs[1:]:
        for a, b in zip(r, runs[0]):
            assert np.array_equal(a, b)
    # fp32 output: with N = 256+ the early tokens' outputs reach ~12x the RMS,
    # where a bf16 output's own rounding (2^-9 of the value) exceeds 2e-2 x RMS
    _check(case, two_phase=True, out_dtype=torch.float32)


@pytest.mark.parametrize("K", [(0, 4, 4), (4, 0, 4), (4, 4, 0), (61, 256, 256), (1, 1, 1)])
def test_split_descent_k_edges(K):
    """The two-part descent (16384 rows, two KV heads) with empty levels, K
    above the candidate counts (buckets far past 32 members) and K = 1."""
    case = _small(seed=37, dtype="bf16", B=2, N=512, S_kv=515, Hq=16, Hkv=2, M_R=61, M_I=907, M=9001,
                  K=(6, 9, 24))
    assert case.rows >= 16384
    _check(case, rows=parity.sample_rows(case, 64, seed=41), two_phase=True, K=K, out_dtype=torch.float32)


def test_threads_sharing_a_view():
    """Two host threads call the split descent (16384 rows) and a decode call
    on one view, each on its own stream and workspace: the view's part and
    sequence streams are shared through its mutex, and every result equals
    the one-thread result bit for bit."""
    import threading
    case = _small(seed=43, dtype="bf16", B=2, N=256, S_kv=260, Hq=32, Hkv=8, M_R=61, M_I=907, M=20011,
                  K=(6, 9, 24))
    dec = _small(seed=44, dtype="bf16", B=16, N=1, S_kv=300, Hq=32, Hkv=8, M_R=61, M_I=907, M=20011,
                 K=(6, 9, 24))
    dec.root_k, dec.mid_k, dec.leaf_k, dec.leaf_v = case.root_k, case.mid_k, case.leaf_k, case.leaf_v
    dec.root_off, dec.mid_off = case.root_off, case.mid_off
    tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, case.mid_off)

    def run(c, stream, reps):
        ws = atlaskv.alloc_workspace(tree, c.q, c.seq_k, c.K)
        outs = []
        with torch.cuda.stream(stream):
            for _ in range(reps):
                out = torch.empty(c.q.shape, dtype=torch.float32, device=DEV)
                atlaskv.hikvp_attend_ex(c.q, tree, c.seq_k, c.seq_v, c.K, out, workspace=ws, stream=stream)
                outs.append(out)
        stream.synchronize()
        return [o.cpu().numpy() for o in outs]

    say("threads sharing a view: one-thread references")
    ref_a = run(case, torch.cuda.Stream(), 1)[0]
    ref_b = run(dec, torch.cuda.Stream(), 1)[0]
    results = {}
    s_a, s_b = torch.cuda.Stream(), torch.cuda.Stream()
    ta = threading.Thread(target=lambda: results.__setitem__("a", run(case, s_a, 3)))
    tb = threading.Thread(target=lambda: results.__setitem__("b", run(dec, s_b, 3)))
    say("threads sharing a view: two threads, three calls each")
    ta.start(); tb.start(); ta.join(); tb.join()
    tree.close()
    assert len(results["a"]) == 3 and len(results["b"]) == 3
    for o in results["a"]:
        assert np.array_equal(o, ref_a)
    for o in results["b"]:
        assert np.array_equal(o, ref_b)


def test_empty_batch_writes_nothing():
    case = _small(seed=15, N=1, S_kv=4)
    tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, case.mid_off)
    q = case.q[:0]
    out = torch.empty_like(q)
    atlaskv.hikvp_attend_ex(q, tree, case.seq_k[:0], case.seq_v[:0], case.K, out)
    torch.cuda.synchronize()


def test_malformed_offsets_rejected():
    case = _small(seed=16)
    bad = case.mid_off.clone()
    bad[5] = bad[6] + 1
    with pytest.raises(atlaskv.AtlasKVError) as e:
        atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, bad)
    assert e.value.status == atlaskv.ERR_TREE


def test_view_workspace_entry_point():
    """atlaskv_hikvp_attend with the view's stream and workspace."""
    case = _small(seed=17, dtype="bf16")
    tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, case.mid_off)
    tree.set_workspace(atlaskv.alloc_workspace(tree, case.q, case.seq_k, case.K))
    out = torch.empty_like(case.q)
    atlaskv.hikvp_attend(case.q, tree, case.seq_k, case.seq_v, case.K, out)
    torch.cuda.synchronize()
    ref = parity.gpu_run(case, tree=tree)
    assert np.array_equal(out.float().reshape(case.rows, -1).cpu().numpy(), ref["out"])


@pytest.mark.parametrize("K,F1,F2", [
    ((2, 4, 8), 300, 1000),    # mid list 600: one wave, 16 per lane; leaf 4000: 256 threads, 16 each
    ((3, 2, 8), 500, 3000),    # mid 1500: 256 threads, 8 each; leaf 6000: 256 threads, 32 each
    ((2, 2, 8), 5000, 20),     # mid 10000: 256 threads, re-read from the workspace; leaf 40: 8 per lane
])
def test_select_launch_shapes(K, F1, F2):
    """Balanced trees whose per-row candidate lists (K_R*F1 mids, K_I*F2
    leaves) land in each register / workgroup shape of the select kernels."""
    MR = 4
    case = synth.make_case("shapes", device=DEV, seed=31, ragged=False, dtype="bf16", B=1, N=5, S_kv=7,
                           Hq=4, Hkv=1, d=64, M_R=MR, M_I=MR * F1, M=MR * F1 * F2, K=K)
    _check(case, two_phase=True)
    del case
    _release()


# ---------------------------------------------------------------------------
# host-tiered trees: tree arrays in pinned host memory, read over the host link
# ---------------------------------------------------------------------------

def _pinned(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


_TREE_FIELDS = ("root_k", "mid_k", "leaf_k", "leaf_v", "root_off", "mid_off")


def _view(case):
    return atlaskv.TreeView(*[getattr(case, f) for f in _TREE_FIELDS])


@pytest.mark.parametrize("fields,mask", [(("leaf_k", "leaf_v"), 0b001100),
                                         (_TREE_FIELDS, 0b111111)])
def test_host_tiered_tree_matches_device_tree(fields, mask):
    """Leaves (or the whole tree) in pinned host memory: the view reports the
    placement, selections and outputs equal the device-resident tree's bit for
    bit, and the oracle agrees."""
    case = _small(seed=41, dtype="bf16")
    dev_tree = _view(case)
    assert dev_tree.placement == 0
    ref = parity.gpu_run(case, tree=dev_tree)
    dev_tree.close()
    for f in fields:
        setattr(case, f, _pinned(getattr(case, f)))
    host_tree = _view(case)
    assert host_tree.placement == mask
    got = parity.gpu_run(case, tree=host_tree)
    host_tree.close()
    assert np.array_equal(got["out"], ref["out"])
    for a, b in zip(got["sel"], ref["sel"]):
        assert np.array_equal(a, b)
    _check(case)


def test_host_tiered_leaves_fp32_ragged():
    case = _small(seed=42, dtype="f32", K=(4, 9, 33))
    case.leaf_k, case.leaf_v = _pinned(case.leaf_k), _pinned(case.leaf_v)
    _check(case)


def test_pageable_host_tree_rejected():
    """Pageable host memory cannot be read by the kernels: the view refuses it
    before anything is enqueued and leaves no pending HIP error behind."""
    case = _small(seed=43, dtype="bf16")
    with pytest.raises(atlaskv.AtlasKVError) as e:
        atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k.cpu(), case.leaf_v, case.root_off,
                         case.mid_off)
    assert e.value.status == atlaskv.ERR_UNSUPPORTED
    assert "leaf_k" in atlaskv.last_error()
    x = torch.arange(1000, device=DEV, dtype=torch.float32)
    assert float(x.sum().item()) == 499500.0
    _check(case)


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

def test_m1e4_all_rows():
    _check(synth.make_case("m1e4", device=DEV))


def test_m1e6_all_rows():
    case = synth.make_case("m1e6", device=DEV)
    _check(case, two_phase=True)
    del case
    _release()


def test_m1e7_decode_all_rows():
    case = synth.make_case("m1e7_decode", device=DEV)
    _check(case, two_phase=True)
    del case
    _release()


def test_m1e8_slice_all_rows():
    case = synth.make_case("m1e8_slice", device=DEV)
    _check(case, two_phase=True)
    del case
    _release()
