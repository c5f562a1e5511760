"""CPU tests of the benchmark's accounting: the algorithmic bytes it divides by
(each compulsory byte of a step counted once) against a brute-force count over
the distinct (KV head, node) pairs of given selections, and the committed
rocprofv3 counter summaries it reads the measured HBM traffic from.  No GPU."""
import glob
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from hierarchical_kv_pruning_amd import synth  # noqa: E402


def _selections(case, rng, counts, share_rows=None):
    """Random selections per level, each row a set of distinct valid nodes
    followed by -1 padding (what the library writes)."""
    rows = case.rows if share_rows is None else share_rows
    sel = []
    for k, n in zip(case.K, counts):
        s = np.full((rows, k), -1, dtype=np.int32)
        for r in range(rows):
            m = rng.integers(0, k + 1)
            s[r, :m] = rng.choice(n, size=m, replace=False)
        sel.append(s)
    return sel


def _brute(case, sel, heads):
    """Bytes of the spans of the distinct (head, node) pairs at each level."""
    eb = 2 if case.dtype == "bf16" else 4
    rb = case.d * eb
    ro = case.root_off.numpy()
    mo = case.mid_off.numpy()
    pairs = [set(), set(), set()]
    for lev in range(3):
        for r, h in enumerate(heads):
            for x in sel[lev][r]:
                if x >= 0:
                    pairs[lev].add((int(h), int(x)))
    mids = sum(int(ro[j + 1] - ro[j]) for _, j in pairs[0]) * rb
    leaves = sum(int(mo[m + 1] - mo[m]) for _, m in pairs[1]) * rb
    return mids, leaves, len(pairs[2]) * rb


@pytest.mark.parametrize("seed", [0, 1])
def test_per_row_bytes_match_brute_force(seed):
    case = synth.make_case("tiny", device="cpu", seed=seed, ragged=True, Hq=8, Hkv=2)
    rng = np.random.default_rng(seed)
    sel = _selections(case, rng, (case.M_R, case.M_I, case.M))
    G = case.Hq // case.Hkv
    heads = (np.arange(case.rows) % case.Hq) // G
    got = bench.algorithmic_bytes(case, sel)
    mids, leaves, values = _brute(case, sel, heads)
    rb = case.d * 4
    assert got["mid_bucket_gemm"] == mids
    assert got["leaf_score_stream"] == leaves
    assert got["leaf_topk_kg_attention"] == values
    assert got["root_score_topk"] == case.Hkv * case.M_R * rb + case.rows * rb
    assert got["seq_attention"] == 2 * case.B * case.S_kv * case.Hkv * rb
    assert got["_total"] == sum(v for k, v in got.items() if not k.startswith("_"))


def test_shared_bytes_use_group_heads():
    """Group selections (rows = groups (b, g)): the head of group i is i mod Hkv."""
    case = synth.make_case("tiny", device="cpu", seed=3, ragged=True, Hq=8, Hkv=2)
    rng = np.random.default_rng(3)
    groups = case.B * case.Hkv
    sel = _selections(case, rng, (case.M_R, case.M_I, case.M), share_rows=groups)
    got = bench.algorithmic_bytes(case, sel, share=2)
    mids, leaves, values = _brute(case, sel, np.arange(groups) % case.Hkv)
    assert (got["mid_bucket_gemm"], got["leaf_score_stream"], got["leaf_topk_kg_attention"]) == (mids, leaves, values)
    assert got["shared_kg_attention"] == values


def test_counter_summaries_parse():
    """Every committed HBM counter summary is complete."""
    files = glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.txt"))
    assert files
    for path in files:
        text = open(path).read()
        for field in ("fetch_kib_per_dispatch", "write_kib_per_dispatch", "hbm_bytes_per_launch",
                      "kernel_source_sha256_16", "# fetch pass: rocprofv3 --pmc FETCH_SIZE"):
            assert field in text, (path, field)


def test_counter_summaries_match_the_kernel_sources():
    """The dominant kernels' summaries were taken on the current sources
    (every file under csrc/ and include/), else the bench line's traffic is
    null; a stale summary is reported as a skip naming it."""
    stale = []
    for kernel, workload in (("leaf_score_stream", "m1e6"), ("leaf_score_stream", "m1e8_slice"),
                             ("seq_attention", "m1e7_decode")):
        t = bench.read_traffic(kernel, workload)
        if t is None:
            stale.append(f"{kernel}_{workload}")
        else:
            assert t > 0
    if stale:
        pytest.skip(f"counter summaries taken on older kernel sources: {stale}")


def test_source_hash_covers_every_library_source():
    names = {os.path.basename(f) for f in bench.kernel_sources()}
    csrc = os.path.join(ROOT, "hierarchical_kv_pruning_amd", "csrc")
    want = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))} | {"atlaskv.h"}
    assert want <= names
