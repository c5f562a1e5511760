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


def _write_counter_csv(path, dispatches):
    """rocprofv3-style counter_collection.csv: dispatches = [(kernel, {counter: value})]."""
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for i, (kernel, counters) in enumerate(dispatches):
            for name, value in counters.items():
                w.writerow([i + 1, kernel, name, value, 1000 * i, 1000 * i + 500 + i])


def test_hbm_summary_scales_by_the_copy_and_averages_the_phase_steps(tmp_path, monkeypatch):
    """--summarize hbm: a kernel's fetch and write KiB are scaled by what the
    same counters read for the 1 GiB calibration copy, and only its last
    phase-steps dispatches (the phase-timed ones) are averaged."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    leaf = "void hikvp::(anonymous namespace)::k_leaf_score<hikvp::BF16, 128, false>(hikvp::StepArgs)"
    copy = "__amd_rocclr_copyBuffer"
    # five dispatches of the leaf stream (the last two are the phase-timed ones), then the copy
    fetch = [(leaf, {"FETCH_SIZE": v}) for v in (1.0, 2.0, 3.0, 100.0, 300.0)] + [(copy, {"FETCH_SIZE": 524288.0})]
    write = [(leaf, {"WRITE_SIZE": v}) for v in (9.0, 9.0, 9.0, 10.0, 30.0)] + [(copy, {"WRITE_SIZE": 1048576.0})]
    _write_counter_csv(str(tmp_path / "f" / "run_counter_collection.csv"), fetch)
    _write_counter_csv(str(tmp_path / "w" / "run_counter_collection.csv"), write)
    args = bench.parse_args(["--summarize", "hbm", "--workload", "m1e6", "--steps", "3", "--warmup", "1",
                             "--phase-steps", "2", "--fetch-dir", str(tmp_path / "f"),
                             "--write-dir", str(tmp_path / "w")])
    bench.summarize(args)
    path = os.path.join(bench.PROFILES, "leaf_score_stream_m1e6_hbm_counters.txt")
    fields = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
    assert float(fields["fetch_scale"]) == pytest.approx(2.0)
    assert float(fields["write_scale"]) == pytest.approx(1.0)
    assert float(fields["fetch_kib_per_dispatch"]) == pytest.approx(200.0)
    assert float(fields["write_kib_per_dispatch"]) == pytest.approx(20.0)
    assert int(fields["hbm_bytes_per_launch"]) == (200 * 2 + 20) * 1024
    assert fields["kernel_source_sha256_16"].strip() == bench.kernel_source_hash()
    assert bench.read_traffic("leaf_score_stream", "m1e6") == (200 * 2 + 20) * 1024
    text = open(path).read()
    assert "# fetch pass: rocprofv3 --pmc FETCH_SIZE" in text and "--calib-copy-gib 1" in text


def test_busy_summary_uses_the_tools_metric_definitions(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    k = "void hikvp::(anonymous namespace)::k_mid_gemm<hikvp::BF16, 128, false>(hikvp::StepArgs)"
    # GRBM_GUI_ACTIVE as the csv holds it: the 8 XCDs' counts summed (100 cycles each)
    c = {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 50.0, "SQ_ACTIVE_INST_VALU": 256 * 25.0, "GRBM_GUI_ACTIVE": 800.0,
         "SQ_WAVES": 10.0, "SQ_INSTS_VALU": 1000.0, "SQ_INSTS_MFMA": 40.0, "MfmaUtil": 49.0, "VALUBusy": 24.0}
    _write_counter_csv(str(tmp_path / "b" / "run_counter_collection.csv"), [(k, c), (k, c)])
    args = bench.parse_args(["--summarize", "busy", "--workload", "m1e6", "--steps", "3", "--warmup", "1",
                             "--phase-steps", "2", "--pmc-dir", str(tmp_path / "b")])
    bench.summarize(args)
    rows = [l for l in open(os.path.join(bench.PROFILES, "busy_counters_m1e6.txt")) if l.startswith("k_mid_gemm")]
    cols = [x.strip() for x in rows[0].split("|")]
    assert cols[1] == "mid_bucket_gemm" and cols[2] == "2"
    assert float(cols[4]) == pytest.approx(49.0)     # the tool's MfmaUtil as collected
    assert float(cols[5]) == pytest.approx(24.0)     # the tool's VALUBusy as collected
    assert float(cols[6]) == pytest.approx(50.0)     # MfmaUtil from the raw counters, per-XCD GRBM
    assert float(cols[7]) == pytest.approx(25.0)     # VALUBusy from the raw counters, per-XCD GRBM
    assert float(cols[9]) == pytest.approx(100.0)    # VALU instructions a wave
    assert float(cols[10]) == pytest.approx(4.0)     # MFMA instructions a wave
