"""Benchmark of HiKVP knowledge-injected attention on one MI355X.

One step = one atlaskv_hikvp_attend_ex call over one batch of synthetic input:
root scoring + Top-K, mid scoring + Top-K, leaf scoring + Top-K, KG softmax over
the selected leaves, causal sequence attention and the λ merge.  Inputs are
resident in HBM before timing starts.

Printed (one JSON line): query tokens/s, ms per step, the whole path's
compulsory HBM bytes and their rate against the 8 TB/s peak, the roofline of
the dominant kernel (algorithmic bytes / live HIP-event duration), and the
fp64 CPU oracle's rate on a bounded row sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload m1e6] [--tree-placement hbm|host-leaves]

Timing: W warm-up steps, then max(K, 50) steps each timed alone with HIP
events on the launch stream after a 1 GiB read has evicted the 256 MB MALL
(cold); the headline is their median (p10 / p90 beside it).  K steps back
to back give the warm figure.  Run without --workload, the benchmark first
measures the m1e7_decode and m1e8_slice workloads and the m1e6 layer folded
onto one base-embedding tree of width D_E = 384 (one JSON line each on
stderr) and ends with the m1e6 line on stdout.

With --tree-placement host-leaves the leaf keys and values sit in pinned host
memory and the kernels read the selected spans over the host link; the
roofline is then the link's (PCIe 5.0 x16).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from hierarchical_kv_pruning_amd import atlaskv, synth  # noqa: E402

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, AMD's published figure
PEAK_LINK_GBPS = 64.0           # MI355X host interface, PCIe 5.0 x16, one direction (published)
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix-core peak (published)
PEAK_FP32_TFLOPS = 157.3        # MI355X fp32 vector peak (published)
CSRC = os.path.join(ROOT, "hierarchical_kv_pruning_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sources():
    """Every source the library is built from (kernels, launch planning, ABI)."""
    out = []
    for d in (CSRC, INCLUDE):
        out += [os.path.join(d, f) for f in sorted(os.listdir(d)) if f.endswith((".hip", ".h"))]
    return out


def kernel_source_hash():
    h = hashlib.sha256()
    for f in kernel_sources():
        h.update(os.path.relpath(f, ROOT).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic bytes: what the method must move per step (each byte once)
# ---------------------------------------------------------------------------

def algorithmic_bytes(case, sel, share=0):
    """Per-phase compulsory bytes of one step, from the step's selections.

    roots: every root key; mids: the child spans of the distinct selected
    (KV head, root) pairs; leaf keys: the child spans of the distinct selected
    (KV head, mid) pairs; leaf values: the distinct selected (KV head, leaf)
    rows; sequence: K and V once; q read once, out written once.  With shared
    selections `sel` holds the group selections (rows of groups (b, n, g) or
    (b, g)) and the per-row KG softmax re-reads the groups' selected leaf keys
    (their values are counted once already).
    """
    eb = 2 if case.dtype == "bf16" else 4
    row_b = case.d * eb
    G = case.Hq // case.Hkv
    R = case.rows
    head = (np.arange(R) % case.Hq) // G if share == 0 else np.arange(sel[0].shape[0]) % case.Hkv
    ro = case.root_off.cpu().numpy()
    mo = case.mid_off.cpu().numpy()

    def distinct(selx, count):
        s = selx.astype(np.int64)
        h = np.repeat(head, s.shape[1])
        v = s.reshape(-1)
        keep = v >= 0
        return np.unique(h[keep] * count + v[keep]) % count

    roots_b = case.Hkv * case.M_R * row_b
    u_root = distinct(sel[0], case.M_R)
    mids_b = int((ro[u_root + 1] - ro[u_root]).sum()) * row_b
    u_mid = distinct(sel[1], case.M_I)
    leafk_b = int((mo[u_mid + 1] - mo[u_mid]).sum()) * row_b
    leafv_b = len(distinct(sel[2], case.M)) * row_b
    q_b = R * row_b
    out_b = R * row_b
    seq_b = 2 * case.B * case.S_kv * case.Hkv * row_b
    if share:
        return {
            "group_query": q_b,
            "root_score_topk": roots_b,
            "mid_bucket_gemm": mids_b,
            "mid_topk": 0, "leaf_bucket_link": 0,
            "leaf_score_stream": leafk_b,
            "leaf_topk_kg_attention": leafv_b,
            "shared_kg_attention": leafv_b,   # the selected leaves' keys (values counted above)
            "seq_attention": seq_b,
            "seq_split_combine": out_b,
            "_total": roots_b + mids_b + leafk_b + 2 * leafv_b + seq_b + q_b + out_b,
            "_parts": dict(roots=roots_b, mids=mids_b, leaf_keys=leafk_b, leaf_values=leafv_b,
                           selected_leaf_keys=leafv_b, sequence_kv=seq_b, q=q_b, out=out_b),
        }
    return {
        "root_score_topk": roots_b + q_b,
        "mid_bucket_gemm": mids_b,
        "mid_topk": 0,
        "leaf_bucket_link": 0,
        "leaf_score_stream": leafk_b,
        "leaf_topk_kg_attention": leafv_b,
        "seq_attention": seq_b,
        "seq_split_combine": out_b,
        "_total": roots_b + mids_b + leafk_b + leafv_b + seq_b + q_b + out_b,
        "_parts": dict(roots=roots_b, mids=mids_b, leaf_keys=leafk_b, leaf_values=leafv_b,
                       sequence_kv=seq_b, q=q_b, out=out_b),
    }


# ---------------------------------------------------------------------------
# rocprofv3 counter summaries committed under profiles/
# ---------------------------------------------------------------------------

def read_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from a committed counter summary, or
    None when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# The summaries themselves: `python3 bench.py --summarize {hbm,busy,stats} ...`
# reads the csv output of the rocprofv3 runs named in each summary's header
# and writes profiles/.  Kernels of each phase (the phase-timed steps run the
# descent as one part over all KV heads, serially, one dispatch of each
# kernel a step: their last `phase_steps` dispatches are the ones the
# roofline divides by).
PHASE_OF = {
    "k_root_mfma": "root_score_topk", "k_root": "root_score_topk",
    "k_root_scan": "root_score_topk (grouping)", "k_root_fill": "root_score_topk (grouping)",
    "k_mid_gemm": "mid_bucket_gemm", "k_mid_select": "mid_topk", "k_bucket_link": "leaf_bucket_link",
    "k_leaf_score": "leaf_score_stream", "k_leaf_score_filtered": "leaf_score_stream",
    "k_leaf_select_pairs": "leaf_topk_kg_attention",
    "k_leaf_select": "leaf_topk_kg_attention", "k_seq_mfma": "seq_attention",
    "k_seq_decode_mfma": "seq_attention", "k_seq_decode": "seq_attention", "k_seq_flash": "seq_attention",
    "k_seq_combine": "seq_split_combine",
    "k_flat_mfma": "flat_kg_partial", "k_flat_valu": "flat_kg_partial", "k_flat_combine": "flat_kg_combine",
}
# the kernel each phase's HBM summary counts (a phase's main kernel)
HBM_SUMMARY_KERNELS = {
    "root_score_topk": ("k_root",), "mid_bucket_gemm": ("k_mid_gemm",), "mid_topk": ("k_mid_select",),
    "leaf_bucket_link": ("k_bucket_link",),
    "leaf_score_stream": ("k_leaf_score", "k_leaf_score_filtered"),
    "leaf_topk_kg_attention": ("k_leaf_select", "k_leaf_select_pairs"),
    "seq_attention": ("k_seq_mfma", "k_seq_decode_mfma", "k_seq_decode", "k_seq_flash"),
}
BUSY_KERNELS = ("k_root_mfma", "k_root", "k_mid_gemm", "k_mid_select", "k_bucket_link", "k_leaf_score",
                "k_leaf_score_filtered", "k_leaf_select", "k_leaf_select_pairs", "k_seq_mfma", "k_seq_decode_mfma",
                "k_seq_combine")
COPY_KERNEL = "__amd_rocclr_copyBuffer"
# the busy pass: the tool's two derived metrics and the raw counters behind them
BUSY_COUNTERS = ("MfmaUtil", "VALUBusy", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU",
                 "SQ_INSTS_MFMA", "SQ_WAVES", "GRBM_GUI_ACTIVE")
XCDS = 8  # MI355X accelerator complex dies; the csv sums GRBM_GUI_ACTIVE over them


def _short_kernel(name):
    import re
    m = re.search(r"hikvp::(?:\(anonymous namespace\)::)?(k_\w+)", name)
    if m:
        return m.group(1)
    return COPY_KERNEL if COPY_KERNEL in name else None


def _read_csv(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _counter_dispatches(directory):
    """{kernel: [(dispatch id, {counter: value}, duration ns)]} in dispatch order."""
    per = {}
    for r in _read_csv(directory, "counter_collection.csv"):
        k = _short_kernel(r["Kernel_Name"])
        if not k:
            continue
        d = int(r["Dispatch_Id"])
        ent = per.setdefault(k, {}).setdefault(d, [{}, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])])
        ent[0][r["Counter_Name"]] = ent[0].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return {k: [(d, v[0], v[1]) for d, v in sorted(m.items())] for k, m in per.items()}


def _variant(args):
    """(file-name suffix, bench flags, description) of a summary's path variant."""
    if getattr(args, "path", "hikvp") == "flat":
        return "_flat", " --path flat", ", unpruned equivalent attention (every leaf)"
    if getattr(args, "tree_placement", "hbm") == "host-leaves":
        return ("_host_leaves", " --tree-placement host-leaves",
                " with leaf keys and values in pinned host memory")
    return "", "", ""


def _bench_cmd(args, extra):
    return (f"python3 bench.py --workload {args.workload}{_variant(args)[1]} --steps {args.steps} "
            f"--warmup {args.warmup} --phase-steps {args.phase_steps} --no-cpu-baseline{extra}")


def summarize(args):
    """Write the profiles/ summaries of one workload from rocprofv3 csv output."""
    w, nph = args.workload, args.phase_steps
    if not w or not nph:
        raise SystemExit("--summarize needs --workload and --phase-steps")
    hsh = kernel_source_hash()
    written = []
    if args.summarize == "hbm":
        fetch, write = _counter_dispatches(args.fetch_dir), _counter_dispatches(args.write_dir)
        calib_gib = 1
        # the calibration copy is the largest device copy of each pass
        cf = max(c["FETCH_SIZE"] for _, c, _ in fetch[COPY_KERNEL])
        cw = max(c["WRITE_SIZE"] for _, c, _ in write[COPY_KERNEL])
        fscale, wscale = calib_gib * (1 << 20) / cf, calib_gib * (1 << 20) / cw
        bench_cmd = _bench_cmd(args, f" --calib-copy-gib {calib_gib}")
        for phase, kernels in HBM_SUMMARY_KERNELS.items():
            k = next((k for k in kernels if k in fetch and k in write), None)
            if k is None:
                continue
            fk = float(np.mean([c["FETCH_SIZE"] for _, c, _ in fetch[k][-nph:]]))
            wk = float(np.mean([c["WRITE_SIZE"] for _, c, _ in write[k][-nph:]]))
            path = os.path.join(PROFILES, f"{phase}_{w}_hbm_counters.txt")
            with open(path, "w") as f:
                f.write(f"# HBM traffic of {k} ({phase}), workload {w}, from two rocprofv3 counter passes\n")
                f.write(f"# fetch pass: rocprofv3 --pmc FETCH_SIZE --output-format csv -d {args.fetch_dir} -o run -- "
                        f"{bench_cmd}\n")
                f.write(f"# write pass: rocprofv3 --pmc WRITE_SIZE --output-format csv -d {args.write_dir} -o run -- "
                        f"{bench_cmd}\n")
                f.write(f"# summary: python3 bench.py --summarize hbm --workload {w} --steps {args.steps} "
                        f"--warmup {args.warmup} --phase-steps {nph} --fetch-dir {args.fetch_dir} "
                        f"--write-dir {args.write_dir}\n")
                f.write(f"# calibration: the same passes count a {calib_gib} GiB device-to-device copy ({COPY_KERNEL})\n")
                f.write(f"calib_copy_fetch_kib: {cf:.1f}\ncalib_copy_write_kib: {cw:.1f}\n")
                f.write(f"fetch_scale: {fscale:.4f}\nwrite_scale: {wscale:.4f}\n")
                f.write(f"dispatches: {len(fetch[k])} (the last {nph}, the bench's phase-timed steps, are averaged)\n")
                f.write(f"fetch_kib_per_dispatch: {fk:.1f}\nwrite_kib_per_dispatch: {wk:.1f}\n")
                f.write(f"hbm_bytes_per_launch: {int(round((fk * fscale + wk * wscale) * 1024))}\n")
                f.write(f"kernel_source_sha256_16: {hsh}\n")
            written.append(path)
    elif args.summarize == "busy":
        per = _counter_dispatches(args.pmc_dir)
        path = os.path.join(PROFILES, f"busy_counters_{w}.txt")
        with open(path, "w") as f:
            f.write(f"# MFMA and VALU activity per kernel, workload {w} (MI355X: 8 XCDs, 256 CUs, 1024 SIMDs)\n")
            f.write(f"# counter pass: rocprofv3 --pmc {' '.join(BUSY_COUNTERS)} "
                    f"--output-format csv -d {args.pmc_dir} -o run -- {_bench_cmd(args, '')}\n")
            f.write(f"# summary: python3 bench.py --summarize busy --workload {w} --steps {args.steps} "
                    f"--warmup {args.warmup} --phase-steps {nph} --pmc-dir {args.pmc_dir}\n")
            f.write("# mean over the last phase-steps dispatches of each kernel (the phase-timed steps):\n")
            f.write("#   mfma_busy_pct: rocprofv3's MfmaUtil, 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) /\n")
            f.write("#                  (max(GRBM_GUI_ACTIVE) * 1024 SIMDs)\n")
            f.write("#   valu_busy_pct: rocprofv3's VALUBusy, 100 * sum(SQ_ACTIVE_INST_VALU) / 256 CUs /\n")
            f.write("#                  max(GRBM_GUI_ACTIVE)\n")
            f.write("#   max(GRBM_GUI_ACTIVE) is one XCD's active cycles; the csv's GRBM_GUI_ACTIVE column sums\n")
            f.write("#   the 8 XCDs' counters, so the raw columns below divide it by 8 (the '(raw)' figures, a\n")
            f.write("#   check on the tool's metrics)\n")
            f.write(f"# kernel sources sha256[:16]: {hsh}\n")
            f.write("kernel | phase | dispatches | us | mfma_busy_pct | valu_busy_pct | mfma_busy_pct (raw) | "
                    "valu_busy_pct (raw) | waves | valu_insts_per_wave | mfma_insts_per_wave\n")
            for k in BUSY_KERNELS:
                if k not in per:
                    continue
                last = per[k][-nph:]
                mean = lambda c: float(np.mean([x[1].get(c, float("nan")) for x in last]))
                g = mean("GRBM_GUI_ACTIVE") / XCDS
                waves = max(mean("SQ_WAVES"), 1.0)
                f.write(f"{k} | {PHASE_OF.get(k, '-')} | {len(per[k])} | {np.mean([x[2] for x in last]) / 1e3:.1f} | "
                        f"{mean('MfmaUtil'):.2f} | {mean('VALUBusy'):.2f} | "
                        f"{100 * mean('SQ_VALU_MFMA_BUSY_CYCLES') / (g * 1024):.2f} | "
                        f"{100 * mean('SQ_ACTIVE_INST_VALU') / (g * 256):.2f} | {waves:.0f} | "
                        f"{mean('SQ_INSTS_VALU') / waves:.0f} | {mean('SQ_INSTS_MFMA') / waves:.1f}\n")
        written.append(path)
    elif args.summarize == "stats":
        per = {}
        for r in _read_csv(args.trace_dir, "kernel_trace.csv"):
            k = _short_kernel(r["Kernel_Name"])
            if k and k != COPY_KERNEL:
                per.setdefault((k, r["Kernel_Name"]), []).append(
                    (int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
        sfx, vflags, vdesc = _variant(args)
        path = os.path.join(PROFILES, f"kernel_stats_{w}{sfx}.txt")
        rows = []
        for (k, full), v in per.items():
            v.sort()
            us = [x[1] for x in v]
            rows.append((float(np.mean(us[-nph:])), full, k, us))
        with open(path, "w") as f:
            f.write(f"# rocprofv3 kernel statistics, workload {w}{vdesc} (MI355X, one GPU)\n")
            f.write(f"# command (from the repository root): rocprofv3 --kernel-trace --stats --output-format csv "
                    f"-d {args.trace_dir} -o run -- {_bench_cmd(args, '')}\n")
            f.write(f"# summary: python3 bench.py --summarize stats --workload {w}{vflags} --steps {args.steps} "
                    f"--warmup {args.warmup} --phase-steps {nph} --trace-dir {args.trace_dir}\n")
            f.write(f"# kernel sources sha256[:16]: {hsh}\n")
            f.write(f"# 'timed us': mean of the kernel's last {nph} dispatches, the bench's phase-timed steps (one\n")
            f.write("# descent part over all KV heads; the roofline divides by this); 'all' columns: every dispatch,\n")
            f.write("# including warm-up and headline steps, where 16384+ rows run the descent as two concurrent parts\n")
            f.write("# kernel | phase | calls | timed us | all average us | all min us | all max us\n")
            for t, full, k, us in sorted(rows, key=lambda x: -x[0]):
                name = full.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
                f.write(f"{name} | {PHASE_OF.get(k, '-')} | {len(us)} | {t:.1f} | {np.mean(us):.1f} | "
                        f"{min(us):.1f} | {max(us):.1f}\n")
        written.append(path)
    for p in written:
        print(os.path.relpath(p, ROOT))


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample, two-phase: leaves fetched per row)
# ---------------------------------------------------------------------------

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, seconds):
    """The oracle on one host core (this thread pinned to it while it runs)."""
    old = os.sched_getaffinity(0)
    core = max(old)
    os.sched_setaffinity(0, {core})
    try:
        res = _cpu_baseline(case, seconds)
    finally:
        os.sched_setaffinity(0, old)
    res["host"] = {"nproc": os.cpu_count(), "cores_allowed": len(old), "pinned_core": core,
                   "cpu_model": cpu_model()}
    return res


def _cpu_baseline(case, seconds):
    from oracle import oracle  # test infrastructure: only this leg uses it

    h = lambda t: None if t is None else t.detach().cpu()
    P = oracle.Problem(h(case.q), h(case.root_k), h(case.mid_k), None, None, h(case.root_off),
                       h(case.mid_off), h(case.seq_k), h(case.seq_v), case.K)
    mo = case.mid_off.cpu().numpy()
    G = case.Hq // case.Hkv
    allr = oracle.all_rows(case.B, case.N, case.Hq)
    rng = np.random.default_rng(0)
    order = rng.permutation(len(allr))

    def run(rows):
        t0 = time.perf_counter()
        ph1 = oracle.select_mids_rows(P, rows)
        t_sel = time.perf_counter() - t0
        off, idx, heads = [0], [], []
        for r, (_, _, hh) in enumerate(rows):
            cand = [np.arange(mo[m], mo[m + 1]) for m in ph1["sel_I"][r] if m >= 0]
            cand = np.concatenate(cand) if cand else np.zeros(0, np.int64)
            idx.append(cand)
            heads.append(np.full(len(cand), hh // G))
            off.append(off[-1] + len(cand))
        idx = torch.from_numpy(np.concatenate(idx).astype(np.int64)).to(case.leaf_k.device)
        hd = torch.from_numpy(np.concatenate(heads).astype(np.int64)).to(case.leaf_k.device)
        ks, vs = case.leaf_k[hd, idx].cpu(), case.leaf_v[hd, idx].cpu()
        t0 = time.perf_counter()
        oracle.finish_rows(P, rows, np.array(off), idx.cpu().numpy(), ks, vs)
        return t_sel + time.perf_counter() - t0   # oracle time only (gather excluded)

    n = 8
    t = run(allr[order[:n]])
    per_row = t / n
    n2 = int(min(len(allr) - n, max(8, seconds / max(per_row, 1e-9))))
    t2 = run(allr[order[n:n + n2]])
    rows_done = n2
    per_row = t2 / n2
    tokens_per_s = 1.0 / (per_row * case.Hq)
    return {"value": tokens_per_s, "unit": "query tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows_done} of {len(allr)} rows (b,n,h) of workload {case.name}, seeded; "
                      f"fp64 single-thread C oracle pinned to one core, {t2:.1f} s; leaf candidates "
                      f"copied to host per row outside the timed calls; tokens/s = rows/s / Hq"}


# ---------------------------------------------------------------------------

def flat_line(args, case, tm, phase_ms, tokens):
    """JSON line of the unpruned path: every leaf key and value is read once;
    the dominant kernel is the flash pass over the leaves, 4*d flops per
    (row, leaf) pair (scores and weighted values)."""
    eb = 2 if case.dtype == "bf16" else 4
    row_b = case.d * eb
    leaves_b = 2 * case.Hkv * case.M * row_b
    seq_b = 2 * case.B * case.S_kv * case.Hkv * row_b
    total_b = leaves_b + seq_b + 2 * case.rows * row_b
    flops = 4.0 * case.rows * case.M * case.d
    t = phase_ms["flat_kg_partial"] * 1e-3
    peak_f = PEAK_BF16_TFLOPS if case.dtype == "bf16" else PEAK_FP32_TFLOPS
    t_mfma, t_hbm = flops / (peak_f * 1e12), leaves_b / (PEAK_HBM_GBPS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma" if case.dtype == "bf16" else "alu", "achieved": flops / t / 1e12,
                "peak": peak_f, "unit": "TFLOP/s", "frac": flops / t / 1e12 / peak_f,
                "algorithmic_flops": flops}
    else:
        roof = {"bound": "hbm", "achieved": leaves_b / t / 1e9, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": leaves_b / t / 1e9 / PEAK_HBM_GBPS, "algorithmic_bytes": leaves_b}
    roof.update(kernel="flat_kg_partial", traffic=None,
                hbm_gbps=leaves_b / t / 1e9, tflops=flops / t / 1e12)
    ms_per_step = tm["ms_per_step"]
    return {
        "metric": "query tokens/s per layer through unpruned equivalent attention (all M leaves)",
        "value": tokens / (ms_per_step * 1e-3), "unit": "query tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "timing": tm,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": case.dtype,
        "data": "synthetic (seeded clustered-Gaussian key tree, Gaussian values, queries and sequence K/V)",
        "config": {"workload": case.name, "path": "flat", "B": case.B, "N": case.N, "S_kv": case.S_kv,
                   "Hq": case.Hq, "Hkv": case.Hkv, "d": case.d, "M": case.M, "tokens_per_step": tokens,
                   "parallelism": "single GPU", "tree_placement": args.tree_placement},
        "path_hbm": {"compulsory_bytes": total_b, "achieved_gbps": total_b / (ms_per_step * 1e-3) / 1e9,
                     "frac_of_peak": total_b / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        "phase_ms": phase_ms, "roofline": roof, "cpu_baseline": None,
    }


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50,
                    help="timed steps: max(steps, 50) cold steps, each alone after a MALL flush (their "
                         "median is the headline), and `steps` warm steps back to back")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, choices=sorted(synth.CONFIGS),
                    help="one workload only (default: m1e7_decode, m1e8_slice and m1e6 folded at "
                         "D_E = 384 on stderr, then m1e6)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--phase-steps", type=int, default=None,
                    help="steps of the per-phase event loop (default: --steps, at most 20)")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--path", default="hikvp", choices=["hikvp", "flat"],
                    help="flat: the unpruned equivalent attention (KG softmax over every leaf)")
    ap.add_argument("--share", default="none", choices=["none", "kv-group", "sequence"],
                    help="shared selections: one descent per KV head and token, or per KV head "
                         "and sequence (pruned path only)")
    ap.add_argument("--fold", action="store_true",
                    help="folded projections: one-head base tree shared by all heads through random "
                         "per-head W_K / W_V [Hkv, d, D_E]")
    ap.add_argument("--fold-width", type=int, default=0,
                    help="base width D_E of the folded tree (default: the head dim, using the workload's "
                         "head-0 tree; otherwise a fresh base tree of that width with the workload's topology)")
    ap.add_argument("--summarize", default=None, choices=["hbm", "busy", "stats"],
                    help="write profiles/ summaries from rocprofv3 csv output (no GPU work): hbm needs "
                         "--fetch-dir and --write-dir, busy --pmc-dir, stats --trace-dir")
    ap.add_argument("--fetch-dir", default=None)
    ap.add_argument("--write-dir", default=None)
    ap.add_argument("--pmc-dir", default=None)
    ap.add_argument("--trace-dir", default=None)
    ap.add_argument("--tree-placement", default="hbm", choices=["hbm", "host-leaves"],
                    help="host-leaves: leaf keys and values in pinned host memory, read by the "
                         "kernels over the host link (roots, mids, offsets stay in HBM)")
    return ap.parse_args(argv)


MIN_COLD_STEPS = 50


def time_steps(step, stream, steps, warmup, dev):
    """Warm-up, then max(steps, 50) cold steps (each after evicting the MALL,
    timed alone: the headline is their median) and `steps` warm steps back to
    back; times in ms."""
    ncold = max(steps, MIN_COLD_STEPS)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # 1 GiB > the 256 MB MALL, read (not written) so that no dirty lines of the
    # flush itself are left to be written back inside the timed step
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty(1, dtype=torch.float32, device=dev)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ncold)]
    torch.cuda.synchronize()
    for a, b in pairs:
        torch.sum(flush, dim=0, keepdim=True, out=sink)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    cold = np.array([a.elapsed_time(b) for a, b in pairs])
    del flush, sink
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    warm = t0.elapsed_time(t1) / steps
    return {"ms_per_step": float(np.median(cold)), "cold_p10_ms": float(np.percentile(cold, 10)),
            "cold_p90_ms": float(np.percentile(cold, 90)), "cold_steps": int(ncold),
            "warm_ms_per_step": float(warm), "protocol": "median of cold steps (1 GiB read between "
            "steps to evict the 256 MB MALL; each step timed alone with HIP events on the launch stream)"}


def fold_inputs(case, args, dev):
    """Base tree and per-head projections of a folded run."""
    DE = args.fold_width or case.d
    if DE == case.d:
        base = [t[:1].contiguous() for t in (case.root_k, case.mid_k, case.leaf_k, case.leaf_v)]
        base_off = (case.root_off, case.mid_off)
    else:
        b = synth.make_case("base", device=dev, seed=synth.CONFIGS[case.name]["seed"] + 500, ragged=False, dtype=case.dtype, B=1, N=1,
                            S_kv=1, Hq=1, Hkv=1, d=DE, M_R=case.M_R, M_I=case.M_I, M=case.M, K=case.K)
        base = [b.root_k, b.mid_k, b.leaf_k, b.leaf_v]
        base_off = (b.root_off, b.mid_off)
    gen = torch.Generator(device=dev).manual_seed(17)
    w_k = (torch.randn(case.Hkv, case.d, DE, generator=gen, device=dev) / DE ** 0.5).to(case.q.dtype)
    w_v = (torch.randn(case.Hkv, case.d, DE, generator=gen, device=dev) / DE ** 0.5).to(case.q.dtype)
    return base, base_off, w_k, w_v, DE


def run_one(args, workload, dev, with_cpu):
    log(f"workload {workload}: generating on {torch.cuda.get_device_name(0)}")
    case = synth.make_case(workload, device=dev)
    link_copy_gbps = None
    if args.tree_placement == "host-leaves":
        log("moving leaf keys and values to pinned host memory")
        for f in ("leaf_k", "leaf_v"):
            t = getattr(case, f)
            h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
            h.copy_(t)
            setattr(case, f, h)
            del t, h
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        # the link's copy-engine ceiling: 1 GiB pinned host -> device
        src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
        dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        link_copy_gbps = (1 << 30) / (a.elapsed_time(b) * 1e-3) / 1e9
        del src, dst
    flat = args.path == "flat"
    share = {"none": 0, "kv-group": atlaskv.SHARE_KV_GROUP, "sequence": atlaskv.SHARE_SEQUENCE}[args.share]
    fold = args.fold
    if fold and (flat or share):
        raise SystemExit("--fold applies to the per-row pruned path only")
    if flat and share:
        raise SystemExit("--share applies to the pruned path only")
    DE = case.d
    if fold:
        base, base_off, w_k, w_v, DE = fold_inputs(case, args, dev)
        case.root_k, case.mid_k, case.leaf_k, case.leaf_v = base
        case.root_off, case.mid_off = base_off
        torch.cuda.empty_cache()
    tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, case.mid_off)
    if flat:
        ws = atlaskv.alloc_flat_workspace(tree, case.q, case.seq_k)
    elif fold:
        ws = atlaskv.alloc_folded_workspace(tree, case.q, w_k, case.seq_k, case.K)
    elif share:
        ws = atlaskv.alloc_shared_workspace(tree, case.q, case.seq_k, case.K, share)
    else:
        ws = atlaskv.alloc_workspace(tree, case.q, case.seq_k, case.K)
    out = torch.empty_like(case.q)
    R = case.rows
    nsel = R if not share else case.B * (case.N if share == atlaskv.SHARE_KV_GROUP else 1) * case.Hkv
    sel = [torch.empty(nsel, k, dtype=torch.int32, device=dev) for k in case.K]
    phases = (atlaskv.flat_phase_names() if flat else atlaskv.folded_phase_names() if fold else
              atlaskv.shared_phase_names() if share else atlaskv.phase_names())
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        if flat:
            atlaskv.flat_attend_ex(case.q, tree, case.seq_k, case.seq_v, out, workspace=ws,
                                   phase_events=events, stream=stream)
        elif fold:
            atlaskv.folded_attend_ex(case.q, tree, w_k, w_v, case.seq_k, case.seq_v, case.K, out, workspace=ws,
                                     sel_root=sel[0], sel_mid=sel[1], sel_leaf=sel[2], phase_events=events,
                                     stream=stream)
        elif share:
            atlaskv.shared_attend_ex(case.q, tree, case.seq_k, case.seq_v, case.K, share, out,
                                     workspace=ws, sel_root=sel[0], sel_mid=sel[1], sel_leaf=sel[2],
                                     phase_events=events, stream=stream)
        else:
            atlaskv.hikvp_attend_ex(case.q, tree, case.seq_k, case.seq_v, case.K, out, workspace=ws,
                                    sel_root=sel[0], sel_mid=sel[1], sel_leaf=sel[2],
                                    phase_events=events, stream=stream)

    log(f"{workload}: warmup {args.warmup}, {args.steps} cold steps, {args.steps} warm steps")
    tm = time_steps(step, stream, args.steps, args.warmup, dev)
    ms_per_step = tm["ms_per_step"]
    # per-phase kernel times from separate steps with phase events (the library
    # then runs everything serially on the call's stream)
    nph = args.phase_steps if args.phase_steps is not None else min(args.steps, 20)
    nph = max(1, nph)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(nph)]
    for row in evs:
        for e in row:
            e.record(stream)           # create the underlying HIP events before timing
    torch.cuda.synchronize()
    log(f"{workload}: phase timing {nph} steps")
    for i in range(nph):
        step(evs[i])
    torch.cuda.synchronize()
    phase_ms = {p: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(nph)]))
                for j, p in enumerate(phases)}

    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")
        del src, dst

    tokens = case.B * case.N
    if flat:
        line = flat_line(args, case, tm, phase_ms, tokens)
        tree.close()
        return line
    host_sel = [s.cpu().numpy() for s in sel]
    if fold:  # every row reads the one base tree: KV head 0 for the byte count
        saved = (case.Hkv, case.Hq, case.d)
        case.Hkv, case.d = 1, DE
        ab = algorithmic_bytes(case, host_sel, 0)
        case.Hkv, case.Hq, case.d = saved
        eb = 2 if case.dtype == "bf16" else 4
        seq_fix = 2 * case.B * case.S_kv * case.Hkv * case.d * eb
        qo_fix = 2 * case.rows * case.d * eb
        ab["_total"] += seq_fix - ab["seq_attention"] + qo_fix - ab["_parts"]["q"] - ab["_parts"]["out"]
        ab["_parts"]["sequence_kv"] = ab["seq_attention"] = seq_fix
        ab["_parts"]["q"] = ab["_parts"]["out"] = case.rows * case.d * eb
        ab["_parts"]["projections"] = 2 * case.Hkv * case.d * DE * eb
        ab["_total"] += ab["_parts"]["projections"]
    else:
        ab = algorithmic_bytes(case, host_sel, share)
    recall = None
    if share:
        # leaves of the per-row selection that the shared selection also holds
        ws1 = atlaskv.alloc_workspace(tree, case.q, case.seq_k, case.K)
        own = torch.empty(R, case.K[2], dtype=torch.int32, device=dev)
        atlaskv.hikvp_attend_ex(case.q, tree, case.seq_k, case.seq_v, case.K, torch.empty_like(case.q),
                                workspace=ws1, sel_leaf=own, stream=stream)
        torch.cuda.synchronize()
        own = own.cpu().numpy()
        G = case.Hq // case.Hkv
        rows = np.arange(R)
        h, t = rows % case.Hq, rows // case.Hq
        grp = (t * case.Hkv + h // G) if share == atlaskv.SHARE_KV_GROUP else \
            ((t // case.N) * case.Hkv + h // G)
        hit = tot = 0
        for r in range(R):
            a = set(own[r][own[r] >= 0].tolist())
            hit += len(a & set(host_sel[2][grp[r]].tolist()))
            tot += len(a)
        recall = hit / max(tot, 1)
    dom = max((p for p in phases if p in ab), key=lambda p: phase_ms[p])
    achieved = ab[dom] / (phase_ms[dom] * 1e-3) / 1e9
    on_host = args.tree_placement == "host-leaves"
    traffic = None if (on_host or fold or share) else read_traffic(dom, case.name)
    path_gbps = ab["_total"] / (ms_per_step * 1e-3) / 1e9

    line = {
        "metric": "query tokens/s per layer through HiKVP+merged attention; % of peak HBM GB/s",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.dtype, "data": "synthetic (seeded clustered-Gaussian key tree, Gaussian values, queries and sequence K/V)",
        "config": {"workload": case.name, "B": case.B, "N": case.N, "S_kv": case.S_kv, "Hq": case.Hq,
                   "Hkv": case.Hkv, "d": case.d, "tree": [case.M_R, case.M_I, case.M], "K": list(case.K),
                   "tokens_per_step": tokens, "parallelism": "single GPU",
                   "tree_placement": args.tree_placement, "share": args.share, "fold": fold,
                   **({"fold_width": DE} if fold else {})},
        "timing": tm,
        "warm_value": tokens / (tm["warm_ms_per_step"] * 1e-3),
        "path_hbm": {"compulsory_bytes": ab["_total"], "achieved_gbps": path_gbps,
                     "frac_of_peak": path_gbps / PEAK_HBM_GBPS, "parts": ab["_parts"],
                     "warm_frac_of_peak": ab["_total"] / (tm["warm_ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        "phase_ms": phase_ms,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic, "algorithmic_bytes": ab[dom],
                     "path_frac": path_gbps / PEAK_HBM_GBPS},
        "cpu_baseline": None,
    }
    if share:
        line["recall_vs_per_row"] = recall
    if on_host:
        # leaf keys and values cross the host link; the dominant kernel is bound by it
        peak = PEAK_LINK_GBPS
        line["roofline"].update(bound="host_link", peak=peak, frac=achieved / peak)
        link_b = ab["_parts"]["leaf_keys"] + ab["_parts"]["leaf_values"]
        line["host_link"] = {"bytes": link_b, "achieved_gbps": link_b / (ms_per_step * 1e-3) / 1e9,
                             "peak_gbps": peak, "copy_engine_gbps": link_copy_gbps}
    tree.close()
    del ws, out, sel
    if with_cpu and not args.no_cpu_baseline:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s of oracle time, one core)")
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    del case
    torch.cuda.empty_cache()
    return line


def main():
    args = parse_args()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    atlaskv.lib()
    if args.workload is not None:
        print(json.dumps(run_one(args, args.workload, dev, with_cpu=True)), flush=True)
        return
    # the other target workloads first (stderr), the headline workload last (stdout):
    # the decode and slice workloads, and the m1e6 layer folded onto one base
    # tree of width D_E = 384
    for extra, over in (("m1e7_decode", {}), ("m1e8_slice", {}), ("m1e6", {"fold": True, "fold_width": 384})):
        line = run_one(argparse.Namespace(**{**vars(args), **over}), extra, dev, with_cpu=False)
        print(json.dumps(line), file=sys.stderr, flush=True)
    print(json.dumps(run_one(args, "m1e6", dev, with_cpu=True)), flush=True)


if __name__ == "__main__":
    main()
