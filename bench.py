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
KERNEL_SOURCES = [os.path.join(ROOT, "hierarchical_kv_pruning_amd", "csrc", f)
                  for f in ("hikvp_device.h", "hikvp_select.hip", "hikvp_seq.hip")]
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
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
            "leaf_score_overflow": 0,
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
        "leaf_score_overflow": 0,
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


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample, two-phase: leaves fetched per row)
# ---------------------------------------------------------------------------

def cpu_baseline(case, seconds):
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
                      f"fp64 single-thread C oracle, {t2:.1f} s; leaf candidates copied to host "
                      f"per row outside the timed calls; tokens/s = rows/s / Hq"}


# ---------------------------------------------------------------------------

def flat_line(args, case, ms_per_step, phase_ms, cold, tokens):
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
    return {
        "metric": "query tokens/s per layer through unpruned equivalent attention (all M leaves)",
        "value": tokens / (ms_per_step * 1e-3), "unit": "query tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": case.dtype,
        "data": "synthetic (seeded clustered-Gaussian key tree, Gaussian values, queries and sequence K/V)",
        "config": {"workload": case.name, "path": "flat", "B": case.B, "N": case.N, "S_kv": case.S_kv,
                   "Hq": case.Hq, "Hkv": case.Hkv, "d": case.d, "M": case.M, "tokens_per_step": tokens,
                   "parallelism": "single GPU", "tree_placement": args.tree_placement},
        "path_hbm": {"compulsory_bytes": total_b, "achieved_gbps": total_b / (ms_per_step * 1e-3) / 1e9,
                     "cold_ms_per_step": cold},
        "phase_ms": phase_ms, "roofline": roof, "cpu_baseline": None,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="m1e6", choices=sorted(synth.CONFIGS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="extra steps timed one by one after evicting the 256 MB MALL")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--path", default="hikvp", choices=["hikvp", "flat"],
                    help="flat: the unpruned equivalent attention (KG softmax over every leaf)")
    ap.add_argument("--share", default="none", choices=["none", "kv-group", "sequence"],
                    help="shared selections: one descent per KV head and token, or per KV head "
                         "and sequence (pruned path only)")
    ap.add_argument("--fold", action="store_true",
                    help="folded projections: one-head base tree (head 0 of the workload's tree, width "
                         "D_E = d) shared by all heads through random per-head W_K / W_V [Hkv, d, D_E]")
    ap.add_argument("--tree-placement", default="hbm", choices=["hbm", "host-leaves"],
                    help="host-leaves: leaf keys and values in pinned host memory, read by the "
                         "kernels over the host link (roots, mids, offsets stay in HBM)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    atlaskv.lib()
    log(f"workload {args.workload}: generating on {torch.cuda.get_device_name(0)}")
    case = synth.make_case(args.workload, device=dev)
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
    tree = atlaskv.TreeView(case.root_k, case.mid_k, case.leaf_k, case.leaf_v, case.root_off, case.mid_off)
    flat = args.path == "flat"
    share = {"none": 0, "kv-group": atlaskv.SHARE_KV_GROUP, "sequence": atlaskv.SHARE_SEQUENCE}[args.share]
    fold = args.fold
    if fold and (flat or share):
        print("--fold applies to the per-row pruned path only", file=sys.stderr)
        sys.exit(2)
    if fold:
        # the base tree: head 0 of the workload's tree; per-head projections of the layer
        tree.close()
        base = [t[:1].contiguous() for t in (case.root_k, case.mid_k, case.leaf_k, case.leaf_v)]
        tree = atlaskv.TreeView(*base, case.root_off, case.mid_off)
        gen = torch.Generator(device=dev).manual_seed(17)
        w_k = (torch.randn(case.Hkv, case.d, case.d, generator=gen, device=dev) / case.d ** 0.5).to(case.q.dtype)
        w_v = (torch.randn(case.Hkv, case.d, case.d, generator=gen, device=dev) / case.d ** 0.5).to(case.q.dtype)
        case.root_k, case.mid_k, case.leaf_k, case.leaf_v = base
        torch.cuda.empty_cache()
    if flat and share:
        print("--share applies to the pruned path only", file=sys.stderr)
        sys.exit(2)
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
            return
        if fold:
            atlaskv.folded_attend_ex(case.q, tree, w_k, w_v, case.seq_k, case.seq_v, case.K, out, workspace=ws,
                                     sel_root=sel[0], sel_mid=sel[1], sel_leaf=sel[2], phase_events=events,
                                     stream=stream)
            return
        if share:
            atlaskv.shared_attend_ex(case.q, tree, case.seq_k, case.seq_v, case.K, share, out,
                                     workspace=ws, sel_root=sel[0], sel_mid=sel[1], sel_leaf=sel[2],
                                     phase_events=events, stream=stream)
            return
        atlaskv.hikvp_attend_ex(case.q, tree, case.seq_k, case.seq_v, case.K, out, workspace=ws,
                                sel_root=sel[0], sel_mid=sel[1], sel_leaf=sel[2],
                                phase_events=events, stream=stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record(stream)           # create the underlying HIP events before timing
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    # per-phase kernel times from separate steps with phase events (the library
    # then runs the sequence half after the KG half instead of beside it)
    log(f"phase timing {args.steps} steps")
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    phase_ms = {p: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
                for j, p in enumerate(phases)}

    # cold steps: MALL evicted between steps, each step timed alone
    cold = None
    if args.cold_reps > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        ts = []
        for _ in range(args.cold_reps):
            flush.add_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        cold = float(np.median(ts))
        del flush

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
        print(json.dumps(flat_line(args, case, ms_per_step, phase_ms, cold, tokens)), flush=True)
        tree.close()
        return
    host_sel = [s.cpu().numpy() for s in sel]
    if fold:  # every row reads the one base tree: KV head 0 for the byte count
        saved = (case.Hkv, case.Hq)
        case.Hkv, case.Hq = 1, case.Hq
        ab = algorithmic_bytes(case, host_sel, 0)
        case.Hkv, case.Hq = saved
        seq_fix = 2 * case.B * case.S_kv * case.Hkv * case.d * (2 if case.dtype == "bf16" else 4)
        ab["_total"] += seq_fix - ab["seq_attention"]
        ab["_parts"]["sequence_kv"] = ab["seq_attention"] = seq_fix
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
    traffic = None if on_host else read_traffic(dom, case.name)
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
                   "tree_placement": args.tree_placement, "share": args.share, "fold": fold},
        "path_hbm": {"compulsory_bytes": ab["_total"], "achieved_gbps": path_gbps,
                     "frac_of_peak": path_gbps / PEAK_HBM_GBPS, "parts": ab["_parts"],
                     "cold_ms_per_step": cold},
        "phase_ms": phase_ms,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic, "algorithmic_bytes": ab[dom]},
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
    if not args.no_cpu_baseline:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s of oracle time)")
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
        line["cpu_baseline"]["host"] = {"nproc": os.cpu_count()}
    tree.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
