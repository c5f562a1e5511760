"""ctypes wrapper of the fp64 CPU oracle (hikvp_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
cpu_baseline leg of the benchmark, never by the GPU library.  It converts
host arrays (numpy or CPU torch tensors) to C-contiguous buffers and marshals
them.  Scoring, Top-K, the KG and sequence softmaxes and the merge run in the
C file; the variant helpers further down (group queries of shared selections,
folded queries and the folded KG half) do their extra steps here in fp64
numpy and math.fsum, each written out in the function that uses it.
"""
import ctypes
import math
import os

import numpy as np

from . import build as _build

F32, BF16, F64 = 0, 1, 2
_I64P = ctypes.POINTER(ctypes.c_int64)
_F64P = ctypes.POINTER(ctypes.c_double)


class _Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int64), ("N", ctypes.c_int64), ("S_kv", ctypes.c_int64),
        ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64), ("d", ctypes.c_int64),
        ("M_R", ctypes.c_int64), ("M_I", ctypes.c_int64), ("M", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("q_kg", ctypes.c_void_p),
        ("root_k", ctypes.c_void_p), ("mid_k", ctypes.c_void_p),
        ("leaf_k", ctypes.c_void_p), ("leaf_v", ctypes.c_void_p),
        ("root_off", _I64P), ("mid_off", _I64P),
        ("seq_k", ctypes.c_void_p), ("seq_v", ctypes.c_void_p),
        ("K", ctypes.c_int32 * 3),
        ("scale", ctypes.c_double),
        ("q_kg_f64", ctypes.c_int32),
    ]


class _Outputs(ctypes.Structure):
    _fields_ = [
        ("sel_R", _I64P), ("sel_I", _I64P), ("sel_L", _I64P),
        ("logit_L", _F64P), ("gap", _F64P), ("n_cand", _I64P),
        ("lse_kg", _F64P), ("lse_seq", _F64P),
        ("lam_kg", _F64P), ("lam_seq", _F64P),
        ("o_kg", _F64P), ("o_seq", _F64P), ("out", _F64P),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        # HIKVP_ORACLE_LIB: another build of the same source (the sanitizer test's)
        path = os.environ.get("HIKVP_ORACLE_LIB") or _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_tree_sizes.argtypes = [ctypes.c_int64, _I64P]
        L.oracle_tree_sizes.restype = ctypes.c_int
        L.oracle_topk.argtypes = [ctypes.c_int64, _F64P, _I64P, ctypes.c_int64, _I64P]
        L.oracle_topk.restype = ctypes.c_int64
        L.oracle_level_scores.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int, _I64P, ctypes.c_int64,
                                          _I64P, _F64P, ctypes.c_int64]
        L.oracle_level_scores.restype = ctypes.c_int64
        L.oracle_candidate_scores.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, _F64P]
        L.oracle_candidate_scores.restype = ctypes.c_int
        rows_sig = [ctypes.POINTER(_Problem), ctypes.c_int64, _I64P, _I64P, _I64P]
        L.oracle_hikvp_rows.argtypes = rows_sig + [ctypes.POINTER(_Outputs)]
        L.oracle_hikvp_rows.restype = ctypes.c_int
        L.oracle_select_mids_rows.argtypes = rows_sig + [ctypes.POINTER(_Outputs)]
        L.oracle_select_mids_rows.restype = ctypes.c_int
        L.oracle_finish_rows.argtypes = rows_sig + [_I64P, _I64P, ctypes.c_void_p, ctypes.c_void_p,
                                                    _I64P, ctypes.POINTER(_Outputs)]
        L.oracle_finish_rows.restype = ctypes.c_int
        L.oracle_flat_rows.argtypes = rows_sig + [ctypes.POINTER(_Outputs)]
        L.oracle_flat_rows.restype = ctypes.c_int
        _lib = L
    return _lib


def _host(x):
    """(numpy array, storage code) for a numpy array or a CPU torch tensor."""
    if x is None:
        return None, None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy(), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            if x.dtype == torch.float64:
                return x.numpy(), F64
            if x.dtype == torch.int64:
                return x.numpy(), None
            raise TypeError(f"unsupported tensor dtype {x.dtype}")
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.int64:
        return x, None
    raise TypeError(f"unsupported array dtype {x.dtype}")


def _offsets(x):
    """int64 numpy copy of CSR offsets given as a list, array or tensor."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _vp(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _ip(a):
    return None if a is None else a.ctypes.data_as(_I64P)


def _fp(a):
    return None if a is None else a.ctypes.data_as(_F64P)


class Problem:
    """One HiKVP layer call: q [B,N,Hq,d], tree keys [Hkv,M_x,d], leaf values,
    int64 child offsets, sequence K/V [B,S_kv,Hkv,d] (None -> no sequence).
    q_kg (optional, [B,N,Hq,d]) is the KG query, in the storage type or in
    fp64: an exact query (a sum or product of stored values) is ranked and
    scored as it is, never rounded to the storage type."""

    def __init__(self, q, root_k, mid_k, leaf_k, leaf_v, root_off, mid_off,
                 seq_k, seq_v, K, scale=None, q_kg=None):
        self._args = (q, root_k, mid_k, leaf_k, leaf_v, root_off, mid_off, seq_k, seq_v, K)
        self._kw = dict(scale=scale, q_kg=q_kg)
        self._keep = []
        qa, dt = _host(q)
        B, N, Hq, d = qa.shape
        rk, dt_r = _host(root_k)
        mk, dt_m = _host(mid_k)
        lk, dt_l = _host(leaf_k)
        lv, _ = _host(leaf_v)
        ro = _offsets(root_off)
        mo = _offsets(mid_off)
        sk, _ = _host(seq_k)
        sv, _ = _host(seq_v)
        qk, dt_qk = _host(q_kg)
        for other in (dt_r, dt_m):
            if other != dt:
                raise TypeError("all floating inputs must share one storage type")
        if qk is not None and dt_qk not in (dt, F64):
            raise TypeError("q_kg must be in the storage type or fp64 (an exact query)")
        Hkv = rk.shape[0]
        self.shape = dict(B=B, N=N, Hq=Hq, Hkv=Hkv, d=d, M_R=rk.shape[1], M_I=mk.shape[1],
                          M=(lk.shape[1] if lk is not None else int(mo[-1])),
                          S_kv=(sk.shape[1] if sk is not None else 0))
        self.K = tuple(int(k) for k in K)
        self.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        self.dtype = dt
        P = _Problem()
        P.dtype = dt
        for k in ("B", "N", "S_kv", "Hq", "Hkv", "d", "M_R", "M_I", "M"):
            setattr(P, k, self.shape[k])
        P.q, P.q_kg = _vp(qa), _vp(qk)
        P.root_k, P.mid_k, P.leaf_k, P.leaf_v = _vp(rk), _vp(mk), _vp(lk), _vp(lv)
        P.root_off, P.mid_off = _ip(ro), _ip(mo)
        P.seq_k, P.seq_v = _vp(sk), _vp(sv)
        P.K = (ctypes.c_int32 * 3)(*self.K)
        P.scale = self.scale
        P.q_kg_f64 = 1 if (qk is not None and dt_qk == F64 and dt != F64) else 0
        self._P = P
        self._keep = [qa, rk, mk, lk, lv, ro, mo, sk, sv, qk]
        self.root_off, self.mid_off = ro, mo


def all_rows(B, N, Hq):
    """(b, n, h) of every row in memory order of [B, N, Hq]."""
    b, n, h = np.meshgrid(np.arange(B), np.arange(N), np.arange(Hq), indexing="ij")
    return np.stack([b.ravel(), n.ravel(), h.ravel()], axis=1).astype(np.int64)


def _alloc_outputs(nrows, K, d):
    KR, KI, KL = K
    o = dict(
        sel_R=np.full((nrows, KR), -1, np.int64), sel_I=np.full((nrows, KI), -1, np.int64),
        sel_L=np.full((nrows, KL), -1, np.int64), logit_L=np.full((nrows, KL), np.nan),
        gap=np.full((nrows, 3), np.inf), n_cand=np.zeros((nrows, 3), np.int64),
        lse_kg=np.zeros(nrows), lse_seq=np.zeros(nrows), lam_kg=np.zeros(nrows),
        lam_seq=np.zeros(nrows), o_kg=np.zeros((nrows, d)), o_seq=np.zeros((nrows, d)),
        out=np.zeros((nrows, d)))
    O = _Outputs()
    for k in ("sel_R", "sel_I", "sel_L", "n_cand"):
        setattr(O, k, _ip(o[k]) if o[k].size else None)
    for k in ("logit_L", "gap", "lse_kg", "lse_seq", "lam_kg", "lam_seq", "o_kg", "o_seq", "out"):
        setattr(O, k, _fp(o[k]) if o[k].size else None)
    return o, O


def _rows(rows):
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    return r, np.ascontiguousarray(r[:, 0]), np.ascontiguousarray(r[:, 1]), np.ascontiguousarray(r[:, 2])


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def hikvp_rows(prob: Problem, rows):
    """Full forward for the given (b, n, h) rows; dict of numpy arrays."""
    r, b, n, h = _rows(rows)
    o, O = _alloc_outputs(len(r), prob.K, prob.shape["d"])
    _check(lib().oracle_hikvp_rows(ctypes.byref(prob._P), len(r), _ip(b), _ip(n), _ip(h),
                                   ctypes.byref(O)), "oracle_hikvp_rows")
    return o


def flat_rows(prob: Problem, rows):
    """Unpruned equivalent attention (the KG softmax runs over every leaf of
    the row's KV head) for the given rows; dict of numpy arrays (selection
    entries stay at their -1 / NaN fill)."""
    r, b, n, h = _rows(rows)
    o, O = _alloc_outputs(len(r), prob.K, prob.shape["d"])
    _check(lib().oracle_flat_rows(ctypes.byref(prob._P), len(r), _ip(b), _ip(n), _ip(h),
                                  ctypes.byref(O)), "oracle_flat_rows")
    return o


# ---------------------------------------------------------------------------
# shared selections: one descent per group of rows
# ---------------------------------------------------------------------------

SHARE_KV_GROUP, SHARE_SEQUENCE = 1, 2


def group_queries(prob: Problem, share):
    """Each row's group query [B, N, Hq, d] as fp64 (torch.float64).

    The group of row (b, n, h) is every row of the same sequence b and KV head
    g = h // G at token n (share = SHARE_KV_GROUP) or at any token
    (SHARE_SEQUENCE).  Its query is the exact sum of the members' stored KG
    queries, not rounded to the storage type: <sum_m q_m, k> is the sum of
    the members' logits, so ranking nodes by it ranks them by the summed
    logits.  math.fsum gives the exact sum rounded to fp64, which is the exact
    sum itself whenever that fits 53 bits (always, unless the members'
    magnitudes span ~2^40).
    """
    q, q_kg = prob._args[0], prob._kw["q_kg"]
    qa, dt = _host(q if q_kg is None else q_kg)
    x = qa.view(np.uint16).astype(np.uint32) << 16 if dt == BF16 else qa
    x = np.asarray(x.view(np.float32) if dt == BF16 else x, dtype=np.float64)
    B, N, Hq, d = x.shape
    s = prob.shape
    G = Hq // s["Hkv"]
    if share not in (SHARE_KV_GROUP, SHARE_SEQUENCE):
        raise ValueError("share must be SHARE_KV_GROUP or SHARE_SEQUENCE")
    xg = x.reshape(B, N, s["Hkv"], G, d)
    g = np.zeros((B, N, s["Hkv"], d))
    for b in range(B):
        for kv in range(s["Hkv"]):
            if share == SHARE_SEQUENCE:
                members = xg[b, :, kv].reshape(N * G, d)
                g[b, :, kv] = [math.fsum(members[:, t]) for t in range(d)]
            else:
                for n in range(N):
                    g[b, n, kv] = [math.fsum(xg[b, n, kv, :, t]) for t in range(d)]
    full = np.repeat(g, G, axis=2)                                   # back to [B, N, Hq, d]
    import torch
    return torch.from_numpy(np.ascontiguousarray(full))


def shared_rows(prob: Problem, rows, share):
    """Shared-selection variant for the given rows: the descent (roots, mids,
    leaves, Top-K per level) runs on the row's group query; the row's KG
    softmax then runs over the group's selected leaves with its own KG query
    and logits, and merges with its own sequence half as in hikvp_rows.
    Returns the finish outputs plus the group selections (sel_R, sel_I,
    sel_L, gap) under the group query."""
    gq = group_queries(prob, share)
    args = prob._args
    grp = Problem(*args, scale=prob._kw["scale"], q_kg=gq)
    sel = hikvp_rows(grp, rows)
    r = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    G = prob.shape["Hq"] // prob.shape["Hkv"]
    lk, lv = args[3], args[4]
    off, idx, ks, vs = [0], [], [], []
    for i, (b, n, h) in enumerate(r):
        lv_i = [int(m) for m in sel["sel_L"][i] if m >= 0]
        idx.extend(lv_i)
        ks.append(lk[h // G, lv_i])
        vs.append(lv[h // G, lv_i])
        off.append(off[-1] + len(lv_i))
    import torch
    ks = torch.cat(ks) if len(idx) else lk[0, :0]
    vs = torch.cat(vs) if len(idx) else lv[0, :0]
    fin = finish_rows(prob, r, off, idx, ks, vs, forced_sel_L=sel["sel_L"])
    for k in ("sel_R", "sel_I", "sel_L", "gap", "n_cand"):
        fin[k] = sel[k]
    return fin


# ---------------------------------------------------------------------------
# folded projections: one base-embedding tree for every head
# ---------------------------------------------------------------------------

def _as_f64(t):
    a, dt = _host(t)
    if dt == BF16:
        return (a.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64), dt
    return np.asarray(a, dtype=np.float64), dt


def folded_query(q_kg, w_k, rows=None):
    """q'[b,n,h] = W_K[g]^T q_kg[b,n,h] as fp64 (torch.float64): the exact
    sum of the products (math.fsum over the head dim), not rounded to the
    storage type.  W_K [Hkv, d, D_E] maps a base key k (width D_E) to the
    head's projected key W_K[g] k, so <q_kg, W_K[g] k> = <q', k> and ranking
    base keys by <q', k> ranks the projected keys by their logits.  rows: only
    these (b, n, h) are formed (the others stay zero)."""
    q, dt = _as_f64(q_kg)
    w, _ = _as_f64(w_k)
    B, N, Hq, d = q.shape
    Hkv, d2, DE = w.shape
    G = Hq // Hkv
    out = np.zeros((B, N, Hq, DE))
    todo = all_rows(B, N, Hq) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    for b, n, h in todo:
        prod = w[h // G] * q[b, n, h][:, None]                  # [d, D_E], exact products
        out[b, n, h] = [math.fsum(prod[:, j]) for j in range(DE)]
    import torch
    return torch.from_numpy(out)


def folded_rows(base_tree, q, w_k, w_v, seq_k, seq_v, K, rows, scale=None, q_kg=None,
                forced_sel_I=None, forced_sel_L=None):
    """Folded-projection variant (方法细节 › KBLaM中的矩形注意力 gives the
    projected keys and values W_K k and W_V v of per-layer heads; one base
    tree serves every head): the descent over the base tree (root_k, mid_k,
    leaf_k, leaf_v with one head, width D_E, offsets) runs on the folded
    queries q'; the KG half of row (b, n, h) is W_V[g] applied to the
    softmax-weighted base values, merged with the causal sequence half over
    seq_k / seq_v [B, S, Hkv, d].  Returns dict(out, lse_kg, lse_seq, sel_R,
    sel_I, sel_L, gap, o_kg).

    Replay: with forced_sel_I and forced_sel_L ([rows, K_I], [rows, K_L],
    -1 padded) the leaf candidates are the children of the given mids and the
    KG softmax runs over the given leaves instead of the oracle's choice."""
    import torch
    root_k, mid_k, leaf_k, leaf_v, root_off, mid_off = base_tree
    d = q.shape[-1]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    qf = folded_query(q if q_kg is None else q_kg, w_k, rows)
    # no sequence half here: the descent reads only the exact KG query qf
    # (q is a placeholder of the storage type that is never read)
    stub_q = torch.zeros(qf.shape, dtype=root_k.dtype)
    P = Problem(stub_q, root_k, mid_k, leaf_k, leaf_v, root_off, mid_off, None, None, K, scale=sc, q_kg=qf)
    r = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    ph1 = select_mids_rows(P, r)                 # roots and mids under q'
    KL = int(K[2])
    lv64, _ = _as_f64(leaf_v)
    DE = lv64.shape[-1]
    sel_L = np.full((len(r), KL), -1, np.int64)
    gap = ph1["gap"].copy()
    a = np.full(len(r), -np.inf)
    o_base = np.zeros((len(r), DE))
    for i, (b, n, h) in enumerate(r):
        sel_mid = ph1["sel_I"][i] if forced_sel_I is None else np.asarray(forced_sel_I[i])
        parents = [int(m) for m in sel_mid if m >= 0]
        cand, score = level_scores(P, b, n, h, 2, parents) if parents and KL > 0 else (np.zeros(0, np.int64), np.zeros(0))
        if forced_sel_L is not None:
            where = {int(c): j for j, c in enumerate(cand)}
            pos = np.asarray([where[int(x)] for x in forced_sel_L[i] if x >= 0], np.int64)
        else:
            pos = topk(score, cand, KL) if len(cand) and KL > 0 else np.zeros(0, np.int64)
        sel_L[i, :len(pos)] = cand[pos]
        ranked = sorted(range(len(cand)), key=lambda j: (-score[j], cand[j]))
        if 0 < KL < len(cand):
            s0, s1 = score[ranked[KL - 1]], score[ranked[KL]]
            gap[i, 2] = abs(s0 - s1) / max(abs(s0), abs(s1)) if max(abs(s0), abs(s1)) > 0 else 0.0
        if len(pos):
            lg = score[pos]
            a[i] = lg.max() + math.log(math.fsum(np.exp(lg - lg.max())))
            w = np.exp(lg - a[i])
            o_base[i] = w @ lv64[0, cand[pos]]
    kg = dict(sel_R=ph1["sel_R"], sel_I=ph1["sel_I"], sel_L=sel_L, gap=gap, lse_kg=a, o_kg=o_base)
    # the sequence half alone: the same oracle with the KG half emptied (K = 0)
    # over a one-node stub tree with the layer's KV heads and head dim
    sq = None
    if seq_k is not None:
        stub = torch.zeros(w_k.shape[0], 1, d, dtype=q.dtype)
        off = torch.tensor([0, 1], dtype=torch.int64)
        sq = hikvp_rows(Problem(q, stub, stub, stub, stub, off, off, seq_k, seq_v, (0, 0, 0), scale=sc),
                        rows)
    wv, _ = _as_f64(w_v)
    G = q.shape[2] // w_k.shape[0]
    o_kg = np.stack([wv[h // G] @ kg["o_kg"][i] for i, (b, n, h) in enumerate(r)]) if len(r) else np.zeros((0, d))
    a = kg["lse_kg"]
    if sq is None:
        c = np.full(len(r), -np.inf)
        o_seq = np.zeros_like(o_kg)
    else:
        c, o_seq = sq["lse_seq"], sq["o_seq"]
    out = np.zeros_like(o_kg)
    for i in range(len(r)):
        if a[i] == -np.inf and c[i] == -np.inf:
            raise RuntimeError("both halves empty")
        lam = 0.0 if a[i] == -np.inf else (1.0 if c[i] == -np.inf else 1.0 / (1.0 + math.exp(c[i] - a[i])))
        out[i] = lam * o_kg[i] + (1.0 - lam) * o_seq[i]
    return dict(out=out, o_kg=o_kg, lse_kg=a, lse_seq=c, sel_R=kg["sel_R"], sel_I=kg["sel_I"],
                sel_L=kg["sel_L"], gap=kg["gap"])


def select_mids_rows(prob: Problem, rows):
    """Two-phase mode, phase 1: sel_R, sel_I, gaps for the given rows."""
    r, b, n, h = _rows(rows)
    o, O = _alloc_outputs(len(r), prob.K, prob.shape["d"])
    _check(lib().oracle_select_mids_rows(ctypes.byref(prob._P), len(r), _ip(b), _ip(n), _ip(h),
                                         ctypes.byref(O)), "oracle_select_mids_rows")
    return o


def finish_rows(prob: Problem, rows, cand_off, cand_idx, cand_k, cand_v, forced_sel_L=None):
    """Two-phase phase 2 / replay: leaf candidates passed explicitly per row."""
    r, b, n, h = _rows(rows)
    co = np.ascontiguousarray(np.asarray(cand_off, dtype=np.int64))
    ci = np.ascontiguousarray(np.asarray(cand_idx, dtype=np.int64))
    ck, dk = _host(cand_k)
    cv, _ = _host(cand_v)
    if dk != prob.dtype:
        raise TypeError("candidate storage type differs from the problem's")
    fs = None if forced_sel_L is None else np.ascontiguousarray(np.asarray(forced_sel_L, dtype=np.int64))
    o, O = _alloc_outputs(len(r), prob.K, prob.shape["d"])
    _check(lib().oracle_finish_rows(ctypes.byref(prob._P), len(r), _ip(b), _ip(n), _ip(h),
                                    _ip(co), _ip(ci), _vp(ck), _vp(cv), _ip(fs), ctypes.byref(O)),
           "oracle_finish_rows")
    return o


def level_scores(prob: Problem, b, n, h, level, parents=()):
    """Candidates of one row at one level with their fp64 scaled scores."""
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int64))
    s = prob.shape
    cap = max(1, s["M_R"], s["M_I"], s["M"])
    if level == 1:
        cap = max(1, int(np.diff(prob.root_off).max(initial=0)) * max(1, len(par)))
    elif level == 2:
        cap = max(1, int(np.diff(prob.mid_off).max(initial=0)) * max(1, len(par)))
    cand = np.zeros(cap, np.int64)
    score = np.zeros(cap)
    c = lib().oracle_level_scores(ctypes.byref(prob._P), int(b), int(n), int(h), int(level),
                                  _ip(par) if len(par) else None, len(par), _ip(cand), _fp(score), cap)
    if c < 0:
        raise RuntimeError("oracle_level_scores: capacity exceeded")
    return cand[:c], score[:c]


def candidate_scores(prob: Problem, b, n, h, cand_k):
    """fp64 scaled scores of explicitly given candidate keys [nc, d] (the
    problem's storage type) for row (b, n, h)."""
    ck, dk = _host(cand_k)
    if len(ck) and dk != prob.dtype:
        raise TypeError("candidate storage type differs from the problem's")
    out = np.zeros(max(1, len(ck)))
    _check(lib().oracle_candidate_scores(ctypes.byref(prob._P), int(b), int(n), int(h), len(ck),
                                         _vp(ck) if len(ck) else None, _fp(out)),
           "oracle_candidate_scores")
    return out[:len(ck)]


def tree_sizes(M):
    """(S, M_I, M_R) from the clustering section's level-size formulas."""
    out = np.zeros(3, np.int64)
    _check(lib().oracle_tree_sizes(int(M), _ip(out)), "oracle_tree_sizes")
    return int(out[0]), int(out[1]), int(out[2])


def topk(score, index, K):
    """Positions of the first min(K, n) by (score desc, index asc)."""
    s = np.ascontiguousarray(np.asarray(score, dtype=np.float64))
    i = np.ascontiguousarray(np.asarray(index, dtype=np.int64))
    out = np.zeros(max(1, min(int(K), len(s))), np.int64)
    k = lib().oracle_topk(len(s), _fp(s), _ip(i), int(K), _ip(out))
    if k < 0:
        raise MemoryError("oracle_topk")
    return out[:k]
