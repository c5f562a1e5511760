"""ctypes binding of libatlaskv.so (C ABI in include/atlaskv.h).

Argument marshalling only: torch tensors are described as atlaskv_tensor
structs (device pointer, dtype, shape, element strides); every step of the
computation runs in the library's HIP kernels.  torch provides the device
memory (including the workspace) and the stream.

The library must be built (`python -m hierarchical_kv_pruning_amd.build`);
loading fails loudly otherwise -- there is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ATLASKV_LIB names another build of the same sources (the host-sanitizer test's)
LIB_PATH = os.environ.get("ATLASKV_LIB") or os.path.join(_HERE, "libatlaskv.so")

OK, ERR_NULL, ERR_DTYPE, ERR_SHAPE, ERR_TREE, ERR_K, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP = range(9)
STATUS_NAMES = ["OK", "ERR_NULL", "ERR_DTYPE", "ERR_SHAPE", "ERR_TREE", "ERR_K", "ERR_WORKSPACE",
                "ERR_UNSUPPORTED", "ERR_HIP"]
F32, BF16 = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}

# every exported symbol of include/atlaskv.h
EXPORTS = ["atlaskv_build_tree_view", "atlaskv_destroy_tree_view", "atlaskv_tree_view_set_workspace",
           "atlaskv_hikvp_workspace_size", "atlaskv_hikvp_attend", "atlaskv_hikvp_attend_ex",
           "atlaskv_check_args", "atlaskv_tree_view_describe", "atlaskv_tree_view_placement",
           "atlaskv_flat_workspace_size", "atlaskv_flat_attend_ex", "atlaskv_flat_check_args",
           "atlaskv_flat_phase_count", "atlaskv_flat_phase_name", "atlaskv_shared_workspace_size",
           "atlaskv_shared_attend_ex", "atlaskv_shared_check_args", "atlaskv_shared_phase_count",
           "atlaskv_shared_phase_name", "atlaskv_folded_workspace_size", "atlaskv_folded_attend_ex",
           "atlaskv_folded_check_args", "atlaskv_folded_phase_count", "atlaskv_folded_phase_name",
           "atlaskv_hikvp_attend_noalloc", "atlaskv_phase_count", "atlaskv_noalloc_scratch_bytes",
           "atlaskv_phase_name", "atlaskv_last_error", "atlaskv_version"]


class AtlasKVError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {message}")


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class AttendOpts(ctypes.Structure):
    _fields_ = [("q_kg", ctypes.POINTER(Tensor)), ("scale", ctypes.c_float),
                ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t),
                ("sel_root", ctypes.c_void_p), ("sel_mid", ctypes.c_void_p),
                ("sel_leaf", ctypes.c_void_p), ("lse_kg", ctypes.c_void_p),
                ("lse_seq", ctypes.c_void_p), ("phase_events", ctypes.POINTER(ctypes.c_void_p)),
                ("n_phase_events", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m hierarchical_kv_pruning_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        T = P(Tensor)
        i32x3 = P(ctypes.c_int32)
        L.atlaskv_build_tree_view.argtypes = [T, T, T, T, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, P(ctypes.c_void_p)]
        L.atlaskv_destroy_tree_view.argtypes = [ctypes.c_void_p]
        L.atlaskv_tree_view_set_workspace.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
        L.atlaskv_hikvp_workspace_size.argtypes = [ctypes.c_void_p, T, T, i32x3, P(ctypes.c_size_t)]
        L.atlaskv_hikvp_attend.argtypes = [T, ctypes.c_void_p, T, T, i32x3, T]
        L.atlaskv_hikvp_attend_ex.argtypes = [T, ctypes.c_void_p, T, T, i32x3, T, P(AttendOpts)]
        L.atlaskv_hikvp_attend_noalloc.argtypes = [T, ctypes.c_void_p, T, T, i32x3, T, P(AttendOpts)]
        L.atlaskv_noalloc_scratch_bytes.argtypes = []
        L.atlaskv_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.atlaskv_check_args.argtypes = [T, ctypes.c_void_p, T, T, i32x3, T, P(AttendOpts)]
        L.atlaskv_tree_view_describe.argtypes = [T, T, T, T, ctypes.c_int64, ctypes.c_int64,
                                                 P(ctypes.c_void_p)]
        L.atlaskv_tree_view_placement.argtypes = [ctypes.c_void_p]
        L.atlaskv_flat_workspace_size.argtypes = [ctypes.c_void_p, T, T, P(ctypes.c_size_t)]
        L.atlaskv_flat_attend_ex.argtypes = [T, ctypes.c_void_p, T, T, T, P(AttendOpts)]
        L.atlaskv_flat_check_args.argtypes = [T, ctypes.c_void_p, T, T, T, P(AttendOpts)]
        L.atlaskv_shared_workspace_size.argtypes = [ctypes.c_void_p, T, T, i32x3, ctypes.c_int32,
                                                    P(ctypes.c_size_t)]
        L.atlaskv_shared_attend_ex.argtypes = [T, ctypes.c_void_p, T, T, i32x3, ctypes.c_int32, T,
                                               P(AttendOpts)]
        L.atlaskv_shared_check_args.argtypes = [T, ctypes.c_void_p, T, T, i32x3, ctypes.c_int32, T,
                                                P(AttendOpts)]
        L.atlaskv_folded_workspace_size.argtypes = [ctypes.c_void_p, T, T, T, i32x3, P(ctypes.c_size_t)]
        L.atlaskv_folded_attend_ex.argtypes = [T, ctypes.c_void_p, T, T, T, T, i32x3, T, P(AttendOpts)]
        L.atlaskv_folded_check_args.argtypes = [T, ctypes.c_void_p, T, T, T, T, i32x3, T, P(AttendOpts)]
        for name in EXPORTS[:-4]:
            getattr(L, name).restype = ctypes.c_int
        L.atlaskv_flat_phase_count.restype = ctypes.c_int32
        L.atlaskv_flat_phase_name.argtypes = [ctypes.c_int32]
        L.atlaskv_flat_phase_name.restype = ctypes.c_char_p
        L.atlaskv_shared_phase_count.restype = ctypes.c_int32
        L.atlaskv_shared_phase_name.argtypes = [ctypes.c_int32]
        L.atlaskv_shared_phase_name.restype = ctypes.c_char_p
        L.atlaskv_folded_phase_count.restype = ctypes.c_int32
        L.atlaskv_folded_phase_name.argtypes = [ctypes.c_int32]
        L.atlaskv_folded_phase_name.restype = ctypes.c_char_p
        L.atlaskv_phase_count.restype = ctypes.c_int32
        L.atlaskv_phase_name.argtypes = [ctypes.c_int32]
        L.atlaskv_phase_name.restype = ctypes.c_char_p
        L.atlaskv_last_error.restype = ctypes.c_char_p
        L.atlaskv_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _raise(status):
    if status != OK:
        raise AtlasKVError(status, lib().atlaskv_last_error().decode())


def describe(t):
    """atlaskv_tensor for a torch tensor (None -> None)."""
    if t is None:
        return None
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    d = Tensor()
    d.data = t.data_ptr()
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(x):
    return None if x is None else ctypes.byref(x)


def _k(K):
    return (ctypes.c_int32 * 3)(*[int(k) for k in K])


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


class TreeView:
    """atlaskv_build_tree_view / atlaskv_destroy_tree_view.  Keeps the tree
    tensors alive as long as the view exists."""

    def __init__(self, root_k, mid_k, leaf_k, leaf_v, root_child_off, mid_child_off, stream=None):
        self._keep = (root_k, mid_k, leaf_k, leaf_v, root_child_off, mid_child_off)
        for off in (root_child_off, mid_child_off):
            if off.dtype != torch.int64 or not off.is_contiguous():
                raise TypeError("child offsets must be contiguous int64 tensors")
        # any tree array may be pinned host memory; the view runs on the device of
        # its device-resident arrays (else the current device)
        dev = next((t.device for t in self._keep if t.is_cuda), None)
        if dev is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.handle = ctypes.c_void_p()
        self._descs = [describe(t) for t in (root_k, mid_k, leaf_k, leaf_v)]
        st = lib().atlaskv_build_tree_view(*[ctypes.byref(x) for x in self._descs],
                                           ctypes.c_void_p(root_child_off.data_ptr()),
                                           ctypes.c_void_p(mid_child_off.data_ptr()),
                                           _stream_handle(stream, dev),
                                           ctypes.byref(self.handle))
        _raise(st)
        self.device = dev
        self._workspace = None

    @classmethod
    def describe_only(cls, root_k, mid_k, leaf_k, leaf_v, max_root_fanout, max_mid_fanout):
        """atlaskv_tree_view_describe: a host-only view for argument checks."""
        self = cls.__new__(cls)
        self._keep = (root_k, mid_k, leaf_k, leaf_v)
        self.handle = ctypes.c_void_p()
        self._descs = [describe(t) for t in (root_k, mid_k, leaf_k, leaf_v)]
        _raise(lib().atlaskv_tree_view_describe(*[ctypes.byref(x) for x in self._descs],
                                                int(max_root_fanout), int(max_mid_fanout),
                                                ctypes.byref(self.handle)))
        self.device = root_k.device
        self._workspace = None
        return self

    @property
    def placement(self):
        """atlaskv_tree_view_placement: bit i set when tree array i (root_k,
        mid_k, leaf_k, leaf_v, root offsets, mid offsets) is pinned host memory."""
        return lib().atlaskv_tree_view_placement(self.handle)

    def set_workspace(self, ws):
        """atlaskv_tree_view_set_workspace with a uint8 device tensor (None detaches)."""
        self._workspace = ws
        ptr = ctypes.c_void_p(ws.data_ptr() if ws is not None else 0)
        _raise(lib().atlaskv_tree_view_set_workspace(self.handle, ptr, 0 if ws is None else ws.numel()))

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().atlaskv_destroy_tree_view(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def build_tree_view(root_k, mid_k, leaf_k, leaf_v, root_child_off, mid_child_off, stream=None):
    return TreeView(root_k, mid_k, leaf_k, leaf_v, root_child_off, mid_child_off, stream)


def hikvp_workspace_size(tree, q, seq_k, K):
    n = ctypes.c_size_t()
    dq, dk = describe(q), describe(seq_k)
    _raise(lib().atlaskv_hikvp_workspace_size(tree.handle, ctypes.byref(dq), _ref(dk), _k(K), ctypes.byref(n)))
    return n.value


def alloc_workspace(tree, q, seq_k, K):
    """A torch uint8 device buffer large enough for an attend call (256-byte aligned)."""
    n = hikvp_workspace_size(tree, q, seq_k, K)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def _opts(q_kg=None, scale=None, stream=None, workspace=None, sel_root=None, sel_mid=None,
          sel_leaf=None, lse_kg=None, lse_seq=None, phase_events=None, device=None):
    o = AttendOpts()
    keep = []
    if phase_events:
        arr = (ctypes.c_void_p * len(phase_events))(*[ev.cuda_event for ev in phase_events])
        keep.append(arr)
        o.phase_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        o.n_phase_events = len(phase_events)
    if q_kg is not None:
        dk = describe(q_kg)
        keep.append(dk)
        o.q_kg = ctypes.pointer(dk)
    o.scale = 0.0 if scale is None else float(scale)
    if stream is not None:
        o.stream = stream.cuda_stream
    elif device is not None and device.type == "cuda":
        o.stream = torch.cuda.current_stream(device).cuda_stream
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel()
    for name, t, dt in (("sel_root", sel_root, torch.int32), ("sel_mid", sel_mid, torch.int32),
                        ("sel_leaf", sel_leaf, torch.int32), ("lse_kg", lse_kg, torch.float32),
                        ("lse_seq", lse_seq, torch.float32)):
        if t is not None:
            if t.dtype != dt or not t.is_contiguous():
                raise TypeError(f"{name} must be a contiguous {dt} tensor")
            setattr(o, name, t.data_ptr())
    return o, keep


def hikvp_attend(q, tree, seq_k, seq_v, K, out):
    """atlaskv_hikvp_attend: view's stream and workspace."""
    dq, dk, dv, do = describe(q), describe(seq_k), describe(seq_v), describe(out)
    _raise(lib().atlaskv_hikvp_attend(ctypes.byref(dq), tree.handle, _ref(dk), _ref(dv), _k(K),
                                      ctypes.byref(do)))
    return out


def hikvp_attend_ex(q, tree, seq_k, seq_v, K, out, **opts):
    """atlaskv_hikvp_attend_ex; keyword options as in atlaskv_attend_opts."""
    dq, dk, dv, do = describe(q), describe(seq_k), describe(seq_v), describe(out)
    o, keep = _opts(device=q.device, **opts)
    _raise(lib().atlaskv_hikvp_attend_ex(ctypes.byref(dq), tree.handle, _ref(dk), _ref(dv), _k(K),
                                         ctypes.byref(do), ctypes.byref(o)))
    del keep
    return out


def hikvp_attend_noalloc(q, tree, seq_k, seq_v, K, out, **opts):
    """atlaskv_hikvp_attend_noalloc: the library's fixed device workspace (no
    allocation); keyword options as in atlaskv_attend_opts, except workspace."""
    dq, dk, dv, do = describe(q), describe(seq_k), describe(seq_v), describe(out)
    o, keep = _opts(device=q.device, **opts)
    _raise(lib().atlaskv_hikvp_attend_noalloc(ctypes.byref(dq), tree.handle, _ref(dk), _ref(dv), _k(K),
                                              ctypes.byref(do), ctypes.byref(o)))
    del keep
    return out


def noalloc_scratch_bytes():
    return int(lib().atlaskv_noalloc_scratch_bytes())


def check_args(q, tree, seq_k, seq_v, K, out, **opts):
    """atlaskv_check_args: status code of the host-side checks (no GPU work)."""
    dq, dk, dv, do = describe(q), describe(seq_k), describe(seq_v), describe(out)
    o, keep = _opts(**opts)
    st = lib().atlaskv_check_args(_ref(dq), tree.handle if tree is not None else None, _ref(dk),
                                  _ref(dv), _k(K) if K is not None else None, _ref(do), ctypes.byref(o))
    del keep
    return st


def flat_workspace_size(tree, q, seq_k):
    n = ctypes.c_size_t()
    dq, dk = describe(q), describe(seq_k)
    _raise(lib().atlaskv_flat_workspace_size(tree.handle, ctypes.byref(dq), _ref(dk), ctypes.byref(n)))
    return n.value


def alloc_flat_workspace(tree, q, seq_k):
    """A torch uint8 device buffer large enough for a flat attend call."""
    n = flat_workspace_size(tree, q, seq_k)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def flat_attend_ex(q, tree, seq_k, seq_v, out, **opts):
    """atlaskv_flat_attend_ex: the KG half over every leaf (no pruning)."""
    dq, dk, dv, do = describe(q), describe(seq_k), describe(seq_v), describe(out)
    o, keep = _opts(device=q.device, **opts)
    _raise(lib().atlaskv_flat_attend_ex(ctypes.byref(dq), tree.handle, _ref(dk), _ref(dv),
                                        ctypes.byref(do), ctypes.byref(o)))
    del keep
    return out


def flat_check_args(q, tree, seq_k, seq_v, out, **opts):
    """atlaskv_flat_check_args: status code of the host-side checks."""
    dq, dk, dv, do = describe(q), describe(seq_k), describe(seq_v), describe(out)
    o, keep = _opts(**opts)
    st = lib().atlaskv_flat_check_args(_ref(dq), tree.handle if tree is not None else None, _ref(dk),
                                       _ref(dv), _ref(do), ctypes.byref(o))
    del keep
    return st


def flat_phase_names():
    L = lib()
    return [L.atlaskv_flat_phase_name(i).decode() for i in range(L.atlaskv_flat_phase_count())]


SHARE_KV_GROUP, SHARE_SEQUENCE = 1, 2


def shared_workspace_size(tree, q, seq_k, K, share):
    n = ctypes.c_size_t()
    dq, dk = describe(q), describe(seq_k)
    _raise(lib().atlaskv_shared_workspace_size(tree.handle, ctypes.byref(dq), _ref(dk), _k(K), int(share),
                                               ctypes.byref(n)))
    return n.value


def alloc_shared_workspace(tree, q, seq_k, K, share):
    n = shared_workspace_size(tree, q, seq_k, K, share)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def shared_attend_ex(q, tree, seq_k, seq_v, K, share, out, **opts):
    """atlaskv_shared_attend_ex: one descent per KV group (share=1) or per
    sequence (share=2); sel_* options receive the group selections."""
    dq, dk, dv, do = describe(q), describe(seq_k), describe(seq_v), describe(out)
    o, keep = _opts(device=q.device, **opts)
    _raise(lib().atlaskv_shared_attend_ex(ctypes.byref(dq), tree.handle, _ref(dk), _ref(dv), _k(K),
                                          int(share), ctypes.byref(do), ctypes.byref(o)))
    del keep
    return out


def shared_check_args(q, tree, seq_k, seq_v, K, share, out, **opts):
    dq, dk, dv, do = describe(q), describe(seq_k), describe(seq_v), describe(out)
    o, keep = _opts(**opts)
    st = lib().atlaskv_shared_check_args(_ref(dq), tree.handle if tree is not None else None, _ref(dk),
                                         _ref(dv), _k(K) if K is not None else None, int(share), _ref(do),
                                         ctypes.byref(o))
    del keep
    return st


def shared_phase_names():
    L = lib()
    return [L.atlaskv_shared_phase_name(i).decode() for i in range(L.atlaskv_shared_phase_count())]


def folded_workspace_size(tree, q, w_k, seq_k, K):
    n = ctypes.c_size_t()
    dq, dw, dk = describe(q), describe(w_k), describe(seq_k)
    _raise(lib().atlaskv_folded_workspace_size(tree.handle, ctypes.byref(dq), ctypes.byref(dw), _ref(dk),
                                               _k(K), ctypes.byref(n)))
    return n.value


def alloc_folded_workspace(tree, q, w_k, seq_k, K):
    n = folded_workspace_size(tree, q, w_k, seq_k, K)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def folded_attend_ex(q, tree, w_k, w_v, seq_k, seq_v, K, out, **opts):
    """atlaskv_folded_attend_ex: a one-head base tree of width D_E, per-head
    projections w_k / w_v [Hkv, d, D_E]."""
    dq, dwk, dwv = describe(q), describe(w_k), describe(w_v)
    dk, dv, do = describe(seq_k), describe(seq_v), describe(out)
    o, keep = _opts(device=q.device, **opts)
    _raise(lib().atlaskv_folded_attend_ex(ctypes.byref(dq), tree.handle, ctypes.byref(dwk), ctypes.byref(dwv),
                                          _ref(dk), _ref(dv), _k(K), ctypes.byref(do), ctypes.byref(o)))
    del keep
    return out


def folded_check_args(q, tree, w_k, w_v, seq_k, seq_v, K, out, **opts):
    dq, dwk, dwv = describe(q), describe(w_k), describe(w_v)
    dk, dv, do = describe(seq_k), describe(seq_v), describe(out)
    o, keep = _opts(**opts)
    st = lib().atlaskv_folded_check_args(_ref(dq), tree.handle if tree is not None else None, _ref(dwk),
                                         _ref(dwv), _ref(dk), _ref(dv), _k(K) if K is not None else None,
                                         _ref(do), ctypes.byref(o))
    del keep
    return st


def folded_phase_names():
    L = lib()
    return [L.atlaskv_folded_phase_name(i).decode() for i in range(L.atlaskv_folded_phase_count())]


def phase_names():
    """Kernel phases of one attend call, in launch order."""
    L = lib()
    return [L.atlaskv_phase_name(i).decode() for i in range(L.atlaskv_phase_count())]


def last_error():
    return lib().atlaskv_last_error().decode()


def version():
    return lib().atlaskv_version().decode()
