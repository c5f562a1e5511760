"""CPU tests of the C-ABI boundary: the library loads without a GPU, exports
every symbol include/atlaskv.h declares, and its host-only argument checks
return the documented status codes.  No kernel is launched here."""
import ctypes
import os
import re

import pytest
import torch

from hierarchical_kv_pruning_amd import atlaskv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(atlaskv.LIB_PATH):
        from hierarchical_kv_pruning_amd import build
        build.build()
    return atlaskv.lib()


def test_header_declarations_are_exported(lib):
    header = open(os.path.join(ROOT, "include", "atlaskv.h")).read()
    declared = set(re.findall(r"\b(atlaskv_[a-z_]+)\s*\(", header))
    assert declared == set(atlaskv.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version(lib):
    assert "gfx950" in atlaskv.version()


def _tree(dtype=torch.bfloat16, Hkv=2, d=128, MR=4, MI=10, M=50):
    z = lambda n: torch.zeros(Hkv, n, d, dtype=dtype)
    return z(MR), z(MI), z(M), z(M)


def _view(**kw):
    rk, mk, lk, lv = _tree(**kw)
    return atlaskv.TreeView.describe_only(rk, mk, lk, lv, 5, 9)


def _call(view, q=None, seq=True, K=(2, 2, 4), out=None, ws_bytes=1 << 30, **opts):
    B, N, Hq, d = 1, 4, 4, view._keep[0].shape[2]
    dt = view._keep[0].dtype
    if q is None:
        q = torch.zeros(B, N, Hq, d, dtype=dt)
    sk = torch.zeros(B, 6, view._keep[0].shape[0], d, dtype=dt) if seq else None
    sv = torch.zeros_like(sk) if seq else None
    if out is None:
        out = torch.zeros(q.shape, dtype=dt)
    ws = torch.zeros(ws_bytes // 1 if ws_bytes < 4096 else 4096, dtype=torch.uint8)
    # a host buffer stands in for the workspace pointer: only its address and size are checked
    fake = type("W", (), {"data_ptr": lambda self: (ws.data_ptr() + 255) // 256 * 256,
                          "numel": lambda self: ws_bytes})()
    return atlaskv.check_args(q, view, sk, sv, K, out, workspace=fake, **opts)


def test_valid_call_passes(lib):
    assert _call(_view()) == atlaskv.OK


def test_valid_call_fp32_and_d64(lib):
    assert _call(_view(dtype=torch.float32, d=64)) == atlaskv.OK


def test_null_pointers(lib):
    v = _view()
    q = torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16)
    assert atlaskv.check_args(None, v, None, None, (1, 1, 1), q) == atlaskv.ERR_NULL
    assert atlaskv.check_args(q, None, None, None, (1, 1, 1), q) == atlaskv.ERR_NULL
    assert atlaskv.check_args(q, v, None, None, None, q) == atlaskv.ERR_NULL
    sk = torch.zeros(1, 6, 2, 128, dtype=torch.bfloat16)
    assert atlaskv.check_args(q, v, sk, None, (1, 1, 1), q) == atlaskv.ERR_NULL


def test_dtype_mismatch(lib):
    v = _view()
    q = torch.zeros(1, 4, 4, 128, dtype=torch.float32)
    assert _call(v, q=q) == atlaskv.ERR_DTYPE
    out16 = torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16)
    assert _call(v, out=out16) == atlaskv.OK
    out32 = torch.zeros(1, 4, 4, 128, dtype=torch.float32)
    assert _call(v, out=out32) == atlaskv.OK  # fp32 output of bf16 inputs is allowed


def test_shape_errors(lib):
    v = _view()
    assert _call(v, q=torch.zeros(1, 4, 3, 128, dtype=torch.bfloat16)) == atlaskv.ERR_SHAPE  # Hq % Hkv
    assert _call(v, q=torch.zeros(1, 4, 4, 64, dtype=torch.bfloat16)) == atlaskv.ERR_SHAPE   # head dim
    assert _call(v, out=torch.zeros(1, 4, 4, 64, dtype=torch.bfloat16)) == atlaskv.ERR_SHAPE
    q = torch.zeros(1, 8, 4, 128, dtype=torch.bfloat16)                                      # S_kv < N
    out = torch.zeros_like(q)
    assert _call(v, q=q, out=out) == atlaskv.ERR_SHAPE
    # non-unit innermost stride
    qt = torch.zeros(1, 4, 128, 4, dtype=torch.bfloat16).transpose(2, 3)
    assert _call(v, q=qt) == atlaskv.ERR_SHAPE


def test_k_errors(lib):
    v = _view()
    assert _call(v, K=(-1, 2, 2)) == atlaskv.ERR_K
    assert _call(v, K=(2, -1, 2)) == atlaskv.ERR_K
    assert _call(v, K=(2, 2, 257)) == atlaskv.OK             # clamps to the 2 * 9 leaf candidates
    assert _call(v, K=(2, 2, 256)) == atlaskv.OK
    assert _call(v, K=(0, 2, 2)) == atlaskv.OK              # empty KG half: plain causal attention
    assert _call(v, K=(2, 2, 0), seq=False) == atlaskv.ERR_K  # both halves empty
    assert _call(v, K=(2, 2, 2), seq=False) == atlaskv.OK


def test_k_clamps_to_each_levels_candidates(lib):
    """K clamps before the 256 limit applies: the tree has 4 roots (fanout
    <= 5) and 10 mids (fanout <= 9), so K = (1000, 1000, 1000) is (4, 10, 50)
    -- every candidate -- and plans the same workspace."""
    v = _view()
    q = torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16)
    assert _call(v, K=(1000, 1000, 1000)) == atlaskv.OK
    assert _call(v, K=(2**31 - 1, 7, 2**31 - 1)) == atlaskv.OK
    a = atlaskv.hikvp_workspace_size(v, q, None, (1000, 1000, 1000))
    b = atlaskv.hikvp_workspace_size(v, q, None, (4, 10, 50))
    assert a == b
    # K_I clamps to K_R' * 5 = 10 under K_R = 2 ... and to M_I = 10 in any case
    assert atlaskv.hikvp_workspace_size(v, q, None, (2, 1000, 4)) == atlaskv.hikvp_workspace_size(v, q, None, (2, 10, 4))


def test_k_above_256_with_more_candidates_is_refused(lib):
    """Only a clamped K above 256 is refused: 300 roots, K_R = 257..300."""
    rk, mk, lk, lv = _tree(MR=300, MI=300, M=600)
    v = atlaskv.TreeView.describe_only(rk, mk, lk, lv, 1, 2)
    assert _call(v, K=(256, 4, 4)) == atlaskv.OK
    assert _call(v, K=(257, 4, 4)) == atlaskv.ERR_K
    assert "256" in atlaskv.last_error()
    assert _call(v, K=(300, 300, 600)) == atlaskv.ERR_K
    # K_I = 300 with K_R = 4 roots of fanout 1: clamps to 4
    assert _call(v, K=(4, 300, 600)) == atlaskv.OK


def test_workspace_errors(lib):
    v = _view()
    assert _call(v, ws_bytes=16) == atlaskv.ERR_WORKSPACE
    q = torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16)
    assert atlaskv.check_args(q, v, None, None, (1, 1, 1), q) == atlaskv.ERR_WORKSPACE  # none attached


def test_workspace_size_grows_with_k(lib):
    v = _view()
    q = torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16)
    a = atlaskv.hikvp_workspace_size(v, q, None, (1, 1, 1))
    b = atlaskv.hikvp_workspace_size(v, q, None, (4, 4, 8))
    assert 0 < a < b


def test_scale_must_be_positive(lib):
    v = _view()
    assert _call(v, scale=-1.0) == atlaskv.ERR_UNSUPPORTED
    assert _call(v, scale=0.5) == atlaskv.OK


def test_unsupported_head_dim(lib):
    for d in (96, 192, 4224):   # not 64 / 128 / a multiple of 128 up to 4096
        with pytest.raises(atlaskv.AtlasKVError) as e:
            _view(d=d)
        assert e.value.status == atlaskv.ERR_UNSUPPORTED, d


def test_wide_tree_serves_the_folded_entry_point_only(lib):
    """A tree wider than 128 (a base-embedding tree of width D_E, a multiple
    of 128 up to 4096) is a valid view, but only the folded entry point
    takes it: the per-row, flat and shared paths refuse it."""
    for DE in (256, 384, 3072, 4096):
        v = _view(Hkv=1, d=DE)
        q = torch.zeros(1, 4, 2, DE, dtype=torch.bfloat16)
        assert _call(v, q=q, seq=False) == atlaskv.ERR_UNSUPPORTED
        ws = torch.zeros(4096, dtype=torch.uint8)
        fake = type("W", (), {"data_ptr": lambda self: (ws.data_ptr() + 255) // 256 * 256,
                              "numel": lambda self: 1 << 34})()
        assert atlaskv.flat_check_args(q, v, None, None, q, workspace=fake) == atlaskv.ERR_UNSUPPORTED
        assert atlaskv.shared_check_args(q, v, None, None, (2, 2, 4), atlaskv.SHARE_KV_GROUP, q,
                                         workspace=fake) == atlaskv.ERR_UNSUPPORTED
        ql = torch.zeros(1, 4, 8, 128, dtype=torch.bfloat16)
        wk = torch.zeros(2, 128, DE, dtype=torch.bfloat16)
        sk = torch.zeros(1, 6, 2, 128, dtype=torch.bfloat16)
        assert atlaskv.folded_check_args(ql, v, wk, wk, sk, sk, (2, 2, 4), ql, workspace=fake) == atlaskv.OK
        # the workspace holds the exact folded queries (fp64) besides the rounded ones
        assert atlaskv.folded_workspace_size(v, ql, wk, sk, (2, 2, 4)) >= 4 * 8 * DE * (8 + 2)


def test_describe_rejects_bad_fanouts_and_tree_mismatch(lib):
    rk, mk, lk, lv = _tree()
    with pytest.raises(atlaskv.AtlasKVError) as e:
        atlaskv.TreeView.describe_only(rk, mk, lk, lv, 11, 9)   # fanout above the mid count
    assert e.value.status == atlaskv.ERR_TREE
    with pytest.raises(atlaskv.AtlasKVError) as e:
        atlaskv.TreeView.describe_only(rk, mk, lk, lv[:, :49], 5, 9)
    assert e.value.status == atlaskv.ERR_SHAPE
    with pytest.raises(atlaskv.AtlasKVError) as e:
        atlaskv.TreeView.describe_only(rk, mk.float(), lk, lv, 5, 9)
    assert e.value.status == atlaskv.ERR_DTYPE


def test_q_kg_must_match_q(lib):
    v = _view()
    assert _call(v, q_kg=torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16)) == atlaskv.OK
    assert _call(v, q_kg=torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)) == atlaskv.ERR_SHAPE


def test_error_message_is_thread_local_text(lib):
    v = _view()
    _call(v, K=(-1, 2, 2))
    assert "K[0]" in atlaskv.last_error()


def test_described_view_cannot_run(lib):
    v = _view()
    q = torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16)
    sk = torch.zeros(1, 6, 2, 128, dtype=torch.bfloat16)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(atlaskv.AtlasKVError) as e:
        atlaskv.hikvp_attend_ex(q, v, sk, torch.zeros_like(sk), (1, 1, 1), torch.zeros_like(q),
                                workspace=ws)
    assert e.value.status in (atlaskv.ERR_UNSUPPORTED, atlaskv.ERR_WORKSPACE)


def test_phase_names_in_launch_order(lib):
    """The timing phases follow the descent: roots (with their row grouping),
    mid GEMM, mid Top-K, leaf bucket link, leaf scoring (first members, then
    overflow members), leaf Top-K with the KG softmax, sequence attention (with
    the merge when keys are not split), the combine of key splits."""
    assert atlaskv.phase_names() == [
        "root_score_topk", "mid_bucket_gemm", "mid_topk", "leaf_bucket_link", "leaf_score_stream",
        "leaf_topk_kg_attention", "seq_attention", "seq_split_combine"]
    assert lib.atlaskv_phase_name(-1) is None
    assert lib.atlaskv_phase_name(lib.atlaskv_phase_count()) is None


def test_flat_phase_names_in_launch_order(lib):
    assert atlaskv.flat_phase_names() == ["flat_kg_partial", "flat_kg_combine", "seq_attention",
                                          "seq_split_combine"]
    assert lib.atlaskv_flat_phase_name(-1) is None
    assert lib.atlaskv_flat_phase_name(lib.atlaskv_flat_phase_count()) is None


def _flat_call(view, q=None, seq=True, out=None, ws_bytes=1 << 30, **opts):
    B, N, Hq, d = 1, 4, 4, view._keep[0].shape[2]
    dt = view._keep[0].dtype
    if q is None:
        q = torch.zeros(B, N, Hq, d, dtype=dt)
    sk = torch.zeros(B, 6, view._keep[0].shape[0], d, dtype=dt) if seq else None
    sv = torch.zeros_like(sk) if seq else None
    if out is None:
        out = torch.zeros(q.shape, dtype=dt)
    ws = torch.zeros(4096, dtype=torch.uint8)
    fake = type("W", (), {"data_ptr": lambda self: (ws.data_ptr() + 255) // 256 * 256,
                          "numel": lambda self: ws_bytes})()
    return atlaskv.flat_check_args(q, view, sk, sv, out, workspace=fake, **opts)


def test_flat_argument_checks(lib):
    """The unpruned path takes no K; shape, dtype and workspace rules are the
    pruned path's, and a tree with leaves always has a KG half."""
    v = _view()
    assert _flat_call(v) == atlaskv.OK
    assert _flat_call(v, seq=False) == atlaskv.OK
    assert _flat_call(_view(dtype=torch.float32, d=64)) == atlaskv.OK
    assert _flat_call(v, q=torch.zeros(1, 4, 3, 128, dtype=torch.bfloat16)) == atlaskv.ERR_SHAPE
    assert _flat_call(v, q=torch.zeros(1, 4, 4, 128, dtype=torch.float32)) == atlaskv.ERR_DTYPE
    assert _flat_call(v, ws_bytes=16) == atlaskv.ERR_WORKSPACE
    assert _flat_call(v, scale=-2.0) == atlaskv.ERR_UNSUPPORTED
    q = torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16)
    assert atlaskv.flat_check_args(q, v, None, None, q) == atlaskv.ERR_WORKSPACE  # none attached


def test_flat_workspace_grows_with_leaves(lib):
    q = torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16)
    small = atlaskv.flat_workspace_size(_view(M=50), q, None)
    big = atlaskv.flat_workspace_size(_view(M=50000), q, None)
    assert 0 < small <= big


def test_shared_phase_names_and_checks(lib):
    assert atlaskv.shared_phase_names() == [
        "group_query", "root_score_topk", "mid_bucket_gemm", "mid_topk", "leaf_bucket_link",
        "leaf_score_stream", "leaf_topk_kg_attention", "shared_kg_attention",
        "seq_attention", "seq_split_combine"]
    v = _view()
    q = torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16)
    sk = torch.zeros(1, 6, 2, 128, dtype=torch.bfloat16)
    ws = torch.zeros(4096, dtype=torch.uint8)
    fake = type("W", (), {"data_ptr": lambda self: (ws.data_ptr() + 255) // 256 * 256,
                          "numel": lambda self: 1 << 30})()
    for share in (atlaskv.SHARE_KV_GROUP, atlaskv.SHARE_SEQUENCE):
        assert atlaskv.shared_check_args(q, v, sk, sk, (2, 2, 4), share, q, workspace=fake) == atlaskv.OK
        assert atlaskv.shared_check_args(q, v, sk, sk, (2, 2, 300), share, q, workspace=fake) == atlaskv.OK
        assert atlaskv.shared_check_args(q, v, sk, sk, (2, -2, 3), share, q, workspace=fake) == atlaskv.ERR_K
        assert atlaskv.shared_workspace_size(v, q, sk, (2, 2, 4), share) > 0
    assert atlaskv.shared_check_args(q, v, sk, sk, (2, 2, 4), 3, q, workspace=fake) == atlaskv.ERR_UNSUPPORTED
    # a sequence group holds every token: no larger group rows than per token
    a = atlaskv.shared_workspace_size(v, q, sk, (2, 2, 4), atlaskv.SHARE_SEQUENCE)
    b = atlaskv.shared_workspace_size(v, q, sk, (2, 2, 4), atlaskv.SHARE_KV_GROUP)
    assert a <= b


def test_folded_phase_names_and_checks(lib):
    assert atlaskv.folded_phase_names() == [
        "fold_query", "root_score_topk", "mid_bucket_gemm", "mid_topk", "leaf_bucket_link",
        "leaf_score_stream", "leaf_topk_kg_attention", "unfold_values",
        "seq_attention", "seq_split_combine"]
    base = _view(Hkv=1, d=128)                      # one-head base tree, D_E = 128
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)          # layer: Hq 8, d 64
    wk = torch.zeros(2, 64, 128, dtype=torch.bfloat16)          # Hkv 2
    sk = torch.zeros(1, 6, 2, 64, dtype=torch.bfloat16)
    ws = torch.zeros(4096, dtype=torch.uint8)
    fake = type("W", (), {"data_ptr": lambda self: (ws.data_ptr() + 255) // 256 * 256,
                          "numel": lambda self: 1 << 30})()
    call = lambda **kw: atlaskv.folded_check_args(kw.get("q", q), kw.get("tree", base), kw.get("wk", wk),
                                                  kw.get("wv", wk), kw.get("sk", sk), kw.get("sk", sk),
                                                  kw.get("K", (2, 2, 4)), kw.get("q", q), workspace=fake)
    assert call() == atlaskv.OK
    assert call(tree=_view(Hkv=2, d=128)) == atlaskv.ERR_SHAPE                   # not a base tree
    assert call(wk=torch.zeros(2, 64, 64, dtype=torch.bfloat16)) == atlaskv.ERR_SHAPE   # D_E mismatch
    assert call(sk=torch.zeros(1, 6, 1, 64, dtype=torch.bfloat16)) == atlaskv.ERR_SHAPE  # seq heads
    assert call(q=torch.zeros(1, 4, 7, 64, dtype=torch.bfloat16)) == atlaskv.ERR_SHAPE   # Hq % Hkv
    assert call(K=(0, 2, 2)) == atlaskv.OK                                        # pure causal
    assert atlaskv.folded_workspace_size(base, q, wk, sk, (2, 2, 4)) > 0

