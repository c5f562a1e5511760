// atlaskv_api.hip -- the C ABI of libatlaskv.so (declared in include/atlaskv.h):
// argument checks, workspace planning and the launch sequence of one HiKVP
// attention call on the caller's stream.
//
// Page: "AtlasKV: Augmenting LLMs with Billion-Scale Knowledge Graphs in 20GB
// VRAM" (digest of arXiv 2510.17934), 速读 › 怎么做的: root scores -> Top-K ->
// children -> Top-K -> leaves -> Top-K, then the λ merge of the KG and sequence
// softmaxes.  The launch order below follows those steps.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <string>

#include "atlaskv.h"
#include "hikvp_internal.h"

using namespace hikvp;

struct atlaskv_tree_view_s {
  TreeDev dev;                 // pointers, strides, sizes (norm -> stats buffer)
  int64_t maxfan[2];           // largest root and mid fanouts
  BuildStats* stats;           // device buffer owned by the view (NULL if described only)
  hipStream_t stream;
  void* workspace;
  size_t workspace_bytes;
  int described_only;
  int host_mask;               // bit i: tree tensor i (root_k, mid_k, leaf_k, leaf_v) in pinned host memory
  // the sequence half runs on aux, forked from and joined back to the call's
  // stream with two events; parts 1.. of a split descent run on part_s[],
  // forked with part_fork and joined with part_join[]; mu keeps one call's
  // fork sequences whole
  hipStream_t aux;
  hipEvent_t fork, join, part_fork;
  hipStream_t part_s[kMaxParts - 1];
  hipEvent_t part_join[kMaxParts - 1];
  std::mutex mu;
};

namespace {

thread_local std::string g_err;

// Frees a view and whatever of its HIP objects exist (not its tree stats).
void release_view(atlaskv_tree_view_s* v) {
  for (int i = 0; i < kMaxParts - 1; ++i) {
    if (v->part_join[i]) (void)hipEventDestroy(v->part_join[i]);
    if (v->part_s[i]) (void)hipStreamDestroy(v->part_s[i]);
  }
  if (v->part_fork) (void)hipEventDestroy(v->part_fork);
  if (v->join) (void)hipEventDestroy(v->join);
  if (v->fork) (void)hipEventDestroy(v->fork);
  if (v->aux) (void)hipStreamDestroy(v->aux);
  delete v;
}

atlaskv_status fail(atlaskv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

atlaskv_status hip_fail(hipError_t e, const char* what) {
  return fail(ATLASKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t esize(int32_t dtype) { return dtype == ATLASKV_BF16 ? 2 : 4; }

constexpr int64_t kIndexLimit = (int64_t)1 << 31;  // node counts and rows are int32 on the GPU

// ndim, dtype, innermost stride 1, non-negative sizes/strides, 16-byte rows.
atlaskv_status check_tensor(const atlaskv_tensor* t, const char* name, int ndim, bool rows16) {
  if (!t) return fail(ATLASKV_ERR_NULL, "%s is NULL", name);
  if (t->dtype != ATLASKV_F32 && t->dtype != ATLASKV_BF16)
    return fail(ATLASKV_ERR_DTYPE, "%s: unknown dtype %d", name, (int)t->dtype);
  if (t->ndim != ndim) return fail(ATLASKV_ERR_SHAPE, "%s: expected %d dims, got %d", name, ndim, (int)t->ndim);
  int64_t numel = 1;
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0 || t->stride[i] < 0)
      return fail(ATLASKV_ERR_SHAPE, "%s: negative shape or stride in dim %d", name, i);
    numel *= t->shape[i];
  }
  if (numel > 0 && !t->data) return fail(ATLASKV_ERR_NULL, "%s: data is NULL", name);
  if (t->stride[ndim - 1] != 1) return fail(ATLASKV_ERR_SHAPE, "%s: innermost stride must be 1", name);
  if (rows16 && numel > 0) {
    const int64_t es = esize(t->dtype);
    if (((uintptr_t)t->data) % 16) return fail(ATLASKV_ERR_SHAPE, "%s: data not 16-byte aligned", name);
    for (int i = 0; i < ndim - 1; ++i)
      if ((t->stride[i] * es) % 16)
        return fail(ATLASKV_ERR_SHAPE, "%s: stride of dim %d is not a multiple of 16 bytes", name, i);
  }
  return ATLASKV_OK;
}

atlaskv_status check_tree_tensors(const atlaskv_tensor* root_k, const atlaskv_tensor* mid_k,
                                  const atlaskv_tensor* leaf_k, const atlaskv_tensor* leaf_v) {
  atlaskv_status st;
  if ((st = check_tensor(root_k, "root_k", 3, true))) return st;
  if ((st = check_tensor(mid_k, "mid_k", 3, true))) return st;
  if ((st = check_tensor(leaf_k, "leaf_k", 3, true))) return st;
  if ((st = check_tensor(leaf_v, "leaf_v", 3, true))) return st;
  const int32_t dt = root_k->dtype;
  if (mid_k->dtype != dt || leaf_k->dtype != dt || leaf_v->dtype != dt)
    return fail(ATLASKV_ERR_DTYPE, "tree tensors must share one dtype");
  const int64_t Hkv = root_k->shape[0], d = root_k->shape[2];
  if (Hkv < 1) return fail(ATLASKV_ERR_SHAPE, "root_k: need at least one KV head");
  if (d != 64 && d != 128 && !(d > 128 && d <= kMaxWideD && d % 128 == 0))
    return fail(ATLASKV_ERR_UNSUPPORTED, "key width %lld: 64, 128, or a multiple of 128 up to %d (a base-embedding "
                "tree for the folded entry point)", (long long)d, kMaxWideD);
  if (mid_k->shape[0] != Hkv || leaf_k->shape[0] != Hkv || leaf_v->shape[0] != Hkv)
    return fail(ATLASKV_ERR_SHAPE, "tree tensors disagree on the KV head count");
  if (mid_k->shape[2] != d || leaf_k->shape[2] != d || leaf_v->shape[2] != d)
    return fail(ATLASKV_ERR_SHAPE, "tree tensors disagree on the head dim");
  if (leaf_v->shape[1] != leaf_k->shape[1])
    return fail(ATLASKV_ERR_SHAPE, "leaf_v and leaf_k disagree on the leaf count");
  if (root_k->shape[1] >= kIndexLimit || mid_k->shape[1] >= kIndexLimit || leaf_k->shape[1] >= kIndexLimit)
    return fail(ATLASKV_ERR_UNSUPPORTED, "node counts must be below 2^31");
  return ATLASKV_OK;
}

void fill_tree(TreeDev& t, const atlaskv_tensor* root_k, const atlaskv_tensor* mid_k,
               const atlaskv_tensor* leaf_k, const atlaskv_tensor* leaf_v) {
  const atlaskv_tensor* ts[4] = {root_k, mid_k, leaf_k, leaf_v};
  for (int i = 0; i < 4; ++i) {
    if (i < 3) t.key[i] = ts[i]->data;
    t.hs[i] = ts[i]->stride[0];
    t.rs[i] = ts[i]->stride[1];
  }
  t.leaf_v = leaf_v->data;
  t.count[0] = root_k->shape[1];
  t.count[1] = mid_k->shape[1];
  t.count[2] = leaf_k->shape[1];
  t.Hkv = (int)root_k->shape[0];
  t.d = (int)root_k->shape[2];
  t.dtype = root_k->dtype;
  t.off[0] = t.off[1] = nullptr;
  t.norm = nullptr;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The address kernels on the current device use for `p`: device memory of
// this device as is, pinned host memory through its device mapping (the
// kernels then read it over the host link).  Pageable host memory and memory
// of another device are refused.  *host is set when `p` is host memory.
atlaskv_status device_address(const void* p, const char* name, const void** dev, int* host) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipPointerAttribute_t at;
  e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess || at.type == hipMemoryTypeUnregistered) {
    if (e != hipSuccess) (void)hipGetLastError();  // leave no pending error for the caller's next call
    return fail(ATLASKV_ERR_UNSUPPORTED,
                "%s is neither device memory nor pinned host memory (pageable host memory "
                "cannot be read by the kernels; allocate it pinned)", name);
  }
  if (at.type == hipMemoryTypeHost) {
    // the mapping may be reported for the allocation's start or for `p` itself:
    // keep p's offset from the reported host address either way
    *dev = at.devicePointer && at.hostPointer
               ? (const void*)((const char*)at.devicePointer + ((const char*)p - (const char*)at.hostPointer))
               : p;
    *host = 1;
    return ATLASKV_OK;
  }
  if (at.type == hipMemoryTypeDevice && at.device != cur)
    return fail(ATLASKV_ERR_UNSUPPORTED, "%s is memory of device %d, the current device is %d", name,
                at.device, cur);
  *dev = p;
  *host = 0;
  return ATLASKV_OK;
}

struct Plan {
  int B, N, Hq, S, R, G;
  int K[3];                    // Top-K per level, clamped to the level's candidate capacity
  int Kuser[3];                // as given (row stride of the caller's selection outputs)
  int64_t c1max, c2max;
  double scale;
  int nsplit;
  size_t off_mid, off_mid_meta, off_leaf, off_sel[3], off_okg, off_lse, off_part, total;
  size_t off_mid_base, off_bcnt, off_bslot, off_bhead, off_bnext, off_blist, off_bcount, off_bovf, off_junk;
  size_t off_rcnt, off_rtot, off_rtoff, off_rtkey, off_rnt, off_rmem;
  int64_t root_tiles_max;
  int32_t desc_per_sub, bucket_q, bslots;
  // descent parts: KV heads [part_g[i], part_g[i+1]) with their own tile,
  // descriptor, count and overflow-key regions (totals above: one part over
  // all heads uses the regions concatenated)
  int nparts;
  int part_g[kMaxParts + 1];
  int64_t part_tiles[kMaxParts], part_ovf[kMaxParts];
  int32_t part_desc[kMaxParts];
  int flat_nsplit, flat_split_len, flat_row_tiles;  // unpruned path only
  size_t off_fpart;
  int group_rows;                                    // shared selections only
  size_t off_gq, off_gpart;
  size_t off_gqx, off_glo, off_gdelta;
  int fold_Hkv, fold_d, fold_kg_empty;               // folded projections only
  size_t off_qf, off_qx, off_qlo, off_qdelta;
  int exact_logits;                                  // the KG softmax takes its logits from rows.q_exact
  int leaf_nst, leaf_fpad, leaf_spt;                 // leaf candidates filtered in the leaf stream
  size_t off_lcnt;
};

// Candidate capacity per row at the mid level (children of K_R distinct
// roots) and at the leaf level (children of K_I distinct mids).
void candidate_capacity(const atlaskv_tree_view_s* v, const int K[3], int64_t* c1, int64_t* c2) {
  const int64_t MR = v->dev.count[0], MI = v->dev.count[1], M = v->dev.count[2];
  int64_t a = (K[0] < MR ? K[0] : MR) * v->maxfan[0];
  if (a > MI) a = MI;
  int64_t b = (K[1] < MI ? K[1] : MI) * v->maxfan[1];
  if (b > M) b = M;
  *c1 = a < 1 ? 1 : a;
  *c2 = b < 1 ? 1 : b;
}

// kModeFoldedDescent: the pruned path on the folded rows of a base-embedding
// tree, the only one that takes a tree wider than 128.
enum { kModeHikvp = 0, kModeFlat = 1, kModeSharedKvGroup = 2, kModeSharedSequence = 3, kModeFoldedDescent = 4 };

// The group rows of a shared-selection call: [B, Ng, Hkv, d] contiguous in
// the tree's dtype, Ng = N (one group per KV head and token) or 1 (per KV
// head and sequence).  Only the shape matters for planning.
atlaskv_tensor group_rows_desc(int64_t B, int64_t Ng, int Hkv, int d, int dtype, void* data) {
  atlaskv_tensor g;
  memset(&g, 0, sizeof g);
  g.data = data;
  g.dtype = dtype;
  g.ndim = 4;
  g.shape[0] = B; g.shape[1] = Ng; g.shape[2] = Hkv; g.shape[3] = d;
  g.stride[3] = 1; g.stride[2] = d; g.stride[1] = (int64_t)Hkv * d; g.stride[0] = Ng * Hkv * (int64_t)d;
  return g;
}

// mode: kModeHikvp (the pruned path), kModeFlat (every leaf; K is not used and
// may be NULL) or a shared-selection mode (the descent runs on group rows).
atlaskv_status plan_call(const atlaskv_tensor* q, const atlaskv_tree_view_s* v,
                         const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                         const int32_t Kpl[3], const atlaskv_tensor* out,
                         const atlaskv_attend_opts* opts, bool need_out, Plan& p, int mode = kModeHikvp) {
  const bool flat = mode == kModeFlat;
  atlaskv_status st;
  memset(&p, 0, sizeof p);
  if (!v) return fail(ATLASKV_ERR_NULL, "tree view is NULL");
  if (!Kpl && !flat) return fail(ATLASKV_ERR_NULL, "K_per_level is NULL");
  if ((st = check_tensor(q, "q", 4, true))) return st;
  const TreeDev& t = v->dev;
  if (t.d > kMaxD && mode != kModeFoldedDescent)
    return fail(ATLASKV_ERR_UNSUPPORTED, "a tree of width %d (above %d) serves the folded entry point only", t.d,
                kMaxD);
  if (q->dtype != t.dtype) return fail(ATLASKV_ERR_DTYPE, "q dtype differs from the tree's");
  if (q->shape[3] != t.d) return fail(ATLASKV_ERR_SHAPE, "q head dim %lld != tree head dim %d",
                                      (long long)q->shape[3], t.d);
  const int64_t B = q->shape[0], N = q->shape[1], Hq = q->shape[2];
  if (Hq < 1 || Hq % t.Hkv) return fail(ATLASKV_ERR_SHAPE, "Hq=%lld is not a multiple of Hkv=%d",
                                         (long long)Hq, t.Hkv);
  if (B * N * Hq >= kIndexLimit) return fail(ATLASKV_ERR_UNSUPPORTED, "B*N*Hq must be below 2^31");
  if (opts && opts->q_kg) {
    if ((st = check_tensor(opts->q_kg, "q_kg", 4, true))) return st;
    if (opts->q_kg->dtype != q->dtype) return fail(ATLASKV_ERR_DTYPE, "q_kg dtype differs from q's");
    for (int i = 0; i < 4; ++i)
      if (opts->q_kg->shape[i] != q->shape[i]) return fail(ATLASKV_ERR_SHAPE, "q_kg shape differs from q's");
  }
  if ((seq_k == nullptr) != (seq_v == nullptr))
    return fail(ATLASKV_ERR_NULL, "seq_k and seq_v must both be given or both be NULL");
  int64_t S = 0;
  if (seq_k) {
    if ((st = check_tensor(seq_k, "seq_k", 4, true))) return st;
    if ((st = check_tensor(seq_v, "seq_v", 4, true))) return st;
    if (seq_k->dtype != q->dtype || seq_v->dtype != q->dtype)
      return fail(ATLASKV_ERR_DTYPE, "sequence K/V dtype differs from q's");
    for (int i = 0; i < 4; ++i)
      if (seq_v->shape[i] != seq_k->shape[i]) return fail(ATLASKV_ERR_SHAPE, "seq_v shape differs from seq_k's");
    if (seq_k->shape[0] != B || seq_k->shape[2] != t.Hkv || seq_k->shape[3] != t.d)
      return fail(ATLASKV_ERR_SHAPE, "seq_k must be [B, S_kv, Hkv, d]");
    S = seq_k->shape[1];
    if (S < N) return fail(ATLASKV_ERR_SHAPE, "S_kv=%lld < N=%lld", (long long)S, (long long)N);
    if (S >= kIndexLimit) return fail(ATLASKV_ERR_UNSUPPORTED, "S_kv must be below 2^31");
    if ((seq_k->stride[1] | seq_v->stride[1]) * esize(seq_k->dtype) >= ((int64_t)1 << 25))
      return fail(ATLASKV_ERR_UNSUPPORTED, "sequence position strides must be below 32 MB");
  }
  if (need_out) {
    if ((st = check_tensor(out, "out", 4, false))) return st;
    if (out->dtype != q->dtype && out->dtype != ATLASKV_F32)
      return fail(ATLASKV_ERR_DTYPE, "out dtype must be q's dtype or fp32");
    for (int i = 0; i < 4; ++i)
      if (out->shape[i] != q->shape[i]) return fail(ATLASKV_ERR_SHAPE, "out shape differs from q's");
  }
  if (!flat)
    for (int i = 0; i < 3; ++i)
      if (Kpl[i] < 0) return fail(ATLASKV_ERR_K, "K[%d]=%d is negative", i, Kpl[i]);
  const bool kg_empty = flat ? t.count[2] == 0
                             : (Kpl[0] == 0 || Kpl[1] == 0 || Kpl[2] == 0 || t.count[0] == 0 ||
                                t.count[1] == 0 || t.count[2] == 0);
  if (kg_empty && !seq_k)
    return fail(ATLASKV_ERR_K, "both the KG half (K or tree empty) and the sequence half are empty");
  double scale = 1.0 / sqrt((double)t.d);
  if (opts && opts->scale != 0.0f) {
    if (!(opts->scale > 0.0f) || isinf(opts->scale))
      return fail(ATLASKV_ERR_UNSUPPORTED, "scale must be positive and finite");
    scale = (double)opts->scale;
  }
  p.B = (int)B; p.N = (int)N; p.Hq = (int)Hq; p.S = (int)S;
  p.R = (int)(B * N * Hq);
  p.G = (int)(Hq / t.Hkv);
  p.scale = scale;
  if (flat) {
    if (t.count[2] >= kIndexLimit) return fail(ATLASKV_ERR_UNSUPPORTED, "M must be below 2^31");
    const int64_t eb = t.dtype == ATLASKV_BF16 ? 2 : 4;
    if (t.rs[2] * eb >= ((int64_t)1 << 25) || t.rs[3] * eb >= ((int64_t)1 << 25))
      return fail(ATLASKV_ERR_UNSUPPORTED, "leaf row strides must be below 32 MB");
    const size_t R = (size_t)p.R;
    size_t o = 0;
    p.flat_nsplit = flat_splits(p.B, p.N, p.Hq, t.Hkv, t.count[2], t.dtype);
    p.flat_split_len = flat_split_len(t.count[2], p.flat_nsplit);
    p.flat_row_tiles = flat_row_tiles(p.B, p.N, p.G);
    p.off_okg = o;   o = align256(o + R * (size_t)t.d * 4);
    p.off_lse = o;   o = align256(o + R * 4);
    p.off_fpart = o; o = align256(o + R * (size_t)p.flat_nsplit * (t.d + 4) * 4);
    p.nsplit = seq_splits(p.B, p.N, t.Hkv, p.G, p.S, t.dtype);
    p.off_part = o;  o = align256(o + R * (size_t)p.nsplit * (t.d + 2) * 4);
    p.total = o;
    return ATLASKV_OK;
  }
  // K clamps to the most candidates a row can have at each level (all roots;
  // the children of K_R roots; the children of K_I mids), so any K at or above
  // that selects every candidate; the kernels take at most kMaxK a level.
  {
    int64_t cap = t.count[0];
    for (int i = 0; i < 3; ++i) {
      p.Kuser[i] = Kpl[i];
      int64_t k = Kpl[i];
      if (k > 0 && k > (cap > 1 ? cap : 1)) k = cap > 1 ? cap : 1;
      if (k > kMaxK)
        return fail(ATLASKV_ERR_K, "K[%d]=%d: more than %d selections from %lld candidates a row is unsupported",
                    i, Kpl[i], kMaxK, (long long)cap);
      p.K[i] = (int)k;
      if (i < 2) {
        cap = k * v->maxfan[i];
        if (cap > t.count[i + 1]) cap = t.count[i + 1];
      }
    }
  }
  if (mode == kModeSharedKvGroup || mode == kModeSharedSequence) {
    // the group descent's own workspace, then group queries, per-row KG half, sequence partials
    const int64_t Ng = mode == kModeSharedSequence ? 1 : N;
    atlaskv_tensor gd = group_rows_desc(B, Ng, t.Hkv, t.d, t.dtype, (void*)(uintptr_t)256);
    Plan pg;
    if ((st = plan_call(&gd, v, seq_k, seq_v, Kpl, nullptr, nullptr, false, pg, kModeHikvp))) return st;
    const size_t R = (size_t)p.R;
    size_t o = align256(pg.total);
    p.group_rows = (int)(B * Ng * t.Hkv);
    p.off_gq = o;    o = align256(o + (size_t)p.group_rows * t.d * esize(t.dtype));
    p.off_gqx = o;   o = align256(o + (size_t)p.group_rows * t.d * 8);
    p.off_glo = o;   o = align256(o + (t.dtype == ATLASKV_BF16 ? (size_t)p.group_rows * t.d * 2 : 0));
    p.off_gdelta = o; o = align256(o + (size_t)p.group_rows * 4);
    int tn = 1;
    const int chunks = group_chunks(p.N, (int)Ng, &tn);
    p.off_gpart = o; o = align256(o + (size_t)p.group_rows * chunks * t.d * 8);
    p.off_okg = o;   o = align256(o + R * (size_t)t.d * 4);
    p.off_lse = o;   o = align256(o + R * 4);
    p.nsplit = seq_splits(p.B, p.N, t.Hkv, p.G, p.S, t.dtype);
    p.off_part = o;  o = align256(o + R * (size_t)p.nsplit * (t.d + 2) * 4);
    p.total = o;
    return ATLASKV_OK;
  }
  if ((int64_t)p.R * p.K[1] >= kIndexLimit || (int64_t)t.Hkv * t.count[1] >= kIndexLimit ||
      (int64_t)p.R * (p.K[0] + kRootTile) >= kIndexLimit)
    return fail(ATLASKV_ERR_UNSUPPORTED, "B*N*Hq*(K_R+16), B*N*Hq*K_I and Hkv*M_I must be below 2^31");
  candidate_capacity(v, p.K, &p.c1max, &p.c2max);
  if (p.c1max >= kMaxMidCands || p.c2max >= kIndexLimit)
    return fail(ATLASKV_ERR_UNSUPPORTED, "candidates per row must be below 2^24 (mid) and 2^31 (leaf)");
  p.scale = scale;
  const size_t R = (size_t)p.R;
  size_t o = 0;
  // mid scores; the root kernel also spills its scores here when M_R is large
  if (v->dev.count[0] > p.c1max) p.c1max = v->dev.count[0];
  p.off_mid = o;       o = align256(o + R * (size_t)p.c1max * 8);
  p.off_mid_meta = o;  o = align256(o + R * (size_t)p.K[0] * 16);
  // Leaf candidates are filtered in the leaf stream on per-head trees whose
  // mids can have at least kLeafFilterRatio * K_L children: each leaf-stream
  // wave stages at most kLeafStageFloats scores, so a scoring group takes
  // leaf_nst members; the survivors are (score, index) pairs, 8 bytes a
  // candidate slot, and the mid's place in the row's selection rides in the
  // top byte of a member's slot base.  With shorter spans the staging and
  // the per-member threshold cost the stream more than the smaller select
  // saves (measured: 100-leaf spans at K_L = 32 step 0.529 -> 0.574 ms;
  // 215-leaf spans at K_L = 32 0.444 -> 0.435 ms; 463-leaf spans at K_L = 64
  // 1.398 -> 1.313 ms).  Not for leaf keys in host memory: there the link
  // bounds the stream, and the filter's pauses between spans cost it more
  // (m1e7 decode 17.5 -> 19.2 ms).
  if (mode != kModeFoldedDescent && (t.d == 64 || t.d == 128) && p.K[1] > 0 && p.K[2] > 0 &&
      !(v->host_mask & (1 << 2)) &&
      v->maxfan[1] >= kLeafFilterRatio * (int64_t)p.K[2] && v->maxfan[1] <= kLeafFilterMaxFan &&
      p.c2max < kMaxMidCands) {
    p.leaf_fpad = (int)((v->maxfan[1] + 3) & ~(int64_t)3);
    const int nst = kLeafStageFloats / p.leaf_fpad;
    p.leaf_nst = nst < 1 ? 1 : nst > 8 ? 8 : nst;
    // survivors a row: K_L of each span longer than K_L, a few more near its
    // threshold; rows past the register list read theirs from the workspace
    const int64_t est = (int64_t)p.K[1] * (p.K[2] + 2) + 64;
    p.leaf_spt = est <= 512 ? 8 : est <= 1024 ? 16 : est <= 1536 ? 24 : 40;
  }
  p.off_leaf = o;      o = align256(o + R * (size_t)p.c2max * (p.leaf_nst > 0 ? 8 : 4));
  p.off_lcnt = o;      o = align256(o + (p.leaf_nst > 0 ? R * (size_t)p.K[1] * 4 : 0));
  for (int i = 0; i < 3; ++i) { p.off_sel[i] = o; o = align256(o + R * (size_t)p.K[i] * 4); }
  p.off_mid_base = o;  o = align256(o + R * (size_t)p.K[1] * 4);
  const size_t nroot = (size_t)t.Hkv * (size_t)t.count[0];
  // the descent runs in concurrent parts (ranges of KV heads) when there
  // are enough rows for each part's kernels to fill the GPU
  p.bslots = mode == kModeFoldedDescent ? kBucketSlotsFolded : kBucketSlots;
  p.nparts = descent_parts(t.Hkv, (int64_t)R);
  int64_t tiles_all = 0, ovf_all = 0, desc_all = 0;
  for (int i = 0; i < p.nparts; ++i) {
    p.part_g[i] = i * t.Hkv / p.nparts;
    p.part_g[i + 1] = (i + 1) * t.Hkv / p.nparts;
    const int64_t heads = p.part_g[i + 1] - p.part_g[i], rows = heads * p.B * p.N * p.G;
    p.part_tiles[i] = rows * p.K[0] / kRootTile + heads * t.count[0] + 1;
    p.part_desc[i] = (int32_t)(((int64_t)row_chunks((int)rows, p.K[1]) + kDescSub - 1) / kDescSub *
                               row_chunk_entries(p.K[1]));
    p.part_ovf[i] = rows * p.K[1] / (p.bslots + 1) + 1;
    tiles_all += p.part_tiles[i];
    desc_all += p.part_desc[i];
    ovf_all += p.part_ovf[i];
  }
  p.root_tiles_max = tiles_all;
  p.off_rcnt = o;      o = align256(o + nroot * kRootSub * 4);
  p.off_rtot = o;      o = align256(o + nroot * 4);
  p.off_rtoff = o;     o = align256(o + nroot * 4);
  p.off_rtkey = o;     o = align256(o + (size_t)p.root_tiles_max * 4);
  p.off_rnt = o;       o = align256(o + kMaxParts * 4);
  p.off_rmem = o;      o = align256(o + (size_t)p.root_tiles_max * kRootTile * 8);
  p.bucket_q = (int32_t)(((size_t)t.Hkv * (size_t)t.count[1] + 63) / 64);
  const size_t nbix = (size_t)p.bucket_q * 64;
  p.off_bcnt = o;      o = align256(o + nbix * 4);
  p.off_bslot = o;     o = align256(o + nbix * 8 * (size_t)p.bslots);
  p.off_bhead = o;     o = align256(o + nbix * 4);
  p.off_bnext = o;     o = align256(o + R * (size_t)p.K[1] * 4);
  // link chunk c appends to sub-list c mod kDescSub (of its part)
  if (desc_all >= kIndexLimit) return fail(ATLASKV_ERR_UNSUPPORTED, "bucket descriptor capacity above 2^31");
  p.desc_per_sub = (int32_t)desc_all;
  p.off_blist = o;     o = align256(o + (size_t)desc_all * kDescSub * 16);
  p.off_bcount = o;    o = align256(o + (size_t)kMaxParts * (kDescSub + 1) * 4);
  p.off_bovf = o;      o = align256(o + (size_t)ovf_all * 4);
  p.off_junk = o;      o = align256(o + (size_t)kJunkSlots * 64);
  p.off_okg = o;       o = align256(o + R * (size_t)t.d * 4);
  p.off_lse = o;       o = align256(o + R * 4);
  p.nsplit = seq_splits(p.B, p.N, t.Hkv, p.G, p.S, t.dtype);
  p.off_part = o;      o = align256(o + R * (size_t)p.nsplit * (t.d + 2) * 4);
  p.total = o;
  return ATLASKV_OK;
}

void fill_rows(RowsDev& r, const atlaskv_tensor* q, const atlaskv_attend_opts* opts, const Plan& p) {
  const atlaskv_tensor* qk = (opts && opts->q_kg) ? opts->q_kg : q;
  r.q = q->data;
  r.q_kg = qk->data;
  for (int i = 0; i < 3; ++i) { r.qs[i] = q->stride[i]; r.qks[i] = qk->stride[i]; }
  r.B = p.B; r.N = p.N; r.Hq = p.Hq; r.G = p.G; r.R = p.R;
  r.scale = p.scale;
  r.q_exact = nullptr;
  r.q_delta = nullptr;
  r.q_lo = nullptr;
}

// Selection arrays of one descent (plan pd): the caller's outputs where their
// row stride (the K the caller gave) equals the clamped K the kernels use,
// else the workspace's, copied into the caller's -1-padded rows afterwards.
struct SelTargets {
  int32_t* sel[3];
  int32_t* user[3];            // caller outputs still to fill from sel (NULL: none)
};

SelTargets sel_targets(const Plan& pd, const atlaskv_attend_opts* opts, char* ws) {
  SelTargets t;
  int32_t* u[3] = {opts ? opts->sel_root : nullptr, opts ? opts->sel_mid : nullptr,
                   opts ? opts->sel_leaf : nullptr};
  for (int i = 0; i < 3; ++i) {
    const bool direct = u[i] && pd.Kuser[i] == pd.K[i];
    t.sel[i] = direct ? u[i] : (int32_t*)(ws + pd.off_sel[i]);
    t.user[i] = direct ? nullptr : u[i];
  }
  return t;
}

hipError_t finish_sel(const SelTargets& t, const Plan& pd, hipStream_t s) {
  hipError_t e = hipSuccess;
  for (int i = 0; i < 3 && e == hipSuccess; ++i)
    if (t.user[i]) e = launch_expand_sel(t.sel[i], pd.K[i], t.user[i], pd.Kuser[i], pd.R, s);
  return e;
}

// Folded projections: the tree is a one-head base tree of width D_E; the
// layer has Hkv heads of width d with W_K, W_V [Hkv, d, D_E].  pd receives the
// plan of the descent on the folded rows [B, N, Hq, D_E] (unset when the KG
// half is empty).
atlaskv_status plan_folded(const atlaskv_tensor* q, const atlaskv_tree_view_s* v,
                           const atlaskv_tensor* w_k, const atlaskv_tensor* w_v,
                           const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v, const int32_t Kpl[3],
                           const atlaskv_tensor* out, const atlaskv_attend_opts* opts, bool need_out,
                           Plan& p, Plan& pd) {
  atlaskv_status st;
  memset(&p, 0, sizeof p);
  memset(&pd, 0, sizeof pd);
  if (!v) return fail(ATLASKV_ERR_NULL, "tree view is NULL");
  if (!Kpl) return fail(ATLASKV_ERR_NULL, "K_per_level is NULL");
  const TreeDev& t = v->dev;
  if (t.Hkv != 1) return fail(ATLASKV_ERR_SHAPE, "folded projections need a one-head base tree (Hkv=%d)", t.Hkv);
  if ((st = check_tensor(w_k, "w_k", 3, true))) return st;
  if ((st = check_tensor(w_v, "w_v", 3, true))) return st;
  if (w_k->dtype != t.dtype || w_v->dtype != t.dtype)
    return fail(ATLASKV_ERR_DTYPE, "w_k / w_v dtype differs from the tree's");
  const int64_t Hkv = w_k->shape[0], d = w_k->shape[1];
  for (int i = 0; i < 3; ++i)
    if (w_v->shape[i] != w_k->shape[i]) return fail(ATLASKV_ERR_SHAPE, "w_v shape differs from w_k's");
  if (w_k->shape[2] != t.d)
    return fail(ATLASKV_ERR_SHAPE, "w_k is [Hkv, d, D_E] with D_E = the tree width %d", t.d);
  if (d != 64 && d != 128) return fail(ATLASKV_ERR_UNSUPPORTED, "head dim d must be 64 or 128");
  if (Hkv < 1) return fail(ATLASKV_ERR_SHAPE, "w_k has no heads");
  if ((st = check_tensor(q, "q", 4, true))) return st;
  if (q->dtype != t.dtype) return fail(ATLASKV_ERR_DTYPE, "q dtype differs from the tree's");
  if (q->shape[3] != d) return fail(ATLASKV_ERR_SHAPE, "q head dim differs from w_k's d");
  const int64_t B = q->shape[0], N = q->shape[1], Hq = q->shape[2];
  if (Hq < 1 || Hq % Hkv) return fail(ATLASKV_ERR_SHAPE, "Hq is not a multiple of Hkv");
  if (B * N * Hq >= kIndexLimit) return fail(ATLASKV_ERR_UNSUPPORTED, "B*N*Hq must be below 2^31");
  if (opts && opts->q_kg) {
    if ((st = check_tensor(opts->q_kg, "q_kg", 4, true))) return st;
    if (opts->q_kg->dtype != q->dtype) return fail(ATLASKV_ERR_DTYPE, "q_kg dtype differs from q's");
    for (int i = 0; i < 4; ++i)
      if (opts->q_kg->shape[i] != q->shape[i]) return fail(ATLASKV_ERR_SHAPE, "q_kg shape differs from q's");
  }
  if ((seq_k == nullptr) != (seq_v == nullptr))
    return fail(ATLASKV_ERR_NULL, "seq_k and seq_v must both be given or both be NULL");
  int64_t S = 0;
  if (seq_k) {
    if ((st = check_tensor(seq_k, "seq_k", 4, true))) return st;
    if ((st = check_tensor(seq_v, "seq_v", 4, true))) return st;
    if (seq_k->dtype != q->dtype || seq_v->dtype != q->dtype)
      return fail(ATLASKV_ERR_DTYPE, "sequence K/V dtype differs from q's");
    for (int i = 0; i < 4; ++i)
      if (seq_v->shape[i] != seq_k->shape[i]) return fail(ATLASKV_ERR_SHAPE, "seq_v shape differs from seq_k's");
    if (seq_k->shape[0] != B || seq_k->shape[2] != Hkv || seq_k->shape[3] != d)
      return fail(ATLASKV_ERR_SHAPE, "seq_k must be [B, S_kv, Hkv, d]");
    S = seq_k->shape[1];
    if (S < N) return fail(ATLASKV_ERR_SHAPE, "S_kv=%lld < N=%lld", (long long)S, (long long)N);
    if (S >= kIndexLimit) return fail(ATLASKV_ERR_UNSUPPORTED, "S_kv must be below 2^31");
    if ((seq_k->stride[1] | seq_v->stride[1]) * esize(seq_k->dtype) >= ((int64_t)1 << 25))
      return fail(ATLASKV_ERR_UNSUPPORTED, "sequence position strides must be below 32 MB");
  }
  if (need_out) {
    if ((st = check_tensor(out, "out", 4, false))) return st;
    if (out->dtype != q->dtype && out->dtype != ATLASKV_F32)
      return fail(ATLASKV_ERR_DTYPE, "out dtype must be q's dtype or fp32");
    for (int i = 0; i < 4; ++i)
      if (out->shape[i] != q->shape[i]) return fail(ATLASKV_ERR_SHAPE, "out shape differs from q's");
  }
  for (int i = 0; i < 3; ++i)
    if (Kpl[i] < 0) return fail(ATLASKV_ERR_K, "K[%d]=%d is negative", i, Kpl[i]);
  const bool kg_empty = Kpl[0] == 0 || Kpl[1] == 0 || Kpl[2] == 0 || t.count[0] == 0 || t.count[1] == 0 ||
                        t.count[2] == 0;
  if (kg_empty && !seq_k)
    return fail(ATLASKV_ERR_K, "both the KG half (K or tree empty) and the sequence half are empty");
  double scale = 1.0 / sqrt((double)d);
  if (opts && opts->scale != 0.0f) {
    if (!(opts->scale > 0.0f) || isinf(opts->scale))
      return fail(ATLASKV_ERR_UNSUPPORTED, "scale must be positive and finite");
    scale = (double)opts->scale;
  }
  p.B = (int)B; p.N = (int)N; p.Hq = (int)Hq; p.S = (int)S;
  p.R = (int)(B * N * Hq);
  p.G = (int)(Hq / Hkv);
  p.scale = scale;
  // K clamps to the most candidates a row can have at each level (all roots;
  // the children of K_R roots; the children of K_I mids), so any K at or above
  // that selects every candidate; the kernels take at most kMaxK a level.
  {
    int64_t cap = t.count[0];
    for (int i = 0; i < 3; ++i) {
      p.Kuser[i] = Kpl[i];
      int64_t k = Kpl[i];
      if (k > 0 && k > (cap > 1 ? cap : 1)) k = cap > 1 ? cap : 1;
      if (k > kMaxK)
        return fail(ATLASKV_ERR_K, "K[%d]=%d: more than %d selections from %lld candidates a row is unsupported",
                    i, Kpl[i], kMaxK, (long long)cap);
      p.K[i] = (int)k;
      if (i < 2) {
        cap = k * v->maxfan[i];
        if (cap > t.count[i + 1]) cap = t.count[i + 1];
      }
    }
  }
  p.fold_Hkv = (int)Hkv;
  p.fold_d = (int)d;
  p.fold_kg_empty = kg_empty;
  size_t o = 0;
  if (!kg_empty) {
    atlaskv_tensor qd = group_rows_desc(B, N, (int)Hq, t.d, t.dtype, (void*)(uintptr_t)256);
    if ((st = plan_call(&qd, v, nullptr, nullptr, Kpl, nullptr, nullptr, false, pd, kModeFoldedDescent))) return st;
    // fp32 trees: the KG softmax takes fp64 logits of the exact folded query
    // (their fp32 scores can be off by more than an fp32 output resolves at
    // wide D_E).  bf16 trees keep the scores of the rounded pair hi + lo
    // (each component within about 2^-18 of the exact one; q_delta bounds the
    // norm of the rest), whose logit error lies far below the rounding of a
    // bf16 output, and skip re-reading the selected keys
    pd.exact_logits = t.dtype == ATLASKV_F32;
    o = align256(pd.total);
  }
  const size_t R = (size_t)p.R;
  p.off_qf = o;   o = align256(o + R * (size_t)t.d * esize(t.dtype));
  p.off_qx = o;   o = align256(o + R * (size_t)t.d * 8);
  p.off_qlo = o;  o = align256(o + (t.dtype == ATLASKV_BF16 ? R * (size_t)t.d * 2 : 0));
  p.off_qdelta = o; o = align256(o + R * 4);
  p.off_okg = o;  o = align256(o + R * (size_t)d * 4);
  p.off_lse = o;  o = align256(o + R * 4);
  p.nsplit = seq_splits(p.B, p.N, (int)Hkv, p.G, p.S, t.dtype);
  p.off_part = o; o = align256(o + R * (size_t)p.nsplit * (d + 2) * 4);
  p.total = o;
  return ATLASKV_OK;
}

// Optional timing events at phase boundaries: event 0 before the first
// kernel, event i after phase i-1.
struct PhaseMarks {
  void** ev;
  int nev, phase;
  hipStream_t s;
  PhaseMarks(const atlaskv_attend_opts* opts, hipStream_t st)
      : ev((opts && opts->phase_events && opts->n_phase_events > 0) ? opts->phase_events : nullptr),
        nev(ev ? opts->n_phase_events : 0), phase(0), s(st) {}
  hipError_t mark(hipError_t prev) {
    if (prev != hipSuccess || phase >= nev || !ev[phase]) { ++phase; return prev; }
    hipError_t r = hipEventRecord((hipEvent_t)ev[phase], s);
    ++phase;
    return r;
  }
};

// Sequence half (背景知识与设计原则 › 自注意力层机制) and the λ merge with the
// KG half held in o_kg / lse_kg.  The causal attention does not depend on the
// KG half, so unless phase timing is requested it runs concurrently on the
// view's aux stream and writes (o, m, l) partials; the call's stream waits for
// it before k_seq_combine merges both halves.  Decode blocks (under 16
// tokens: one light HBM-bound wave per SIMD) fork before the KG kernels.
// Prefill blocks fork from the last descent part: with one part just before
// its leaf stream (the matrix-core prefill kernels hold most of a SIMD's
// registers and LDS, which slowed the one chain of latency-bound descent
// kernels beside them), with several parts after its root phase (the other
// parts' kernels fill the gaps, and the half is done before the leaf streams
// take every wave slot: 0.531 -> 0.519 ms at 16384 rows over 8 KV heads,
// where before the leaf stream it finished only with the last leaf select).  With phase timing both
// phases (attention, split combine) run after the KG half, through the same
// partials and merge.
struct SeqHalf {
  SeqArgs sa;
  bool overlap;                // on the aux stream, joined before k_seq_combine
  bool at_leaf;                // forked from the last descent part (else before the KG half)
  mutable bool forked;         // the fork was enqueued (else the half runs after the KG half)
};

SeqHalf seq_prepare(const Plan& p, const RowsDev& rows, int Hkv, int d, int dtype,
                    const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v, const atlaskv_tensor* out,
                    const atlaskv_attend_opts* opts, float* o_kg, float* lse_kg, char* ws,
                    const atlaskv_tree_view_s* v) {
  SeqHalf h;
  SeqArgs& sa = h.sa;
  memset(&sa, 0, sizeof sa);
  sa.r = rows;
  sa.S = p.S;
  sa.Hkv = Hkv;
  sa.d = d;
  sa.dtype = dtype;
  if (seq_k) {
    sa.k = seq_k->data;
    sa.v = seq_v->data;
    sa.ks[0] = seq_k->stride[0]; sa.ks[1] = seq_k->stride[1]; sa.ks[2] = seq_k->stride[2];
    sa.vs[0] = seq_v->stride[0]; sa.vs[1] = seq_v->stride[1]; sa.vs[2] = seq_v->stride[2];
  }
  sa.o_kg = o_kg;
  sa.lse_kg = lse_kg;
  sa.out = out->data;
  sa.os[0] = out->stride[0]; sa.os[1] = out->stride[1]; sa.os[2] = out->stride[2];
  sa.out_dtype = out->dtype;
  sa.lse_seq_out = opts ? opts->lse_seq : nullptr;
  sa.nsplit = p.nsplit;
  h.overlap = seq_k && v->aux && !(opts && opts->phase_events && opts->n_phase_events > 0);
  h.at_leaf = h.overlap && p.N >= 16;
  h.forked = false;
  // with a sequence the merge is always k_seq_combine's, so the serial and
  // the overlapped order produce the same bits
  sa.part = seq_k ? (float*)(ws + p.off_part) : nullptr;
  sa.split_len = p.nsplit > 1 ? seq_split_len(p.S, p.nsplit) : (p.S > 0 ? p.S : 1);
  return h;
}

// The fork itself, from stream `from`; the caller holds the view's mutex (one
// call's record / wait / launch / record stay together).
hipError_t seq_fork_locked(const SeqHalf& h, atlaskv_tree_view_s* v, hipStream_t from) {
  hipError_t e = hipEventRecord(v->fork, from);
  if (e == hipSuccess) e = hipStreamWaitEvent(v->aux, v->fork, 0);
  if (e == hipSuccess) e = launch_seq_attend(h.sa, v->aux);
  if (e == hipSuccess) e = hipEventRecord(v->join, v->aux);
  h.forked = e == hipSuccess;
  return e;
}

// Before the KG half: the fork of a decode block's sequence half.
hipError_t seq_start(const SeqHalf& h, atlaskv_tree_view_s* v, hipStream_t s) {
  if (!h.overlap || h.at_leaf) return hipSuccess;
  std::lock_guard<std::mutex> lock(v->mu);
  return seq_fork_locked(h, v, s);
}

// After the KG half: the join and the combine, or the serial sequence half
// (also when no descent ran to fork a prefill half from).
hipError_t seq_finish(const SeqHalf& h, atlaskv_tree_view_s* v, hipStream_t s, PhaseMarks& pm) {
  if (h.forked) {
    // a later call's join only comes later on aux: waiting on it is still enough
    hipError_t e = hipStreamWaitEvent(s, v->join, 0);
    if (e == hipSuccess) e = launch_seq_combine(h.sa, s);
    return e;
  }
  hipError_t e = pm.mark(launch_seq_attend(h.sa, s));
  if (e == hipSuccess) e = pm.mark(launch_seq_combine(h.sa, s));
  return e;
}

// A prefill block's sequence half, forked from a descent part's stream just
// before its leaf stream, or after its root phase (early) (h NULL: none to
// fork there).
struct LateFork {
  const SeqHalf* h;
  atlaskv_tree_view_s* v;
  bool early;
};

// One part of the descent (KV heads [a.g0, a.g1)) on stream s; the caller
// holds the view's mutex when `fork` is given.
hipError_t descent_part(const StepArgs& a, hipStream_t s, PhaseMarks& pm, const LateFork* fork = nullptr) {
  auto mark = [&](hipError_t prev) { return pm.mark(prev); };
  auto fork_at = [&](bool early, hipError_t prev) {
    if (prev != hipSuccess || !fork || !fork->h || fork->early != early) return prev;
    return seq_fork_locked(*fork->h, fork->v, s);
  };
  hipError_t e = launch_root(a, s);
  if (e == hipSuccess) e = mark(launch_root_groups(a, s));
  e = fork_at(true, e);
  if (e == hipSuccess) e = mark(launch_mid_gemm(a, s));
  if (e == hipSuccess) e = mark(launch_mid_select(a, s));
  if (e == hipSuccess) e = mark(launch_leaf_link(a, s));
  e = fork_at(false, e);
  if (e == hipSuccess) e = mark(launch_leaf_score(a, s));
  if (e == hipSuccess) e = mark(launch_leaf_select(a, s));
  return e;
}

// The pruned descent for `rows` (速读 › 怎么做的: roots -> Top-K -> their
// children -> Top-K -> leaves -> Top-K, then the KG softmax over the selected
// leaves into o_kg / lse_kg): six timing phases.  Every index structure of
// the descent is keyed by KV head, so the heads split into parts that share
// no state; part 0 runs on s and parts 1.. on the view's part streams
// (forked from s, joined back to it), so that one part's kernel tails and
// launch gaps are filled by the others' work.  With phase timing requested
// the descent runs as one part over all heads, serially on s.
hipError_t launch_descent(const Plan& p, const RowsDev& rows, atlaskv_tree_view_s* v, char* ws,
                          int32_t* const sel[3], float* o_kg, float* lse_kg, hipStream_t s, PhaseMarks& pm,
                          const SeqHalf* seq = nullptr) {
  // a prefill sequence half to fork from the last part (after its root phase
  // when there are several parts, else before its leaf stream)
  LateFork late{(seq && seq->overlap && seq->at_leaf) ? seq : nullptr, v, false};
  StepArgs a;
  memset(&a, 0, sizeof a);
  a.t = v->dev;
  a.r = rows;
  for (int i = 0; i < 3; ++i) { a.K[i] = p.K[i]; a.sel[i] = sel[i]; }
  a.c1max = p.c1max;
  a.c2max = p.c2max;
  a.mid_pairs = (uint2*)(ws + p.off_mid);
  a.mid_meta = (int4*)(ws + p.off_mid_meta);
  a.leaf_scores = (float*)(ws + p.off_leaf);
  if (p.leaf_nst > 0) {
    a.leaf_pairs = (uint2*)(ws + p.off_leaf);
    a.leaf_cnt = (int32_t*)(ws + p.off_lcnt);
    a.leaf_nst = p.leaf_nst;
    a.leaf_fpad = p.leaf_fpad;
    a.leaf_spt = p.leaf_spt;
  }
  a.mid_base = (int32_t*)(ws + p.off_mid_base);
  a.root_cnt = (int32_t*)(ws + p.off_rcnt);
  a.root_tot = (int32_t*)(ws + p.off_rtot);
  a.root_tile_off = (int32_t*)(ws + p.off_rtoff);
  a.root_tile_key = (int32_t*)(ws + p.off_rtkey);
  a.root_ntiles = (int32_t*)(ws + p.off_rnt);
  a.root_members = (int2*)(ws + p.off_rmem);
  a.root_tiles_max = p.root_tiles_max;
  a.bucket_cnt = (int32_t*)(ws + p.off_bcnt);
  a.bucket_slot = (int2*)(ws + p.off_bslot);
  a.bucket_head = (int32_t*)(ws + p.off_bhead);
  a.bucket_next = (int32_t*)(ws + p.off_bnext);
  a.bucket_desc = (int4*)(ws + p.off_blist);
  a.bucket_count = (int32_t*)(ws + p.off_bcount);
  a.desc_per_sub = p.desc_per_sub;
  a.bucket_q = p.bucket_q;
  a.bslots = p.bslots;
  a.bucket_ovf = (int32_t*)(ws + p.off_bovf);
  a.junk = (float*)(ws + p.off_junk);
  a.o_kg = o_kg;
  a.lse_kg = lse_kg;
  a.exact_logits = p.exact_logits;
  {
    // the mid tiles keep, of each selected root's children, about the K_I
    // best and the band around them: K_R * min(fanout, 4 K_I) estimates a
    // row's survivors generously; the smaller register list (less LDS a
    // wave, more rows in flight) when that fits it
    const int64_t f = v->maxfan[0] < 4 * (int64_t)p.K[1] ? v->maxfan[0] : 4 * (int64_t)p.K[1];
    a.mid_spt = (int64_t)p.K[0] * f <= 64 * 4 ? 4 : 16;
  }
  const int per_head = rows.B * rows.N * rows.G;  // row blocks per KV head
  if (p.nparts < 2 || !v->part_s[0] || pm.ev) {
    a.g0 = 0;
    a.g1 = a.t.Hkv;
    a.blk0 = 0;
    a.blk1 = rows.R;
    if (!late.h) return descent_part(a, s, pm);
    std::lock_guard<std::mutex> lock(v->mu);
    return descent_part(a, s, pm, &late);
  }
  StepArgs part[kMaxParts];
  int64_t tiles = 0, ovf = 0, desc = 0;
  for (int i = 0; i < p.nparts; ++i) {
    StepArgs& b = part[i];
    b = a;
    b.g0 = p.part_g[i];
    b.g1 = p.part_g[i + 1];
    b.blk0 = b.g0 * per_head;
    b.blk1 = b.g1 * per_head;
    b.root_tile_key = a.root_tile_key + tiles;
    b.root_members = a.root_members + tiles * kRootTile;
    b.root_tiles_max = p.part_tiles[i];
    b.root_ntiles = a.root_ntiles + i;
    b.bucket_desc = a.bucket_desc + desc * kDescSub;
    b.desc_per_sub = p.part_desc[i];
    b.bucket_count = a.bucket_count + i * (kDescSub + 1);
    b.bucket_ovf = a.bucket_ovf + ovf;
    tiles += p.part_tiles[i];
    desc += p.part_desc[i];
    ovf += p.part_ovf[i];
  }
  late.early = true;
  std::lock_guard<std::mutex> lock(v->mu);  // one call's records / waits / launches stay together
  hipError_t e = hipEventRecord(v->part_fork, s);
  for (int i = 1; i < p.nparts && e == hipSuccess; ++i) {
    hipStream_t ps = v->part_s[i - 1];
    PhaseMarks none(nullptr, ps);
    e = hipStreamWaitEvent(ps, v->part_fork, 0);
    if (e == hipSuccess) e = descent_part(part[i], ps, none, i == p.nparts - 1 ? &late : nullptr);
    if (e == hipSuccess) e = hipEventRecord(v->part_join[i - 1], ps);
  }
  if (e == hipSuccess) e = descent_part(part[0], s, pm);
  for (int i = 1; i < p.nparts && e == hipSuccess; ++i) e = hipStreamWaitEvent(s, v->part_join[i - 1], 0);
  return e;
}

// Workspace of atlaskv_hikvp_attend_noalloc: a device array of fixed size,
// one copy per GPU the library runs on, held until the process ends.  Host
// code must use its device address (hipGetSymbolAddress, per device), never
// the array's name, which names a host-side stand-in.
constexpr size_t kNoAllocScratchBytes = (size_t)256 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device (NULL: not yet)

// The current device's scratch address, looked up once per device.
atlaskv_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ATLASKV_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e == hipSuccess ? hipErrorInvalidSymbol : e, "hipGetSymbolAddress");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATLASKV_OK;
}

}  // namespace

extern "C" {

const char* atlaskv_last_error(void) { return g_err.c_str(); }

const char* atlaskv_version(void) { return "atlaskv-mi355x 0.1 (gfx950)"; }

static const char* const kPhaseNames[] = {"root_score_topk", "mid_bucket_gemm", "mid_topk",
                                          "leaf_bucket_link", "leaf_score_stream", "leaf_topk_kg_attention",
                                          "seq_attention", "seq_split_combine"};
static const int kPhases = (int)(sizeof kPhaseNames / sizeof kPhaseNames[0]);

int32_t atlaskv_phase_count(void) { return kPhases; }

const char* atlaskv_phase_name(int32_t i) { return (i >= 0 && i < kPhases) ? kPhaseNames[i] : nullptr; }

atlaskv_status atlaskv_build_tree_view(const atlaskv_tensor* root_k, const atlaskv_tensor* mid_k,
                                       const atlaskv_tensor* leaf_k, const atlaskv_tensor* leaf_v,
                                       const int64_t* root_child_off, const int64_t* mid_child_off,
                                       void* stream, atlaskv_tree_view* out) {
  if (!out) return fail(ATLASKV_ERR_NULL, "out is NULL");
  atlaskv_status st = check_tree_tensors(root_k, mid_k, leaf_k, leaf_v);
  if (st) return st;
  if (!root_child_off || !mid_child_off) return fail(ATLASKV_ERR_NULL, "child offsets are NULL");
  atlaskv_tree_view_s* v = new (std::nothrow) atlaskv_tree_view_s();
  if (!v) return fail(ATLASKV_ERR_HIP, "host allocation failed");
  fill_tree(v->dev, root_k, mid_k, leaf_k, leaf_v);
  {
    const void* given[6] = {root_k->data, mid_k->data, leaf_k->data, leaf_v->data, root_child_off,
                            mid_child_off};
    static const char* const names[6] = {"root_k", "mid_k", "leaf_k", "leaf_v", "root_child_off",
                                         "mid_child_off"};
    const void* addr[6];
    for (int i = 0; i < 6; ++i) {
      int host = 0;
      st = device_address(given[i], names[i], &addr[i], &host);
      if (st) { release_view(v); return st; }
      if (host) v->host_mask |= 1 << i;
    }
    for (int i = 0; i < 3; ++i) v->dev.key[i] = addr[i];
    v->dev.leaf_v = addr[3];
    v->dev.off[0] = (const int64_t*)addr[4];
    v->dev.off[1] = (const int64_t*)addr[5];
  }
  v->stream = (hipStream_t)stream;
  const int Hkv = v->dev.Hkv;
  const size_t stats_bytes = offsetof(BuildStats, norm_bits) + sizeof(unsigned int) * 3 * (size_t)Hkv;
  // all streams at the default priority.  The fork/join events only order
  // kernels of this device's streams (no host waits on them), so they skip
  // the system-scope fence an event record otherwise issues (an L2
  // write-back for host visibility in the middle of the step)
  const unsigned evf = hipEventDisableTiming | hipEventDisableSystemFence;
  hipError_t e = hipStreamCreateWithFlags(&v->aux, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&v->fork, evf);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&v->join, evf);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&v->part_fork, evf);
  for (int i = 0; i < kMaxParts - 1 && e == hipSuccess; ++i) {
    e = hipStreamCreateWithFlags(&v->part_s[i], hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&v->part_join[i], evf);
  }
  if (e != hipSuccess) { release_view(v); return hip_fail(e, "stream/event creation"); }
  e = hipMalloc((void**)&v->stats, stats_bytes);
  if (e != hipSuccess) { release_view(v); return hip_fail(e, "hipMalloc(tree stats)"); }
  BuildStats* host = (BuildStats*)calloc(1, stats_bytes);
  if (!host) { (void)hipFree(v->stats); release_view(v); return fail(ATLASKV_ERR_HIP, "host allocation failed"); }
  hipStream_t s = v->stream;
  e = hipMemcpyAsync(v->stats, host, stats_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = launch_validate(v->dev.off[0], v->dev.count[0], v->dev.count[1], 0, v->stats, s);
  if (e == hipSuccess) e = launch_validate(v->dev.off[1], v->dev.count[1], v->dev.count[2], 1, v->stats, s);
  for (int lev = 0; lev < 3 && e == hipSuccess; ++lev)
    e = launch_key_norms(v->dev.key[lev], v->dev.dtype, v->dev.d, Hkv, v->dev.count[lev], v->dev.hs[lev],
                         v->dev.rs[lev], v->stats->norm_bits + (size_t)lev * Hkv, s);
  if (e == hipSuccess) e = hipMemcpyAsync(host, v->stats, stats_bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    free(host);
    (void)hipFree(v->stats);
    release_view(v);
    return hip_fail(e, "tree validation");
  }
  const int bad = host->bad;
  v->maxfan[0] = (int64_t)host->maxfan[0];
  v->maxfan[1] = (int64_t)host->maxfan[1];
  free(host);
  if (bad) {
    (void)hipFree(v->stats);
    release_view(v);
    return fail(ATLASKV_ERR_TREE, "malformed child offsets (%s%s)", (bad & 1) ? "root->mid " : "",
                (bad & 2) ? "mid->leaf" : "");
  }
  v->dev.norm = (const float*)v->stats->norm_bits;
  *out = v;
  return ATLASKV_OK;
}

atlaskv_status atlaskv_tree_view_describe(const atlaskv_tensor* root_k, const atlaskv_tensor* mid_k,
                                          const atlaskv_tensor* leaf_k, const atlaskv_tensor* leaf_v,
                                          int64_t max_root_fanout, int64_t max_mid_fanout,
                                          atlaskv_tree_view* out) {
  if (!out) return fail(ATLASKV_ERR_NULL, "out is NULL");
  atlaskv_status st = check_tree_tensors(root_k, mid_k, leaf_k, leaf_v);
  if (st) return st;
  if (max_root_fanout < 0 || max_mid_fanout < 0 || max_root_fanout > mid_k->shape[1] ||
      max_mid_fanout > leaf_k->shape[1])
    return fail(ATLASKV_ERR_TREE, "maximum fanouts outside 0..level size");
  atlaskv_tree_view_s* v = new (std::nothrow) atlaskv_tree_view_s();
  if (!v) return fail(ATLASKV_ERR_HIP, "host allocation failed");
  fill_tree(v->dev, root_k, mid_k, leaf_k, leaf_v);
  v->maxfan[0] = max_root_fanout;
  v->maxfan[1] = max_mid_fanout;
  v->described_only = 1;
  *out = v;
  return ATLASKV_OK;
}

int32_t atlaskv_tree_view_placement(atlaskv_tree_view v) { return v ? v->host_mask : -1; }

atlaskv_status atlaskv_destroy_tree_view(atlaskv_tree_view v) {
  if (!v) return ATLASKV_OK;
  hipError_t e = hipSuccess;
  if (v->stats) e = hipFree(v->stats);
  release_view(v);
  return e == hipSuccess ? ATLASKV_OK : hip_fail(e, "hipFree(tree stats)");
}

atlaskv_status atlaskv_tree_view_set_workspace(atlaskv_tree_view v, void* ws, size_t bytes) {
  if (!v) return fail(ATLASKV_ERR_NULL, "tree view is NULL");
  if (bytes && !ws) return fail(ATLASKV_ERR_NULL, "workspace is NULL");
  if (((uintptr_t)ws) % 256) return fail(ATLASKV_ERR_WORKSPACE, "workspace not 256-byte aligned");
  v->workspace = bytes ? ws : nullptr;
  v->workspace_bytes = bytes;
  return ATLASKV_OK;
}

atlaskv_status atlaskv_hikvp_workspace_size(atlaskv_tree_view v, const atlaskv_tensor* q,
                                            const atlaskv_tensor* seq_k, const int32_t K[3],
                                            size_t* bytes) {
  if (!bytes) return fail(ATLASKV_ERR_NULL, "bytes is NULL");
  Plan p;
  atlaskv_status st = plan_call(q, v, seq_k, seq_k, K, nullptr, nullptr, false, p);
  if (st) return st;
  *bytes = p.total;
  return ATLASKV_OK;
}

static atlaskv_status check_all(const atlaskv_tensor* q, atlaskv_tree_view v,
                                const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                const int32_t K[3], const atlaskv_tensor* out,
                                const atlaskv_attend_opts* opts, Plan& p, void** ws,
                                int mode = kModeHikvp) {
  atlaskv_status st = plan_call(q, v, seq_k, seq_v, K, out, opts, true, p, mode);
  if (st) return st;
  void* w = (opts && opts->workspace) ? opts->workspace : v->workspace;
  size_t wb = (opts && opts->workspace) ? opts->workspace_bytes : v->workspace_bytes;
  if (p.R > 0) {
    if (!w) return fail(ATLASKV_ERR_WORKSPACE, "no workspace (need %zu bytes)", p.total);
    if (((uintptr_t)w) % 256) return fail(ATLASKV_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (wb < p.total) return fail(ATLASKV_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", wb, p.total);
  }
  *ws = w;
  return ATLASKV_OK;
}

atlaskv_status atlaskv_check_args(const atlaskv_tensor* q, atlaskv_tree_view v,
                                  const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                  const int32_t K[3], const atlaskv_tensor* out,
                                  const atlaskv_attend_opts* opts) {
  Plan p;
  void* ws = nullptr;
  return check_all(q, v, seq_k, seq_v, K, out, opts, p, &ws);
}

atlaskv_status atlaskv_hikvp_attend_ex(const atlaskv_tensor* q, atlaskv_tree_view v,
                                       const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                       const int32_t K[3], atlaskv_tensor* out,
                                       const atlaskv_attend_opts* opts) {
  Plan p;
  void* wsv = nullptr;
  atlaskv_status st = check_all(q, v, seq_k, seq_v, K, out, opts, p, &wsv);
  if (st) return st;
  if (v->described_only) return fail(ATLASKV_ERR_UNSUPPORTED, "a described-only view cannot run");
  if (p.R == 0) return ATLASKV_OK;
  hipStream_t s = (opts && opts->stream) ? (hipStream_t)opts->stream : v->stream;
  char* ws = (char*)wsv;

  RowsDev rows;
  fill_rows(rows, q, opts, p);
  const SelTargets st3 = sel_targets(p, opts, ws);
  float* lse_kg = (opts && opts->lse_kg) ? opts->lse_kg : (float*)(ws + p.off_lse);
  float* o_kg = (float*)(ws + p.off_okg);

  PhaseMarks pm(opts, s);
  const SeqHalf sh = seq_prepare(p, rows, v->dev.Hkv, v->dev.d, v->dev.dtype, seq_k, seq_v, out, opts, o_kg,
                                 lse_kg, ws, v);
  hipError_t e = pm.mark(hipSuccess);
  if (e == hipSuccess) e = seq_start(sh, v, s);
  if (e == hipSuccess) e = launch_descent(p, rows, v, ws, st3.sel, o_kg, lse_kg, s, pm, &sh);
  if (e == hipSuccess) e = seq_finish(sh, v, s, pm);
  if (e == hipSuccess) e = finish_sel(st3, p, s);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return ATLASKV_OK;
}

atlaskv_status atlaskv_hikvp_attend(const atlaskv_tensor* q, atlaskv_tree_view v,
                                    const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                    const int32_t K[3], atlaskv_tensor* out) {
  return atlaskv_hikvp_attend_ex(q, v, seq_k, seq_v, K, out, nullptr);
}

atlaskv_status atlaskv_hikvp_attend_noalloc(const atlaskv_tensor* q, atlaskv_tree_view v,
                                            const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                            const int32_t K[3], atlaskv_tensor* out,
                                            const atlaskv_attend_opts* opts) {
  if (opts && opts->workspace)
    return fail(ATLASKV_ERR_WORKSPACE, "the no-allocation entry point uses its own fixed workspace");
  Plan p;
  void* wsv = nullptr;
  atlaskv_attend_opts o;
  memset(&o, 0, sizeof o);
  if (opts) o = *opts;
  o.workspace = (void*)(uintptr_t)256;     // a stand-in: the checks read only its size and alignment
  o.workspace_bytes = kNoAllocScratchBytes;
  atlaskv_status st = check_all(q, v, seq_k, seq_v, K, out, &o, p, &wsv);
  if (st == ATLASKV_ERR_WORKSPACE)
    return fail(ATLASKV_ERR_WORKSPACE, "the call needs %zu workspace bytes; the fixed scratch holds %zu",
                p.total, kNoAllocScratchBytes);
  if (st) return st;
  if ((st = scratch_address(&o.workspace))) return st;
  return atlaskv_hikvp_attend_ex(q, v, seq_k, seq_v, K, out, &o);
}

size_t atlaskv_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

static const char* const kSharedPhaseNames[] = {
    "group_query", "root_score_topk", "mid_bucket_gemm", "mid_topk", "leaf_bucket_link",
    "leaf_score_stream", "leaf_topk_kg_attention", "shared_kg_attention",
    "seq_attention", "seq_split_combine"};
static const int kSharedPhases = (int)(sizeof kSharedPhaseNames / sizeof kSharedPhaseNames[0]);

int32_t atlaskv_shared_phase_count(void) { return kSharedPhases; }

const char* atlaskv_shared_phase_name(int32_t i) {
  return (i >= 0 && i < kSharedPhases) ? kSharedPhaseNames[i] : nullptr;
}

static int shared_mode(int32_t share) {
  return share == ATLASKV_SHARE_KV_GROUP ? kModeSharedKvGroup
         : share == ATLASKV_SHARE_SEQUENCE ? kModeSharedSequence : -1;
}

atlaskv_status atlaskv_shared_workspace_size(atlaskv_tree_view v, const atlaskv_tensor* q,
                                             const atlaskv_tensor* seq_k, const int32_t K[3],
                                             int32_t share, size_t* bytes) {
  if (!bytes) return fail(ATLASKV_ERR_NULL, "bytes is NULL");
  const int mode = shared_mode(share);
  if (mode < 0) return fail(ATLASKV_ERR_UNSUPPORTED, "share must be ATLASKV_SHARE_KV_GROUP or _SEQUENCE");
  Plan p;
  atlaskv_status st = plan_call(q, v, seq_k, seq_k, K, nullptr, nullptr, false, p, mode);
  if (st) return st;
  *bytes = p.total;
  return ATLASKV_OK;
}

atlaskv_status atlaskv_shared_check_args(const atlaskv_tensor* q, atlaskv_tree_view v,
                                         const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                         const int32_t K[3], int32_t share, const atlaskv_tensor* out,
                                         const atlaskv_attend_opts* opts) {
  const int mode = shared_mode(share);
  if (mode < 0) return fail(ATLASKV_ERR_UNSUPPORTED, "share must be ATLASKV_SHARE_KV_GROUP or _SEQUENCE");
  Plan p;
  void* ws = nullptr;
  return check_all(q, v, seq_k, seq_v, K, out, opts, p, &ws, mode);
}

atlaskv_status atlaskv_shared_attend_ex(const atlaskv_tensor* q, atlaskv_tree_view v,
                                        const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                        const int32_t K[3], int32_t share, atlaskv_tensor* out,
                                        const atlaskv_attend_opts* opts) {
  const int mode = shared_mode(share);
  if (mode < 0) return fail(ATLASKV_ERR_UNSUPPORTED, "share must be ATLASKV_SHARE_KV_GROUP or _SEQUENCE");
  Plan p;
  void* wsv = nullptr;
  atlaskv_status st = check_all(q, v, seq_k, seq_v, K, out, opts, p, &wsv, mode);
  if (st) return st;
  if (v->described_only) return fail(ATLASKV_ERR_UNSUPPORTED, "a described-only view cannot run");
  if (p.R == 0) return ATLASKV_OK;
  hipStream_t s = (opts && opts->stream) ? (hipStream_t)opts->stream : v->stream;
  char* ws = (char*)wsv;
  const int Ng = mode == kModeSharedSequence ? 1 : p.N;
  // the group rows and their descent's workspace (at the start of ws)
  atlaskv_tensor gd = group_rows_desc(p.B, Ng, v->dev.Hkv, v->dev.d, v->dev.dtype, ws + p.off_gq);
  Plan pg;
  if ((st = plan_call(&gd, v, seq_k, seq_v, K, nullptr, nullptr, false, pg, kModeHikvp))) return st;
  RowsDev rows, grows;
  fill_rows(rows, q, opts, p);
  fill_rows(grows, &gd, nullptr, pg);
  grows.scale = p.scale;
  grows.q_exact = (const double*)(ws + p.off_gqx);   // the selection is exact for the unrounded sums
  grows.q_delta = (const float*)(ws + p.off_gdelta);
  grows.q_lo = v->dev.dtype == ATLASKV_BF16 ? (const void*)(ws + p.off_glo) : nullptr;
  const SelTargets st3 = sel_targets(pg, opts, ws);
  int32_t* const* sel = st3.sel;
  float* lse_kg = (opts && opts->lse_kg) ? opts->lse_kg : (float*)(ws + p.off_lse);
  float* o_kg = (float*)(ws + p.off_okg);
  SharedArgs sa;
  memset(&sa, 0, sizeof sa);
  sa.t = v->dev;
  sa.r = rows;
  sa.B = p.B;
  sa.Ng = Ng;
  sa.gq = ws + p.off_gq;
  sa.gqx = (double*)(ws + p.off_gqx);
  sa.glo = ws + p.off_glo;
  sa.gdelta = (float*)(ws + p.off_gdelta);
  sa.gpart = (double*)(ws + p.off_gpart);
  sa.chunks = group_chunks(p.N, Ng, &sa.tn);
  sa.sel_leaf = sel[2];
  sa.KL = p.K[2];
  sa.o_kg = o_kg;
  sa.lse_kg = lse_kg;
  PhaseMarks pm(opts, s);
  const SeqHalf sh = seq_prepare(p, rows, v->dev.Hkv, v->dev.d, v->dev.dtype, seq_k, seq_v, out, opts, o_kg,
                                 lse_kg, ws, v);
  hipError_t e = pm.mark(hipSuccess);
  if (e == hipSuccess) e = seq_start(sh, v, s);
  if (e == hipSuccess) e = pm.mark(launch_group_query(sa, s));
  // the descent on the group rows; its own KG softmax lands in its workspace
  if (e == hipSuccess)
    e = launch_descent(pg, grows, v, ws, sel, (float*)(ws + pg.off_okg), (float*)(ws + pg.off_lse), s, pm, &sh);
  if (e == hipSuccess) e = pm.mark(launch_shared_kg(sa, s));
  if (e == hipSuccess) e = seq_finish(sh, v, s, pm);
  if (e == hipSuccess) e = finish_sel(st3, pg, s);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return ATLASKV_OK;
}

static const char* const kFoldedPhaseNames[] = {
    "fold_query", "root_score_topk", "mid_bucket_gemm", "mid_topk", "leaf_bucket_link",
    "leaf_score_stream", "leaf_topk_kg_attention", "unfold_values",
    "seq_attention", "seq_split_combine"};
static const int kFoldedPhases = (int)(sizeof kFoldedPhaseNames / sizeof kFoldedPhaseNames[0]);

int32_t atlaskv_folded_phase_count(void) { return kFoldedPhases; }

const char* atlaskv_folded_phase_name(int32_t i) {
  return (i >= 0 && i < kFoldedPhases) ? kFoldedPhaseNames[i] : nullptr;
}

atlaskv_status atlaskv_folded_workspace_size(atlaskv_tree_view v, const atlaskv_tensor* q,
                                             const atlaskv_tensor* w_k, const atlaskv_tensor* seq_k,
                                             const int32_t K[3], size_t* bytes) {
  if (!bytes) return fail(ATLASKV_ERR_NULL, "bytes is NULL");
  Plan p, pd;
  atlaskv_status st = plan_folded(q, v, w_k, w_k, seq_k, seq_k, K, nullptr, nullptr, false, p, pd);
  if (st) return st;
  *bytes = p.total;
  return ATLASKV_OK;
}

static atlaskv_status check_folded(const atlaskv_tensor* q, atlaskv_tree_view v, const atlaskv_tensor* w_k,
                                   const atlaskv_tensor* w_v, const atlaskv_tensor* seq_k,
                                   const atlaskv_tensor* seq_v, const int32_t K[3], const atlaskv_tensor* out,
                                   const atlaskv_attend_opts* opts, Plan& p, Plan& pd, void** ws) {
  atlaskv_status st = plan_folded(q, v, w_k, w_v, seq_k, seq_v, K, out, opts, true, p, pd);
  if (st) return st;
  void* w = (opts && opts->workspace) ? opts->workspace : v->workspace;
  size_t wb = (opts && opts->workspace) ? opts->workspace_bytes : v->workspace_bytes;
  if (p.R > 0) {
    if (!w) return fail(ATLASKV_ERR_WORKSPACE, "no workspace (need %zu bytes)", p.total);
    if (((uintptr_t)w) % 256) return fail(ATLASKV_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (wb < p.total) return fail(ATLASKV_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", wb, p.total);
  }
  *ws = w;
  return ATLASKV_OK;
}

atlaskv_status atlaskv_folded_check_args(const atlaskv_tensor* q, atlaskv_tree_view v,
                                         const atlaskv_tensor* w_k, const atlaskv_tensor* w_v,
                                         const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                         const int32_t K[3], const atlaskv_tensor* out,
                                         const atlaskv_attend_opts* opts) {
  Plan p, pd;
  void* ws = nullptr;
  return check_folded(q, v, w_k, w_v, seq_k, seq_v, K, out, opts, p, pd, &ws);
}

atlaskv_status atlaskv_folded_attend_ex(const atlaskv_tensor* q, atlaskv_tree_view v,
                                        const atlaskv_tensor* w_k, const atlaskv_tensor* w_v,
                                        const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                        const int32_t K[3], atlaskv_tensor* out,
                                        const atlaskv_attend_opts* opts) {
  Plan p, pd;
  void* wsv = nullptr;
  atlaskv_status st = check_folded(q, v, w_k, w_v, seq_k, seq_v, K, out, opts, p, pd, &wsv);
  if (st) return st;
  if (v->described_only) return fail(ATLASKV_ERR_UNSUPPORTED, "a described-only view cannot run");
  if (p.R == 0) return ATLASKV_OK;
  hipStream_t s = (opts && opts->stream) ? (hipStream_t)opts->stream : v->stream;
  char* ws = (char*)wsv;
  RowsDev rows;
  fill_rows(rows, q, opts, p);
  float* lse_kg = (opts && opts->lse_kg) ? opts->lse_kg : (float*)(ws + p.off_lse);
  float* o_kg = (float*)(ws + p.off_okg);
  FoldArgs fa;
  memset(&fa, 0, sizeof fa);
  fa.r = rows;
  fa.w_k = w_k->data;
  fa.w_v = w_v->data;
  fa.wks[0] = w_k->stride[0]; fa.wks[1] = w_k->stride[1];
  fa.wvs[0] = w_v->stride[0]; fa.wvs[1] = w_v->stride[1];
  fa.d = p.fold_d;
  fa.DE = v->dev.d;
  fa.dtype = v->dev.dtype;
  fa.qf = ws + p.off_qf;
  fa.qx = (double*)(ws + p.off_qx);
  fa.qlo = ws + p.off_qlo;
  fa.qdelta = (float*)(ws + p.off_qdelta);
  fa.o_base = p.fold_kg_empty ? nullptr : (const float*)(ws + pd.off_okg);
  fa.o_kg = o_kg;
  fa.lse_kg = lse_kg;
  PhaseMarks pm(opts, s);
  const SeqHalf sh = seq_prepare(p, rows, p.fold_Hkv, p.fold_d, v->dev.dtype, seq_k, seq_v, out, opts, o_kg,
                                 lse_kg, ws, v);
  hipError_t e = pm.mark(hipSuccess);
  if (e == hipSuccess) e = seq_start(sh, v, s);
  if (p.fold_kg_empty) {
    // no descent: seven empty phases (the fold and the six descent phases)
    // keep the event numbering
    for (int i = 0; i < 7 && e == hipSuccess; ++i) e = pm.mark(hipSuccess);
  } else if (e == hipSuccess) {
    e = pm.mark(launch_fold_query(fa, s));
    atlaskv_tensor qd = group_rows_desc(p.B, p.N, p.Hq, v->dev.d, v->dev.dtype, fa.qf);
    RowsDev frows;
    fill_rows(frows, &qd, nullptr, pd);
    frows.scale = p.scale;
    frows.q_exact = fa.qx;
    frows.q_delta = fa.qdelta;
    frows.q_lo = v->dev.dtype == ATLASKV_BF16 ? fa.qlo : nullptr;
    const SelTargets st3 = sel_targets(pd, opts, ws);
    if (e == hipSuccess) e = launch_descent(pd, frows, v, ws, st3.sel, (float*)(ws + pd.off_okg), lse_kg, s, pm, &sh);
    if (e == hipSuccess) e = finish_sel(st3, pd, s);
  }
  if (e == hipSuccess) e = pm.mark(launch_unfold_values(fa, p.fold_kg_empty != 0, s));
  if (e == hipSuccess)
    e = seq_finish(sh, v, s, pm);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return ATLASKV_OK;
}

static const char* const kFlatPhaseNames[] = {"flat_kg_partial", "flat_kg_combine", "seq_attention",
                                              "seq_split_combine"};
static const int kFlatPhases = (int)(sizeof kFlatPhaseNames / sizeof kFlatPhaseNames[0]);

int32_t atlaskv_flat_phase_count(void) { return kFlatPhases; }

const char* atlaskv_flat_phase_name(int32_t i) {
  return (i >= 0 && i < kFlatPhases) ? kFlatPhaseNames[i] : nullptr;
}

atlaskv_status atlaskv_flat_workspace_size(atlaskv_tree_view v, const atlaskv_tensor* q,
                                           const atlaskv_tensor* seq_k, size_t* bytes) {
  if (!bytes) return fail(ATLASKV_ERR_NULL, "bytes is NULL");
  Plan p;
  atlaskv_status st = plan_call(q, v, seq_k, seq_k, nullptr, nullptr, nullptr, false, p, kModeFlat);
  if (st) return st;
  *bytes = p.total;
  return ATLASKV_OK;
}

atlaskv_status atlaskv_flat_attend_ex(const atlaskv_tensor* q, atlaskv_tree_view v,
                                      const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                      atlaskv_tensor* out, const atlaskv_attend_opts* opts) {
  Plan p;
  void* wsv = nullptr;
  atlaskv_status st = check_all(q, v, seq_k, seq_v, nullptr, out, opts, p, &wsv, kModeFlat);
  if (st) return st;
  if (v->described_only) return fail(ATLASKV_ERR_UNSUPPORTED, "a described-only view cannot run");
  if (p.R == 0) return ATLASKV_OK;
  hipStream_t s = (opts && opts->stream) ? (hipStream_t)opts->stream : v->stream;
  char* ws = (char*)wsv;
  RowsDev rows;
  fill_rows(rows, q, opts, p);
  float* lse_kg = (opts && opts->lse_kg) ? opts->lse_kg : (float*)(ws + p.off_lse);
  float* o_kg = (float*)(ws + p.off_okg);
  PhaseMarks pm(opts, s);
  const SeqHalf sh = seq_prepare(p, rows, v->dev.Hkv, v->dev.d, v->dev.dtype, seq_k, seq_v, out, opts, o_kg,
                                 lse_kg, ws, v);
  hipError_t e = pm.mark(hipSuccess);
  if (e == hipSuccess) e = seq_start(sh, v, s);
  FlatArgs fa;
  memset(&fa, 0, sizeof fa);
  fa.t = v->dev;
  fa.r = rows;
  fa.nsplit = p.flat_nsplit;
  fa.split_len = p.flat_split_len;
  fa.row_tiles = p.flat_row_tiles;
  fa.part = (float*)(ws + p.off_fpart);
  fa.o_kg = o_kg;
  fa.lse_kg = lse_kg;
  // KG half over every leaf, then the sequence half and the λ merge as in the pruned path
  if (e == hipSuccess) e = pm.mark(launch_flat_partial(fa, s));
  if (e == hipSuccess) e = pm.mark(launch_flat_combine(fa, s));
  if (e == hipSuccess) e = seq_finish(sh, v, s, pm);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return ATLASKV_OK;
}

atlaskv_status atlaskv_flat_check_args(const atlaskv_tensor* q, atlaskv_tree_view v,
                                       const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                       const atlaskv_tensor* out, const atlaskv_attend_opts* opts) {
  Plan p;
  void* ws = nullptr;
  return check_all(q, v, seq_k, seq_v, nullptr, out, opts, p, &ws, kModeFlat);
}

}  // extern "C"
