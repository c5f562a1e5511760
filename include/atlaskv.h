/*
 * atlaskv.h -- C ABI of libatlaskv.so: HiKVP knowledge-injected attention for
 * one attention layer on an MI355X (gfx950) GPU.
 *
 * The operation (page: "AtlasKV: Augmenting LLMs with Billion-Scale Knowledge
 * Graphs in 20GB VRAM", digest of arXiv 2510.17934):
 *   - 速读 › 怎么做的 (quick read, how it is done): the knowledge keys form a
 *     three-level tree (root, mid, leaf).  For each query, score the root keys,
 *     keep the Top-K branches, score their children, keep the Top-K, and so on
 *     down to the leaves.  The layer output is then
 *         y = λ_kg · Softmax(logits_kg) · v̄  +  λ_seq · Softmax(logits_seq) · v
 *     where logits_kg are the selected leaves' logits and logits_seq the
 *     ordinary causal attention logits.
 *   - 背景知识与设计原则 › 自注意力层机制: causal attention, logits
 *     <q_n, k_i>/sqrt(D) over positions i <= n.
 *   - 方法细节 › 等效注意力机制的知识增强: the λ definitions are missing from
 *     the page; this library uses the log-sum-exp shares
 *         λ_kg = Σexp(logits_kg) / (Σexp(logits_kg) + Σexp(logits_seq)),
 *         λ_seq = 1 - λ_kg,
 *     which makes the merge equal to one softmax over both logit sets, i.e.
 *     the rectangular attention of 背景知识与设计原则 › KBLaM中的矩形注意力
 *     restricted to the selected leaves.
 *
 * Semantics fixed by this library where the page is silent:
 *   - a row is one (batch b, token n, query head h); every row selects its own
 *     nodes.  Query head h reads KV head g = h / (Hq / Hkv) of the tree and of
 *     the sequence (grouped-query attention); the tree topology is shared by
 *     all KV heads;
 *   - ranking key: the scaled logit scale * <q_kg, k>, with scale = 1/sqrt(d)
 *     unless given; equal keys rank the lower node index first.  Selections
 *     are exact with respect to the fp64 value of that logit computed from the
 *     stored inputs (products exact, summed left to right over the head dim);
 *   - K clamps to the number of candidates; K = 0 at any level empties the KG
 *     half (then the output is plain causal attention).  Before anything
 *     runs, each level's K is clamped to the most candidates a row can have
 *     there (M_R roots; the children of K_R roots under the largest root
 *     fanout, at most M_I; the children of K_I mids likewise, at most M), so
 *     K at or above that bound selects every candidate whatever its value.
 *     Only a clamped K above 256 (more than 256 selections out of more than
 *     256 candidates) is refused, with ATLASKV_ERR_K;
 *   - causal alignment is bottom-right: token n sees sequence positions
 *     0 .. S_kv - N + n (so S_kv >= N); seq_k == NULL means no sequence half;
 *   - only leaves carry values; the KG softmax runs over the K_L selected
 *     leaves and reuses the logits computed for the selection.
 *
 * Memory and threading:
 *   - every tensor is device memory owned by the caller, except that the
 *     tree's tensors may instead live in pinned host memory (below); the
 *     library never copies or frees them.  A tree view references its tensors
 *     until destroyed;
 *   - atlaskv_hikvp_attend* allocate nothing: scratch memory is the caller's
 *     workspace (size from atlaskv_hikvp_workspace_size).  Only
 *     atlaskv_build_tree_view allocates (a few bytes of device memory per KV
 *     head, two streams and four events, freed by atlaskv_destroy_tree_view)
 *     and synchronises its stream;
 *   - attend calls are asynchronous on their stream; device faults surface at
 *     the caller's next synchronisation.  Calls on different streams need
 *     separate workspaces; calls sharing a workspace must be stream-ordered.
 *     Unless phase events are requested, the causal sequence half runs on a
 *     second stream that the view owns (default priority), forked by an
 *     event and joined back before the merge, so it overlaps the KG half:
 *     for query blocks under 16 tokens (decode) it is forked from the call's
 *     stream before the KG kernels, for longer blocks from the last descent
 *     part (after its root phase when the descent runs in two parts, else
 *     just before its leaf scoring).
 *     With 16384 query rows or more (B*N*Hq, or groups for shared
 *     selections) and two KV heads or more, the KG descent itself runs in two
 *     concurrent parts (the two halves of the KV heads, which share no index
 *     structure), the second on the view's other stream, forked and joined
 *     the same way.  The call's stream still orders
 *     everything the call reads and writes.  With phase events the halves and
 *     parts run one after the other on the call's stream (same results, bit
 *     for bit).
 *
 * Errors: every entry point returns an atlaskv_status.  Argument errors are
 * detected on the host before anything is enqueued, so a failed call writes
 * nothing.  atlaskv_last_error() returns a message for the calling thread's
 * most recent failure.
 */
#ifndef ATLASKV_H
#define ATLASKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATLASKV_OK = 0,
  ATLASKV_ERR_NULL = 1,        /* a required pointer is NULL */
  ATLASKV_ERR_DTYPE = 2,       /* unknown dtype, or inputs of different dtypes */
  ATLASKV_ERR_SHAPE = 3,       /* shapes, strides or alignment inconsistent */
  ATLASKV_ERR_TREE = 4,        /* malformed child offsets */
  ATLASKV_ERR_K = 5,           /* K < 0, a clamped K above 256, or both halves empty */
  ATLASKV_ERR_WORKSPACE = 6,   /* workspace missing, too small or misaligned */
  ATLASKV_ERR_UNSUPPORTED = 7, /* head dim not 64/128 (or a wide tree outside the folded entry
                                  point), node counts >= 2^31, scale <= 0 */
  ATLASKV_ERR_HIP = 8          /* a HIP runtime call failed */
} atlaskv_status;

typedef enum { ATLASKV_F32 = 0, ATLASKV_BF16 = 1 } atlaskv_dtype;

/* A strided view of caller-owned device memory.  Strides are in elements and
 * the innermost stride must be 1; rows must start on 16-byte boundaries. */
typedef struct {
  void* data;
  int32_t dtype;       /* atlaskv_dtype */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} atlaskv_tensor;

typedef struct atlaskv_tree_view_s* atlaskv_tree_view;

/*
 * Build a view of a three-level key tree (方法细节 › KGKVs的层次化聚类 gives
 * the levels; the tree itself is built offline by the caller).
 *   root_k  [Hkv, M_R, d]   root keys
 *   mid_k   [Hkv, M_I, d]   mid keys
 *   leaf_k  [Hkv, M,   d]   leaf keys
 *   leaf_v  [Hkv, M,   d]   leaf values
 *   root_child_off  device int64 [M_R + 1]: mids of root j are
 *                   root_child_off[j] .. root_child_off[j+1]-1
 *   mid_child_off   device int64 [M_I + 1]: leaves of mid m likewise
 * All float tensors share one dtype and head dim d (64 or 128; a base-
 * embedding tree for atlaskv_folded_attend_ex may also be a multiple of 128
 * up to 4096 wide).  Offsets must start at 0,
 * be non-decreasing and end at M_I (resp. M); empty ranges are allowed.
 * stream: hipStream_t (NULL = default stream) used for validation and as the
 * default stream of attend calls.  The call validates the offsets and
 * computes per-level key-norm bounds on the GPU, then synchronises once.
 * Returns ATLASKV_ERR_TREE for malformed offsets; *out is set only on success.
 *
 * Host-tiered trees (速读 › 怎么做的 keeps only the root keys in GPU memory
 * and brings each lower level in from CPU memory as the descent reaches it;
 * 速读 › 效果如何 names that traffic as the method's I/O cost): any of the six
 * tree arrays may be pinned host memory (hipHostMalloc, or a torch tensor
 * with pin_memory=True) instead of device memory.  The kernels then read it
 * through its device mapping over the host link: each level's selected spans
 * are fetched by the kernel that scores them, once per (KV head, node) group,
 * so only the selected mids' leaf spans and the selected leaves' values cross
 * the link.  Results are identical to a device-resident tree.  Pageable host
 * memory, or device memory of another GPU, gives ATLASKV_ERR_UNSUPPORTED
 * before anything is enqueued.
 */
atlaskv_status atlaskv_build_tree_view(const atlaskv_tensor* root_k, const atlaskv_tensor* mid_k,
                                       const atlaskv_tensor* leaf_k, const atlaskv_tensor* leaf_v,
                                       const int64_t* root_child_off, const int64_t* mid_child_off,
                                       void* stream, atlaskv_tree_view* out);

/* Where a view's tree lives: bit i set when tree array i (0 root_k, 1 mid_k,
 * 2 leaf_k, 3 leaf_v, 4 root_child_off, 5 mid_child_off) is pinned host
 * memory; 0 for an all-device tree, -1 for NULL. */
int32_t atlaskv_tree_view_placement(atlaskv_tree_view tree);

/* Release a view (and its small device buffers).  NULL is accepted. */
atlaskv_status atlaskv_destroy_tree_view(atlaskv_tree_view tree);

/* Attach a caller-owned device workspace (256-byte aligned) used by
 * atlaskv_hikvp_attend.  bytes = 0 detaches. */
atlaskv_status atlaskv_tree_view_set_workspace(atlaskv_tree_view tree, void* workspace, size_t bytes);

/* Workspace bytes an attend call with these shapes and K needs.  q gives
 * B, N, Hq; seq_k may be NULL.  Host only. */
atlaskv_status atlaskv_hikvp_workspace_size(atlaskv_tree_view tree, const atlaskv_tensor* q,
                                            const atlaskv_tensor* seq_k,
                                            const int32_t K_per_level[3], size_t* bytes);

/*
 * HiKVP attention for one layer, enqueued on the view's stream with the view's
 * workspace.
 *   q      [B, N, Hq, d]  queries (post-RoPE); also the KG query
 *   seq_k  [B, S_kv, Hkv, d], seq_v likewise: causal sequence keys/values
 *          (both NULL: no sequence half)
 *   K_per_level  host int32 {K_R, K_I, K_L}, each >= 0 (clamped per level, see above)
 *   out    [B, N, Hq, d]  dtype of q, or fp32
 */
atlaskv_status atlaskv_hikvp_attend(const atlaskv_tensor* q, atlaskv_tree_view tree,
                                    const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                    const int32_t K_per_level[3], atlaskv_tensor* out);

/* Optional controls and outputs of atlaskv_hikvp_attend_ex.  Zero-initialise
 * and set what is needed. */
typedef struct {
  const atlaskv_tensor* q_kg; /* [B,N,Hq,d] KG query (the page's W̃_Q x); NULL -> q */
  float scale;                /* logit scale; 0 -> 1/sqrt(d); must be > 0 otherwise */
  void* stream;               /* hipStream_t; NULL -> the view's stream */
  void* workspace;            /* NULL -> the view's workspace */
  size_t workspace_bytes;
  int32_t* sel_root;          /* optional device [B*N*Hq, K_R] selected roots, -1 padded */
  int32_t* sel_mid;           /* optional device [B*N*Hq, K_I] */
  int32_t* sel_leaf;          /* optional device [B*N*Hq, K_L] */
  float* lse_kg;              /* optional device [B*N*Hq]: log Σexp(logits_kg), -inf if empty */
  float* lse_seq;             /* optional device [B*N*Hq]: log Σexp(logits_seq), -inf if empty */
  void** phase_events;        /* optional hipEvent_t[n_phase_events]: event 0 is recorded on the
                                 launch stream before the first kernel, event i after kernel
                                 phase i-1 (names from atlaskv_phase_name); for timing only */
  int32_t n_phase_events;
} atlaskv_attend_opts;

/* As atlaskv_hikvp_attend, with options (opts may be NULL).  The selections
 * are written as sets: each row's K entries (K as given, the row stride of
 * the selection outputs) are the selected node indices in candidate order,
 * -1 padded when fewer than K candidates exist. */
atlaskv_status atlaskv_hikvp_attend_ex(const atlaskv_tensor* q, atlaskv_tree_view tree,
                                       const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                       const int32_t K_per_level[3], atlaskv_tensor* out,
                                       const atlaskv_attend_opts* opts);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): as
 * atlaskv_hikvp_attend_ex, but the workspace is a fixed device array inside
 * the library -- one per GPU, atlaskv_noalloc_scratch_bytes() bytes (256 MiB),
 * held until the process ends -- so the call performs no allocation of any
 * kind.  opts->workspace must be NULL (ATLASKV_ERR_WORKSPACE otherwise); a
 * call whose workspace would exceed the array fails with
 * ATLASKV_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU
 * shares that GPU's array and leaves its contents behind (each call
 * initialises what it reads), so calls that overlap in time on one GPU --
 * on different streams or host threads -- race and must be serialised by the
 * caller.  Results equal atlaskv_hikvp_attend_ex's bit for bit.
 */
atlaskv_status atlaskv_hikvp_attend_noalloc(const atlaskv_tensor* q, atlaskv_tree_view tree,
                                            const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                            const int32_t K_per_level[3], atlaskv_tensor* out,
                                            const atlaskv_attend_opts* opts);

/* Size in bytes of the fixed workspace of atlaskv_hikvp_attend_noalloc. */
size_t atlaskv_noalloc_scratch_bytes(void);

/* The argument checks of atlaskv_hikvp_attend_ex alone: pure host code, no
 * HIP call, nothing enqueued.  tree may describe shapes only (see
 * atlaskv_tree_view_describe). */
atlaskv_status atlaskv_check_args(const atlaskv_tensor* q, atlaskv_tree_view tree,
                                  const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                  const int32_t K_per_level[3], const atlaskv_tensor* out,
                                  const atlaskv_attend_opts* opts);

/* A host-only view for argument checking (no device work, no validation of
 * offsets beyond their count): same tensors as atlaskv_build_tree_view plus
 * the maximum fanouts the caller asserts.  Usable with atlaskv_check_args and
 * atlaskv_hikvp_workspace_size; attend calls on it return
 * ATLASKV_ERR_UNSUPPORTED. */
atlaskv_status atlaskv_tree_view_describe(const atlaskv_tensor* root_k, const atlaskv_tensor* mid_k,
                                          const atlaskv_tensor* leaf_k, const atlaskv_tensor* leaf_v,
                                          int64_t max_root_fanout, int64_t max_mid_fanout,
                                          atlaskv_tree_view* out);

/* Kernel phases of one attend call, in launch order (for phase_events).
 * atlaskv_phase_count() phases; atlaskv_phase_name(i) names phase i (NULL if
 * out of range). */
int32_t atlaskv_phase_count(void);
const char* atlaskv_phase_name(int32_t phase);

/*
 * Unpruned equivalent attention (flat KG half).  背景知识与设计原则 ›
 * KBLaM中的矩形注意力 defines one softmax over the logits of every knowledge
 * key together with the visible sequence logits; 方法细节 ›
 * 等效注意力机制的知识增强 writes that same output as the λ merge of a KG
 * softmax and a sequence softmax and uses it, with nothing pruned, while
 * fine-tuning.  Here the KG half is the softmax over the logits
 * scale * <q_kg, leaf_k[g][m]> of ALL M leaves of the row's KV head g (the
 * roots and mids of the view are not read), weighted over leaf_v; the
 * sequence half and the merge are those of atlaskv_hikvp_attend.  The result
 * equals atlaskv_hikvp_attend with K at least every fanout sum, for any M.
 * Arguments as atlaskv_hikvp_attend_ex without K: q, seq_k/seq_v, out and
 * opts (q_kg, scale, stream, workspace, lse_kg, lse_seq, phase_events;
 * sel_* are ignored).  The workspace size comes from
 * atlaskv_flat_workspace_size.  bf16 trees run on matrix cores (scores and
 * softmax weights rounded to bf16 operands, fp32 accumulation); fp32 trees on
 * plain fp32 arithmetic.
 */
atlaskv_status atlaskv_flat_workspace_size(atlaskv_tree_view tree, const atlaskv_tensor* q,
                                           const atlaskv_tensor* seq_k, size_t* bytes);
atlaskv_status atlaskv_flat_attend_ex(const atlaskv_tensor* q, atlaskv_tree_view tree,
                                      const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                      atlaskv_tensor* out, const atlaskv_attend_opts* opts);
/* The argument checks of atlaskv_flat_attend_ex alone (pure host code). */
atlaskv_status atlaskv_flat_check_args(const atlaskv_tensor* q, atlaskv_tree_view tree,
                                       const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                       const atlaskv_tensor* out, const atlaskv_attend_opts* opts);
/* Kernel phases of one flat call, in launch order (for phase_events). */
int32_t atlaskv_flat_phase_count(void);
const char* atlaskv_flat_phase_name(int32_t phase);

/*
 * Shared selections.  速读 › 怎么做的 picks the Top-K branches of the current
 * query; its memory bound (the C_m·M^(1/3) + N term) reads like one selected
 * key set shared by many tokens.  In this variant a group of rows shares one
 * descent:
 *   ATLASKV_SHARE_KV_GROUP  the G query heads of one KV head at one token
 *                           (B*N*Hkv groups);
 *   ATLASKV_SHARE_SEQUENCE  every token and query head of one KV head in one
 *                           sequence (B*Hkv groups).
 * The group's query is the exact sum of its members' KG queries; ranking
 * nodes by it ranks them by the members' summed logits.  The sum is formed in
 * fp64 (token chunks, then chunks), exact whenever it fits 53 bits, i.e.
 * unless the members' magnitudes span more than ~2^40.  The scores are
 * computed with the sum rounded to the tree's dtype (in bf16 as the rounded
 * sum plus its rounded residual, two bf16 rows); the selection is exact for
 * the unrounded sum all the same: the band of candidates that the rounding
 * could reorder is widened by its bound and re-scored in fp64 with the
 * fp64 sum.
 * The descent (roots -> mids -> leaves, Top-K per level, ties to the lower
 * index) runs on the group queries; every row then takes the softmax of its
 * own KG logits over its group's K_L selected leaves, and its own sequence
 * half and λ merge as in atlaskv_hikvp_attend.  Arguments as
 * atlaskv_hikvp_attend_ex plus `share`; opts->sel_root/sel_mid/sel_leaf, when
 * given, receive the GROUP selections, [groups, K_x] in group order
 * (b, n, g) or (b, g).  Workspace size from atlaskv_shared_workspace_size.
 */
typedef enum { ATLASKV_SHARE_KV_GROUP = 1, ATLASKV_SHARE_SEQUENCE = 2 } atlaskv_share;
atlaskv_status atlaskv_shared_workspace_size(atlaskv_tree_view tree, const atlaskv_tensor* q,
                                             const atlaskv_tensor* seq_k, const int32_t K_per_level[3],
                                             int32_t share, size_t* bytes);
atlaskv_status atlaskv_shared_attend_ex(const atlaskv_tensor* q, atlaskv_tree_view tree,
                                        const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                        const int32_t K_per_level[3], int32_t share,
                                        atlaskv_tensor* out, const atlaskv_attend_opts* opts);
/* The argument checks of atlaskv_shared_attend_ex alone (pure host code). */
atlaskv_status atlaskv_shared_check_args(const atlaskv_tensor* q, atlaskv_tree_view tree,
                                         const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                         const int32_t K_per_level[3], int32_t share,
                                         const atlaskv_tensor* out, const atlaskv_attend_opts* opts);
/* Kernel phases of one shared-selection call, in launch order. */
int32_t atlaskv_shared_phase_count(void);
const char* atlaskv_shared_phase_name(int32_t phase);

/*
 * Folded projections: one base-embedding tree for every head.
 * 背景知识与设计原则 › KBLaM中的矩形注意力 scores a head's query against
 * projected knowledge keys W_K k and weights projected values W_V v, with
 * per-layer heads W_K, W_V mapping the encoder width D_E to the head dim d;
 * 方法细节 › KGKVs的层次化聚类 builds the tree over the base embeddings.
 * Because <q, W_K k> = <W_K^T q, k> and sum p W_V v = W_V sum p v, the tree
 * need not be projected per head:
 *   tree   a view whose root_k / mid_k / leaf_k / leaf_v are the base
 *          embeddings, ONE head ([1, M_x, D_E]), D_E 64, 128 or a multiple
 *          of 128 up to 4096 (views of such wide trees serve this entry
 *          point only; the others return ATLASKV_ERR_UNSUPPORTED);
 *   w_k, w_v  [Hkv, d, D_E]: head g's projected key is w_k[g] k, its
 *          projected value w_v[g] v; d in {64, 128};
 *   q, seq_k, seq_v, out as atlaskv_hikvp_attend with the layer's Hkv and d.
 * Row (b, n, h) with g = h / (Hq/Hkv) folds its KG query into
 * q' = w_k[g]^T q_kg (exact product sum in fp64), runs the pruned descent
 * over the base tree with q' (logit scale 1/sqrt(d) unless given), applies
 * w_v[g] to its softmax-weighted base values, and merges with its causal
 * sequence half.  The scores are computed with q' rounded to the tree dtype
 * (in bf16 as the rounded q' plus its rounded residual); the selections are
 * exact for the unrounded q' (the rounding's bound widens the band that is
 * re-scored in fp64 with q').  On fp32 trees the KG softmax takes the
 * selected leaves' logits from the unrounded q' in fp64; on bf16 trees it
 * uses their scores (rounded q' plus residual, fp32 sums), whose error lies
 * far below a bf16 output's rounding.  The result equals
 * atlaskv_hikvp_attend on the per-head projected trees (w_k[g] k, w_v[g] v)
 * up to fp32 rounding.  opts->sel_* receive per-row selections of base
 * nodes.  Workspace size from atlaskv_folded_workspace_size (it holds q' in
 * fp64, 8 * D_E bytes a row).
 */
atlaskv_status atlaskv_folded_workspace_size(atlaskv_tree_view tree, const atlaskv_tensor* q,
                                             const atlaskv_tensor* w_k, const atlaskv_tensor* seq_k,
                                             const int32_t K_per_level[3], size_t* bytes);
atlaskv_status atlaskv_folded_attend_ex(const atlaskv_tensor* q, atlaskv_tree_view tree,
                                        const atlaskv_tensor* w_k, const atlaskv_tensor* w_v,
                                        const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                        const int32_t K_per_level[3], atlaskv_tensor* out,
                                        const atlaskv_attend_opts* opts);
/* The argument checks of atlaskv_folded_attend_ex alone (pure host code). */
atlaskv_status atlaskv_folded_check_args(const atlaskv_tensor* q, atlaskv_tree_view tree,
                                         const atlaskv_tensor* w_k, const atlaskv_tensor* w_v,
                                         const atlaskv_tensor* seq_k, const atlaskv_tensor* seq_v,
                                         const int32_t K_per_level[3], const atlaskv_tensor* out,
                                         const atlaskv_attend_opts* opts);
/* Kernel phases of one folded call, in launch order. */
int32_t atlaskv_folded_phase_count(void);
const char* atlaskv_folded_phase_name(int32_t phase);

/* Message for the calling thread's most recent failed call ("" if none). */
const char* atlaskv_last_error(void);

/* Library version string. */
const char* atlaskv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ATLASKV_H */
