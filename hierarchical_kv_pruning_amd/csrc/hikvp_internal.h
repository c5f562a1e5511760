// hikvp_internal.h -- argument blocks shared by the C-ABI layer and the HIP
// kernels of libatlaskv.so.  Internal: not installed, not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hikvp {

constexpr int kMaxK = 256;        // largest Top-K per level
constexpr int kMaxD = 128;        // largest head dim of the per-head trees and the sequence half
constexpr int kMaxWideD = 4096;   // largest width of a base-embedding tree (a multiple of 128)
// Members of a (head, mid) bucket stored in fixed slots (no list walk): 32
// for per-head trees, 64 for a folded call's base tree, where every query
// head selects from the one tree and a bucket holds ~13 rows with a long
// tail (64 slots: folded D_E = 384 overflow 42 -> 6 us, step 0.917 -> 0.888
// ms; the per-row paths lost ~1 % with 64, reading twice the slot bytes).
constexpr int kBucketSlots = 32, kBucketSlotsFolded = 64;
constexpr int kJunkSlots = 1024;  // per-wave sinks for masked-off score stores
constexpr int kRootTile = 64;     // member rows per mid-GEMM work item (four waves of 16 rows)
constexpr int kRootSub = 16;      // counters per (head, root) group, picked by token
constexpr int kDescSub = 64;      // bucket descriptor sub-lists, picked by link chunk
constexpr int kFilterK = 32;      // largest K_I the mid tiles filter their scores for (else all are kept)
constexpr int64_t kMaxMidCands = (int64_t)1 << 24;  // mid candidates per row (slot bases pack in 24 bits)
constexpr int kMaxParts = 2;      // descent parts (KV-head ranges run concurrently)
constexpr int kLeafStageFloats = 2048;  // staged scores a leaf-stream wave holds (per-member groups)
constexpr int kLeafFilterMaxFan = 1024; // largest mid fanout the leaf-stream filter stages
constexpr int kLeafFilterRatio = 4;     // the filter runs when the largest mid fanout is >= this x K_L
constexpr int kDtypeF32 = 0;

// Row-aligned work chunks of the kernels that scan a row's K selections in
// one wave (root fill, bucket link): floor(64 / K) whole rows each when
// K <= 64, else one row each; and the most selections one chunk holds.
// Parts of a split descent: as many KV-head ranges as keep kPartRows rows or
// more each (at most kMaxParts, at most one per head).  Two concurrent parts
// measured faster than one at 16384 rows (0.588 -> 0.542 ms) and much slower
// at 4096 rows with a small tree (0.094 -> 0.152 ms: the leaf stream is too
// short to hide the other part's work); more parts measured slower.
constexpr int64_t kPartRows = 8192;
inline int descent_parts(int Hkv, int64_t rows) {
  int64_t n = rows / kPartRows;
  if (n > kMaxParts) n = kMaxParts;
  if (n > Hkv) n = Hkv;
  return n < 1 ? 1 : (int)n;
}

__host__ __device__ inline int row_chunks(int R, int K1) {
  return K1 <= 0 ? 0 : K1 <= 64 ? (R + 64 / K1 - 1) / (64 / K1) : R;
}
__host__ __device__ inline int row_chunk_entries(int K1) {
  return K1 <= 0 ? 0 : K1 <= 64 ? 64 / K1 * K1 : K1;
}

constexpr int kDtypeBF16 = 1;

// A three-level key tree in device memory.  Levels: 0 root, 1 mid, 2 leaf.
// Element strides: hs = per KV head, rs = per node (innermost stride 1).
struct TreeDev {
  const void* key[3];         // root_k, mid_k, leaf_k
  const void* leaf_v;
  int64_t hs[4], rs[4];       // [0..2] keys of each level, [3] leaf values
  const int64_t* off[2];      // child offsets of roots (into mids) and mids (into leaves)
  int64_t count[3];           // M_R, M_I, M
  const float* norm;          // [3][Hkv] upper bounds of the key 2-norms per level and head
  int Hkv, d, dtype;
};

// The query rows of one call: row r = (b*N + n)*Hq + h.
struct RowsDev {
  const void* q;              // sequence query [B,N,Hq,d]
  const void* q_kg;           // KG query (== q when not given)
  int64_t qs[3], qks[3];      // strides of b, n, h for q and q_kg
  int B, N, Hq, G;            // G = Hq / Hkv
  int R;                      // B*N*Hq
  double scale;               // logit scale (the fp64 ranking uses exactly this value)
  // When q_kg holds a rounding (to the tree's dtype) of an exact query -- a
  // folded W_K^T q or a sum of member queries -- the exact one, by row
  // index, and a bound on the rounding: the selection is then exact with
  // respect to the exact query.  NULL otherwise.  In bf16 the scores take
  // the exact query as the sum of two bf16 rows, q_kg (rounded) + q_lo (the
  // residual rounded), two MFMA passes on the same keys: the part left out
  // is ~2^-8 of one bf16 rounding, so the band of exactly re-scored
  // candidates stays as narrow as for a stored query.
  const double* q_exact;      // [R, d] fp64
  const float* q_delta;       // [R] upper bound of |q_kg + q_lo - q_exact|_2 (q_lo NULL: 0)
  const void* q_lo;           // [R, d] tree dtype (bf16 only), or NULL
};

// One attend call's selection path (root -> mid -> leaf -> KG attention),
// for the rows of KV heads [g0, g1): row blocks [blk0, blk1) in the
// KV-head-major block order of row_of_block.  Every index structure below
// is keyed by KV head (or by row), so parts with disjoint heads can run
// concurrently; the per-part ones (tiles, descriptors, counts, overflow
// keys) point into the part's own region.
struct StepArgs {
  TreeDev t;
  RowsDev r;
  int g0, g1;                 // KV heads of this part
  int blk0, blk1;             // row blocks of this part
  int K[3];                   // Top-K per level (plan-clamped; a row takes min(K, its candidates))
  int mid_spt;                // surviving mid candidates a lane of the mid select holds in registers (4, 16)
  int64_t c1max;              // mid candidates per row: capacity and row stride of mid_pairs
  int64_t c2max;              // leaf candidates per row: capacity
  uint2* mid_pairs;           // [R, c1max] surviving mid candidates: (unscaled fp32 score bits, child
                              // index within its root's span), those of the row's k-th selected root
                              // from slot pre[k] on; the row's first 2*c1max floats also carry the
                              // root scores between the root kernels
  int4* mid_meta;             // [R, K[0]] per (row, selected root): survivors, first candidate slot,
                              // first child (mid index), the row's |q_kg| bound (fp32 bits)
  float* leaf_scores;         // [R, c2max] unscaled fp32 leaf scores, candidate order
  int32_t* sel[3];            // [R, K[i]] selected node indices, candidate order, -1 padded
  int32_t* mid_base;          // [R, K[1]] first leaf-candidate slot of each selected mid
  // rows grouped by selected (head, root), each group padded to kRootTile rows
  int32_t* root_cnt;          // [kRootSub, Hkv * M_R] rows per sub-counter; the scan turns
                              // them into each sub-counter's first rank in the group
  int32_t* root_tot;          // [Hkv * M_R] rows that selected the (head, root)
  int32_t* root_tile_off;     // [Hkv * M_R] first work item (tile) of each group
  int32_t* root_tile_key;     // [root_tiles_max] group (key g*M_R + root) of each tile
  int32_t* root_ntiles;       // [1] tiles in use
  int2* root_members;         // [root_tiles_max * kRootTile] (row, first mid slot | selection index << 24)
  int64_t root_tiles_max;     // rows*K[0]/kRootTile + heads*M_R + 1 (rows, heads of the part)
  // (head, mid) bucket arrays are indexed by bucket_index(key) (below), which
  // spreads neighbouring mids (siblings, selected together) over cache lines
  int32_t* bucket_cnt;        // [64 * bucket_q] rows that selected the (head, mid)
  int2* bucket_slot;          // [64 * bucket_q * bslots] first members: (row, first leaf slot)
  int32_t* bucket_head;       // [64 * bucket_q] overflow members: list head, -1 none
  int32_t* bucket_next;       // [R * K[1]] next overflow entry of the same (head, mid)
  int4* bucket_desc;          // [kDescSub, desc_per_sub] distinct (head, mid): key g*M_I+mid, fanout,
                              // first leaf element (lo, hi); sub-list s holds buckets first
                              // registered by a link chunk c with c mod kDescSub = s
  int32_t* bucket_count;      // [kDescSub + 1] descriptors per sub-list; [kDescSub]: keys with more
                              // than bslots rows
  int32_t desc_per_sub;       // ceil(row_chunks(rows, K[1]) / kDescSub) * row_chunk_entries(K[1])
  int32_t bucket_q;           // ceil(Hkv * M_I / 64)
  int32_t bslots;             // fixed member slots a bucket (kBucketSlots or kBucketSlotsFolded)
  float* junk;                // [kJunkSlots * 16] write-only sinks for the mid GEMM's idle score lanes
  int32_t* bucket_ovf;        // [rows * K[1] / (bslots + 1) + 1] keys (g*M_I + mid) with overflow members
  float* o_kg;                // [R, d] softmax-weighted leaf values (fp32)
  float* lse_kg;              // [R] log-sum-exp of the selected leaf logits
  // Leaf candidates filtered in the leaf stream (leaf_nst > 0; per-head trees):
  // a member's scores over a bucket's span are staged in LDS and only those
  // that can still be among the row's K_L best are written, as (unscaled fp32
  // score bits, leaf index in the span) pairs from the mid's first candidate
  // slot on; the bucket members then carry (row, first slot | k << 24), k the
  // mid's place in the row's selection.
  uint2* leaf_pairs;          // [R, c2max] survivors (leaf_nst > 0; else leaf_scores is used)
  int32_t* leaf_cnt;          // [R, K[1]] survivors per (row, selected mid)
  int leaf_nst;               // members scored per pass (their scores staged), 0: no filter
  int leaf_fpad;              // staged scores per member: max mid fanout rounded up to 4
  int leaf_spt;               // survivors a lane of the filtered leaf select holds in registers
  int exact_logits;           // non-zero (folded calls on fp32 trees): the KG softmax takes the selected
                              // leaves' logits from the exact query r.q_exact (fp64 dot products),
                              // not from the scores
};

// Bucket array index of key = g*M_I + mid: a bijective transpose of [0, 64*q)
// (consecutive keys land 4*q bytes apart).
__device__ inline int64_t bucket_index(const StepArgs& a, int64_t key) {
  return (key & 63) * a.bucket_q + (key >> 6);
}

struct SeqArgs {
  RowsDev r;
  const void* k;              // [B, S, Hkv, d] (NULL: no sequence half)
  const void* v;
  int64_t ks[3], vs[3];       // strides of b, position, KV head
  int S, Hkv, d, dtype;
  const float* o_kg;          // [R, d]
  const float* lse_kg;        // [R]
  void* out;                  // [B, N, Hq, d]
  int64_t os[3];
  int out_dtype;
  float* lse_seq_out;         // optional [R]
  float* part;                // [R, nsplit, d + 2] partials for k_seq_combine (NULL: the attention
                              // kernel merges and stores the output itself; needs nsplit == 1)
  int nsplit;                 // key splits per row
  int split_len;              // keys per split (multiple of 64); >= S when not split
};

// One unpruned (flat) KG attention call: every leaf of the row's KV head.
struct FlatArgs {
  TreeDev t;
  RowsDev r;
  int nsplit;                 // leaf-key ranges per (KV head, row tile)
  int split_len;              // keys per range (multiple of 64)
  int row_tiles;              // 128-row tiles of one KV head's B*N*G rows
  float* part;                // [R, nsplit, d + 4] per range: o (relative to m), m (log2 units), sum, pad
  float* o_kg;                // [R, d]
  float* lse_kg;              // [R]
};

// Shared selections: the real rows and their groups' leaf selections.
struct SharedArgs {
  TreeDev t;
  RowsDev r;                  // the real rows (their own q / q_kg)
  int B, Ng;                  // groups: [B, Ng, Hkv], Ng = N (per token) or 1 (per sequence)
  void* gq;                   // [B, Ng, Hkv, d] group queries, tree dtype
  double* gqx;                // [B, Ng, Hkv, d] the exact sums (fp64) gq rounds
  void* glo;                  // [B, Ng, Hkv, d] bf16 only: gqx - gq rounded to bf16
  float* gdelta;              // [B, Ng, Hkv] upper bound of |gq + glo - gqx|_2 (fp32: |gq - gqx|_2)
  double* gpart;              // [B*Ng*Hkv, chunks, d] fp64 partial sums over chunks of tn tokens
  int chunks, tn;
  const int32_t* sel_leaf;    // [B*Ng*Hkv, KL] leaves selected for each group, -1 padded
  int KL;
  float* o_kg;                // [R, d]
  float* lse_kg;              // [R]
};

// Folded projections: the layer's rows, its per-head W_K / W_V [Hkv, d, D_E].
struct FoldArgs {
  RowsDev r;                  // the layer's rows (q_kg of width d)
  const void* w_k;            // [Hkv, d, D_E]: projected key of head g = W_K[g] k
  const void* w_v;            // [Hkv, d, D_E]
  int64_t wks[2], wvs[2];     // element strides of head and row (innermost 1)
  int d, DE, dtype;
  void* qf;                   // [R, D_E] folded queries W_K[g]^T q_kg, tree dtype
  double* qx;                 // [R, D_E] the exact products' sums (fp64) qf rounds
  void* qlo;                  // [R, D_E] bf16 only: qx - qf rounded to bf16
  float* qdelta;              // [R] upper bound of |qf + qlo - qx|_2 (fp32: |qf - qx|_2)
  const float* o_base;        // [R, D_E] softmax-weighted base values (the descent's KG half)
  float* o_kg;                // [R, d]
  float* lse_kg;              // [R] (written only when the KG half is empty)
};

struct BuildStats {           // device-side result of tree validation
  int bad;                    // non-zero: malformed offsets
  int pad;
  unsigned long long maxfan[2];
  unsigned int norm_bits[1];  // [3*Hkv] float bits of the norm bounds (flexible)
};

hipError_t launch_validate(const int64_t* off, int64_t count, int64_t children, int which,
                           BuildStats* stats, hipStream_t s);
hipError_t launch_key_norms(const void* key, int dtype, int d, int Hkv, int64_t rows,
                            int64_t hs, int64_t rs, unsigned int* out_bits, hipStream_t s);
// dst[r, i] = src[r, i] for i < Ks, -1 for Ks <= i < Kd (rows r < R)
hipError_t launch_expand_sel(const int32_t* src, int Ks, int32_t* dst, int Kd, int R, hipStream_t s);
hipError_t launch_root(const StepArgs& a, hipStream_t s);          // (clears the group and bucket counters)
hipError_t launch_root_groups(const StepArgs& a, hipStream_t s);  // rows by selected (head, root)
hipError_t launch_mid_gemm(const StepArgs& a, hipStream_t s);
hipError_t launch_mid_select(const StepArgs& a, hipStream_t s);
hipError_t launch_leaf_link(const StepArgs& a, hipStream_t s);    // rows grouped by selected (head, mid)
hipError_t launch_leaf_score(const StepArgs& a, hipStream_t s);   // every member of every bucket
hipError_t launch_leaf_select(const StepArgs& a, hipStream_t s);
hipError_t launch_seq_attend(const SeqArgs& a, hipStream_t s);   // + λ merge when keys are not split
hipError_t launch_seq_combine(const SeqArgs& a, hipStream_t s);  // split partials: LSE combine + λ merge
hipError_t launch_flat_partial(const FlatArgs& a, hipStream_t s);  // per (head, rows, key range)
hipError_t launch_flat_combine(const FlatArgs& a, hipStream_t s);  // ranges -> o_kg, lse_kg
hipError_t launch_group_query(const SharedArgs& a, hipStream_t s);  // member sums -> gq
int group_chunks(int N, int Ng, int* tn);                           // token chunks of a group sum
hipError_t launch_shared_kg(const SharedArgs& a, hipStream_t s);    // per-row softmax over group leaves
hipError_t launch_fold_query(const FoldArgs& a, hipStream_t s);                  // q' = W_K^T q
hipError_t launch_unfold_values(const FoldArgs& a, bool kg_empty, hipStream_t s);  // o_kg = W_V o_base
int flat_row_tiles(int B, int N, int G);
int flat_splits(int B, int N, int Hq, int Hkv, int64_t M, int dtype);
int flat_split_len(int64_t M, int nsplit);
int seq_splits(int B, int N, int Hkv, int G, int S, int dtype);  // key splits of the sequence attention
int seq_split_len(int S, int nsplit);

}  // namespace hikvp
