/*
 * hikvp_oracle.h -- plain fp64 CPU oracle for HiKVP knowledge-injected attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The GPU library shares
 * no code, header, table or helper with it.
 *
 * Sources (page: "AtlasKV: Augmenting LLMs with Billion-Scale Knowledge Graphs
 * in 20GB VRAM", a Chinese digest of arXiv 2510.17934):
 *   - 速读 › 怎么做的 (quick read, "how it is done"): the three-level descent
 *     (score the current query against the root keys, keep the Top-K branches,
 *     load their children, repeat down to the leaves) and the inference merge
 *     y = λ_kg·Softmax(logits_kg)·v̄ + λ_seq·Softmax(logits_seq)·v.
 *   - 背景知识与设计原则 › 自注意力层机制: causal softmax attention with
 *     logits <q_n,k_i>/sqrt(D) over i <= n.
 *   - 背景知识与设计原则 › KBLaM中的矩形注意力: one softmax over all KB logits
 *     plus the causal sequence logits (the rectangular formula).
 *   - 方法细节 › KGKVs的层次化聚类: level sizes S = ceil(cbrt(M)),
 *     M_I = [M^(2/3)], M_R = ceil(ceil(M^(2/3)) * M^(-1/3)).
 *   - 方法细节 › 等效注意力机制的知识增强: the λ-weighted pair of softmaxes
 *     named "equivalent" to the rectangular formula; its λ definitions are
 *     missing from the page.  Reading used here: λ_kg and λ_seq are the
 *     log-sum-exp shares of the two logit sets, which is the only choice that
 *     makes the pair equal to the single rectangular softmax.
 *
 * Conventions (readings where the page is silent):
 *   - one selection per row (b, n, h); KV head g = h / (Hq / Hkv);
 *   - ranking key: the fp64 scaled logit s = scale * sum_t q[t]*k[t]
 *     accumulated sequentially in t, ties broken by the lower node index;
 *   - K clamps to the candidate count; K = 0 at any level empties the KG set;
 *   - causal alignment is bottom-right: query n sees sequence positions
 *     0 .. S_kv - N + n;  S_kv == 0 means "no sequence part";
 *   - only leaves carry values; the KG softmax runs over the K_L selected
 *     leaves, whose logits are the scores already computed for the selection.
 *
 * Every array is host memory, C-contiguous, and owned by the caller.
 */
#ifndef HIKVP_ORACLE_H
#define HIKVP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage types the oracle reads (each value is converted exactly to fp64) */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

typedef struct {
  int32_t dtype;           /* storage type of every floating array below */
  int64_t B, N, S_kv;      /* sequences, new tokens per sequence, sequence length */
  int64_t Hq, Hkv, d;      /* query heads, KV heads, head dim */
  int64_t M_R, M_I, M;     /* root, mid and leaf counts */
  const void* q;           /* [B, N, Hq, d]  sequence query */
  const void* q_kg;        /* [B, N, Hq, d]  KG query; NULL -> q */
  const void* root_k;      /* [Hkv, M_R, d] */
  const void* mid_k;       /* [Hkv, M_I, d] */
  const void* leaf_k;      /* [Hkv, M,   d]  may be NULL in the two-phase mode */
  const void* leaf_v;      /* [Hkv, M,   d]  may be NULL in the two-phase mode */
  const int64_t* root_off; /* [M_R + 1]  children of root j: mids root_off[j] .. root_off[j+1]-1 */
  const int64_t* mid_off;  /* [M_I + 1]  children of mid m: leaves mid_off[m] .. mid_off[m+1]-1 */
  const void* seq_k;       /* [B, S_kv, Hkv, d] */
  const void* seq_v;       /* [B, S_kv, Hkv, d] */
  int32_t K[3];            /* Top-K per level: root, mid, leaf */
  double scale;            /* logit scale, normally 1/sqrt(d) */
  int32_t q_kg_f64;        /* nonzero: q_kg holds fp64 values (an exact KG query, e.g. a sum
                              or a product of stored values, not rounded to dtype) */
} oracle_problem;

/* Per-row outputs; any pointer may be NULL.  Row i of a call fills entry i. */
typedef struct {
  int64_t* sel_R;     /* [rows, K_R]  selected roots, rank order, -1 padded */
  int64_t* sel_I;     /* [rows, K_I]  selected mids */
  int64_t* sel_L;     /* [rows, K_L]  selected leaves */
  double* logit_L;    /* [rows, K_L]  scaled logits of the selected leaves (NaN pad) */
  double* gap;        /* [rows, 3]    relative gap between the K-th and (K+1)-th score per level (+inf if none) */
  int64_t* n_cand;    /* [rows, 3]    candidates scored per level */
  double* lse_kg;     /* [rows]  log-sum-exp of the selected leaf logits (-inf if empty) */
  double* lse_seq;    /* [rows]  log-sum-exp of the visible sequence logits (-inf if empty) */
  double* lam_kg;     /* [rows] */
  double* lam_seq;    /* [rows] */
  double* o_kg;       /* [rows, d]  Softmax(logits_kg) . v  (zeros if empty) */
  double* o_seq;      /* [rows, d]  Softmax(logits_seq) . v (zeros if empty) */
  double* out;        /* [rows, d]  joint-softmax output */
} oracle_outputs;

/* Level sizes from the clustering section, in exact integer arithmetic
 * (the bracket in M_I read as ceil).  out = {S, M_I, M_R}.  Returns 0, or -1
 * for M < 1 or M > 2^62. */
int oracle_tree_sizes(int64_t M, int64_t out[3]);

/* Sort n (score, index) pairs by score descending, index ascending and write
 * the first min(K, n) positions (into the input arrays) to out_pos.  Returns
 * the count written. */
int64_t oracle_topk(int64_t n, const double* score, const int64_t* index,
                    int64_t K, int64_t* out_pos);

/* Candidates of one row at one level and their fp64 scaled scores.
 * level 0: all roots (parents ignored); level 1: children of the given roots;
 * level 2: children of the given mids (needs leaf_k).  Returns the candidate
 * count, or -1 if it would exceed cap. */
int64_t oracle_level_scores(const oracle_problem* P, int64_t b, int64_t n,
                            int64_t h, int level, const int64_t* parents,
                            int64_t n_parents, int64_t* cand, double* score,
                            int64_t cap);

/* Scores of nc candidate keys given explicitly ([nc, d] in P->dtype), for
 * row (b, n, h): score[i] = scale * <q_kg, cand_k[i]>, the same sequential
 * fp64 dot product as oracle_level_scores (used where the leaf array is not
 * on the host, e.g. to rank a row's leaf candidates under given parents).
 * Returns 0, or -1 for a bad argument. */
int oracle_candidate_scores(const oracle_problem* P, int64_t b, int64_t n,
                            int64_t h, int64_t nc, const void* cand_k,
                            double* score);

/* Full forward for rows (b[i], n[i], h[i]).  Returns 0, or a negative code:
 * -1 bad argument, -2 both the KG set and the sequence part empty for a row,
 * -3 out of memory. */
int oracle_hikvp_rows(const oracle_problem* P, int64_t rows, const int64_t* b,
                      const int64_t* n, const int64_t* h, const oracle_outputs* O);

/* Two-phase mode, phase 1: root and mid selection only (leaf arrays unused). */
int oracle_select_mids_rows(const oracle_problem* P, int64_t rows,
                            const int64_t* b, const int64_t* n, const int64_t* h,
                            const oracle_outputs* O);

/* Two-phase mode, phase 2 (and replay mode).  For row i the caller passes its
 * leaf candidates explicitly: cand_off[i] .. cand_off[i+1]-1 index into
 * cand_idx (global leaf indices), cand_k and cand_v ([*, d] in P->dtype).
 * If forced_sel_L is non-NULL ([rows, K_L], -1 padded, global indices) the
 * leaf selection is taken from it instead of being computed (replay mode);
 * every forced index must be one of the row's candidates. */
int oracle_finish_rows(const oracle_problem* P, int64_t rows, const int64_t* b,
                       const int64_t* n, const int64_t* h,
                       const int64_t* cand_off, const int64_t* cand_idx,
                       const void* cand_k, const void* cand_v,
                       const int64_t* forced_sel_L, const oracle_outputs* O);

/* Unpruned equivalent attention for the given rows: the KG half is the
 * softmax over the logits of all M leaves of the row's KV head, merged with
 * the causal sequence half exactly as above.  Fills lse_kg, lse_seq, lam_kg,
 * lam_seq, o_kg, o_seq and out; selection outputs are left untouched. */
int oracle_flat_rows(const oracle_problem* P, int64_t rows, const int64_t* b,
                     const int64_t* n, const int64_t* h, const oracle_outputs* O);

#ifdef __cplusplus
}
#endif
#endif
