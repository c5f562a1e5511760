/*
 * hikvp_oracle.c -- plain, slow, single-threaded fp64 reference for HiKVP
 * knowledge-injected attention.  TEST INFRASTRUCTURE ONLY (see the header):
 * nothing in the GPU library links, includes or calls this file.
 *
 * Every floating value is read from its storage type exactly into a double;
 * every sum is a left-to-right fp64 loop; every sort is qsort on
 * (score descending, index ascending).  No blocking, fusion or reordering.
 *
 * Page: "AtlasKV: Augmenting LLMs with Billion-Scale Knowledge Graphs in 20GB
 * VRAM" (digest of arXiv 2510.17934).  Section names below are the page's.
 */
#include "hikvp_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- storage access ---------------------------------------------------- */

static double load(const void* base, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
  if (dtype == ORACLE_BF16) {
    /* a bfloat16 is the high half of a float32 */
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return ((const double*)base)[i];
}

/* <a, b> over d elements, sequential in t, fp64. */
static double dot(const void* a, int64_t a0, const void* b, int64_t b0,
                  int dtype, int64_t d) {
  double acc = 0.0;
  for (int64_t t = 0; t < d; ++t) acc += load(a, dtype, a0 + t) * load(b, dtype, b0 + t);
  return acc;
}

/* The same with the two operands in their own storage types (an fp64 query
 * against keys of the problem's storage type). */
static double dot2(const void* a, int adt, int64_t a0, const void* b, int bdt, int64_t b0,
                   int64_t d) {
  double acc = 0.0;
  for (int64_t t = 0; t < d; ++t) acc += load(a, adt, a0 + t) * load(b, bdt, b0 + t);
  return acc;
}

/* ---- level sizes (方法细节 › KGKVs的层次化聚类) --------------------------- */

typedef unsigned __int128 u128;

/* smallest x >= 0 with x^3 >= v */
static int64_t icbrt_ceil(u128 v) {
  int64_t lo = 0, hi = (int64_t)1 << 42;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    u128 c = (u128)mid * (u128)mid * (u128)mid;
    if (c >= v) hi = mid; else lo = mid + 1;
  }
  return lo;
}

int oracle_tree_sizes(int64_t M, int64_t out[3]) {
  if (M < 1 || M > ((int64_t)1 << 62)) return -1;
  /* S = ceil(cbrt(M)) */
  int64_t S = icbrt_ceil((u128)M);
  /* M_I = ceil(M^(2/3)) = smallest m with m^3 >= M^2 */
  int64_t MI = icbrt_ceil((u128)M * (u128)M);
  /* M_R = ceil(M_I * M^(-1/3)) = smallest r with r^3 * M >= M_I^3 */
  u128 target = (u128)MI * (u128)MI * (u128)MI;
  int64_t lo = 0, hi = MI;
  while (lo < hi) {
    int64_t r = lo + (hi - lo) / 2;
    if ((u128)r * (u128)r * (u128)r * (u128)M >= target) hi = r; else lo = r + 1;
  }
  out[0] = S;
  out[1] = MI;
  out[2] = lo;
  return 0;
}

/* ---- Top-K by (score desc, index asc) ------------------------------------ */

typedef struct { double s; int64_t idx; int64_t pos; } ranked;

static int cmp_ranked(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  if (a->idx < b->idx) return -1;
  if (a->idx > b->idx) return 1;
  return 0;
}

int64_t oracle_topk(int64_t n, const double* score, const int64_t* index,
                    int64_t K, int64_t* out_pos) {
  if (n <= 0 || K <= 0) return 0;
  ranked* r = (ranked*)malloc((size_t)n * sizeof(ranked));
  if (!r) return -1;
  for (int64_t i = 0; i < n; ++i) { r[i].s = score[i]; r[i].idx = index[i]; r[i].pos = i; }
  qsort(r, (size_t)n, sizeof(ranked), cmp_ranked);
  int64_t k = K < n ? K : n;
  for (int64_t i = 0; i < k; ++i) out_pos[i] = r[i].pos;
  free(r);
  return k;
}

/* relative gap between the K-th and (K+1)-th of the sorted scores; +inf if
 * there is no boundary (K == 0 or fewer than K+1 candidates) */
static double boundary_gap(int64_t n, const double* score, const int64_t* index, int64_t K) {
  if (K <= 0 || n <= K) return INFINITY;
  ranked* r = (ranked*)malloc((size_t)n * sizeof(ranked));
  if (!r) return NAN;
  for (int64_t i = 0; i < n; ++i) { r[i].s = score[i]; r[i].idx = index[i]; r[i].pos = i; }
  qsort(r, (size_t)n, sizeof(ranked), cmp_ranked);
  double a = r[K - 1].s, b = r[K].s;
  free(r);
  double den = fmax(fabs(a), fabs(b));
  if (den == 0.0) return 0.0;
  return fabs(a - b) / den;
}

/* ---- one level of the descent (速读 › 怎么做的) --------------------------- */

static int64_t q_base(const oracle_problem* P, int64_t b, int64_t n, int64_t h) {
  return ((b * P->N + n) * P->Hq + h) * P->d;
}

static const void* kg_query(const oracle_problem* P) { return P->q_kg ? P->q_kg : P->q; }

/* storage type of the KG query: fp64 when q_kg is given as an exact query */
static int kg_dtype(const oracle_problem* P) { return (P->q_kg && P->q_kg_f64) ? ORACLE_F64 : P->dtype; }

/* scale * <KG query of the row at qb, key row at kb of `keys`> */
static double kg_score(const oracle_problem* P, int64_t qb, const void* keys, int64_t kb) {
  return P->scale * dot2(kg_query(P), kg_dtype(P), qb, keys, P->dtype, kb, P->d);
}

int64_t oracle_level_scores(const oracle_problem* P, int64_t b, int64_t n,
                            int64_t h, int level, const int64_t* parents,
                            int64_t n_parents, int64_t* cand, double* score,
                            int64_t cap) {
  const int64_t d = P->d;
  const int64_t g = h / (P->Hq / P->Hkv);
  const int64_t qb = q_base(P, b, n, h);
  int64_t cnt = 0;
  if (level == 0) {
    /* the current query against every root key */
    for (int64_t j = 0; j < P->M_R; ++j) {
      if (cnt >= cap) return -1;
      cand[cnt] = j;
      score[cnt] = kg_score(P, qb, P->root_k, (g * P->M_R + j) * d);
      ++cnt;
    }
    return cnt;
  }
  /* children of the selected parents, in the order the parents were ranked */
  const int64_t* off = level == 1 ? P->root_off : P->mid_off;
  const void* keys = level == 1 ? P->mid_k : P->leaf_k;
  const int64_t level_size = level == 1 ? P->M_I : P->M;
  for (int64_t p = 0; p < n_parents; ++p) {
    int64_t par = parents[p];
    if (par < 0) continue;
    for (int64_t c = off[par]; c < off[par + 1]; ++c) {
      if (cnt >= cap) return -1;
      cand[cnt] = c;
      score[cnt] = kg_score(P, qb, keys, (g * level_size + c) * d);
      ++cnt;
    }
  }
  return cnt;
}

int oracle_candidate_scores(const oracle_problem* P, int64_t b, int64_t n,
                            int64_t h, int64_t nc, const void* cand_k,
                            double* score) {
  if (!P || nc < 0 || (nc > 0 && (!cand_k || !score))) return -1;
  const int64_t d = P->d;
  const int64_t qb = q_base(P, b, n, h);
  for (int64_t i = 0; i < nc; ++i)
    score[i] = kg_score(P, qb, cand_k, i * d);
  return 0;
}

/* ---- the per-row pieces --------------------------------------------------- */

static int64_t max_children(const int64_t* off, int64_t count) {
  int64_t m = 0;
  for (int64_t i = 0; i < count; ++i)
    if (off[i + 1] - off[i] > m) m = off[i + 1] - off[i];
  return m;
}

/* select K of n scored candidates into sel (rank order, -1 pad to K) */
static int select_level(int64_t n, const int64_t* cand, const double* score, int64_t K,
                        int64_t* pos_scratch, int64_t* sel, double* gap) {
  int64_t k = oracle_topk(n, score, cand, K, pos_scratch);
  if (k < 0) return -3;
  for (int64_t i = 0; i < K; ++i) sel[i] = i < k ? cand[pos_scratch[i]] : -1;
  if (gap) *gap = boundary_gap(n, score, cand, K);
  return 0;
}

/* log-sum-exp of n values (-inf if n == 0) */
static double lse(int64_t n, const double* x) {
  if (n == 0) return -INFINITY;
  double m = -INFINITY;
  for (int64_t i = 0; i < n; ++i) if (x[i] > m) m = x[i];
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += exp(x[i] - m);
  return m + log(s);
}

/*
 * KG half, sequence half and merge for one row.
 *   KG half (速读 › 怎么做的, merge formula): softmax over the selected leaf
 *   logits, weighted sum of their values.
 *   Sequence half (自注意力层机制): causal softmax over positions
 *   0 .. S_kv - N + n with logits scale*<q, k_i>.
 *   Merge: λ_kg = e^{a-Z}, λ_seq = e^{c-Z}, Z = log(e^a + e^c); the output is
 *   the single softmax over both logit sets (KBLaM中的矩形注意力 form).
 */
static int finish_row(const oracle_problem* P, int64_t b, int64_t n, int64_t h,
                      int64_t nsel, const double* logits, const void* const* vrows,
                      const int64_t* voff, int64_t i_out, const oracle_outputs* O) {
  const int64_t d = P->d;
  const int64_t g = h / (P->Hq / P->Hkv);
  const int64_t qb = q_base(P, b, n, h);
  int64_t npos = P->S_kv > 0 ? P->S_kv - P->N + n + 1 : 0;
  if (npos < 0) npos = 0;
  if (nsel == 0 && npos == 0) return -2;

  double* sig = (double*)malloc((size_t)(npos > 0 ? npos : 1) * sizeof(double));
  double* okg = (double*)calloc((size_t)d, sizeof(double));
  double* oseq = (double*)calloc((size_t)d, sizeof(double));
  double* out = (double*)calloc((size_t)d, sizeof(double));
  if (!sig || !okg || !oseq || !out) { free(sig); free(okg); free(oseq); free(out); return -3; }

  for (int64_t i = 0; i < npos; ++i) {
    int64_t kb = ((b * P->S_kv + i) * P->Hkv + g) * d;
    sig[i] = P->scale * dot(P->q, qb, P->seq_k, kb, P->dtype, d);
  }
  double a = lse(nsel, logits);
  double c = lse(npos, sig);
  double Z = (nsel == 0) ? c : (npos == 0) ? a : fmax(a, c) + log(exp(a - fmax(a, c)) + exp(c - fmax(a, c)));

  for (int64_t i = 0; i < nsel; ++i) {
    double wk = exp(logits[i] - a);   /* Softmax(logits_kg)_i */
    double wz = exp(logits[i] - Z);   /* joint softmax weight */
    for (int64_t t = 0; t < d; ++t) {
      double v = load(vrows[i], P->dtype, voff[i] + t);
      okg[t] += wk * v;
      out[t] += wz * v;
    }
  }
  for (int64_t i = 0; i < npos; ++i) {
    int64_t vb = ((b * P->S_kv + i) * P->Hkv + g) * d;
    double ws = exp(sig[i] - c);
    double wz = exp(sig[i] - Z);
    for (int64_t t = 0; t < d; ++t) {
      double v = load(P->seq_v, P->dtype, vb + t);
      oseq[t] += ws * v;
      out[t] += wz * v;
    }
  }
  if (O->lse_kg) O->lse_kg[i_out] = a;
  if (O->lse_seq) O->lse_seq[i_out] = c;
  if (O->lam_kg) O->lam_kg[i_out] = nsel ? exp(a - Z) : 0.0;
  if (O->lam_seq) O->lam_seq[i_out] = npos ? exp(c - Z) : 0.0;
  for (int64_t t = 0; t < d; ++t) {
    if (O->o_kg) O->o_kg[i_out * d + t] = okg[t];
    if (O->o_seq) O->o_seq[i_out * d + t] = oseq[t];
    if (O->out) O->out[i_out * d + t] = out[t];
  }
  free(sig); free(okg); free(oseq); free(out);
  return 0;
}

static int check_problem(const oracle_problem* P, int need_leaves) {
  if (!P || !P->q || !P->root_k || !P->mid_k || !P->root_off || !P->mid_off) return -1;
  if (need_leaves && (!P->leaf_k || !P->leaf_v)) return -1;
  if (P->d <= 0 || P->Hq <= 0 || P->Hkv <= 0 || P->Hq % P->Hkv) return -1;
  if (P->K[0] < 0 || P->K[1] < 0 || P->K[2] < 0) return -1;
  if (P->S_kv > 0 && (P->S_kv < P->N || !P->seq_k || !P->seq_v)) return -1;
  if (!(P->scale > 0.0)) return -1;
  return 0;
}

/* root and mid selection of one row; pos/cand/score are scratch of size cap */
static int select_upper(const oracle_problem* P, int64_t b, int64_t n, int64_t h,
                        int64_t* cand, double* score, int64_t* pos, int64_t cap,
                        int64_t* selR, int64_t* selI, double* gap, int64_t* ncand) {
  int64_t KR = P->K[0], KI = P->K[1];
  int64_t c = oracle_level_scores(P, b, n, h, 0, NULL, 0, cand, score, cap);
  if (c < 0) return -3;
  ncand[0] = c;
  int rc = select_level(c, cand, score, KR, pos, selR, &gap[0]);
  if (rc) return rc;
  c = oracle_level_scores(P, b, n, h, 1, selR, KR, cand, score, cap);
  if (c < 0) return -3;
  ncand[1] = c;
  return select_level(c, cand, score, KI, pos, selI, &gap[1]);
}

static void store_sel(int64_t* dst, const int64_t* src, int64_t K, int64_t row) {
  if (!dst) return;
  for (int64_t i = 0; i < K; ++i) dst[row * K + i] = src[i];
}

int oracle_select_mids_rows(const oracle_problem* P, int64_t rows,
                            const int64_t* b, const int64_t* n, const int64_t* h,
                            const oracle_outputs* O) {
  if (check_problem(P, 0)) return -1;
  int64_t cap = P->M_R;
  int64_t fI = max_children(P->root_off, P->M_R);
  if (P->K[0] * fI > cap) cap = P->K[0] * fI;
  if (cap < 1) cap = 1;
  int64_t KR = P->K[0], KI = P->K[1];
  int64_t* cand = (int64_t*)malloc((size_t)cap * sizeof(int64_t));
  int64_t* pos = (int64_t*)malloc((size_t)cap * sizeof(int64_t));
  double* score = (double*)malloc((size_t)cap * sizeof(double));
  int64_t* selR = (int64_t*)malloc((size_t)(KR + 1) * sizeof(int64_t));
  int64_t* selI = (int64_t*)malloc((size_t)(KI + 1) * sizeof(int64_t));
  int rc = (!cand || !pos || !score || !selR || !selI) ? -3 : 0;
  for (int64_t r = 0; r < rows && !rc; ++r) {
    double gap[3] = {INFINITY, INFINITY, INFINITY};
    int64_t nc[3] = {0, 0, 0};
    rc = select_upper(P, b[r], n[r], h[r], cand, score, pos, cap, selR, selI, gap, nc);
    if (rc) break;
    store_sel(O->sel_R, selR, KR, r);
    store_sel(O->sel_I, selI, KI, r);
    if (O->gap) { O->gap[r * 3] = gap[0]; O->gap[r * 3 + 1] = gap[1]; O->gap[r * 3 + 2] = INFINITY; }
    if (O->n_cand) { O->n_cand[r * 3] = nc[0]; O->n_cand[r * 3 + 1] = nc[1]; O->n_cand[r * 3 + 2] = 0; }
  }
  free(cand); free(pos); free(score); free(selR); free(selI);
  return rc;
}

/* Leaf level + finish for one row given its leaf candidates (global index,
 * key row, value row).  forced: optional K_L selection (replay). */
static int leaf_and_finish(const oracle_problem* P, int64_t b, int64_t n, int64_t h,
                           int64_t nc, const int64_t* cidx, const void* const* krow,
                           const int64_t* koff, const void* const* vrow, const int64_t* voff,
                           const int64_t* forced, int64_t r, const oracle_outputs* O) {
  const int64_t KL = P->K[2];
  const int64_t qb = q_base(P, b, n, h);
  double* score = (double*)malloc((size_t)(nc > 0 ? nc : 1) * sizeof(double));
  int64_t* pos = (int64_t*)malloc((size_t)(nc > 0 ? nc : 1) * sizeof(int64_t));
  int64_t* sel = (int64_t*)malloc((size_t)(KL + 1) * sizeof(int64_t));
  double* lg = (double*)malloc((size_t)(KL + 1) * sizeof(double));
  const void** vsel = (const void**)malloc((size_t)(KL + 1) * sizeof(void*));
  int64_t* vsel_off = (int64_t*)malloc((size_t)(KL + 1) * sizeof(int64_t));
  int rc = (!score || !pos || !sel || !lg || !vsel || !vsel_off) ? -3 : 0;
  int64_t k = 0;
  if (!rc) {
    for (int64_t i = 0; i < nc; ++i)
      score[i] = kg_score(P, qb, krow[i], koff[i]);
    if (O->gap) O->gap[r * 3 + 2] = boundary_gap(nc, score, cidx, KL);
    if (O->n_cand) O->n_cand[r * 3 + 2] = nc;
    if (forced) {
      for (int64_t i = 0; i < KL; ++i) {
        int64_t want = forced[r * KL + i];
        if (want < 0) continue;
        int64_t at = -1;
        for (int64_t j = 0; j < nc; ++j) if (cidx[j] == want) { at = j; break; }
        if (at < 0) { rc = -1; break; }
        pos[k++] = at;
      }
    } else {
      k = oracle_topk(nc, score, cidx, KL, pos);
      if (k < 0) rc = -3;
    }
  }
  if (!rc) {
    for (int64_t i = 0; i < KL; ++i) {
      sel[i] = i < k ? cidx[pos[i]] : -1;
      lg[i] = i < k ? score[pos[i]] : NAN;
      if (i < k) { vsel[i] = vrow[pos[i]]; vsel_off[i] = voff[pos[i]]; }
    }
    store_sel(O->sel_L, sel, KL, r);
    if (O->logit_L) for (int64_t i = 0; i < KL; ++i) O->logit_L[r * KL + i] = lg[i];
    rc = finish_row(P, b, n, h, k, lg, vsel, vsel_off, r, O);
  }
  free(score); free(pos); free(sel); free(lg); free(vsel); free(vsel_off);
  return rc;
}

int oracle_hikvp_rows(const oracle_problem* P, int64_t rows, const int64_t* b,
                      const int64_t* n, const int64_t* h, const oracle_outputs* O) {
  if (check_problem(P, 1)) return -1;
  const int64_t d = P->d;
  const int64_t KR = P->K[0], KI = P->K[1];
  int64_t fI = max_children(P->root_off, P->M_R);
  int64_t fL = max_children(P->mid_off, P->M_I);
  int64_t cap = P->M_R;
  if (KR * fI > cap) cap = KR * fI;
  if (KI * fL > cap) cap = KI * fL;
  if (cap < 1) cap = 1;
  int64_t* cand = (int64_t*)malloc((size_t)cap * sizeof(int64_t));
  int64_t* pos = (int64_t*)malloc((size_t)cap * sizeof(int64_t));
  double* score = (double*)malloc((size_t)cap * sizeof(double));
  int64_t* selR = (int64_t*)malloc((size_t)(KR + 1) * sizeof(int64_t));
  int64_t* selI = (int64_t*)malloc((size_t)(KI + 1) * sizeof(int64_t));
  const void** krow = (const void**)malloc((size_t)cap * sizeof(void*));
  const void** vrow = (const void**)malloc((size_t)cap * sizeof(void*));
  int64_t* koff = (int64_t*)malloc((size_t)cap * sizeof(int64_t));
  int rc = (!cand || !pos || !score || !selR || !selI || !krow || !vrow || !koff) ? -3 : 0;
  for (int64_t r = 0; r < rows && !rc; ++r) {
    double gap[3] = {INFINITY, INFINITY, INFINITY};
    int64_t nc[3] = {0, 0, 0};
    rc = select_upper(P, b[r], n[r], h[r], cand, score, pos, cap, selR, selI, gap, nc);
    if (rc) break;
    store_sel(O->sel_R, selR, KR, r);
    store_sel(O->sel_I, selI, KI, r);
    if (O->gap) { O->gap[r * 3] = gap[0]; O->gap[r * 3 + 1] = gap[1]; }
    if (O->n_cand) { O->n_cand[r * 3] = nc[0]; O->n_cand[r * 3 + 1] = nc[1]; }
    /* leaf candidates: children of the selected mids, in rank order */
    const int64_t g = h[r] / (P->Hq / P->Hkv);
    int64_t c = 0;
    for (int64_t p = 0; p < KI; ++p) {
      if (selI[p] < 0) continue;
      for (int64_t lf = P->mid_off[selI[p]]; lf < P->mid_off[selI[p] + 1]; ++lf) {
        cand[c] = lf;
        krow[c] = P->leaf_k;
        vrow[c] = P->leaf_v;
        koff[c] = (g * P->M + lf) * d;
        ++c;
      }
    }
    rc = leaf_and_finish(P, b[r], n[r], h[r], c, cand, krow, koff, vrow, koff, NULL, r, O);
  }
  free(cand); free(pos); free(score); free(selR); free(selI); free(krow); free(vrow); free(koff);
  return rc;
}

int oracle_finish_rows(const oracle_problem* P, int64_t rows, const int64_t* b,
                       const int64_t* n, const int64_t* h,
                       const int64_t* cand_off, const int64_t* cand_idx,
                       const void* cand_k, const void* cand_v,
                       const int64_t* forced_sel_L, const oracle_outputs* O) {
  if (check_problem(P, 0) || !cand_off || !cand_idx || !cand_k || !cand_v) return -1;
  const int64_t d = P->d;
  int rc = 0;
  for (int64_t r = 0; r < rows && !rc; ++r) {
    int64_t c0 = cand_off[r], nc = cand_off[r + 1] - cand_off[r];
    if (nc < 0) return -1;
    const void** krow = (const void**)malloc((size_t)(nc > 0 ? nc : 1) * sizeof(void*));
    const void** vrow = (const void**)malloc((size_t)(nc > 0 ? nc : 1) * sizeof(void*));
    int64_t* koff = (int64_t*)malloc((size_t)(nc > 0 ? nc : 1) * sizeof(int64_t));
    if (!krow || !vrow || !koff) rc = -3;
    for (int64_t i = 0; i < nc && !rc; ++i) {
      krow[i] = cand_k;
      vrow[i] = cand_v;
      koff[i] = (c0 + i) * d;
    }
    if (!rc)
      rc = leaf_and_finish(P, b[r], n[r], h[r], nc, cand_idx + c0, krow, koff, vrow, koff,
                           forced_sel_L, r, O);
    free(krow); free(vrow); free(koff);
  }
  return rc;
}

/*
 * Unpruned equivalent attention (背景知识与设计原则 › KBLaM中的矩形注意力: one
 * softmax over every knowledge logit and the visible sequence logits;
 * 方法细节 › 等效注意力机制的知识增强 writes the same output as the λ merge of
 * a KG softmax and a sequence softmax, with nothing pruned while fine-tuning).
 * The KG logits of row (b, n, h) are scale * <q_kg, leaf_k[g][m]> for every
 * leaf m < M of KV head g, in index order; roots, mids and K are not used.
 */
int oracle_flat_rows(const oracle_problem* P, int64_t rows, const int64_t* b,
                     const int64_t* n, const int64_t* h, const oracle_outputs* O) {
  if (!P || !P->q || !P->leaf_k || !P->leaf_v || !b || !n || !h) return -1;
  if (P->d <= 0 || P->Hq <= 0 || P->Hkv <= 0 || P->Hq % P->Hkv || P->M < 0) return -1;
  if (P->S_kv > 0 && (P->S_kv < P->N || !P->seq_k || !P->seq_v)) return -1;
  const int64_t d = P->d, M = P->M;
  const size_t cap = (size_t)(M > 0 ? M : 1);
  double* logit = (double*)malloc(cap * sizeof(double));
  const void** vrow = (const void**)malloc(cap * sizeof(void*));
  int64_t* voff = (int64_t*)malloc(cap * sizeof(int64_t));
  int rc = (!logit || !vrow || !voff) ? -3 : 0;
  for (int64_t r = 0; r < rows && !rc; ++r) {
    const int64_t g = h[r] / (P->Hq / P->Hkv);
    const int64_t qb = q_base(P, b[r], n[r], h[r]);
    for (int64_t m = 0; m < M; ++m) {
      voff[m] = (g * M + m) * d;
      vrow[m] = P->leaf_v;
      logit[m] = kg_score(P, qb, P->leaf_k, voff[m]);
    }
    rc = finish_row(P, b[r], n[r], h[r], M, logit, vrow, voff, r, O);
  }
  free(logit); free(vrow); free(voff);
  return rc;
}
