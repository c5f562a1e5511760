// hikvp_select.hip -- the tree-descent kernels of HiKVP attention on gfx950.
//
// Page: "AtlasKV: Augmenting LLMs with Billion-Scale Knowledge Graphs in 20GB
// VRAM" (digest of arXiv 2510.17934), 速读 › 怎么做的: score the query against
// the root keys and keep the Top-K branches, score the children of those
// branches and keep the Top-K, and so on down to the leaves; the selected
// leaves' softmax then forms the KG half of the merged output.
//
//   k_root      one wave per row: scores of all M_R root keys of the row's KV
//               head (coalesced 16-byte lanes), exact-boundary Top-K_R.  The
//               per-row select kernels keep a few KB of LDS per wave so many
//               rows are in flight per CU.
//   k_mid_gemm  one workgroup per (root j, KV head g): every row of head g that
//               selected root j is gathered (in row order) and scored against
//               j's child span with bf16 (or fp32) MFMA 16x16 tiles; the span
//               is read once per bucket instead of once per row.  Scores land
//               in each row's candidate slots of the workspace.
//   k_mid_select   one wave per row (a workgroup per row for long candidate
//               lists): Top-K_I over the row's mid scores.
//   k_bucket_clear / k_bucket_link  link the rows that selected each distinct
//               (KV head, mid) into one list per bucket.
//   k_leaf_score   one wave per bucket: streams the mid's leaf span once (it is
//               contiguous in the head-major layout) and writes the scores of
//               every member row into that row's candidate slots.
//   k_leaf_select  one wave (or workgroup) per row: Top-K_L, then the KG softmax over the
//               selected leaves and the weighted sum of their values.
#include <hip/hip_runtime.h>

#include "hikvp_device.h"

namespace hikvp {
namespace {

__device__ inline void decode_row(const RowsDev& r, int row, int& b, int& n, int& h) {
  h = row % r.Hq;
  const int bn = row / r.Hq;
  n = bn % r.N;
  b = bn / r.N;
}

__device__ inline const char* key_base(const TreeDev& t, int lev, int g, int64_t& rsb, int eb) {
  rsb = t.rs[lev] * eb;
  return (const char*)t.key[lev] + (int64_t)g * t.hs[lev] * eb;
}

// ---------------------------------------------------------------------------
// per-row select kernels: one wave per row, LDS work area carved per wave
// ---------------------------------------------------------------------------
constexpr int kStageMax = 0;     // mid/leaf scores are not staged in LDS (registers instead)
constexpr int kRegScores = 32;   // candidate scores held per thread in the select kernels

struct RowWork {
  SelWork sel;
  int* out_node;                 // [K]
  float* out_logit;              // [K]
  int* pre;                      // [Kp + 1]
  int64_t* base;                 // [Kp]
  float* stage;                  // [stage] staged scores (or unused)
};

__host__ __device__ inline size_t rowwork_bytes(int K, int Kp, int D, int stage, int NT = 64) {
  return selwork_bytes(NT, K, D) + 2 * align16((size_t)K * 4) + align16((size_t)(Kp + 1) * 4) +
         align16((size_t)Kp * 8) + align16((size_t)stage * 4);
}

__device__ inline RowWork carve_rowwork(char* p, int K, int Kp, int D, int stage, int NT = 64) {
  RowWork w;
  w.sel = carve_selwork(p, NT, K, D);
  auto take = [&](size_t bytes) { char* q = p; p += align16(bytes); return q; };
  w.out_node = (int*)take((size_t)K * 4);
  w.out_logit = (float*)take((size_t)K * 4);
  w.pre = (int*)take((size_t)(Kp + 1) * 4);
  w.base = (int64_t*)take((size_t)Kp * 8);
  w.stage = (float*)take((size_t)stage * 4);
  return w;
}

// The row's KG query (exact fp32 copy in LDS) and its 2-norm (rounded up).
template <class E, int D>
__device__ inline double load_query(const RowsDev& r, int b, int n, int h, float* qrow, int lane) {
  const char* qp = (const char*)r.q_kg + q_off(r.qks, b, n, h) * E::kBytes;
  float qq = 0.f;
  for (int t = lane; t < D; t += 64) {
    const float v = load_f32<E>(qp, t);
    qrow[t] = v;
    qq = fmaf(v, v, qq);
  }
  qq = wave_sum(qq);
  return sqrt((double)qq) * 1.0001;
}

template <class E, int D>
__global__ __launch_bounds__(256) void k_root(StepArgs a, size_t wave_bytes, int stage) {
  constexpr int EPV = E::kEPV, LPK = D / EPV;
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int blk = blockIdx.x * nwave + wave;
  if (blk >= a.r.R) return;  // whole wave; waves never meet at a barrier
  const int MR = (int)a.t.count[0];
  const int K = a.K[0];
  RowWork W = carve_rowwork(smem + (size_t)wave * wave_bytes, K, 0, D, stage);
  float* sc = stage ? W.stage : a.mid_scores + (int64_t)blk * a.c1max;  // spill: reuse the mid buffer

  const int row = row_of_block(a.r, blk);
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  const int g = h / a.r.G;
  const double qnorm = load_query<E, D>(a.r, b, n, h, W.sel.qrow, lane);
  wave_sync();
  float qf[EPV];
#pragma unroll
  for (int t = 0; t < EPV; ++t) qf[t] = W.sel.qrow[(lane % LPK) * EPV + t];

  int64_t rsb;
  const char* kb = key_base(a.t, 0, g, rsb, E::kBytes);
  const SlotMap ident{nullptr, nullptr, -1};
  score_run<E, D, 4>(qf, kb, rsb, ident, MR, sc, 0, 1, lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  wave_sync();
  const int k = select_topk<E, D, 64>(MemScores<64>{sc}, MR, K, twice_err_bound<D>(qnorm, a.t.norm[g]),
                                      a.r.scale, ident, KeyRows{kb, rsb}, W.sel, W.out_node, W.out_logit,
                                      lane);
  int32_t* out = a.sel[0] + (int64_t)row * K;
  for (int i = lane; i < K; i += 64) out[i] = i < k ? W.out_node[i] : -1;
}

// ---------------------------------------------------------------------------
// mid level: bucket GEMM on MFMA
// ---------------------------------------------------------------------------
constexpr int kMemCap = 512;  // bucket members staged per GEMM round

struct MidSmem {
  int mem_row[kMemCap];
  int mem_base[kMemCap];
  int wave_cnt[4];
};

template <class E, int D>
__device__ void mid_bucket_tiles(const StepArgs& a, const MidSmem& M, int cnt, int g,
                                 int64_t first, int F, int wave, int nwave, int lane) {
  constexpr int KCH = D * E::kBytes / 64;  // 16-byte pieces per lane per row
  const int quad = lane >> 4, col = lane & 15;
  int64_t rsb;
  const char* kb = key_base(a.t, 1, g, rsb, E::kBytes);
  const int n_mt = (cnt + 15) >> 4, n_nt = (F + 15) >> 4;
  for (int mt = wave; mt < n_mt; mt += nwave) {
    uint4 afr[KCH];
    const int ia = mt * 16 + col;
    if (ia < cnt) {
      int b, n, h;
      decode_row(a.r, M.mem_row[ia], b, n, h);
      const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes;
#pragma unroll
      for (int m = 0; m < KCH; ++m) afr[m] = *(const uint4*)(qp + m * 64 + quad * 16);
    } else {
#pragma unroll
      for (int m = 0; m < KCH; ++m) afr[m] = make_uint4(0, 0, 0, 0);
    }
    for (int nt = 0; nt < n_nt; ++nt) {
      uint4 bfr[KCH];
      const int cb = nt * 16 + col;
      if (cb < F) {
        const char* kp = kb + (first + cb) * rsb;
#pragma unroll
        for (int m = 0; m < KCH; ++m) bfr[m] = *(const uint4*)(kp + m * 64 + quad * 16);
      } else {
#pragma unroll
        for (int m = 0; m < KCH; ++m) bfr[m] = make_uint4(0, 0, 0, 0);
      }
      const float4_t acc = tile_dot<E, KCH>(afr, bfr);
      // lane holds tile rows 4*quad .. 4*quad+3 of column col
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = mt * 16 + quad * 4 + v;
        if (i < cnt && cb < F)
          a.mid_scores[(int64_t)M.mem_row[i] * a.c1max + M.mem_base[i] + cb] = acc[v];
      }
    }
  }
}

template <class E, int D>
__global__ __launch_bounds__(256) void k_mid_gemm(StepArgs a) {
  __shared__ MidSmem M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwave = blockDim.x >> 6;
  const int j = blockIdx.x, g = blockIdx.y;
  const int64_t* off0 = a.t.off[0];
  const int64_t first = off0[j];
  const int F = (int)(off0[j + 1] - first);
  const int K0 = a.K[0];
  if (F == 0 || K0 == 0) return;
  const int G = a.r.G;
  const int Rg = a.r.B * a.r.N * G;
  const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int cnt = 0;
  for (int t0 = 0; t0 < Rg; t0 += blockDim.x) {
    const int t = t0 + tid;
    bool member = false;
    int r = 0, base = 0;
    if (t < Rg) {
      r = (t / G) * a.r.Hq + g * G + (t % G);
      const int32_t* sr = a.sel[0] + (int64_t)r * K0;
      int acc = 0;
      for (int k = 0; k < K0; ++k) {
        const int p = sr[k];
        if (p == j) { member = true; base = acc; break; }
        if (p >= 0) acc += (int)(off0[p + 1] - off0[p]);
      }
    }
    // members in row order: wave ballots + per-wave offsets
    const unsigned long long bal = __ballot(member);
    if (lane == 0) M.wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int woff = 0, total = 0;
    for (int w = 0; w < nwave; ++w) {
      if (w < wave) woff += M.wave_cnt[w];
      total += M.wave_cnt[w];
    }
    if (member) {
      const int at = cnt + woff + __popcll(bal & below);
      M.mem_row[at] = r;
      M.mem_base[at] = base;
    }
    cnt += total;
    __syncthreads();
    if (cnt > kMemCap - (int)blockDim.x || t0 + (int)blockDim.x >= Rg) {
      if (cnt > 0) mid_bucket_tiles<E, D>(a, M, cnt, g, first, F, wave, nwave, lane);
      cnt = 0;
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// mid-level Top-K, one wave per row
// ---------------------------------------------------------------------------
// Prologue of the mid/leaf select kernels (NT threads per row): query row
// in LDS, its norm, the candidate list of level `lev` (children of the row's
// level-1 selection).  Returns the candidate count.
template <class E, int D, int NT>
__device__ inline int select_prologue(const StepArgs& a, const RowWork& W, int row, int lev, int& g,
                                      double& qnorm, int gtid) {
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  g = h / a.r.G;
  const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes;
  for (int t = gtid; t < D; t += NT) W.sel.qrow[t] = load_f32<E>(qp, t);
  group_sync<NT>();
  const int Kp = a.K[lev - 1];
  if (gtid < 64) {
    float qq = 0.f;
    for (int t = gtid; t < D; t += 64) qq = fmaf(W.sel.qrow[t], W.sel.qrow[t], qq);
    qq = wave_sum(qq);
    if (gtid == 0) W.sel.ctl[7] = __float_as_int((float)(sqrt((double)qq) * 1.0001));
    build_candidates(a.sel[lev - 1] + (int64_t)row * Kp, Kp, a.t.off[lev - 1], gtid, W.pre, W.base);
  }
  group_sync<NT>();
  qnorm = (double)__int_as_float(W.sel.ctl[7]);
  return W.pre[Kp];
}

// The row's candidate scores: in registers (SPT per thread, loaded once) or,
// for very long candidate lists, read from the workspace in every pass.
template <int NT, int SPT>
struct RowScores {
  using type = RegScores<NT, SPT>;
  __device__ static inline type make(const float* p, int cap, int tid) {
    type r;
    r.load(p, cap, tid);
    return r;
  }
};
template <int NT>
struct RowScores<NT, 0> {
  using type = MemScores<NT>;
  __device__ static inline type make(const float* p, int, int) { return type{p}; }
};

template <class E, int D, int NT, int SPT>
__device__ inline void mid_select_body(const StepArgs& a, size_t group_bytes) {
  extern __shared__ __align__(16) char smem[];
  const int groups = blockDim.x / NT, grp = threadIdx.x / NT, gtid = threadIdx.x % NT;
  const int blk = blockIdx.x * groups + grp;
  if (blk >= a.r.R) return;  // whole group (whole waves) leaves together
  const int K1 = a.K[1];
  RowWork W = carve_rowwork(smem + (size_t)grp * group_bytes, K1, a.K[0], D, 0, NT);
  const int row = row_of_block(a.r, blk);
  // the scores do not depend on the candidate list: load them first
  const auto sc = RowScores<NT, SPT>::make(a.mid_scores + (int64_t)row * a.c1max, (int)a.c1max, gtid);
  int g;
  double qnorm;
  const int n1 = select_prologue<E, D, NT>(a, W, row, 1, g, qnorm, gtid);
  int64_t rsb;
  const char* kb = key_base(a.t, 1, g, rsb, E::kBytes);
  const int k1 = select_topk<E, D, NT>(sc, n1, K1,
                                       twice_err_bound<D>(qnorm, a.t.norm[a.t.Hkv + g]), a.r.scale,
                                       SlotMap{W.pre, W.base, a.K[0]}, KeyRows{kb, rsb}, W.sel,
                                       W.out_node, W.out_logit, gtid);
  if (gtid >= 64) return;
  const int lane = gtid;
  int32_t* o1 = a.sel[1] + (int64_t)row * K1;
  int32_t* ob = a.mid_base + (int64_t)row * K1;
  const int64_t* off1 = a.t.off[1];
  int carry = 0;
  for (int i0 = 0; i0 < K1; i0 += 64) {
    const int i = i0 + lane;
    const int node = i < k1 ? W.out_node[i] : -1;
    const int fan = node >= 0 ? (int)(off1[node + 1] - off1[node]) : 0;
    int incl = fan;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (i < K1) {
      o1[i] = node;
      ob[i] = carry + incl - fan;  // first leaf-candidate slot of this mid in the row's list
    }
    carry += __shfl(incl, 63);
  }
}

// one wave per row (candidate lists up to a few thousand) or one workgroup per row
template <class E, int D>
__global__ __launch_bounds__(256) void k_mid_select(StepArgs a, size_t gb) {
  mid_select_body<E, D, 64, 0>(a, gb);
}
template <class E, int D>
__global__ __launch_bounds__(256) void k_mid_select_wide(StepArgs a, size_t gb) {
  mid_select_body<E, D, 256, 0>(a, gb);
}
template <class E, int D>
__global__ __launch_bounds__(256) void k_mid_select_mem(StepArgs a, size_t gb) {
  mid_select_body<E, D, 256, 0>(a, gb);
}

// ---------------------------------------------------------------------------
// leaf scoring, deduplicated: every distinct (KV head, mid) selected by any
// row is one bucket.  The link kernel writes one 16-byte descriptor per bucket
// (key, fanout, element offset of the span) and stores the first
// kBucketSlots member rows as (row, first leaf slot) pairs; later members go
// to a linked list scored by k_leaf_score_overflow.  One wave per bucket
// streams the mid's leaf span (contiguous in the head-major layout) once and
// scores it for every member row, prefetching its next bucket's descriptor.
// Each member's dot products are computed independently, so results do not
// depend on the (atomic) member or bucket order.
// ---------------------------------------------------------------------------
__global__ void k_bucket_clear(StepArgs a, int64_t nkeys) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nkeys;
       i += (int64_t)gridDim.x * blockDim.x) {
    a.bucket_cnt[i] = 0;
    a.bucket_head[i] = -1;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.bucket_count = 0;
}

__global__ void k_bucket_link(StepArgs a) {
  const int K1 = a.K[1];
  const int64_t n = (int64_t)a.r.R * K1;
  const int MI = (int)a.t.count[1];
  const int64_t* off1 = a.t.off[1];
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int mid = a.sel[1][e];
    if (mid < 0) continue;
    const int row = (int)(e / K1);
    const int g = (row % a.r.Hq) / a.r.G;
    const int64_t key = (int64_t)g * MI + mid;
    const int rank = atomicAdd(&a.bucket_cnt[key], 1);
    if (rank == 0) {
      const int64_t f0 = off1[mid];
      const int64_t first = (int64_t)g * a.t.hs[2] + f0 * a.t.rs[2];
      const int v = atomicAdd(a.bucket_count, 1);
      a.bucket_desc[v] = make_int4((int)key, (int)(off1[mid + 1] - f0), (int)(uint32_t)first,
                                   (int)(first >> 32));
    }
    if (rank < kBucketSlots) {
      a.bucket_slot[key * kBucketSlots + rank] = make_int2(row, a.mid_base[e]);
    } else {
      a.bucket_next[e] = atomicExch(&a.bucket_head[key], (int)e);
    }
  }
}

template <class E, int D, int MB>
__device__ inline void score_members(const StepArgs& a, const char* kb, int F, int m, const int* rows,
                                     const int* bases, const float (*qf)[E::kEPV], int lane) {
  constexpr int EPV = E::kEPV, LPK = D / EPV, KPW = 64 / LPK, U = 4;
  const int j = lane % LPK, sub = lane / LPK;
  const int64_t rsb = a.t.rs[2] * E::kBytes;
  for (int c0 = 0; c0 < F; c0 += KPW * U) {
    uint4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * KPW + sub;
      kv[u] = c < F ? *(const uint4*)(kb + c * rsb + j * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * KPW + sub;
      float kf[EPV];
      unpack<E>(kv[u], kf);
#pragma unroll
      for (int mm = 0; mm < MB; ++mm) {
        if (mm >= m) break;
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < EPV; ++t) s = fmaf(qf[mm][t], kf[t], s);
#pragma unroll
        for (int o = LPK / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
        if (j == 0 && c < F) a.leaf_scores[(int64_t)rows[mm] * a.c2max + bases[mm] + c] = s;
      }
    }
  }
}

template <class E>
__device__ inline void load_q_chunk(const StepArgs& a, int row, int j, float* qf) {
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes;
  unpack<E>(*(const uint4*)(qp + j * 16), qf);
}

// One wave per bucket: the member rows (up to 16) are the M side and the
// span's keys the N side of 16x16 MFMA tiles, so each 16-key tile costs four
// 16-byte loads per lane, 8 MFMAs and one 64-byte store per member.
template <class E, int D>
__global__ __launch_bounds__(256) void k_leaf_score(StepArgs a) {
  constexpr int KCH = D * E::kBytes / 64;  // 16-byte pieces per lane per row
  constexpr int TU = 2;                    // key tiles in flight per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int quad = lane >> 4, col = lane & 15;
  const int nb = *a.bucket_count;
  const char* kbase = (const char*)a.t.key[2];
  const int64_t rsb = a.t.rs[2] * E::kBytes;
  const int stride = gridDim.x * nwave;
  int v = blockIdx.x * nwave + wave;
  int4 cur = v < nb ? a.bucket_desc[v] : make_int4(0, 0, 0, 0);
  while (v < nb) {
    const int vn = v + stride;
    const int4 nxt = vn < nb ? a.bucket_desc[vn] : make_int4(0, 0, 0, 0);  // prefetch
    const int key = cur.x, F = cur.y;
    const int64_t first = (int64_t)(uint32_t)cur.z | ((int64_t)cur.w << 32);
    const char* kb = kbase + first * E::kBytes;
    int cnt = a.bucket_cnt[key];
    cnt = cnt < kBucketSlots ? cnt : kBucketSlots;
    // tile row `col` = member col: its query pieces (zeros past the members)
    int2 mem = make_int2(-1, 0);
    uint4 afr[KCH];
    if (col < cnt) {
      mem = a.bucket_slot[(int64_t)key * kBucketSlots + col];
      int b, n, h;
      decode_row(a.r, mem.x, b, n, h);
      const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes;
#pragma unroll
      for (int m = 0; m < KCH; ++m) afr[m] = *(const uint4*)(qp + m * 64 + quad * 16);
    } else {
#pragma unroll
      for (int m = 0; m < KCH; ++m) afr[m] = make_uint4(0, 0, 0, 0);
    }
    // the 4 members whose scores this lane stores: tile rows 4*quad .. 4*quad+3
    int srow[4], sbase[4];
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      srow[vv] = __shfl(mem.x, 4 * quad + vv);
      sbase[vv] = __shfl(mem.y, 4 * quad + vv);
    }
    for (int t0 = 0; t0 < F; t0 += 16 * TU) {
      uint4 bfr[TU][KCH];
#pragma unroll
      for (int u = 0; u < TU; ++u) {
        const int c = t0 + u * 16 + col;
#pragma unroll
        for (int m = 0; m < KCH; ++m)
          bfr[u][m] = c < F ? *(const uint4*)(kb + c * rsb + m * 64 + quad * 16) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < TU; ++u) {
        const int c = t0 + u * 16 + col;
        const float4_t acc = tile_dot<E, KCH>(afr, bfr[u]);
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          if (4 * quad + vv < cnt && c < F)
            a.leaf_scores[(int64_t)srow[vv] * a.c2max + sbase[vv] + c] = acc[vv];
        }
      }
    }
    cur = nxt;
    v = vn;
  }
}

// Members of buckets with more than kBucketSlots rows: one wave per bucket
// walks the overflow list, two rows per pass over the span.
template <class E, int D>
__global__ __launch_bounds__(256) void k_leaf_score_overflow(StepArgs a) {
  constexpr int EPV = E::kEPV, LPK = D / EPV, MB = 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int j = lane % LPK;
  const int nb = *a.bucket_count;
  const int K1 = a.K[1];
  const char* kbase = (const char*)a.t.key[2];
  for (int v = blockIdx.x * nwave + wave; v < nb; v += gridDim.x * nwave) {
    const int4 d = a.bucket_desc[v];
    if (a.bucket_cnt[d.x] <= kBucketSlots) continue;
    const int64_t first = (int64_t)(uint32_t)d.z | ((int64_t)d.w << 32);
    const char* kb = kbase + first * E::kBytes;
    int e = a.bucket_head[d.x];
    while (e != -1) {  // wave-uniform walk
      int rows[MB], bases[MB];
      float qf[MB][EPV];
      int m = 0;
#pragma unroll
      for (int mm = 0; mm < MB; ++mm) {
        rows[mm] = -1;
        bases[mm] = 0;
#pragma unroll
        for (int t = 0; t < EPV; ++t) qf[mm][t] = 0.f;
        if (e != -1) {
          rows[mm] = e / K1;
          bases[mm] = a.mid_base[e];
          load_q_chunk<E>(a, rows[mm], j, qf[mm]);
          e = a.bucket_next[e];
          ++m;
        }
      }
      score_members<E, D, MB>(a, kb, d.y, m, rows, bases, qf, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// leaf Top-K and the KG softmax over the selected leaves, one wave per row
// ---------------------------------------------------------------------------
template <class E, int D, int NT, int SPT>
__device__ inline void leaf_select_body(const StepArgs& a, size_t group_bytes) {
  constexpr int DPL = D / 64;
  extern __shared__ __align__(16) char smem[];
  const int groups = blockDim.x / NT, grp = threadIdx.x / NT, gtid = threadIdx.x % NT;
  const int blk = blockIdx.x * groups + grp;
  if (blk >= a.r.R) return;
  const int K2 = a.K[2];
  RowWork W = carve_rowwork(smem + (size_t)grp * group_bytes, K2, a.K[1], D, 0, NT);
  const int row = row_of_block(a.r, blk);
  const auto sc = RowScores<NT, SPT>::make(a.leaf_scores + (int64_t)row * a.c2max, (int)a.c2max, gtid);
  int g;
  double qnorm;
  const int n2 = select_prologue<E, D, NT>(a, W, row, 2, g, qnorm, gtid);
  int64_t rsb;
  const char* kb = key_base(a.t, 2, g, rsb, E::kBytes);
  const int k2 = select_topk<E, D, NT>(sc, n2, K2,
                                       twice_err_bound<D>(qnorm, a.t.norm[2 * a.t.Hkv + g]), a.r.scale,
                                       SlotMap{W.pre, W.base, a.K[1]}, KeyRows{kb, rsb}, W.sel,
                                       W.out_node, W.out_logit, gtid);
  int32_t* o2 = a.sel[2] + (int64_t)row * K2;
  for (int i = gtid; i < K2; i += NT) o2[i] = i < k2 ? W.out_node[i] : -1;
  if (gtid >= 64) return;  // the KG half is formed by the group's first wave
  const int lane = gtid;

  // KG half: softmax over the selected leaves' logits, weighted values
  float* okg = a.o_kg + (int64_t)row * D;
  if (k2 == 0) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) okg[lane * DPL + e] = 0.f;
    if (lane == 0) a.lse_kg[row] = -INFINITY;
    return;
  }
  float mx = -INFINITY;
  for (int i = lane; i < k2; i += 64) mx = fmaxf(mx, W.out_logit[i]);
  mx = wave_max(mx);
  float sum = 0.f;
  for (int i = lane; i < k2; i += 64) {
    const float p = __expf(W.out_logit[i] - mx);
    W.out_logit[i] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  wave_sync();
  const char* vb = (const char*)a.t.leaf_v + (int64_t)g * a.t.hs[3] * E::kBytes;
  const int64_t vrs = a.t.rs[3] * E::kBytes;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  int i = 0;
  for (; i + 8 <= k2; i += 8) {
    float v[8][DPL];
#pragma unroll
    for (int u = 0; u < 8; ++u) load_lane<E, DPL>(vb + (int64_t)W.out_node[i + u] * vrs, lane, v[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = W.out_logit[i + u];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
    }
  }
  for (; i < k2; ++i) {
    float v[DPL];
    load_lane<E, DPL>(vb + (int64_t)W.out_node[i] * vrs, lane, v);
    const float w = W.out_logit[i];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, v[e], acc[e]);
  }
  const float inv = 1.f / sum;
#pragma unroll
  for (int e = 0; e < DPL; ++e) okg[lane * DPL + e] = acc[e] * inv;
  if (lane == 0) a.lse_kg[row] = mx + logf(sum);
}

template <class E, int D>
__global__ __launch_bounds__(256) void k_leaf_select(StepArgs a, size_t gb) {
  leaf_select_body<E, D, 64, 0>(a, gb);
}
template <class E, int D>
__global__ __launch_bounds__(256) void k_leaf_select_wide(StepArgs a, size_t gb) {
  leaf_select_body<E, D, 256, 0>(a, gb);
}
template <class E, int D>
__global__ __launch_bounds__(256) void k_leaf_select_mem(StepArgs a, size_t gb) {
  leaf_select_body<E, D, 256, 0>(a, gb);
}

}  // namespace

#define HIKVP_DISPATCH(dtype, d, KERNEL, ...)                                                        \
  do {                                                                                               \
    if ((dtype) == kDtypeBF16 && (d) == 128) hipLaunchKernelGGL((KERNEL<BF16, 128>), __VA_ARGS__);   \
    else if ((dtype) == kDtypeBF16 && (d) == 64) hipLaunchKernelGGL((KERNEL<BF16, 64>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 128) hipLaunchKernelGGL((KERNEL<F32, 128>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 64) hipLaunchKernelGGL((KERNEL<F32, 64>), __VA_ARGS__);  \
    else return hipErrorInvalidValue;                                                                \
  } while (0)

// Waves per block and per-wave LDS of a per-row select kernel.
static bool row_launch_shape(int K, int Kp, int D, int64_t cands, int& wpb, size_t& wave_bytes,
                             int& stage, bool must_stage = false) {
  stage = (must_stage || cands <= kStageMax) ? (int)cands : 0;
  wave_bytes = rowwork_bytes(K, Kp, D, stage);
  const size_t limit = 64 * 1024;
  wpb = 4;
  while (wpb > 1 && wave_bytes * wpb > limit) --wpb;
  return wave_bytes * wpb <= limit;
}

hipError_t launch_root(const StepArgs& a, hipStream_t s) {
  if (a.r.R <= 0) return hipSuccess;
  int wpb, stage;
  size_t wb;
  // root scores are produced in-kernel: keep them in LDS when they fit
  if (!row_launch_shape(a.K[0], 0, a.t.d, a.t.count[0], wpb, wb, stage, a.t.count[0] <= 2048))
    return hipErrorInvalidValue;
  if (!stage && a.t.count[0] > a.c1max) return hipErrorInvalidValue;  // spill buffer too small
  const unsigned blocks = (unsigned)((a.r.R + wpb - 1) / wpb);
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_root, dim3(blocks), dim3(64 * wpb), wb * wpb, s, a, wb, stage);
  return hipGetLastError();
}

hipError_t launch_mid_gemm(const StepArgs& a, hipStream_t s) {
  if (a.r.R <= 0 || a.t.count[0] <= 0 || a.K[0] <= 0) return hipSuccess;
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_mid_gemm, dim3((unsigned)a.t.count[0], (unsigned)a.t.Hkv), dim3(256),
                 0, s, a);
  return hipGetLastError();
}


hipError_t launch_mid_select(const StepArgs& a, hipStream_t s) {
  if (a.r.R <= 0) return hipSuccess;
  if (a.c1max > 64 * kRegScores) {
    const size_t gb = rowwork_bytes(a.K[1], a.K[0], a.t.d, 0, 256);
    if (a.c1max <= 256 * kRegScores)
      HIKVP_DISPATCH(a.t.dtype, a.t.d, k_mid_select_wide, dim3((unsigned)a.r.R), dim3(256), gb, s, a, gb);
    else
      HIKVP_DISPATCH(a.t.dtype, a.t.d, k_mid_select_mem, dim3((unsigned)a.r.R), dim3(256), gb, s, a, gb);
    return hipGetLastError();
  }
  int wpb, stage;
  size_t wb;
  if (!row_launch_shape(a.K[1], a.K[0], a.t.d, 0, wpb, wb, stage)) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((a.r.R + wpb - 1) / wpb);
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_mid_select, dim3(blocks), dim3(64 * wpb), wb * wpb, s, a, wb);
  return hipGetLastError();
}

hipError_t launch_leaf_buckets(const StepArgs& a, hipStream_t s) {
  if (a.r.R <= 0 || a.K[1] <= 0) return hipSuccess;
  const int64_t nkeys = (int64_t)a.t.Hkv * a.t.count[1];
  int64_t blocks = (nkeys + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_bucket_clear, dim3((unsigned)blocks), dim3(256), 0, s, a, nkeys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)a.r.R * a.K[1];
  blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_bucket_link, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_leaf_score(const StepArgs& a, hipStream_t s) {
  if (a.r.R <= 0 || a.K[1] <= 0) return hipSuccess;
  // at most R * K_I distinct (head, mid) buckets
  const int64_t nb_max = (int64_t)a.r.R * a.K[1];
  int64_t blocks = (nb_max + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_leaf_score, dim3((unsigned)blocks), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  blocks = (nb_max + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_leaf_score_overflow, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_leaf_select(const StepArgs& a, hipStream_t s) {
  if (a.r.R <= 0) return hipSuccess;
  if (a.c2max > 64 * kRegScores) {
    const size_t gb = rowwork_bytes(a.K[2], a.K[1], a.t.d, 0, 256);
    if (a.c2max <= 256 * kRegScores)
      HIKVP_DISPATCH(a.t.dtype, a.t.d, k_leaf_select_wide, dim3((unsigned)a.r.R), dim3(256), gb, s, a, gb);
    else
      HIKVP_DISPATCH(a.t.dtype, a.t.d, k_leaf_select_mem, dim3((unsigned)a.r.R), dim3(256), gb, s, a, gb);
    return hipGetLastError();
  }
  int wpb, stage;
  size_t wb;
  if (!row_launch_shape(a.K[2], a.K[1], a.t.d, 0, wpb, wb, stage)) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((a.r.R + wpb - 1) / wpb);
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_leaf_select, dim3(blocks), dim3(64 * wpb), wb * wpb, s, a, wb);
  return hipGetLastError();
}

}  // namespace hikvp
