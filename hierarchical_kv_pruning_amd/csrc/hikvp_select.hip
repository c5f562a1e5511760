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
//   k_mid_select   one wave per row: Top-K_I over the row's mid scores.
//   k_leaf_score   one workgroup per row, small LDS (high occupancy): streams
//               the selected mids' leaf spans (contiguous in the head-major
//               layout) and writes the row's leaf scores.
//   k_leaf_select  one wave per row: Top-K_L, then the KG softmax over the
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
constexpr int kStageMax = 2048;  // candidate scores staged in LDS up to this count

struct RowWork {
  SelWork sel;
  int* out_node;                 // [K]
  float* out_logit;              // [K]
  int* pre;                      // [Kp + 1]
  int64_t* base;                 // [Kp]
  float* stage;                  // [stage] staged scores (or unused)
};

__host__ __device__ inline size_t rowwork_bytes(int K, int Kp, int D, int stage) {
  return selwork_bytes(64, K, D) + 2 * align16((size_t)K * 4) + align16((size_t)(Kp + 1) * 4) +
         align16((size_t)Kp * 8) + align16((size_t)stage * 4);
}

__device__ inline RowWork carve_rowwork(char* p, int K, int Kp, int D, int stage) {
  RowWork w;
  w.sel = carve_selwork(p, 64, K, D);
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
  const int k = select_topk<E, D, 64>(sc, MR, K, twice_err_bound<D>(qnorm, a.t.norm[g]), a.r.scale,
                                      ident, KeyRows{kb, rsb}, W.sel, W.out_node, W.out_logit, lane);
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

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// One 16x16 tile of <q_member, key_child> over the head dim.  Lane l feeds
// tile row/column l%16 with the 16-byte pieces m*64 + (l/16)*16 of its row
// (m < KCH); the same element permutation on both operands leaves the dot
// products unchanged.
template <class E, int KCH>
__device__ inline float4_t tile_dot(const uint4* a, const uint4* b) {
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (E::kBytes == 2) {
#pragma unroll
    for (int m = 0; m < KCH; ++m) {
      short4_t alo, ahi, blo, bhi;
      alo = __builtin_bit_cast(short4_t, make_uint2(a[m].x, a[m].y));
      ahi = __builtin_bit_cast(short4_t, make_uint2(a[m].z, a[m].w));
      blo = __builtin_bit_cast(short4_t, make_uint2(b[m].x, b[m].y));
      bhi = __builtin_bit_cast(short4_t, make_uint2(b[m].z, b[m].w));
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, blo, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, bhi, acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int m = 0; m < KCH; ++m) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[m].x), __uint_as_float(b[m].x), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[m].y), __uint_as_float(b[m].y), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[m].z), __uint_as_float(b[m].z), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[m].w), __uint_as_float(b[m].w), acc, 0, 0, 0);
    }
  }
  return acc;
}

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
// Prologue of the mid/leaf select kernels: query row, candidate list of level
// `lev` (children of the row's level-1 selection), scores staged in LDS when
// they fit.  Returns the candidate count.
template <class E, int D>
__device__ inline int select_prologue(const StepArgs& a, const RowWork& W, int row, int lev,
                                      const float* gscores, int stage, int& g, double& qnorm,
                                      const float*& sc, int lane) {
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  g = h / a.r.G;
  qnorm = load_query<E, D>(a.r, b, n, h, W.sel.qrow, lane);
  const int Kp = a.K[lev - 1];
  const int nc = build_candidates(a.sel[lev - 1] + (int64_t)row * Kp, Kp, a.t.off[lev - 1], lane,
                                  W.pre, W.base);
  sc = gscores;
  if (stage) {
    for (int i = lane; i < nc; i += 64) W.stage[i] = gscores[i];
    sc = W.stage;
  }
  wave_sync();
  return nc;
}

template <class E, int D>
__global__ __launch_bounds__(256) void k_mid_select(StepArgs a, size_t wave_bytes, int stage) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int blk = blockIdx.x * nwave + wave;
  if (blk >= a.r.R) return;
  const int K1 = a.K[1];
  RowWork W = carve_rowwork(smem + (size_t)wave * wave_bytes, K1, a.K[0], D, stage);
  const int row = row_of_block(a.r, blk);
  int g;
  double qnorm;
  const float* sc;
  const int n1 = select_prologue<E, D>(a, W, row, 1, a.mid_scores + (int64_t)row * a.c1max, stage, g,
                                       qnorm, sc, lane);
  int64_t rsb;
  const char* kb = key_base(a.t, 1, g, rsb, E::kBytes);
  const int k1 = select_topk<E, D, 64>(sc, n1, K1, twice_err_bound<D>(qnorm, a.t.norm[a.t.Hkv + g]),
                                       a.r.scale, SlotMap{W.pre, W.base, a.K[0]}, KeyRows{kb, rsb},
                                       W.sel, W.out_node, W.out_logit, lane);
  int32_t* o1 = a.sel[1] + (int64_t)row * K1;
  for (int i = lane; i < K1; i += 64) o1[i] = i < k1 ? W.out_node[i] : -1;
}

// ---------------------------------------------------------------------------
// leaf scoring: stream the selected mids' leaf spans, one workgroup per row
// ---------------------------------------------------------------------------
struct StreamSmem {
  int pre[kMaxK + 1];
  int64_t base[kMaxK];
  float qrow[kMaxD];
};

template <class E, int D>
__global__ __launch_bounds__(256) void k_leaf_score(StepArgs a) {
  constexpr int EPV = E::kEPV, LPK = D / EPV;
  __shared__ StreamSmem L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwave = blockDim.x >> 6;
  const int row = row_of_block(a.r, blockIdx.x);
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  const int g = h / a.r.G;
  const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes;
  for (int t = tid; t < D; t += blockDim.x) L.qrow[t] = load_f32<E>(qp, t);
  const int K1 = a.K[1];
  if (wave == 0) build_candidates(a.sel[1] + (int64_t)row * K1, K1, a.t.off[1], lane, L.pre, L.base);
  __syncthreads();
  const int n2 = L.pre[K1];
  float qf[EPV];
#pragma unroll
  for (int t = 0; t < EPV; ++t) qf[t] = L.qrow[(lane % LPK) * EPV + t];
  int64_t rsb;
  const char* kb = key_base(a.t, 2, g, rsb, E::kBytes);
  score_run<E, D, 8>(qf, kb, rsb, SlotMap{L.pre, L.base, K1}, n2, a.leaf_scores + (int64_t)row * a.c2max,
                     wave, nwave, lane);
}

// ---------------------------------------------------------------------------
// leaf Top-K and the KG softmax over the selected leaves, one wave per row
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(256) void k_leaf_select(StepArgs a, size_t wave_bytes, int stage) {
  constexpr int DPL = D / 64;
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int blk = blockIdx.x * nwave + wave;
  if (blk >= a.r.R) return;
  const int K2 = a.K[2];
  RowWork W = carve_rowwork(smem + (size_t)wave * wave_bytes, K2, a.K[1], D, stage);
  const int row = row_of_block(a.r, blk);
  int g;
  double qnorm;
  const float* sc;
  const int n2 = select_prologue<E, D>(a, W, row, 2, a.leaf_scores + (int64_t)row * a.c2max, stage, g,
                                       qnorm, sc, lane);
  int64_t rsb;
  const char* kb = key_base(a.t, 2, g, rsb, E::kBytes);
  const int k2 = select_topk<E, D, 64>(sc, n2, K2, twice_err_bound<D>(qnorm, a.t.norm[2 * a.t.Hkv + g]),
                                       a.r.scale, SlotMap{W.pre, W.base, a.K[1]}, KeyRows{kb, rsb},
                                       W.sel, W.out_node, W.out_logit, lane);
  int32_t* o2 = a.sel[2] + (int64_t)row * K2;
  for (int i = lane; i < K2; i += 64) o2[i] = i < k2 ? W.out_node[i] : -1;

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
                             int& stage) {
  stage = cands <= kStageMax ? (int)cands : 0;
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
  if (!row_launch_shape(a.K[0], 0, a.t.d, a.t.count[0], wpb, wb, stage)) return hipErrorInvalidValue;
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
  int wpb, stage;
  size_t wb;
  if (!row_launch_shape(a.K[1], a.K[0], a.t.d, a.c1max, wpb, wb, stage)) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((a.r.R + wpb - 1) / wpb);
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_mid_select, dim3(blocks), dim3(64 * wpb), wb * wpb, s, a, wb, stage);
  return hipGetLastError();
}

hipError_t launch_leaf_score(const StepArgs& a, hipStream_t s) {
  if (a.r.R <= 0) return hipSuccess;
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_leaf_score, dim3((unsigned)a.r.R), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_leaf_select(const StepArgs& a, hipStream_t s) {
  if (a.r.R <= 0) return hipSuccess;
  int wpb, stage;
  size_t wb;
  if (!row_launch_shape(a.K[2], a.K[1], a.t.d, a.c2max, wpb, wb, stage)) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((a.r.R + wpb - 1) / wpb);
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_leaf_select, dim3(blocks), dim3(64 * wpb), wb * wpb, s, a, wb, stage);
  return hipGetLastError();
}

}  // namespace hikvp
