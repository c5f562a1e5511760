// hikvp_kernels.hip -- gfx950 kernels of HiKVP knowledge-injected attention.
//
// Page: "AtlasKV: Augmenting LLMs with Billion-Scale Knowledge Graphs in 20GB
// VRAM" (digest of arXiv 2510.17934).
//   速读 › 怎么做的: per level, score the query against the candidate keys and
//     keep the Top-K branches; the selected leaves' softmax is merged with the
//     sequence softmax through λ_kg / λ_seq.
//   背景知识与设计原则 › 自注意力层机制: causal softmax over positions <= n.
//   方法细节 › 等效注意力机制的知识增强: the λ-weighted pair of softmaxes,
//     read as log-sum-exp shares (one joint softmax).
//
// Kernels (all wave64):
//   k_score_rows  one workgroup per row: scaled-dot scores of the row's
//                 candidates at one level (fp32, unscaled) into the workspace.
//                 A wave reads 64/LPK keys per load with 16-byte lanes, so each
//                 key row is one coalesced segment.
//   k_topk        one wave per row: radix select of the K-th largest fp32
//                 score, then an exact fp64 re-score of every candidate whose
//                 fp32 score lies within a proven error band of that
//                 threshold, so the selected set equals the set ranked by the
//                 fp64 logit with lower-index tie-break.  At the leaf level it
//                 also gathers the selected values and forms the KG softmax
//                 half (o_kg, lse_kg).
//   k_seq_merge   one workgroup per (b, n, KV head): causal flash-style
//                 attention for the group's query heads (K/V read once per
//                 group), then the λ merge with the KG half.
//   k_validate / k_key_norms  tree-view set-up: offset checks and per-level
//                 key-norm bounds used by the error band of k_topk.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "hikvp_internal.h"

namespace hikvp {
namespace {

struct BF16 {
  static constexpr int kBytes = 2;
  static constexpr int kEPV = 8;  // elements per 16-byte vector
};
struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kEPV = 4;
};

template <class E>
__device__ inline void unpack(const uint4& v, float* f);
template <>
__device__ inline void unpack<BF16>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xffff0000u);
}
template <>
__device__ inline void unpack<F32>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

template <class E>
__device__ inline float load_f32(const void* base, int64_t i);
template <>
__device__ inline float load_f32<BF16>(const void* base, int64_t i) {
  return __uint_as_float(((uint32_t)((const uint16_t*)base)[i]) << 16);
}
template <>
__device__ inline float load_f32<F32>(const void* base, int64_t i) {
  return ((const float*)base)[i];
}

// DPL = D/64 consecutive elements owned by one lane (value rows, outputs)
template <class E, int DPL>
__device__ inline void load_lane(const void* row, int lane, float* f) {
  if constexpr (DPL == 2 && E::kBytes == 2) {
    const uint32_t u = ((const uint32_t*)row)[lane];
    f[0] = __uint_as_float(u << 16);
    f[1] = __uint_as_float(u & 0xffff0000u);
  } else if constexpr (DPL == 2 && E::kBytes == 4) {
    const float2 v = ((const float2*)row)[lane];
    f[0] = v.x;
    f[1] = v.y;
  } else {
#pragma unroll
    for (int e = 0; e < DPL; ++e) f[e] = load_f32<E>(row, (int64_t)lane * DPL + e);
  }
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Sync of one wave's LDS traffic (waves of a block run independent rows).
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ inline uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float ord_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ inline void decode_row(const RowsDev& r, int row, int& b, int& n, int& h) {
  h = row % r.Hq;
  const int bn = row / r.Hq;
  n = bn % r.N;
  b = bn / r.N;
}

__device__ inline int64_t q_off(const int64_t* s, int b, int n, int h) {
  return (int64_t)b * s[0] + (int64_t)n * s[1] + (int64_t)h * s[2];
}

// Candidate list of a row at level >= 1: the children of its selected
// parents, concatenated in selection order.  pre[k] = first slot of parent k,
// base[k] = global index of parent k's first child.  Run by one whole wave.
__device__ inline int build_candidates(const int32_t* parents, int Kp, const int64_t* off,
                                       int lane, int* pre, int64_t* base) {
  int carry = 0;
  if (lane == 0) pre[0] = 0;
  for (int k0 = 0; k0 < Kp; k0 += 64) {
    const int k = k0 + lane;
    int fan = 0;
    int64_t first = 0;
    if (k < Kp) {
      const int p = parents[k];
      if (p >= 0) {
        first = off[p];
        fan = (int)(off[p + 1] - first);
      }
      base[k] = first;
    }
    int incl = fan;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (k < Kp) pre[k + 1] = carry + incl;
    carry += __shfl(incl, 63);
  }
  return carry;
}

// Global node index of candidate slot c (0 <= c < pre[Kp]).
__device__ inline int64_t slot_node(const int* pre, const int64_t* base, int Kp, int c) {
  int lo = 0, hi = Kp - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return base[lo] + (c - pre[lo]);
}

// ---------------------------------------------------------------------------
// level scoring, one workgroup per row
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(256) void k_score_rows(LevelArgs a) {
  constexpr int EPV = E::kEPV, LPK = D / EPV, KPW = 64 / LPK;
  __shared__ int s_pre[kMaxK + 1];
  __shared__ int64_t s_base[kMaxK];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  const int g = h / a.r.G;
  const int lev = a.level;
  int ncand;
  if (lev == 0) {
    ncand = (int)a.t.count[0];
  } else {
    if (wave == 0)
      build_candidates(a.parent_sel + (int64_t)row * a.Kp, a.Kp, a.t.off[lev - 1], lane, s_pre, s_base);
    __syncthreads();
    ncand = s_pre[a.Kp];
  }
  const int j = lane % LPK;
  float qf[EPV];
  {
    const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes;
    unpack<E>(*(const uint4*)(qp + j * 16), qf);
  }
  const char* kb = (const char*)a.t.key[lev] + (int64_t)g * a.t.hs[lev] * E::kBytes;
  const int64_t rsb = a.t.rs[lev] * E::kBytes;
  float* out = a.scores + (int64_t)row * a.cmax;
  for (int c0 = wave * KPW; c0 < ncand; c0 += nwave * KPW) {
    const int c = c0 + lane / LPK;
    float s = 0.f;
    if (c < ncand) {
      const int64_t node = lev == 0 ? c : slot_node(s_pre, s_base, a.Kp, c);
      const uint4 kv = *(const uint4*)(kb + node * rsb + j * 16);
      float kf[EPV];
      unpack<E>(kv, kf);
#pragma unroll
      for (int t = 0; t < EPV; ++t) s = fmaf(qf[t], kf[t], s);
    }
#pragma unroll
    for (int o = LPK / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (j == 0 && c < ncand) out[c] = s;
  }
}

// ---------------------------------------------------------------------------
// Top-K with exact boundary, one wave per row
// ---------------------------------------------------------------------------
struct TopkSmem {              // per wave
  int pre[kMaxK + 1];
  int pad;
  int64_t base[kMaxK];
  int hist[256];
  int sel_node[kMaxK];
  float sel_logit[kMaxK];
};

template <class E>
__device__ double exact_dot(const void* q, const void* k, int d) {
  double acc = 0.0;
  for (int t = 0; t < d; ++t) acc += (double)load_f32<E>(q, t) * (double)load_f32<E>(k, t);
  return acc;
}

template <class E, int D>
__global__ __launch_bounds__(256) void k_topk(LevelArgs a) {
  constexpr int DPL = D / 64;
  extern __shared__ __align__(16) char smem_raw[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int row = blockIdx.x * nwave + wave;
  const size_t per_wave = sizeof(TopkSmem) + (a.stage_lds ? (size_t)a.cmax * 4 : 0);
  char* mine = smem_raw + (size_t)wave * ((per_wave + 15) & ~(size_t)15);
  TopkSmem& S = *reinterpret_cast<TopkSmem*>(mine);
  float* lds_scores = reinterpret_cast<float*>(mine + sizeof(TopkSmem));
  if (row >= a.r.R) return;  // whole wave leaves together

  int b, n, h;
  decode_row(a.r, row, b, n, h);
  const int g = h / a.r.G;
  const int lev = a.level;
  int ncand;
  if (lev == 0) {
    ncand = (int)a.t.count[0];
  } else {
    ncand = build_candidates(a.parent_sel + (int64_t)row * a.Kp, a.Kp, a.t.off[lev - 1], lane,
                             S.pre, S.base);
  }
  wave_sync();
  const float* gsc = a.scores + (int64_t)row * a.cmax;
  const float* sc = gsc;
  if (a.stage_lds) {
    for (int i = lane; i < ncand; i += 64) lds_scores[i] = gsc[i];
    wave_sync();
    sc = lds_scores;
  }
  const int K = a.K < ncand ? a.K : ncand;
  const double scale = a.r.scale;
  const char* qk = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes;
  const char* kb = (const char*)a.t.key[lev] + (int64_t)g * a.t.hs[lev] * E::kBytes;
  const int64_t rsb = a.t.rs[lev] * E::kBytes;
  int ksel = 0;

  if (K == ncand) {
    // every candidate is selected
    for (int i = lane; i < ncand; i += 64) {
      S.sel_node[i] = (int)(lev == 0 ? i : slot_node(S.pre, S.base, a.Kp, i));
      S.sel_logit[i] = (float)(scale * (double)sc[i]);
    }
    ksel = ncand;
  } else if (K > 0) {
    // 1) radix select: ordered key of the K-th largest fp32 score
    uint32_t prefix = 0, mask = 0;
    int krem = K;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = lane; i < 256; i += 64) S.hist[i] = 0;
      wave_sync();
      for (int i = lane; i < ncand; i += 64) {
        const uint32_t u = ord_key(sc[i]);
        if ((u & mask) == prefix) atomicAdd(&S.hist[(u >> shift) & 255u], 1);
      }
      wave_sync();
      const int c0 = S.hist[4 * lane], c1 = S.hist[4 * lane + 1];
      const int c2 = S.hist[4 * lane + 2], c3 = S.hist[4 * lane + 3];
      const int tot = c0 + c1 + c2 + c3;
      int suf = tot;  // inclusive suffix sum over lanes (higher lanes hold higher bins)
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_down(suf, o);
        if (lane + o < 64) suf += t;
      }
      const int above = suf - tot;
      const unsigned long long hit = __ballot(above < krem && krem <= suf);
      const int src = __ffsll((long long)hit) - 1;
      int bin = 0, newk = 0;
      if (lane == src) {
        int cum = above;
        const int cnt[4] = {c0, c1, c2, c3};
        for (int q = 3; q >= 0; --q) {
          if (cum + cnt[q] >= krem) { bin = 4 * lane + q; newk = krem - cum; break; }
          cum += cnt[q];
        }
      }
      bin = __shfl(bin, src);
      newk = __shfl(newk, src);
      prefix |= (uint32_t)bin << shift;
      mask |= 0xffu << shift;
      krem = newk;
      wave_sync();
    }
    const double T = (double)ord_float(prefix);

    // 2) error band: |fp32 score - fp64 sum| <= E = d*2^-23*|q|*max|k| (a
    //    bound for any summation order of d products with <= 2 ulp per step)
    float qq = 0.f;
    {
      float qf[DPL];
      load_lane<E, DPL>(qk, lane, qf);
#pragma unroll
      for (int e = 0; e < DPL; ++e) qq = fmaf(qf[e], qf[e], qq);
    }
    qq = wave_sum(qq);
    const double qnorm = sqrt((double)qq) * 1.0001;
    const double knorm = (double)a.t.norm[lev * a.t.Hkv + g];
    const double err = qnorm * knorm * (double)D * (1.0 / 8388608.0) * 1.01;
    const double W = 2.0 * err + 4.0 * fabs(T) * (1.0 / 8388608.0) + 1e-37;

    // 3) classify: sure (above the band) and band members, candidate order
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int nsure = 0, nband = 0;
    int32_t* band_node = a.band_slot + (int64_t)row * a.cmax;
    double* band_s = a.band_s + (int64_t)row * a.cmax;
    for (int i0 = 0; i0 < ncand; i0 += 64) {
      const int i = i0 + lane;
      const bool valid = i < ncand;
      const double f = valid ? (double)sc[i] : 0.0;
      const bool sure = valid && f > T + W;
      const bool band = valid && !sure && f >= T - W;
      const unsigned long long bs = __ballot(sure), bb = __ballot(band);
      if (sure) {
        const int at = nsure + __popcll(bs & below);
        S.sel_node[at] = (int)(lev == 0 ? i : slot_node(S.pre, S.base, a.Kp, i));
        S.sel_logit[at] = (float)(scale * f);
      }
      if (band) {
        const int at = nband + __popcll(bb & below);
        band_node[at] = (int)(lev == 0 ? i : slot_node(S.pre, S.base, a.Kp, i));
      }
      nsure += __popcll(bs);
      nband += __popcll(bb);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
    __builtin_amdgcn_wave_barrier();

    // 4) exact fp64 logits of the band (products exact, summed left to right)
    for (int i = lane; i < nband; i += 64) {
      const int64_t node = band_node[i];
      band_s[i] = scale * exact_dot<E>(qk, kb + node * rsb, D);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
    __builtin_amdgcn_wave_barrier();

    // 5) the top (K - nsure) band members by (logit desc, index asc)
    const int need = K - nsure;
    int taken = 0;
    for (int i0 = 0; i0 < nband; i0 += 64) {
      const int i = i0 + lane;
      bool pick = false;
      double si = 0.0;
      if (i < nband) {
        si = band_s[i];
        const int ni = band_node[i];
        int rank = 0;
        for (int j = 0; j < nband && rank < need; ++j) {
          const double sj = band_s[j];
          rank += (sj > si || (sj == si && band_node[j] < ni)) ? 1 : 0;
        }
        pick = rank < need;
      }
      const unsigned long long bp = __ballot(pick);
      if (pick) {
        const int at = nsure + taken + __popcll(bp & below);
        S.sel_node[at] = band_node[i];
        S.sel_logit[at] = (float)si;
      }
      taken += __popcll(bp);
    }
    ksel = nsure + taken;
  }
  wave_sync();

  int32_t* sel = a.sel + (int64_t)row * a.K;
  for (int i = lane; i < a.K; i += 64) sel[i] = i < ksel ? S.sel_node[i] : -1;

  if (lev == 2) {
    // KG half: softmax over the selected leaves' logits, weighted values
    float* okg = a.o_kg + (int64_t)row * D;
    float acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
    if (ksel == 0) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) okg[lane * DPL + e] = 0.f;
      if (lane == 0) a.lse_kg[row] = -INFINITY;
      return;
    }
    float mx = -INFINITY;
    for (int i = lane; i < ksel; i += 64) mx = fmaxf(mx, S.sel_logit[i]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int i = lane; i < ksel; i += 64) {
      const float p = __expf(S.sel_logit[i] - mx);
      S.sel_logit[i] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    wave_sync();
    const char* vb = (const char*)a.t.leaf_v + (int64_t)g * a.t.hs[3] * E::kBytes;
    const int64_t vrs = a.t.rs[3] * E::kBytes;
#pragma unroll 4
    for (int i = 0; i < ksel; ++i) {
      const float p = S.sel_logit[i];
      float v[DPL];
      load_lane<E, DPL>(vb + (int64_t)S.sel_node[i] * vrs, lane, v);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = fmaf(p, v[e], acc[e]);
    }
    const float inv = 1.f / sum;
#pragma unroll
    for (int e = 0; e < DPL; ++e) okg[lane * DPL + e] = acc[e] * inv;
    if (lane == 0) a.lse_kg[row] = mx + logf(sum);
  }
}

// ---------------------------------------------------------------------------
// causal sequence attention + λ merge, one workgroup per (b, n, KV head)
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(256) void k_seq_merge(SeqArgs a) {
  constexpr int EPV = E::kEPV, LPK = D / EPV, KPW = 64 / LPK, DPL = D / 64, CH = 64;
  __shared__ float s_p[4][CH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int g = blockIdx.x % a.Hkv;
  const int bn = blockIdx.x / a.Hkv;
  const int n = bn % a.r.N, b = bn / a.r.N;
  const int G = a.r.G;
  const int j = lane % LPK;
  const float scale = (float)a.r.scale;
  const int vis = a.k ? a.S - a.r.N + n + 1 : 0;
  const char* kbase = (const char*)a.k + ((int64_t)b * a.ks[0] + (int64_t)g * a.ks[2]) * E::kBytes;
  const char* vbase = (const char*)a.v + ((int64_t)b * a.vs[0] + (int64_t)g * a.vs[2]) * E::kBytes;
  const int64_t kstep = a.ks[1] * E::kBytes, vstep = a.vs[1] * E::kBytes;

  for (int hw = wave; hw < G; hw += nwave) {
    const int h = g * G + hw;
    const int row = (b * a.r.N + n) * a.r.Hq + h;
    float qf[EPV];
    {
      const char* qp = (const char*)a.r.q + q_off(a.r.qs, b, n, h) * E::kBytes;
      unpack<E>(*(const uint4*)(qp + j * 16), qf);
    }
    float acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
    float m = -INFINITY, l = 0.f;
    for (int c0 = 0; c0 < vis; c0 += CH) {
#pragma unroll
      for (int it = 0; it < CH / KPW; ++it) {
        const int i = c0 + it * KPW + lane / LPK;
        float s = 0.f;
        if (i < vis) {
          const uint4 kv = *(const uint4*)(kbase + (int64_t)i * kstep + j * 16);
          float kf[EPV];
          unpack<E>(kv, kf);
#pragma unroll
          for (int t = 0; t < EPV; ++t) s = fmaf(qf[t], kf[t], s);
        }
#pragma unroll
        for (int o = LPK / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
        if (j == 0) s_p[wave][it * KPW + lane / LPK] = (i < vis) ? s * scale : -INFINITY;
      }
      wave_sync();
      const float sv = s_p[wave][lane];
      const float mn = fmaxf(m, wave_max(sv));
      const float alpha = __expf(m - mn);
      const float p = __expf(sv - mn);
      l = l * alpha + wave_sum(p);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] *= alpha;
      m = mn;
      wave_sync();
      s_p[wave][lane] = p;
      wave_sync();
      const int cnt = (vis - c0) < CH ? (vis - c0) : CH;
#pragma unroll 4
      for (int i = 0; i < cnt; ++i) {
        const float pi = s_p[wave][i];
        float v[DPL];
        load_lane<E, DPL>(vbase + (int64_t)(c0 + i) * vstep, lane, v);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(pi, v[e], acc[e]);
      }
      wave_sync();
    }
    const float lse_seq = vis > 0 ? m + logf(l) : -INFINITY;
    const float lkg = a.lse_kg[row];
    float lam;
    if (lkg == -INFINITY) lam = 0.f;
    else if (vis == 0) lam = 1.f;
    else lam = 1.f / (1.f + __expf(lse_seq - lkg));
    const float inv_l = vis > 0 ? 1.f / l : 0.f;
    const float* okg = a.o_kg + (int64_t)row * D;
    const int64_t ob = q_off(a.os, b, n, h);
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float o = lam * okg[lane * DPL + e] + (1.f - lam) * (acc[e] * inv_l);
      const int64_t at = ob + (int64_t)lane * DPL + e;
      if (a.out_dtype == kDtypeBF16) ((uint16_t*)a.out)[at] = f32_to_bf16_rne(o);
      else ((float*)a.out)[at] = o;
    }
    if (a.lse_seq_out && lane == 0) a.lse_seq_out[row] = lse_seq;
  }
}

// ---------------------------------------------------------------------------
// tree-view set-up
// ---------------------------------------------------------------------------
__global__ void k_validate(const int64_t* off, int64_t count, int64_t children, int which,
                           BuildStats* st) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i <= count;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t v = off[i];
    bool bad = v < 0 || v > children;
    if (i == 0 && v != 0) bad = true;
    if (i == count && v != children) bad = true;
    if (i < count) {
      const int64_t w = off[i + 1];
      if (w < v) bad = true;
      else atomicMax(&st->maxfan[which], (unsigned long long)(w - v));
    }
    if (bad) atomicOr(&st->bad, 1 << which);
  }
}

template <class E, int D>
__global__ __launch_bounds__(256) void k_key_norms(const void* key, int64_t rows, int64_t hs,
                                                   int64_t rs, unsigned int* out_bits) {
  constexpr int EPV = E::kEPV, LPK = D / EPV, KPW = 64 / LPK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int g = blockIdx.y;
  const int j = lane % LPK;
  const char* kb = (const char*)key + (int64_t)g * hs * E::kBytes;
  float mx = 0.f;
  for (int64_t r0 = ((int64_t)blockIdx.x * nwave + wave) * KPW; r0 < rows;
       r0 += (int64_t)gridDim.x * nwave * KPW) {
    const int64_t r = r0 + lane / LPK;
    float s = 0.f;
    if (r < rows) {
      const uint4 kv = *(const uint4*)(kb + r * rs * E::kBytes + j * 16);
      float kf[EPV];
      unpack<E>(kv, kf);
#pragma unroll
      for (int t = 0; t < EPV; ++t) s = fmaf(kf[t], kf[t], s);
    }
#pragma unroll
    for (int o = LPK / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (lane == 0) atomicMax(&out_bits[g], __float_as_uint(sqrtf(mx) * 1.0001f));
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define HIKVP_DISPATCH(dtype, d, KERNEL, ...)                                         \
  do {                                                                                \
    if ((dtype) == kDtypeBF16 && (d) == 128) hipLaunchKernelGGL((KERNEL<BF16, 128>), __VA_ARGS__); \
    else if ((dtype) == kDtypeBF16 && (d) == 64) hipLaunchKernelGGL((KERNEL<BF16, 64>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 128) hipLaunchKernelGGL((KERNEL<F32, 128>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 64) hipLaunchKernelGGL((KERNEL<F32, 64>), __VA_ARGS__); \
    else return hipErrorInvalidValue;                                                 \
  } while (0)

hipError_t launch_validate(const int64_t* off, int64_t count, int64_t children, int which,
                           BuildStats* stats, hipStream_t s) {
  int64_t blocks = (count + 1 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_validate, dim3((unsigned)blocks), dim3(256), 0, s, off, count, children,
                     which, stats);
  return hipGetLastError();
}

hipError_t launch_key_norms(const void* key, int dtype, int d, int Hkv, int64_t rows, int64_t hs,
                            int64_t rs, unsigned int* out_bits, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  int64_t blocks = (rows + 63) / 64;
  if (blocks > 2048) blocks = 2048;
  HIKVP_DISPATCH(dtype, d, k_key_norms, dim3((unsigned)blocks, (unsigned)Hkv), dim3(256), 0, s, key,
                 rows, hs, rs, out_bits);
  return hipGetLastError();
}

hipError_t launch_score_rows(const LevelArgs& a, hipStream_t s) {
  if (a.r.R <= 0) return hipSuccess;
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_score_rows, dim3(a.r.R), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk(const LevelArgs& a, hipStream_t s) {
  if (a.r.R <= 0) return hipSuccess;
  LevelArgs b = a;
  size_t per = sizeof(TopkSmem) + (size_t)a.cmax * 4;
  per = (per + 15) & ~(size_t)15;
  int wpb = 4;
  const size_t limit = 64 * 1024;
  if (per * wpb > limit) wpb = (int)(limit / per);
  if (wpb < 1) {
    b.stage_lds = 0;
    per = (sizeof(TopkSmem) + 15) & ~(size_t)15;
    wpb = 4;
  } else {
    b.stage_lds = 1;
  }
  const unsigned blocks = (unsigned)((a.r.R + wpb - 1) / wpb);
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_topk, dim3(blocks), dim3(64 * wpb), per * wpb, s, b);
  return hipGetLastError();
}

hipError_t launch_seq_merge(const SeqArgs& a, hipStream_t s) {
  if (a.r.R <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)(a.r.B * a.r.N * a.Hkv);
  const int waves = a.r.G < 4 ? a.r.G : 4;
  HIKVP_DISPATCH(a.dtype, a.d, k_seq_merge, dim3(blocks), dim3(64 * waves), 0, s, a);
  return hipGetLastError();
}

}  // namespace hikvp
