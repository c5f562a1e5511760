// hikvp_shared.hip -- shared selections: one descent per group of rows.
//
// The pages pick Top-K branches per query (速读 › 怎么做的) and state a memory
// bound that reads like one selected key set shared by the tokens of a layer
// (速读 › 怎么做的, complexity).  In this variant the rows of one KV head at
// one token (or in one whole sequence) share a selection: the descent runs on
// the group's query, the sum of its members' KG queries, which ranks every
// node by the members' summed logits.  The scores are computed with the sum
// rounded once to the tree's storage type; the selection is exact for the
// unrounded sum (its band is widened by the rounding's bound and re-scored
// with the fp64 sum).  Each member then takes its own softmax over the
// group's selected leaves with its own logits, merged with its own sequence
// half as usual.
#include "hikvp_device.h"
#include "hikvp_round.h"

namespace hikvp {
namespace {

// The group query is the exact sum of the members' stored KG queries.  It is
// formed in fp64 in two passes: one wave per (group, chunk of
// a.tn tokens) sums its tokens' G heads, one workgroup per group sums its
// chunks.  Both are exact whenever the exact sum fits fp64's 53 bits (the
// members' magnitudes spanning less than ~2^40), so the order of the
// additions does not change the result; where it does not fit, the order is
// still fixed, so the result is reproducible.  With one chunk per group (a
// group per token) the first pass writes the group query itself.

// Group row gr's sums (this lane's DPL elements): as they are (gqx, the exact
// query the selection is exact for) and as the query the scores are
// computed with: rounded once to the tree's dtype (gq), in bf16 with the
// rounded residual beside it (glo), and an upper bound of what that leaves
// out (gdelta).  One wave.
template <class E, int D>
__device__ inline void store_group_query(const SharedArgs& a, int64_t gr, const double (&x)[D / 64], int lane) {
  constexpr int DPL = D / 64;
  double dq2 = 0.0;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const int64_t o = gr * D + lane * DPL + e;
    double rest;
    if constexpr (E::kBytes == 2) {
      const Bf16Split sp = split_bf16(x[e]);
      ((uint16_t*)a.gq)[o] = sp.hi;
      ((uint16_t*)a.glo)[o] = sp.lo;
      rest = sp.rest;
    } else {
      const float v = (float)x[e];
      ((float*)a.gq)[o] = v;
      rest = x[e] - (double)v;
    }
    a.gqx[o] = x[e];
    dq2 = fma(rest, rest, dq2);
  }
  dq2 = wave_sum_f64(dq2);
  // rounded up: the fp32 conversion's relative error is below 2^-24
  if (lane == 0) a.gdelta[gr] = (float)(sqrt(dq2) * (1.0 + 1e-6));
}

template <class E, int D>
__global__ __launch_bounds__(256) void k_group_partial(SharedArgs a) {
  constexpr int DPL = D / 64;
  constexpr int U = 8;  // member loads in flight
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int Hkv = a.t.Hkv, G = a.r.G;
  if (w >= a.B * a.Ng * Hkv * a.chunks) return;
  const int c = w % a.chunks, gr = w / a.chunks;
  const int g = gr % Hkv, bn = gr / Hkv;
  const int b = bn / a.Ng;
  const int n0 = a.Ng == 1 ? c * a.tn : bn % a.Ng;
  const int n1 = a.Ng == 1 ? min(a.r.N, n0 + a.tn) : n0 + 1;
  const int cnt = (n1 - n0) * G;  // members (token, head) of this chunk
  double acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0;
  for (int m0 = 0; m0 < cnt; m0 += U) {
    float v[U][DPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int m = min(m0 + u, cnt - 1);
      const int64_t base = q_off(a.r.qks, b, n0 + m / G, g * G + m % G) + lane * DPL;
#pragma unroll
      for (int e = 0; e < DPL; ++e) v[u][e] = load_f32<E>(a.r.q_kg, base + e);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (m0 + u < cnt)
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] += (double)v[u][e];
  }
  if (a.chunks > 1) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) a.gpart[(int64_t)w * D + lane * DPL + e] = acc[e];
  } else {
    store_group_query<E, D>(a, w, acc, lane);
  }
}

// One workgroup per group: wave i sums chunks i, i+4, ... in order, then the
// four wave sums are added in wave order.
template <class E, int D>
__global__ __launch_bounds__(256) void k_group_query(SharedArgs a) {
  constexpr int DPL = D / 64;
  constexpr int U = 8;
  __shared__ double part[4][D];
  const int gr = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const double* src = a.gpart + (int64_t)gr * a.chunks * D + lane * DPL;
  double acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0;
  for (int c0 = wave; c0 < a.chunks; c0 += 4 * U) {
    double v[U][DPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + 4 * u, a.chunks - 1);
#pragma unroll
      for (int e = 0; e < DPL; ++e) v[u][e] = src[(int64_t)c * D + e];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + 4 * u < a.chunks)
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] += v[u][e];
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) part[wave][lane * DPL + e] = acc[e];
  __syncthreads();
  if (wave != 0) return;
  double x[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const int i = lane * DPL + e;
    x[e] = ((part[0][i] + part[1][i]) + part[2][i]) + part[3][i];
  }
  store_group_query<E, D>(a, gr, x, lane);
}

// One wave per (token, KV head) and up to kSharedRW of its query heads: the
// group's K_L leaf keys and values are read once for all of those rows.  Key
// rows are read 16 bytes a lane (LPK lanes a row, KPW rows an instruction,
// KU instructions in flight); each row's logits go to LDS, then its softmax
// weights; values are read the same way, each lane accumulating its dims
// over the leaves of its lane group, the KPW groups summed at the end.
constexpr int kSharedRW = 4;
template <class E, int D>
__global__ __launch_bounds__(256) void k_shared_kg(SharedArgs a) {
  constexpr int EPV = E::kEPV;
  constexpr int LPK = D / EPV;      // lanes per key row (16-byte chunks)
  constexpr int KPW = 64 / LPK;     // key rows per instruction
  constexpr int RW = kSharedRW;
  constexpr int KU = 8;             // instructions in flight
  __shared__ float lg_all[4][RW][kMaxK];
  __shared__ int leaf_all[4][kMaxK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = a.r.G, Hkv = a.t.Hkv, N = a.r.N;
  const int cpu = (G + RW - 1) / RW;  // row chunks per (token, KV head)
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= (int64_t)a.B * N * Hkv * cpu) return;
  const int c = (int)(w % cpu), unit = (int)(w / cpu);
  const int g = unit % Hkv, t = unit / Hkv;
  const int b = t / N, n = t % N;
  const int gr = a.Ng == 1 ? b * Hkv + g : t * Hkv + g;
  const int h0 = g * G + c * RW, nr = min(RW, G - c * RW);
  const int32_t* sl = a.sel_leaf + (int64_t)gr * a.KL;
  const float scale = (float)a.r.scale;
  const int sub = lane / LPK, ch = lane % LPK;
  float (*lg)[kMaxK] = lg_all[wave];
  int* lid = leaf_all[wave];
  // this lane's 16-byte chunk of each row's KG query (absent rows: zero)
  float qf[RW][EPV];
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (j < nr) u = *(const uint4*)((const char*)a.r.q_kg + q_off(a.r.qks, b, n, h0 + j) * E::kBytes + ch * 16);
    unpack<E>(u, qf[j]);
  }
  const char* kb = (const char*)a.t.key[2] + (int64_t)g * a.t.hs[2] * E::kBytes;
  const int64_t krs = a.t.rs[2] * E::kBytes;
  for (int i0 = 0; i0 < a.KL; i0 += KPW * KU) {
    int leaf[KU];
    uint4 kr[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int i = i0 + u * KPW + sub;
      leaf[u] = i < a.KL ? sl[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      kr[u] = make_uint4(0, 0, 0, 0);
      if (leaf[u] >= 0) kr[u] = *(const uint4*)(kb + (int64_t)leaf[u] * krs + ch * 16);
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int i = i0 + u * KPW + sub;
      float kf[EPV];
      unpack<E>(kr[u], kf);
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) dot = fmaf(qf[j][e], kf[e], dot);
        dot = group_sum<LPK>(dot);
        if (ch == 0 && i < a.KL) lg[j][i] = leaf[u] >= 0 ? dot * scale : -INFINITY;
      }
      if (ch == 0 && i < a.KL) lid[i] = leaf[u];
    }
  }
  wave_sync();
  // softmax weights over the leaves, in place
  float mj[RW], lj[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    float m = -INFINITY;
    for (int i = lane; i < a.KL; i += 64) m = fmaxf(m, lg[j][i]);
    m = wave_max(m);
    float l = 0.f;
    for (int i = lane; i < a.KL; i += 64) {
      const float p = m == -INFINITY ? 0.f : expf(lg[j][i] - m);
      lg[j][i] = p;
      l += p;
    }
    mj[j] = m;
    lj[j] = wave_sum(l);
  }
  wave_sync();
  float o[RW][EPV];
#pragma unroll
  for (int j = 0; j < RW; ++j)
#pragma unroll
    for (int e = 0; e < EPV; ++e) o[j][e] = 0.f;
  const char* vb = (const char*)a.t.leaf_v + (int64_t)g * a.t.hs[3] * E::kBytes;
  const int64_t vrs = a.t.rs[3] * E::kBytes;
  for (int i0 = 0; i0 < a.KL; i0 += KPW * KU) {
    int leaf[KU];
    uint4 vr[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int i = i0 + u * KPW + sub;
      leaf[u] = i < a.KL ? lid[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      vr[u] = make_uint4(0, 0, 0, 0);
      if (leaf[u] >= 0) vr[u] = *(const uint4*)(vb + (int64_t)leaf[u] * vrs + ch * 16);
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int i = i0 + u * KPW + sub;
      float vf[EPV];
      unpack<E>(vr[u], vf);
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const float p = leaf[u] >= 0 ? lg[j][i] : 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) o[j][e] = fmaf(p, vf[e], o[j][e]);
      }
    }
  }
  // sum the KPW lane groups (lanes ch, ch + LPK, ...)
#pragma unroll
  for (int s = LPK; s < 64; s <<= 1)
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
      for (int e = 0; e < EPV; ++e) o[j][e] += __shfl_xor(o[j][e], s);
  const int r0 = t * a.r.Hq + h0;
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    if (j >= nr || sub != j % KPW) continue;
    const float inv = lj[j] > 0.f ? 1.f / lj[j] : 0.f;
    float4* dst = (float4*)(a.o_kg + (int64_t)(r0 + j) * D + ch * EPV);
#pragma unroll
    for (int e = 0; e < EPV; e += 4)
      dst[e / 4] = make_float4(o[j][e] * inv, o[j][e + 1] * inv, o[j][e + 2] * inv, o[j][e + 3] * inv);
  }
  if (lane < nr) {
    float m = mj[0], l = lj[0];
#pragma unroll
    for (int j = 1; j < RW; ++j)
      if (lane == j) m = mj[j], l = lj[j];
    a.lse_kg[r0 + lane] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

}  // namespace

int group_chunks(int N, int Ng, int* tn) {
  *tn = Ng == 1 ? 8 : 1;
  return Ng == 1 ? (N + 7) / 8 : 1;
}

hipError_t launch_group_query(const SharedArgs& a, hipStream_t s) {
  const int rows = a.B * a.Ng * a.t.Hkv;
  const dim3 gp((rows * a.chunks + 3) / 4), grid(rows), block(256);
  const bool two = a.chunks > 1;
  if (a.t.dtype == kDtypeBF16) {
    if (a.t.d == 128) {
      hipLaunchKernelGGL((k_group_partial<BF16, 128>), gp, block, 0, s, a);
      if (two) hipLaunchKernelGGL((k_group_query<BF16, 128>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL((k_group_partial<BF16, 64>), gp, block, 0, s, a);
      if (two) hipLaunchKernelGGL((k_group_query<BF16, 64>), grid, block, 0, s, a);
    }
  } else {
    if (a.t.d == 128) {
      hipLaunchKernelGGL((k_group_partial<F32, 128>), gp, block, 0, s, a);
      if (two) hipLaunchKernelGGL((k_group_query<F32, 128>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL((k_group_partial<F32, 64>), gp, block, 0, s, a);
      if (two) hipLaunchKernelGGL((k_group_query<F32, 64>), grid, block, 0, s, a);
    }
  }
  return hipGetLastError();
}

hipError_t launch_shared_kg(const SharedArgs& a, hipStream_t s) {
  const int64_t waves = (int64_t)a.B * a.r.N * a.t.Hkv * ((a.r.G + kSharedRW - 1) / kSharedRW);
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (a.t.dtype == kDtypeBF16) {
    if (a.t.d == 128) hipLaunchKernelGGL((k_shared_kg<BF16, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_shared_kg<BF16, 64>), grid, block, 0, s, a);
  } else {
    if (a.t.d == 128) hipLaunchKernelGGL((k_shared_kg<F32, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_shared_kg<F32, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hikvp
