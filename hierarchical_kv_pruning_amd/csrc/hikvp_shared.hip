// hikvp_shared.hip -- shared selections: one descent per group of rows.
//
// The pages pick Top-K branches per query (速读 › 怎么做的) and state a memory
// bound that reads like one selected key set shared by the tokens of a layer
// (速读 › 怎么做的, complexity).  In this variant the rows of one KV head at
// one token (or in one whole sequence) share a selection: the descent runs on
// the group's query, the sum of its members' KG queries rounded once to the
// tree's storage type, which ranks every node by the members' summed logits.
// Each member then takes its own softmax over the group's selected leaves
// with its own logits, merged with its own sequence half as usual.
#include "hikvp_device.h"
#include "hikvp_round.h"

namespace hikvp {
namespace {

// The group query is the exact sum of the members' stored KG queries, rounded
// once.  It is formed in fp64 in two passes: one wave per (group, chunk of
// a.tn tokens) sums its tokens' G heads, one wave per group sums its chunks.
// Both are exact whenever the exact sum fits fp64's 53 bits (the members'
// magnitudes spanning less than ~2^40), so the order of the additions does
// not change the result.
template <class E, int D>
__global__ __launch_bounds__(256) void k_group_partial(SharedArgs a) {
  constexpr int DPL = D / 64;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int Hkv = a.t.Hkv;
  if (w >= a.B * a.Ng * Hkv * a.chunks) return;
  const int c = w % a.chunks, gr = w / a.chunks;
  const int g = gr % Hkv, bn = gr / Hkv;
  const int b = bn / a.Ng;
  const int n0 = a.Ng == 1 ? c * a.tn : bn % a.Ng;
  const int n1 = a.Ng == 1 ? min(a.r.N, n0 + a.tn) : n0 + 1;
  double acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0;
  for (int n = n0; n < n1; ++n)
    for (int j = 0; j < a.r.G; ++j) {
      const int64_t base = q_off(a.r.qks, b, n, g * a.r.G + j) + lane * DPL;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += (double)load_f32<E>(a.r.q_kg, base + e);
    }
#pragma unroll
  for (int e = 0; e < DPL; ++e) a.gpart[(int64_t)w * D + lane * DPL + e] = acc[e];
}

template <class E, int D>
__global__ __launch_bounds__(256) void k_group_query(SharedArgs a) {
  constexpr int DPL = D / 64;
  const int gr = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (gr >= a.B * a.Ng * a.t.Hkv) return;
  double acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0;
  for (int c = 0; c < a.chunks; ++c)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] += a.gpart[((int64_t)gr * a.chunks + c) * D + lane * DPL + e];
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const int64_t o = (int64_t)gr * D + lane * DPL + e;
    if constexpr (E::kBytes == 2) ((uint16_t*)a.gq)[o] = f64_to_bf16_rne(acc[e]);
    else ((float*)a.gq)[o] = (float)acc[e];
  }
}

// One wave per row: logits of the group's K_L leaves under the row's own KG
// query, their softmax, the weighted leaf values -> o_kg, lse_kg.
template <class E, int D>
__global__ __launch_bounds__(256) void k_shared_kg(SharedArgs a) {
  constexpr int LPK = D / E::kEPV;  // lanes per key row (16-byte chunks)
  constexpr int KPW = 64 / LPK;     // key rows per wave step
  constexpr int DPL = D / 64;
  __shared__ float lg_all[4][kMaxK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= a.r.R) return;
  float* lg = lg_all[wave];
  const int h = r % a.r.Hq, t = r / a.r.Hq;
  const int b = t / a.r.N, n = t % a.r.N, g = h / a.r.G;
  const int gr = a.Ng == 1 ? b * a.t.Hkv + g : (b * a.r.N + n) * a.t.Hkv + g;
  const int32_t* sl = a.sel_leaf + (int64_t)gr * a.KL;
  const float scale = (float)a.r.scale;
  // this lane's 16-byte chunk of the row's KG query
  float qf[E::kEPV];
  unpack<E>(*(const uint4*)((const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes +
                            (lane % LPK) * 16),
            qf);
  const char* kb = (const char*)a.t.key[2] + (int64_t)g * a.t.hs[2] * E::kBytes;
  const int64_t krs = a.t.rs[2] * E::kBytes;
  for (int i0 = 0; i0 < a.KL; i0 += KPW) {
    const int i = i0 + lane / LPK;
    const int leaf = i < a.KL ? sl[i] : -1;
    float dot = 0.f;
    if (leaf >= 0) {
      float kf[E::kEPV];
      unpack<E>(*(const uint4*)(kb + (int64_t)leaf * krs + (lane % LPK) * 16), kf);
#pragma unroll
      for (int e = 0; e < E::kEPV; ++e) dot = fmaf(qf[e], kf[e], dot);
    }
    dot = group_sum<LPK>(dot);
    if (lane % LPK == 0 && i < a.KL) lg[i] = leaf >= 0 ? dot * scale : -INFINITY;
  }
  wave_sync();
  float m = -INFINITY;
  for (int i = lane; i < a.KL; i += 64) m = fmaxf(m, lg[i]);
  m = wave_max(m);
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  float l = 0.f;
  if (m != -INFINITY) {
    for (int i = lane; i < a.KL; i += 64) l += expf(lg[i] - m);
    l = wave_sum(l);
    const char* vb = (const char*)a.t.leaf_v + (int64_t)g * a.t.hs[3] * E::kBytes;
    const int64_t vrs = a.t.rs[3] * E::kBytes;
#pragma unroll 4
    for (int i = 0; i < a.KL; ++i) {
      const int leaf = sl[i];
      if (leaf < 0) continue;
      const float p = expf(lg[i] - m);
      float v[DPL];
      load_lane<E, DPL>(vb + (int64_t)leaf * vrs, lane, v);
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(p, v[e], o[e]);
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) a.o_kg[(int64_t)r * D + lane * DPL + e] = o[e] * inv;
  if (lane == 0) a.lse_kg[r] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

int group_chunks(int N, int Ng, int* tn) {
  *tn = Ng == 1 ? 16 : 1;
  return Ng == 1 ? (N + 15) / 16 : 1;
}

hipError_t launch_group_query(const SharedArgs& a, hipStream_t s) {
  const int rows = a.B * a.Ng * a.t.Hkv;
  const dim3 gp((rows * a.chunks + 3) / 4), grid((rows + 3) / 4), block(256);
  if (a.t.dtype == kDtypeBF16) {
    if (a.t.d == 128) {
      hipLaunchKernelGGL((k_group_partial<BF16, 128>), gp, block, 0, s, a);
      hipLaunchKernelGGL((k_group_query<BF16, 128>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL((k_group_partial<BF16, 64>), gp, block, 0, s, a);
      hipLaunchKernelGGL((k_group_query<BF16, 64>), grid, block, 0, s, a);
    }
  } else {
    if (a.t.d == 128) {
      hipLaunchKernelGGL((k_group_partial<F32, 128>), gp, block, 0, s, a);
      hipLaunchKernelGGL((k_group_query<F32, 128>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL((k_group_partial<F32, 64>), gp, block, 0, s, a);
      hipLaunchKernelGGL((k_group_query<F32, 64>), grid, block, 0, s, a);
    }
  }
  return hipGetLastError();
}

hipError_t launch_shared_kg(const SharedArgs& a, hipStream_t s) {
  const dim3 grid((a.r.R + 3) / 4), block(256);
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
