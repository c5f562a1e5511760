// hikvp_folded.hip -- folded projections: one base-embedding tree for every
// head.  背景知识与设计原则 › KBLaM中的矩形注意力 scores the layer's query
// against projected knowledge keys W_K k and weights projected values W_V v
// (W_K, W_V: D_E -> d per layer and head); 方法细节 › KGKVs的层次化聚类
// builds the tree over the encoder's base embeddings (width D_E).  Since
// <q, W_K k> = <W_K^T q, k> and sum p W_V v = W_V sum p v, a single base tree
// serves all heads: the query is folded into q' = W_K[g]^T q (k_fold_query),
// the pruned descent runs on the base tree with q', and W_V[g] is applied to
// the softmax-weighted base values afterwards (k_unfold_values).
#include "hikvp_device.h"
#include "hikvp_round.h"

namespace hikvp {
namespace {

// One wave per row: q'[j] = sum_t W_K[g][t][j] q_kg[t], products exact in
// fp64 and summed in fp64 (exact for stored bf16 / fp32 inputs of ordinary
// range), rounded once into the tree's dtype.  Lanes own output columns j,
// so every W_K row read is coalesced.
template <class E, int D, int DE>
__global__ __launch_bounds__(256) void k_fold_query(FoldArgs a) {
  constexpr int JPL = DE / 64;
  __shared__ double qs[4][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= a.r.R) return;
  const int h = r % a.r.Hq, t = r / a.r.Hq;
  const int b = t / a.r.N, n = t % a.r.N, g = h / a.r.G;
  const int64_t qb = q_off(a.r.qks, b, n, h);
  for (int i = lane; i < D; i += 64) qs[wave][i] = (double)load_f32<E>(a.r.q_kg, qb + i);
  wave_sync();
  double acc[JPL];
#pragma unroll
  for (int e = 0; e < JPL; ++e) acc[e] = 0.0;
  const int64_t wb = (int64_t)g * a.wks[0];
  for (int i = 0; i < D; ++i) {
    const double qi = qs[wave][i];
#pragma unroll
    for (int e = 0; e < JPL; ++e)
      acc[e] = fma(qi, (double)load_f32<E>(a.w_k, wb + (int64_t)i * a.wks[1] + e * 64 + lane), acc[e]);
  }
#pragma unroll
  for (int e = 0; e < JPL; ++e) {
    const int64_t o = (int64_t)r * DE + e * 64 + lane;
    if constexpr (E::kBytes == 2) ((uint16_t*)a.qf)[o] = f64_to_bf16_rne(acc[e]);
    else ((float*)a.qf)[o] = (float)acc[e];
  }
}

// One wave per row: o_kg[i] = sum_j W_V[g][i][j] o_base[j] in fp32; lanes own
// output rows i of W_V.  empty: the KG half has no leaves at all (o_kg = 0,
// lse_kg = -inf).
template <class E, int D, int DE>
__global__ __launch_bounds__(256) void k_unfold_values(FoldArgs a, int empty) {
  constexpr int IPL = D / 64;
  __shared__ float os[4][DE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= a.r.R) return;
  if (empty) {
#pragma unroll
    for (int e = 0; e < IPL; ++e) a.o_kg[(int64_t)r * D + e * 64 + lane] = 0.f;
    if (lane == 0) a.lse_kg[r] = -INFINITY;
    return;
  }
  const int g = (r % a.r.Hq) / a.r.G;
  for (int j = lane; j < DE; j += 64) os[wave][j] = a.o_base[(int64_t)r * DE + j];
  wave_sync();
#pragma unroll
  for (int e = 0; e < IPL; ++e) {
    const int i = e * 64 + lane;
    const char* wrow = (const char*)a.w_v + ((int64_t)g * a.wvs[0] + (int64_t)i * a.wvs[1]) * E::kBytes;
    float acc = 0.f;
#pragma unroll 4
    for (int j0 = 0; j0 < DE; j0 += E::kEPV) {
      float w[E::kEPV];
      unpack<E>(*(const uint4*)(wrow + j0 * E::kBytes), w);
#pragma unroll
      for (int k = 0; k < E::kEPV; ++k) acc = fmaf(w[k], os[wave][j0 + k], acc);
    }
    a.o_kg[(int64_t)r * D + i] = acc;
  }
}

template <class E, int D>
hipError_t fold_dispatch(const FoldArgs& a, hipStream_t s, bool unfold, int empty) {
  const dim3 grid((a.r.R + 3) / 4), block(256);
  if (a.DE == 128) {
    if (unfold) hipLaunchKernelGGL((k_unfold_values<E, D, 128>), grid, block, 0, s, a, empty);
    else hipLaunchKernelGGL((k_fold_query<E, D, 128>), grid, block, 0, s, a);
  } else {
    if (unfold) hipLaunchKernelGGL((k_unfold_values<E, D, 64>), grid, block, 0, s, a, empty);
    else hipLaunchKernelGGL((k_fold_query<E, D, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t fold_launch(const FoldArgs& a, hipStream_t s, bool unfold, int empty) {
  if (a.dtype == kDtypeBF16)
    return a.d == 128 ? fold_dispatch<BF16, 128>(a, s, unfold, empty) : fold_dispatch<BF16, 64>(a, s, unfold, empty);
  return a.d == 128 ? fold_dispatch<F32, 128>(a, s, unfold, empty) : fold_dispatch<F32, 64>(a, s, unfold, empty);
}

}  // namespace

hipError_t launch_fold_query(const FoldArgs& a, hipStream_t s) { return fold_launch(a, s, false, 0); }

hipError_t launch_unfold_values(const FoldArgs& a, bool kg_empty, hipStream_t s) {
  return fold_launch(a, s, true, kg_empty ? 1 : 0);
}

}  // namespace hikvp
