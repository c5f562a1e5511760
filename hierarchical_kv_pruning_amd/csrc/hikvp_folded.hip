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

// Work tiles: kFoldRows rows sharing one KV head g, the layer's tokens in
// order with the group's G heads each (row u of the tile: token
// (tile*kFoldRows + u) / G, head g*G + u % G); a workgroup stages the head's
// projection in LDS once for its 16 rows (4 waves x 4 rows), instead of
// every row reading the 32-64 KB matrix through L2.
constexpr int kFoldRows = 16, kFoldRPW = 4;

struct FoldRow {
  int row, b, n, h;
  bool ok;
};
__device__ inline FoldRow fold_row(const FoldArgs& a, int g, int tile, int wave, int rho) {
  FoldRow f;
  const int G = a.r.G;
  const int u = tile * kFoldRows + wave * kFoldRPW + rho;
  f.ok = u < a.r.B * a.r.N * G;
  const int tok = f.ok ? u / G : 0;
  f.b = tok / a.r.N;
  f.n = tok % a.r.N;
  f.h = g * G + (f.ok ? u % G : 0);
  f.row = (f.b * a.r.N + f.n) * a.r.Hq + f.h;
  return f;
}

template <class E>
__device__ inline float lds_elem(const char* base, int idx) {
  if constexpr (E::kBytes == 2) return __uint_as_float((uint32_t)((const uint16_t*)base)[idx] << 16);
  else return ((const float*)base)[idx];
}

// q'[j] = sum_i W_K[g][i][j] q_kg[i]: products exact in fp64 and summed in
// fp64 in i order (exact for stored bf16 / fp32 inputs of ordinary range),
// rounded once into the tree's dtype.  Lanes own output columns j.
template <class E, int D, int DE>
__global__ __launch_bounds__(256) void k_fold_query(FoldArgs a, int tiles_per_head) {
  constexpr int JPL = DE / 64;
  __shared__ __align__(16) char w_lds[D * DE * E::kBytes];   // W_K[g] as stored, [i][j]
  __shared__ float q_lds[4][kFoldRPW][D];                     // the waves' KG queries (exact)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x / tiles_per_head, tile = blockIdx.x % tiles_per_head;
  const char* wg = (const char*)a.w_k + (int64_t)g * a.wks[0] * E::kBytes;
  // 16-byte row pieces (the API requires 16-byte aligned projection rows)
  constexpr int CPR = DE / E::kEPV;
  for (int idx = threadIdx.x; idx < D * CPR; idx += 256) {
    const int i = idx / CPR, c = idx % CPR;
    *(uint4*)(w_lds + (i * DE + c * E::kEPV) * E::kBytes) =
        *(const uint4*)(wg + ((int64_t)i * a.wks[1] + c * E::kEPV) * E::kBytes);
  }
  for (int rho = 0; rho < kFoldRPW; ++rho) {
    const FoldRow f = fold_row(a, g, tile, wave, rho);
    const int64_t qb = q_off(a.r.qks, f.b, f.n, f.h);
    for (int t = lane; t < D; t += 64) q_lds[wave][rho][t] = f.ok ? load_f32<E>(a.r.q_kg, qb + t) : 0.f;
  }
  __syncthreads();
  double acc[kFoldRPW][JPL];
#pragma unroll
  for (int rho = 0; rho < kFoldRPW; ++rho)
#pragma unroll
    for (int e = 0; e < JPL; ++e) acc[rho][e] = 0.0;
  for (int i = 0; i < D; ++i) {
    double w[JPL];
#pragma unroll
    for (int e = 0; e < JPL; ++e) w[e] = (double)lds_elem<E>(w_lds, i * DE + e * 64 + lane);
#pragma unroll
    for (int rho = 0; rho < kFoldRPW; ++rho) {
      const double qi = (double)q_lds[wave][rho][i];
#pragma unroll
      for (int e = 0; e < JPL; ++e) acc[rho][e] = fma(qi, w[e], acc[rho][e]);
    }
  }
#pragma unroll
  for (int rho = 0; rho < kFoldRPW; ++rho) {
    const FoldRow f = fold_row(a, g, tile, wave, rho);
    if (!f.ok) continue;
#pragma unroll
    for (int e = 0; e < JPL; ++e) {
      const int64_t o = (int64_t)f.row * DE + e * 64 + lane;
      if constexpr (E::kBytes == 2) ((uint16_t*)a.qf)[o] = f64_to_bf16_rne(acc[rho][e]);
      else ((float*)a.qf)[o] = (float)acc[rho][e];
    }
  }
}

// o_kg[i] = sum_j W_V[g][i][j] o_base[j] in fp32, j in order; lanes own
// output rows i of W_V, staged transposed ([j][i]) so a lane's reads are
// consecutive.  empty: the KG half has no leaves at all (o_kg = 0, lse_kg =
// -inf).
template <class E, int D, int DE>
__global__ __launch_bounds__(256) void k_unfold_values(FoldArgs a, int tiles_per_head, int empty) {
  constexpr int IPL = D / 64;
  __shared__ __align__(16) char wt_lds[DE * D * E::kBytes];  // W_V[g]^T, [j][i]
  __shared__ float o_lds[4][kFoldRPW][DE];                    // the waves' weighted base values
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x / tiles_per_head, tile = blockIdx.x % tiles_per_head;
  if (empty) {
    for (int rho = 0; rho < kFoldRPW; ++rho) {
      const FoldRow f = fold_row(a, g, tile, wave, rho);
      if (!f.ok) continue;
#pragma unroll
      for (int e = 0; e < IPL; ++e) a.o_kg[(int64_t)f.row * D + e * 64 + lane] = 0.f;
      if (lane == 0) a.lse_kg[f.row] = -INFINITY;
    }
    return;
  }
  const char* wg = (const char*)a.w_v + (int64_t)g * a.wvs[0] * E::kBytes;
  // 16-byte row pieces (16-byte aligned rows), scattered transposed
  constexpr int CPR = DE / E::kEPV;
  for (int idx = threadIdx.x; idx < D * CPR; idx += 256) {
    const int i = idx / CPR, c = idx % CPR;
    const uint4 v = *(const uint4*)(wg + ((int64_t)i * a.wvs[1] + c * E::kEPV) * E::kBytes);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < E::kEPV; ++k) {
      const int j = c * E::kEPV + k;
      if constexpr (E::kBytes == 2) ((uint16_t*)wt_lds)[j * D + i] = (uint16_t)(w4[k >> 1] >> (16 * (k & 1)));
      else ((uint32_t*)wt_lds)[j * D + i] = w4[k];
    }
  }
  for (int rho = 0; rho < kFoldRPW; ++rho) {
    const FoldRow f = fold_row(a, g, tile, wave, rho);
    for (int j = lane; j < DE; j += 64) o_lds[wave][rho][j] = f.ok ? a.o_base[(int64_t)f.row * DE + j] : 0.f;
  }
  __syncthreads();
  float acc[kFoldRPW][IPL];
#pragma unroll
  for (int rho = 0; rho < kFoldRPW; ++rho)
#pragma unroll
    for (int e = 0; e < IPL; ++e) acc[rho][e] = 0.f;
  for (int j = 0; j < DE; ++j) {
    float w[IPL];
#pragma unroll
    for (int e = 0; e < IPL; ++e) w[e] = lds_elem<E>(wt_lds, j * D + e * 64 + lane);
#pragma unroll
    for (int rho = 0; rho < kFoldRPW; ++rho) {
      const float ob = o_lds[wave][rho][j];
#pragma unroll
      for (int e = 0; e < IPL; ++e) acc[rho][e] = fmaf(w[e], ob, acc[rho][e]);
    }
  }
#pragma unroll
  for (int rho = 0; rho < kFoldRPW; ++rho) {
    const FoldRow f = fold_row(a, g, tile, wave, rho);
    if (!f.ok) continue;
#pragma unroll
    for (int e = 0; e < IPL; ++e) a.o_kg[(int64_t)f.row * D + e * 64 + lane] = acc[rho][e];
  }
}

template <class E, int D>
hipError_t fold_dispatch(const FoldArgs& a, hipStream_t s, bool unfold, int empty) {
  const int G = a.r.G, Hkv = a.r.Hq / G;
  const int tiles = (a.r.B * a.r.N * G + kFoldRows - 1) / kFoldRows;
  const dim3 grid((unsigned)(Hkv * tiles)), block(256);
  if (a.DE == 128) {
    if (unfold) hipLaunchKernelGGL((k_unfold_values<E, D, 128>), grid, block, 0, s, a, tiles, empty);
    else hipLaunchKernelGGL((k_fold_query<E, D, 128>), grid, block, 0, s, a, tiles);
  } else {
    if (unfold) hipLaunchKernelGGL((k_unfold_values<E, D, 64>), grid, block, 0, s, a, tiles, empty);
    else hipLaunchKernelGGL((k_fold_query<E, D, 64>), grid, block, 0, s, a, tiles);
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
