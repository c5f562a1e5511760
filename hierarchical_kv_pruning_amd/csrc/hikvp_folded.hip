// hikvp_folded.hip -- folded projections: one base-embedding tree for every
// head.  背景知识与设计原则 › KBLaM中的矩形注意力 scores the layer's query
// against projected knowledge keys W_K k and weights projected values W_V v
// (W_K, W_V: D_E -> d per layer and head); 方法细节 › KGKVs的层次化聚类
// builds the tree over the encoder's base embeddings (width D_E).  Since
// <q, W_K k> = <W_K^T q, k> and sum p W_V v = W_V sum p v, a single base tree
// serves all heads: the query is folded into q' = W_K[g]^T q (k_fold_query),
// the pruned descent runs on the base tree with q', and W_V[g] is applied to
// the softmax-weighted base values afterwards (k_unfold_values).  The
// descent scores with q' rounded to the tree's dtype; its selections are
// exact for the unrounded q', and the KG softmax takes the selected leaves'
// logits from it on fp32 trees (from the scores of the rounded pair on bf16
// trees), so the result is the projected trees' up to fp32 rounding.
#include "hikvp_device.h"
#include "hikvp_round.h"

namespace hikvp {
namespace {

// Work tiles: 4*RPW rows sharing one KV head g, the layer's tokens in order
// with the group's G heads each (row u of the tile: token (tile*4*RPW + u) /
// G, head g*G + u % G); a workgroup stages the head's projection in LDS once
// for its rows (4 waves x RPW rows), instead of every row reading the 32-64 KB
// matrix through L2.  Both take 8 rows a wave, each staged weight converted
// once for 8 rows (the fold keeps its rows' queries in LDS as fp64, so its
// inner loop is fp64 FMAs and weight conversions only: 90 -> 79 us at D_E =
// 384, 587 -> 514 us at 3072; the unfold 82 -> 72 and 607 -> 481 us; 16 rows
// a wave were slower).
constexpr int kFoldRPW = 8, kUnfoldRPW = 8;

struct FoldRow {
  int row, b, n, h;
  bool ok;
};
template <int RPW>
__device__ inline FoldRow fold_row(const FoldArgs& a, int g, int tile, int wave, int rho) {
  FoldRow f;
  const int G = a.r.G;
  const int u = tile * 4 * RPW + wave * RPW + rho;
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
// fp64 in i order (exact for stored bf16 / fp32 inputs of ordinary range).
// The sums go out as they are (qx, fp64: the exact query the selection is
// exact for) and as the query the scores are computed with: rounded once
// into the tree's dtype (qf), in bf16 with the rounded residual beside it
// (qlo), and an upper bound of what that leaves out, per row (qdelta).
// Lanes own output columns j; the columns are taken in chunks of JC = 64*JPL,
// each chunk's slice of W_K[g] staged in LDS once for the workgroup's rows.
template <class E, int D, int JPL>
__global__ __launch_bounds__(256) void k_fold_query(FoldArgs a, int tiles_per_head) {
  constexpr int JC = 64 * JPL;
  __shared__ __align__(16) char w_lds[D * JC * E::kBytes];   // W_K[g][:, chunk] as stored, [i][j]
  __shared__ double q_lds[4][kFoldRPW][D];                    // the waves' KG queries (exact)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x / tiles_per_head, tile = blockIdx.x % tiles_per_head;
  const int DE = a.DE;
  const char* wg = (const char*)a.w_k + (int64_t)g * a.wks[0] * E::kBytes;
  for (int rho = 0; rho < kFoldRPW; ++rho) {
    const FoldRow f = fold_row<kFoldRPW>(a, g, tile, wave, rho);
    const int64_t qb = q_off(a.r.qks, f.b, f.n, f.h);
    for (int t = lane; t < D; t += 64) q_lds[wave][rho][t] = f.ok ? (double)load_f32<E>(a.r.q_kg, qb + t) : 0.0;
  }
  double dq2[kFoldRPW];                                       // |qf - qx|^2, this lane's columns
#pragma unroll
  for (int rho = 0; rho < kFoldRPW; ++rho) dq2[rho] = 0.0;
  // 16-byte row pieces (the API requires 16-byte aligned projection rows)
  constexpr int CPR = JC / E::kEPV;
  for (int j0 = 0; j0 < DE; j0 += JC) {
    __syncthreads();                                          // the previous chunk is consumed
    for (int idx = threadIdx.x; idx < D * CPR; idx += 256) {
      const int i = idx / CPR, c = idx % CPR;
      *(uint4*)(w_lds + (i * JC + c * E::kEPV) * E::kBytes) =
          *(const uint4*)(wg + ((int64_t)i * a.wks[1] + j0 + c * E::kEPV) * E::kBytes);
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
      for (int e = 0; e < JPL; ++e) w[e] = (double)lds_elem<E>(w_lds, i * JC + e * 64 + lane);
#pragma unroll
      for (int rho = 0; rho < kFoldRPW; ++rho) {
        const double qi = q_lds[wave][rho][i];
#pragma unroll
        for (int e = 0; e < JPL; ++e) acc[rho][e] = fma(qi, w[e], acc[rho][e]);
      }
    }
#pragma unroll
    for (int rho = 0; rho < kFoldRPW; ++rho) {
      const FoldRow f = fold_row<kFoldRPW>(a, g, tile, wave, rho);
      if (!f.ok) continue;
#pragma unroll
      for (int e = 0; e < JPL; ++e) {
        const int64_t o = (int64_t)f.row * DE + j0 + e * 64 + lane;
        const double x = acc[rho][e];
        double rest;
        if constexpr (E::kBytes == 2) {
          const Bf16Split sp = split_bf16(x);
          ((uint16_t*)a.qf)[o] = sp.hi;
          ((uint16_t*)a.qlo)[o] = sp.lo;
          rest = sp.rest;
        } else {
          const float v = (float)x;
          ((float*)a.qf)[o] = v;
          rest = x - (double)v;
        }
        a.qx[o] = x;
        dq2[rho] = fma(rest, rest, dq2[rho]);
      }
    }
  }
#pragma unroll
  for (int rho = 0; rho < kFoldRPW; ++rho) {
    const FoldRow f = fold_row<kFoldRPW>(a, g, tile, wave, rho);
    const double t = wave_sum_f64(dq2[rho]);
    // rounded up: the fp32 conversion's relative error is below 2^-24
    if (f.ok && lane == 0) a.qdelta[f.row] = (float)(sqrt(t) * (1.0 + 1e-6));
  }
}

// o_kg[i] = sum_j W_V[g][i][j] o_base[j] in fp32, j in order; lanes own
// output rows i of W_V.  The columns j are taken in chunks of JC = 64*JPL,
// each chunk's slice of W_V[g] staged transposed ([j][i]) so a lane's reads
// are consecutive.  empty: the KG half has no leaves at all (o_kg = 0,
// lse_kg = -inf).
template <class E, int D, int JPL>
__global__ __launch_bounds__(256) void k_unfold_values(FoldArgs a, int tiles_per_head, int empty) {
  constexpr int IPL = D / 64;
  constexpr int JC = 64 * JPL;
  __shared__ __align__(16) char wt_lds[JC * D * E::kBytes];  // W_V[g][:, chunk]^T, [j][i]
  __shared__ float o_lds[4][kUnfoldRPW][JC];                    // the waves' weighted base values
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x / tiles_per_head, tile = blockIdx.x % tiles_per_head;
  if (empty) {
    for (int rho = 0; rho < kUnfoldRPW; ++rho) {
      const FoldRow f = fold_row<kUnfoldRPW>(a, g, tile, wave, rho);
      if (!f.ok) continue;
#pragma unroll
      for (int e = 0; e < IPL; ++e) a.o_kg[(int64_t)f.row * D + e * 64 + lane] = 0.f;
      if (lane == 0) a.lse_kg[f.row] = -INFINITY;
    }
    return;
  }
  const int DE = a.DE;
  const char* wg = (const char*)a.w_v + (int64_t)g * a.wvs[0] * E::kBytes;
  float acc[kUnfoldRPW][IPL];
#pragma unroll
  for (int rho = 0; rho < kUnfoldRPW; ++rho)
#pragma unroll
    for (int e = 0; e < IPL; ++e) acc[rho][e] = 0.f;
  // 16-byte row pieces (16-byte aligned rows), scattered transposed
  constexpr int CPR = JC / E::kEPV;
  for (int j0 = 0; j0 < DE; j0 += JC) {
    __syncthreads();                                          // the previous chunk is consumed
    for (int idx = threadIdx.x; idx < D * CPR; idx += 256) {
      const int i = idx / CPR, c = idx % CPR;
      const uint4 v = *(const uint4*)(wg + ((int64_t)i * a.wvs[1] + j0 + c * E::kEPV) * E::kBytes);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < E::kEPV; ++k) {
        const int j = c * E::kEPV + k;
        if constexpr (E::kBytes == 2) ((uint16_t*)wt_lds)[j * D + i] = (uint16_t)(w4[k >> 1] >> (16 * (k & 1)));
        else ((uint32_t*)wt_lds)[j * D + i] = w4[k];
      }
    }
    for (int rho = 0; rho < kUnfoldRPW; ++rho) {
      const FoldRow f = fold_row<kUnfoldRPW>(a, g, tile, wave, rho);
      for (int j = lane; j < JC; j += 64) o_lds[wave][rho][j] = f.ok ? a.o_base[(int64_t)f.row * DE + j0 + j] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < JC; ++j) {
      float w[IPL];
#pragma unroll
      for (int e = 0; e < IPL; ++e) w[e] = lds_elem<E>(wt_lds, j * D + e * 64 + lane);
#pragma unroll
      for (int rho = 0; rho < kUnfoldRPW; ++rho) {
        const float ob = o_lds[wave][rho][j];
#pragma unroll
        for (int e = 0; e < IPL; ++e) acc[rho][e] = fmaf(w[e], ob, acc[rho][e]);
      }
    }
  }
#pragma unroll
  for (int rho = 0; rho < kUnfoldRPW; ++rho) {
    const FoldRow f = fold_row<kUnfoldRPW>(a, g, tile, wave, rho);
    if (!f.ok) continue;
#pragma unroll
    for (int e = 0; e < IPL; ++e) a.o_kg[(int64_t)f.row * D + e * 64 + lane] = acc[rho][e];
  }
}

// Column chunks of 128 for bf16 when D_E allows (32 KB of W per chunk), of
// 64 otherwise (fp32 rows are twice as wide).
template <class E, int D>
hipError_t fold_dispatch(const FoldArgs& a, hipStream_t s, bool unfold, int empty) {
  const int G = a.r.G, Hkv = a.r.Hq / G;
  const int rows_per_tile = 4 * (unfold ? kUnfoldRPW : kFoldRPW);
  const int tiles = (a.r.B * a.r.N * G + rows_per_tile - 1) / rows_per_tile;
  const dim3 grid((unsigned)(Hkv * tiles)), block(256);
  if (E::kBytes == 2 && a.DE % 128 == 0) {
    if (unfold) hipLaunchKernelGGL((k_unfold_values<E, D, 2>), grid, block, 0, s, a, tiles, empty);
    else hipLaunchKernelGGL((k_fold_query<E, D, 2>), grid, block, 0, s, a, tiles);
  } else {
    if (unfold) hipLaunchKernelGGL((k_unfold_values<E, D, 1>), grid, block, 0, s, a, tiles, empty);
    else hipLaunchKernelGGL((k_fold_query<E, D, 1>), grid, block, 0, s, a, tiles);
  }
  return hipGetLastError();
}

hipError_t fold_launch(const FoldArgs& a, hipStream_t s, bool unfold, int empty) {
  if (a.DE % 64 || a.DE < 64) return hipErrorInvalidValue;
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
