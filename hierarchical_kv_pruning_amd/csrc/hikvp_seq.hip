// hikvp_seq.hip -- causal sequence attention and the λ merge (gfx950).
//
// Page: "AtlasKV: Augmenting LLMs with Billion-Scale Knowledge Graphs in 20GB
// VRAM" (digest of arXiv 2510.17934).
//   背景知识与设计原则 › 自注意力层机制: causal softmax attention with logits
//     <q_n, k_i>/sqrt(D) over positions i <= n (bottom-right aligned here when
//     the sequence is longer than the query block).
//   速读 › 怎么做的 and 方法细节 › 等效注意力机制的知识增强: the output is
//     λ_kg·Softmax(logits_kg)·v + λ_seq·Softmax(logits_seq)·v with λ read as the
//     log-sum-exp shares, λ_kg = 1 / (1 + exp(lse_seq - lse_kg)).
#include <hip/hip_runtime.h>

#include "hikvp_device.h"

namespace hikvp {
namespace {

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

}  // namespace

#define HIKVP_DISPATCH(dtype, d, KERNEL, ...)                                                        \
  do {                                                                                               \
    if ((dtype) == kDtypeBF16 && (d) == 128) hipLaunchKernelGGL((KERNEL<BF16, 128>), __VA_ARGS__);   \
    else if ((dtype) == kDtypeBF16 && (d) == 64) hipLaunchKernelGGL((KERNEL<BF16, 64>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 128) hipLaunchKernelGGL((KERNEL<F32, 128>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 64) hipLaunchKernelGGL((KERNEL<F32, 64>), __VA_ARGS__);  \
    else return hipErrorInvalidValue;                                                                \
  } while (0)

hipError_t launch_seq_merge(const SeqArgs& a, hipStream_t s) {
  if (a.r.R <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)(a.r.B * a.r.N * a.Hkv);
  const int waves = a.r.G < 4 ? a.r.G : 4;
  HIKVP_DISPATCH(a.dtype, a.d, k_seq_merge, dim3(blocks), dim3(64 * waves), 0, s, a);
  return hipGetLastError();
}

}  // namespace hikvp
