// hikvp_flat.hip -- unpruned equivalent attention: the KG half as one softmax
// over EVERY leaf of the row's KV head (背景知识与设计原则 › KBLaM中的矩形注意力;
// 方法细节 › 等效注意力机制的知识增强 uses this unpruned form while fine-tuning).
//
// Per KV head g the rows of its G query heads form a dense problem
//   o_kg = softmax(scale · Q_g K_g^T) V_g,   Q_g [B·N·G, d], K_g, V_g [M, d],
// a non-causal flash attention over M keys.  Keys are split into `nsplit`
// ranges; each workgroup owns 128 query rows of one head and one key range and
// writes a partial (o relative to its running max, max, sum) that
// k_flat_combine merges into o_kg / lse_kg.  The sequence half and the λ merge
// then run exactly as for the pruned path.
#include "hikvp_flash.h"

namespace hikvp {
namespace {

using namespace flash;

constexpr int kFlatRows = 128;  // query rows per workgroup, 32 per wave
constexpr int kFlatKeys = kKeys;

// Work item of a workgroup: (KV head, key split) pairs are spread over the 8
// XCDs (workgroup i runs on XCD i mod 8); the row tiles of one pair are
// consecutive on the same XCD so they stream the same keys through its L2.
__device__ inline bool flat_item(const FlatArgs& a, int& g, int& split, int& tile) {
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  tile = local % a.row_tiles;
  const int pair = (local / a.row_tiles) * 8 + xcd;
  if (pair >= a.t.Hkv * a.nsplit) return false;
  g = pair / a.nsplit;
  split = pair % a.nsplit;
  return true;
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_flat_mfma(FlatArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[2 * Lds<D>::kBufDw];
  int g, split, tile;
  if (!flat_item(a, g, split, tile)) return;  // uniform per workgroup, before any barrier
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int G = a.r.G, TG = a.r.B * a.r.N * G;
  const int64_t M = a.t.count[2];
  const int64_t key_lo = (int64_t)split * a.split_len;
  const int nkeys = (int)max<int64_t>(0, min(M, key_lo + a.split_len) - key_lo);

  // this lane's query row (column of the transposed score tile)
  const int u = tile * kFlatRows + wave * 32 + col;
  const bool valid = u < TG;
  const int tok = valid ? u / G : 0, j = valid ? u % G : 0;
  const int b = tok / a.r.N, n = tok % a.r.N, hq = g * G + j;
  const int64_t row = (int64_t)tok * a.r.Hq + hq;
  u32x4 qop[D / 16];
  load_query<D>(valid ? (const uint16_t*)a.r.q_kg + b * a.r.qks[0] + n * a.r.qks[1] + hq * a.r.qks[2] : nullptr,
                half, qop);
  const uint32_t krs = (uint32_t)(a.t.rs[2] * 2), vrs = (uint32_t)(a.t.rs[3] * 2);
  const char* kbase = (const char*)a.t.key[2] + (int64_t)g * a.t.hs[2] * 2 + key_lo * krs;
  const char* vbase = (const char*)a.t.leaf_v + (int64_t)g * a.t.hs[3] * 2 + key_lo * vrs;
  State<D> S;
  run<D, 256, false>(S, qop, kbase, krs, vbase, vrs, nkeys, nkeys, nkeys, (float)a.r.scale * kLog2e, lds);
  if (!valid) return;
  float* pp = a.part + ((size_t)row * a.nsplit + split) * (D + 4);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = dt * 32 + 8 * q4 + 4 * half;
      *(float4*)(pp + d0) = make_float4(S.acc[dt][4 * q4], S.acc[dt][4 * q4 + 1], S.acc[dt][4 * q4 + 2],
                                        S.acc[dt][4 * q4 + 3]);
    }
  if (half == 0) {
    pp[D] = S.m;
    pp[D + 1] = S.l;
  }
}

// Plain fp32 variant (any element type): one workgroup per (row, key split);
// 256 keys per chunk, one key per thread for the scores, then value columns
// d = tid % D accumulated over the chunk's keys in 256/D interleaved subsets.
template <class E, int D>
__global__ __launch_bounds__(256) void k_flat_valu(FlatArgs a) {
  constexpr int SUB = 256 / D;
  __shared__ float qs[D];
  __shared__ float ps[256];
  __shared__ float red[256];
  const int row = blockIdx.x / a.nsplit, split = blockIdx.x % a.nsplit;
  const int tid = threadIdx.x;
  const int h = row % a.r.Hq, tok = row / a.r.Hq;
  const int b = tok / a.r.N, n = tok % a.r.N, g = h / a.r.G;
  const int64_t M = a.t.count[2];
  const int64_t key_lo = (int64_t)split * a.split_len;
  const int64_t key_hi = min(M, key_lo + a.split_len);
  if (tid < D)
    qs[tid] = load_f32<E>(a.r.q_kg, b * a.r.qks[0] + n * a.r.qks[1] + h * a.r.qks[2] + tid);
  __syncthreads();
  const float sl2 = (float)a.r.scale * kLog2e;
  const int64_t kh = (int64_t)g * a.t.hs[2], vh = (int64_t)g * a.t.hs[3];
  float m_run = -INFINITY, l_run = 0.f, o = 0.f;
  const int dcol = tid % D, sub = tid / D;
  for (int64_t c0 = key_lo; c0 < key_hi; c0 += 256) {
    const int64_t key = c0 + tid;
    float x = -INFINITY;
    if (key < key_hi) {
      float acc = 0.f;
      for (int t = 0; t < D; ++t) acc += qs[t] * load_f32<E>(a.t.key[2], kh + key * a.t.rs[2] + t);
      x = acc * sl2;
    }
    red[tid] = x;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
      __syncthreads();
    }
    const float m_new = fmaxf(m_run, red[0]);
    __syncthreads();
    const float alpha = exp2f(m_run - m_new);
    const float p = key < key_hi ? exp2f(x - m_new) : 0.f;
    ps[tid] = p;
    red[tid] = p;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    l_run = l_run * alpha + red[0];
    m_run = m_new;
    o *= alpha;
    const int nk = (int)min<int64_t>(256, key_hi - c0);
    for (int k = sub; k < nk; k += SUB)
      o += ps[k] * load_f32<E>(a.t.leaf_v, vh + (c0 + k) * a.t.rs[3] + dcol);
    __syncthreads();
  }
  red[tid] = o;
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
    for (int s = 0; s < SUB; ++s) acc += red[s * D + tid];
    float* pp = a.part + ((size_t)row * a.nsplit + split) * (D + 4);
    pp[tid] = acc;
    if (tid == 0) {
      pp[D] = key_lo < key_hi ? m_run : -INFINITY;
      pp[D + 1] = l_run;
    }
  }
}

// Log-sum-exp merge of the key splits of one row per wave: o_kg (normalised)
// and lse_kg (natural log).  No leaves at all: lse_kg = -inf, o_kg = 0.
template <int D>
__global__ __launch_bounds__(256) void k_flat_combine(FlatArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.r.R) return;
  constexpr int DPL = D / 64;
  const float* pp = a.part + (size_t)row * a.nsplit * (D + 4);
  float mx = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s)
    if (pp[(size_t)s * (D + 4) + D + 1] > 0.f) mx = fmaxf(mx, pp[(size_t)s * (D + 4) + D]);
  float l = 0.f, o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < a.nsplit; ++s) {
      const float* ps = pp + (size_t)s * (D + 4);
      const float ls = ps[D + 1];
      if (!(ls > 0.f)) continue;
      const float w = exp2f(ps[D] - mx);
      l += w * ls;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] += w * ps[lane * DPL + e];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) a.o_kg[(size_t)row * D + lane * DPL + e] = o[e] * inv;
  if (lane == 0) a.lse_kg[row] = l > 0.f ? (mx + log2f(l)) * 0.6931471805599453f : -INFINITY;
}

}  // namespace

int flat_row_tiles(int B, int N, int G) { return (B * N * G + kFlatRows - 1) / kFlatRows; }

int flat_splits(int B, int N, int Hq, int Hkv, int64_t M, int dtype) {
  if (M <= 0) return 1;
  const int64_t blocks = (M + kFlatKeys - 1) / kFlatKeys;
  int64_t want;
  if (dtype == kDtypeBF16) {
    // about 2048 workgroups (8 per CU); Hkv * nsplit a multiple of the 8 XCDs
    const int64_t tiles = (int64_t)Hkv * flat_row_tiles(B, N, Hq / Hkv);
    want = (2048 + tiles - 1) / tiles;
    int common = 8;  // gcd(8, Hkv)
    while (Hkv % common) common /= 2;
    const int64_t step = 8 / common;
    want = (want + step - 1) / step * step;
  } else {
    const int64_t rows = (int64_t)B * N * Hq;
    want = (2048 + rows - 1) / rows;
  }
  // at least 16 key blocks per range: fewer ranges than that only add partial traffic
  const int64_t cap = (blocks + 15) / 16;
  if (want > cap) want = cap;
  if (want > 1024) want = 1024;
  return (int)(want < 1 ? 1 : want);
}

int flat_split_len(int64_t M, int nsplit) {
  const int64_t per = (M + nsplit - 1) / nsplit;
  return (int)((per + kFlatKeys - 1) / kFlatKeys * kFlatKeys);
}

hipError_t launch_flat_partial(const FlatArgs& a, hipStream_t s) {
  if (a.t.dtype == kDtypeBF16) {
    const int pairs = a.t.Hkv * a.nsplit;
    const int blocks = (pairs + 7) / 8 * 8 * a.row_tiles;
    if (a.t.d == 128) hipLaunchKernelGGL(k_flat_mfma<128>, dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_flat_mfma<64>, dim3(blocks), dim3(256), 0, s, a);
  } else {
    const int blocks = a.r.R * a.nsplit;
    if (a.t.d == 128) hipLaunchKernelGGL((k_flat_valu<F32, 128>), dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_flat_valu<F32, 64>), dim3(blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_flat_combine(const FlatArgs& a, hipStream_t s) {
  const int blocks = (a.r.R + 3) / 4;
  if (a.t.d == 128) hipLaunchKernelGGL(k_flat_combine<128>, dim3(blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_flat_combine<64>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hikvp
