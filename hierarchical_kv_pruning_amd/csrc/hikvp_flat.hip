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
#include "hikvp_device.h"

namespace hikvp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kFlatRows = 128;  // query rows per workgroup, 32 per wave
constexpr int kFlatKeys = 64;   // keys per LDS block
// true: softmax weights enter the value product as bf16 hi + lo (two products
// with the same value operand), weight error ~2^-17 instead of bf16's 2^-9.
// Measured 25% slower at 1e6 leaves; the single bf16 weight already keeps the
// output well inside 2e-2 of its RMS (rounding errors of 1e6 weights average
// out), so it is off.
constexpr bool kPSplit = false;
constexpr float kLog2e = 1.4426950408889634f;
// partial record of one (row, key range): o[D], m, sum, 2 pad floats (16-byte rows)

// LDS geometry of one block (dwords).  Keys: [64 key rows][D/2 + 4]; the
// 4-dword pad puts the 16-byte operand reads of 8 consecutive key rows on
// distinct bank groups.  Values, transposed: [D rows][32 + 4] with two keys'
// bf16 values packed per dword, so a lane reads 4 consecutive keys of one
// value column as 8 bytes.
template <int D> struct FlatLds {
  static constexpr int kKS = D / 2 + 4;
  static constexpr int kVS = kFlatKeys / 2 + 4;
  static constexpr int kKDw = kFlatKeys * kKS;
  static constexpr int kVDw = D * kVS;
  static constexpr int kBufDw = kKDw + kVDw;
};

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight fp32 values as bf16 operand elements, rounded to nearest even by the
// hardware conversion (v_cvt_pk_bf16_f32): element 2j in the low half of dword j.
__device__ inline u32x4 pack_bf16x8(const float* p) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2 * j], p[2 * j + 1]}, bf16x2));
  return r;
}

// One wave's staging share of a key block: 4 x 16 bytes of keys, and 2 key
// pairs x 16 bytes of values (one d-chunk of two consecutive keys each).
template <int D> struct Stage {
  static constexpr int kKChunks = kFlatKeys * D / 8 / 256;    // 16-byte key chunks per thread
  static constexpr int kVItems = (kFlatKeys / 2) * (D / 8) / 256;  // (key pair, d chunk) per thread
  u32x4 k[kKChunks];
  u32x4 va[kVItems], vb[kVItems];
};

// kblk / vblk: the block's first key / value row (uniform); nkeys >= 1 valid
// rows, the ragged tail clamped to the last one.  Offsets inside a block fit
// 32 bits (row strides below 32 MB are checked on the host).
template <int D>
__device__ inline void stage_load(Stage<D>& st, const char* kblk, uint32_t krs, const char* vblk,
                                  uint32_t vrs, int nkeys, int tid) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < Stage<D>::kKChunks; ++i) {
    const int c = tid + 256 * i;
    const uint32_t key = (uint32_t)min(c / CPR, nkeys - 1);
    st.k[i] = *(const u32x4*)(kblk + (key * krs + (uint32_t)(c % CPR) * 16u));
  }
#pragma unroll
  for (int i = 0; i < Stage<D>::kVItems; ++i) {
    const int it = tid + 256 * i;
    const int pr = it % (kFlatKeys / 2), ch = it / (kFlatKeys / 2);
    const uint32_t ka = (uint32_t)min(2 * pr, nkeys - 1), kb = (uint32_t)min(2 * pr + 1, nkeys - 1);
    st.va[i] = *(const u32x4*)(vblk + (ka * vrs + (uint32_t)ch * 16u));
    st.vb[i] = *(const u32x4*)(vblk + (kb * vrs + (uint32_t)ch * 16u));
  }
}

template <int D>
__device__ inline void stage_store(const Stage<D>& st, uint32_t* buf, int tid) {
  using L = FlatLds<D>;
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < Stage<D>::kKChunks; ++i) {
    const int c = tid + 256 * i;
    *(u32x4*)(buf + (c / CPR) * L::kKS + (c % CPR) * 4) = st.k[i];
  }
  uint32_t* vt = buf + L::kKDw;
#pragma unroll
  for (int i = 0; i < Stage<D>::kVItems; ++i) {
    const int it = tid + 256 * i;
    const int pr = it % (kFlatKeys / 2), ch = it / (kFlatKeys / 2);
    uint32_t* col = vt + (ch * 8) * L::kVS + pr;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // value columns 8ch + 2w (low halves) and 8ch + 2w + 1 (high halves)
      col[(2 * w) * L::kVS] = __builtin_amdgcn_perm(st.vb[i][w], st.va[i][w], 0x05040100u);
      col[(2 * w + 1) * L::kVS] = __builtin_amdgcn_perm(st.vb[i][w], st.va[i][w], 0x07060302u);
    }
  }
}

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
  using L = FlatLds<D>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[2 * L::kBufDw];
  int g, split, tile;
  if (!flat_item(a, g, split, tile)) return;  // uniform per workgroup, before any barrier
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int G = a.r.G, TG = a.r.B * a.r.N * G;
  const int64_t M = a.t.count[2];
  const int64_t key_lo = (int64_t)split * a.split_len;
  const int64_t key_hi = min(M, key_lo + a.split_len);
  const int nblk = key_lo < key_hi ? (int)((key_hi - key_lo + kFlatKeys - 1) / kFlatKeys) : 0;

  // this lane's query row (column of the transposed score tile)
  const int u = tile * kFlatRows + wave * 32 + col;
  const bool valid = u < TG;
  const int tok = valid ? u / G : 0, j = valid ? u % G : 0;
  const int b = tok / a.r.N, n = tok % a.r.N, hq = g * G + j;
  const int64_t row = (int64_t)tok * a.r.Hq + hq;

  // Q^T operands: lane (query col, half h) holds d = 16*ds + 8h .. +7
  constexpr int DS = D / 16;
  u32x4 qop[DS];
  {
    const uint16_t* qp = (const uint16_t*)a.r.q_kg + b * a.r.qks[0] + n * a.r.qks[1] + hq * a.r.qks[2];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qop[ds] = valid ? *(const u32x4*)(qp + 16 * ds + 8 * half) : u32x4{0u, 0u, 0u, 0u};
  }
  const char* kbase = (const char*)a.t.key[2] + (int64_t)g * a.t.hs[2] * 2;
  const char* vbase = (const char*)a.t.leaf_v + (int64_t)g * a.t.hs[3] * 2;
  const uint32_t krs = (uint32_t)(a.t.rs[2] * 2), vrs = (uint32_t)(a.t.rs[3] * 2);
  const float sl2 = (float)a.r.scale * kLog2e;

  constexpr int DT = D / 32;
  f32x16 acc_o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  Stage<D> st;
  if (nblk > 0) {
    stage_load<D>(st, kbase + key_lo * krs, krs, vbase + key_lo * vrs, vrs,
                  (int)min<int64_t>(kFlatKeys, key_hi - key_lo), tid);
    stage_store<D>(st, lds, tid);
  }
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int64_t k0 = key_lo + (int64_t)blk * kFlatKeys;
    const int nk = (int)min<int64_t>(kFlatKeys, key_hi - k0);
    if (blk + 1 < nblk)
      stage_load<D>(st, kbase + (k0 + kFlatKeys) * krs, krs, vbase + (k0 + kFlatKeys) * vrs, vrs,
                    (int)min<int64_t>(kFlatKeys, key_hi - k0 - kFlatKeys), tid);
    const uint32_t* kb = lds + (blk & 1) * L::kBufDw;
    const uint32_t* vt = kb + L::kKDw;

    // S^T = K Q^T: two 32-key tiles; element i of tile kt is key kt*32 + 8(i/4) + 4h + i%4
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16{};
      const uint32_t* kr = kb + (kt * 32 + col) * L::kKS + 4 * half;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*(const u32x4*)(kr + 8 * ds)),
                                                        as_bf16x8(qop[ds]), s[kt], 0, 0, 0);
    }
    // online softmax in log2 units; the lane's query column is its own
    if (nk < kFlatKeys) {  // ragged last block (uniform)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * 32 + 8 * (i >> 2) + 4 * half + (i & 3) >= nk) s[kt][i] = -INFINITY;
    }
    float mb = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mb = fmaxf(mb, s[kt][i]);
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float m_new = fmaxf(m_run, mb * sl2);  // finite: every block holds a valid key
    // rescale only when some row's running maximum grew (rare after the first blocks)
    const bool grow = m_new > m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;
    }
    m_run = m_new;
    float ps = 0.f;
    u32x4 pop[2][2], pol[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][8 * h2 + e], sl2, -m_new));
          ps += p[e];
        }
        pop[kt][h2] = pack_bf16x8(p);
        if constexpr (kPSplit) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t w = pop[kt][h2][e >> 1];
            p[e] -= __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
          }
          pol[kt][h2] = pack_bf16x8(p);
        }
      }
    l_run = l_run * alpha + ps;
    // O^T += V^T P^T: k-step (kt, h2) covers keys kt*32 + 16*h2 .. +15; slot e of
    // half h is key kt*32 + 16*h2 + 8(e/4) + 4h + e%4, the same key as P's slot
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t* vr = vt + (dt * 32 + col) * L::kVS + 2 * half;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const u32x2 lo = *(const u32x2*)(vr + 16 * kt + 8 * h2);
          const u32x2 hi = *(const u32x2*)(vr + 16 * kt + 8 * h2 + 4);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(pop[kt][h2]),
                                                              acc_o[dt], 0, 0, 0);
          if constexpr (kPSplit)
            acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(pol[kt][h2]),
                                                                acc_o[dt], 0, 0, 0);
        }
    }
    if (blk + 1 < nblk) stage_store<D>(st, lds + ((blk + 1) & 1) * L::kBufDw, tid);
    __syncthreads();
  }
  l_run += __shfl_xor(l_run, 32);
  if (!valid) return;
  float* pp = a.part + ((size_t)row * a.nsplit + split) * (D + 4);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = dt * 32 + 8 * q4 + 4 * half;
      *(float4*)(pp + d0) = make_float4(acc_o[dt][4 * q4], acc_o[dt][4 * q4 + 1], acc_o[dt][4 * q4 + 2],
                                        acc_o[dt][4 * q4 + 3]);
    }
  if (half == 0) {
    pp[D] = nblk > 0 ? m_run : -INFINITY;
    pp[D + 1] = l_run;
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
