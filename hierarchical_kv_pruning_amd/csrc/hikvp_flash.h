// hikvp_flash.h -- the bf16 flash-attention core shared by the unpruned KG
// kernel (every leaf) and the causal sequence kernel: a workgroup of NT/64
// waves, 32 query rows per wave, streams 64-key blocks of one key range
// through LDS and keeps an online softmax per query row.
//
// Layout (gfx950 v_mfma_f32_32x32x16_bf16; lane l, half h = l/32, col = l%32):
//   * scores are computed transposed, S^T = K Q^T: the K block is the A
//     operand (row = key, 8 consecutive head-dim elements per lane from LDS),
//     the lane's query row the B operand held in registers; accumulator
//     element i of key tile kt is key kt*32 + 8(i/4) + 4h + i%4 of the lane's
//     own query column, so the softmax is in-lane plus one exchange between
//     the two half-waves;
//   * O^T += V^T P^T: the weights stay in registers as the B operand (k-step
//     (kt, h2) covers keys kt*32 + 16*h2 .. +15, slot e of half h being key
//     kt*32 + 16*h2 + 8(e/4) + 4h + e%4, the same key as the score slot) and
//     V^T comes from LDS, where the values are stored transposed with two
//     keys' bf16 packed per dword, so a lane reads 4 consecutive keys of one
//     value column as 8 bytes;
//   * keys are LDS rows of D/2 + 4 dwords (the pad puts the 16-byte operand
//     reads of 8 consecutive rows on distinct bank groups); blocks are double
//     buffered, the next block's global loads in flight during this one's
//     products.
// Weights enter the value product as single bf16 (kSplitP = false: errors of
// many weights average out; measured 25% faster on the unpruned path) or as
// bf16 hi + lo (kSplitP = true: two products with the same value operand,
// weight error ~2^-17 instead of 2^-9).
#pragma once
#include "hikvp_device.h"

namespace hikvp {
namespace flash {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kKeys = 64;  // keys per LDS block
constexpr float kLog2e = 1.4426950408889634f;

template <int D> struct Lds {
  static constexpr int kKS = D / 2 + 4;
  static constexpr int kVS = kKeys / 2 + 4;
  static constexpr int kKDw = kKeys * kKS;
  static constexpr int kVDw = D * kVS;
  static constexpr int kBufDw = kKDw + kVDw;
};

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight fp32 values as bf16 operand elements, rounded to nearest even by the
// hardware conversion (v_cvt_pk_bf16_f32): element 2j in the low half of dword j.
__device__ inline u32x4 pack_bf16x8(const float* p) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2 * j], p[2 * j + 1]}, bf16x2));
  return r;
}

// One thread's staging share of a key block (NT threads).
template <int D, int NT> struct Stage {
  static constexpr int kKChunks = kKeys * D / 8 / NT;          // 16-byte key chunks per thread
  static constexpr int kVItems = (kKeys / 2) * (D / 8) / NT;   // (key pair, d chunk) per thread
  u32x4 k[kKChunks];
  u32x4 va[kVItems], vb[kVItems];
};

// kblk / vblk: the block's first key / value row (uniform); nkeys >= 1 valid
// rows, the ragged tail clamped to the last one.  Offsets inside a block fit
// 32 bits (row strides below 32 MB, checked on the host).
template <int D, int NT>
__device__ inline void stage_load(Stage<D, NT>& st, const char* kblk, uint32_t krs, const char* vblk,
                                  uint32_t vrs, int nkeys, int tid) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < Stage<D, NT>::kKChunks; ++i) {
    const int c = tid + NT * i;
    const uint32_t key = (uint32_t)min(c / CPR, nkeys - 1);
    st.k[i] = *(const u32x4*)(kblk + (key * krs + (uint32_t)(c % CPR) * 16u));
  }
#pragma unroll
  for (int i = 0; i < Stage<D, NT>::kVItems; ++i) {
    const int it = tid + NT * i;
    const int pr = it % (kKeys / 2), ch = it / (kKeys / 2);
    const uint32_t ka = (uint32_t)min(2 * pr, nkeys - 1), kb = (uint32_t)min(2 * pr + 1, nkeys - 1);
    st.va[i] = *(const u32x4*)(vblk + (ka * vrs + (uint32_t)ch * 16u));
    st.vb[i] = *(const u32x4*)(vblk + (kb * vrs + (uint32_t)ch * 16u));
  }
}

template <int D, int NT>
__device__ inline void stage_store(const Stage<D, NT>& st, uint32_t* buf, int tid) {
  using L = Lds<D>;
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < Stage<D, NT>::kKChunks; ++i) {
    const int c = tid + NT * i;
    *(u32x4*)(buf + (c / CPR) * L::kKS + (c % CPR) * 4) = st.k[i];
  }
  uint32_t* vt = buf + L::kKDw;
#pragma unroll
  for (int i = 0; i < Stage<D, NT>::kVItems; ++i) {
    const int it = tid + NT * i;
    const int pr = it % (kKeys / 2), ch = it / (kKeys / 2);
    uint32_t* col = vt + (ch * 8) * L::kVS + pr;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // value columns 8ch + 2w (low halves) and 8ch + 2w + 1 (high halves)
      col[(2 * w) * L::kVS] = __builtin_amdgcn_perm(st.vb[i][w], st.va[i][w], 0x05040100u);
      col[(2 * w + 1) * L::kVS] = __builtin_amdgcn_perm(st.vb[i][w], st.va[i][w], 0x07060302u);
    }
  }
}

// The lane's query row as Q^T operands: lane (col, half h) holds head-dim
// elements 16*ds + 8h .. +7; qp == NULL gives zeros (a padding row).
template <int D>
__device__ inline void load_query(const uint16_t* qp, int half, u32x4 (&qop)[D / 16]) {
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds)
    qop[ds] = qp ? *(const u32x4*)(qp + 16 * ds + 8 * half) : u32x4{0u, 0u, 0u, 0u};
}

// Online softmax state of the lane's query row: o^T (head-dim element
// dt*32 + 8(i/4) + 4h + i%4 in acc[dt][i]), running max m (log2 units, -inf
// before the first visible key) and the half-wave's part of the sum l.
template <int D> struct State {
  f32x16 acc[D / 32];
  float m, l;
};

// Streams keys [0, nkeys) of a range through the workgroup.  kbase / vbase:
// the range's first key / value row; lim: keys of the range visible to the
// lane's query row (0..nkeys; keys at or past lim are masked); lim_min: the
// smallest lim in the workgroup (blocks below it need no mask).  NT threads;
// every thread of the workgroup calls this (it contains barriers).
template <int D, int NT, bool kSplitP>
__device__ inline void run(State<D>& S, const u32x4 (&qop)[D / 16], const char* kbase, uint32_t krs,
                           const char* vbase, uint32_t vrs, int nkeys, int lim, int lim_min, float sl2,
                           uint32_t* lds) {
  using L = Lds<D>;
  constexpr int DS = D / 16, DT = D / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) S.acc[dt] = f32x16{};
  S.m = -INFINITY;
  S.l = 0.f;
  const int nblk = (nkeys + kKeys - 1) / kKeys;
  Stage<D, NT> st;
  if (nblk > 0) {
    stage_load<D, NT>(st, kbase, krs, vbase, vrs, min(kKeys, nkeys), tid);
    stage_store<D, NT>(st, lds, tid);
  }
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int k0 = blk * kKeys;
    if (blk + 1 < nblk)
      stage_load<D, NT>(st, kbase + (int64_t)(k0 + kKeys) * krs, krs, vbase + (int64_t)(k0 + kKeys) * vrs, vrs,
                        min(kKeys, nkeys - k0 - kKeys), tid);
    const uint32_t* kb = lds + (blk & 1) * L::kBufDw;
    const uint32_t* vt = kb + L::kKDw;
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
    if (k0 + kKeys > lim_min) {  // some row sees only part of this block (uniform)
      const int vis = lim - k0;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * 32 + 8 * (i >> 2) + 4 * half + (i & 3) >= vis) s[kt][i] = -INFINITY;
    }
    float mb = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mb = fmaxf(mb, s[kt][i]);
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float m_new = fmaxf(S.m, mb * sl2);
    // rescale only when some row's running maximum grew (rare after the first blocks)
    const bool grow = m_new > S.m;
    const float alpha = grow ? __builtin_amdgcn_exp2f(S.m - m_new) : 1.f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) S.acc[dt] *= alpha;
    }
    S.m = m_new;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // a row with nothing visible yet
    float ps = 0.f;
    u32x4 pop[2][2], pol[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][8 * h2 + e], sl2, -m_use));
          ps += p[e];
        }
        pop[kt][h2] = pack_bf16x8(p);
        if constexpr (kSplitP) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t w = pop[kt][h2][e >> 1];
            p[e] -= __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
          }
          pol[kt][h2] = pack_bf16x8(p);
        }
      }
    S.l = S.l * alpha + ps;
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
          S.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(pop[kt][h2]),
                                                              S.acc[dt], 0, 0, 0);
          if constexpr (kSplitP)
            S.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(pol[kt][h2]),
                                                                S.acc[dt], 0, 0, 0);
        }
    }
    if (blk + 1 < nblk) stage_store<D, NT>(st, lds + ((blk + 1) & 1) * L::kBufDw, tid);
    __syncthreads();
  }
  S.l += __shfl_xor(S.l, 32);
}

}  // namespace flash
}  // namespace hikvp
