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

#include <type_traits>

#include "hikvp_device.h"
#include "hikvp_flash.h"

namespace hikvp {
namespace {

// λ merge of the sequence half (lse_seq, o_seq) with the KG half of the row.
template <class E, int D>
__device__ inline void merge_store(const SeqArgs& a, int row, int b, int n, int h, float lse_seq,
                                   bool has_seq, const float* oseq, int lane) {
  constexpr int DPL = D / 64;
  const float lkg = a.lse_kg[row];
  float lam;
  if (lkg == -INFINITY) lam = 0.f;
  else if (!has_seq) lam = 1.f;
  else lam = 1.f / (1.f + __expf(lse_seq - lkg));
  const float* okg = a.o_kg + (int64_t)row * D;
  const int64_t ob = q_off(a.os, b, n, h);
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const float o = lam * okg[lane * DPL + e] + (1.f - lam) * oseq[e];
    const int64_t at = ob + (int64_t)lane * DPL + e;
    if (a.out_dtype == kDtypeBF16) ((uint16_t*)a.out)[at] = f32_to_bf16_rne(o);
    else ((float*)a.out)[at] = o;
  }
  if (a.lse_seq_out && lane == 0) a.lse_seq_out[row] = lse_seq;
}

// ---------------------------------------------------------------------------
// Decode (fewer than 16 query tokens): one wave per (b, n, KV head, group of
// up to 4 query heads [, key split]).  The wave streams its key range in
// chunks of 16 keys; a 16-lane DPP row holds one 256-byte key (or value) row,
// lane c owning dims [c*EPL, c*EPL+EPL) with EPL = D/16, so each load
// instruction covers four whole rows and K and V are read once for all the
// group's heads.  Scores are 16-lane DPP sums; the softmax statistics are
// wave-uniform (v_readlane); every lane of a row keeps that row's
// probabilities, so P V accumulates on VALU without LDS.  The four rows'
// partial sums are combined at the end.
// ---------------------------------------------------------------------------
// EPL consecutive elements of a row as raw 32-bit words (8, 16 or 32 bytes),
// unpacked to fp32 where used: holding rows packed keeps the registers low.
template <class E, int EPL>
struct RawElems {
  static constexpr int kWords = EPL * E::kBytes / 4;
  uint32_t w[kWords];
  __device__ inline void load(const char* p) {
    if constexpr (kWords == 2) {
      const uint2 v = *(const uint2*)p;
      w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
      for (int k = 0; k < kWords; k += 4) {
        const uint4 v = *(const uint4*)(p + 4 * k);
        w[k] = v.x; w[k + 1] = v.y; w[k + 2] = v.z; w[k + 3] = v.w;
      }
    }
  }
  __device__ inline float operator[](int e) const {
    if constexpr (E::kBytes == 2) return __uint_as_float(e & 1 ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
    else return __uint_as_float(w[e]);
  }
};

// <q, k> over a lane's EPL elements: bf16 pairs on v_dot2_f32_bf16 (products
// exact in fp32), fp32 on FMA.
typedef __bf16 Bf16x2 __attribute__((ext_vector_type(2)));
template <class E, int EPL>
__device__ inline float dot_elems(const RawElems<E, EPL>& x, const RawElems<E, EPL>& y) {
  float d = 0.f;
  if constexpr (E::kBytes == 2) {
#pragma unroll
    for (int k = 0; k < RawElems<E, EPL>::kWords; ++k)
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(Bf16x2, x.w[k]), __builtin_bit_cast(Bf16x2, y.w[k]), d,
                                          false);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) d = fmaf(x[e], y[e], d);
  }
  return d;
}

template <class E, int D>
__global__ __launch_bounds__(64) void k_seq_decode(SeqArgs a) {
  constexpr int EPL = D / 16, HG = 4, CK = 16;
  const int lane = threadIdx.x, r = lane >> 4, c = lane & 15;
  const int G = a.r.G, HGP = (G + HG - 1) / HG;
  int t = blockIdx.x;
  const int hgp = t % HGP; t /= HGP;
  const int g = t % a.Hkv; t /= a.Hkv;
  const int n = t % a.r.N, b = t / a.r.N;
  const int nh = (G - hgp * HG) < HG ? (G - hgp * HG) : HG;   // heads of this wave
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int vis = a.k ? a.S - a.r.N + n + 1 : 0;
  const int k0 = split * a.split_len;
  const int k1 = (k0 + a.split_len) < vis ? (k0 + a.split_len) : vis;
  const float scale = (float)a.r.scale;

  RawElems<E, EPL> qr[HG];                 // queries stay packed (bf16: v_dot2 on pairs)
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    const int h = g * G + hgp * HG + (hh < nh ? hh : 0);
    qr[hh].load((const char*)a.r.q + (q_off(a.r.qs, b, n, h) + c * EPL) * E::kBytes);
  }
  float m[HG], l[HG], acc[HG][EPL];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  }
  if (k0 < k1) {
    const char* kb = (const char*)a.k + ((int64_t)b * a.ks[0] + (int64_t)g * a.ks[2] + c * EPL) * E::kBytes;
    const char* vb = (const char*)a.v + ((int64_t)b * a.vs[0] + (int64_t)g * a.vs[2] + c * EPL) * E::kBytes;
    const int64_t kstep = a.ks[1] * E::kBytes, vstep = a.vs[1] * E::kBytes;
    // chunk loads are issued one chunk ahead (key c0 + 4i + r; past the range
    // its last key, masked)
    RawElems<E, EPL> kn[CK / 4], vn[CK / 4];
    auto load_chunk = [&](int c0) {
#pragma unroll
      for (int i = 0; i < CK / 4; ++i) {
        const int key = min(c0 + 4 * i + r, k1 - 1);
        kn[i].load(kb + (int64_t)key * kstep);
        vn[i].load(vb + (int64_t)key * vstep);
      }
    };
    load_chunk(k0);
    for (int c0 = k0; c0 < k1; c0 += CK) {
      RawElems<E, EPL> kf[CK / 4], vf[CK / 4];
#pragma unroll
      for (int i = 0; i < CK / 4; ++i) {
        kf[i] = kn[i];
        vf[i] = vn[i];
      }
      if (c0 + CK < k1) load_chunk(c0 + CK);
      float p[CK / 4][HG];
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        float sc[CK / 4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < CK / 4; ++i) {
          float d = dot_elems(qr[hh], kf[i]);
          d = group_sum<16>(d);
          sc[i] = (c0 + 4 * i + r < k1) ? d * scale : -INFINITY;
          mx = fmaxf(mx, sc[i]);
        }
        // chunk max over the four rows, wave-uniform
        mx = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 0)),
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 16))),
                   fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 32)),
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 48))));
        const float mn = fmaxf(m[hh], mx);   // finite: key c0 is in range
        const float alpha = __expf(m[hh] - mn);
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < CK / 4; ++i) {
          p[i][hh] = __expf(sc[i] - mn);
          ls += p[i][hh];
        }
        ls = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), 0)) +
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), 16))) +
             (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), 32)) +
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), 48)));
        l[hh] = l[hh] * alpha + ls;
        m[hh] = mn;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
      }
#pragma unroll
      for (int i = 0; i < CK / 4; ++i)
#pragma unroll
        for (int hh = 0; hh < HG; ++hh)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(p[i][hh], vf[i][e], acc[hh][e]);
    }
  }
  // sum the four rows' partial weighted values (keys = r mod 4)
#pragma unroll
  for (int hh = 0; hh < HG; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[hh][e];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[hh][e] = v;
    }
  if (r != 0) return;
  for (int hh = 0; hh < nh; ++hh) {
    const int h = g * G + hgp * HG + hh;
    const int row = (b * a.r.N + n) * a.r.Hq + h;
    if (a.part) {  // partial (acc, m, l) for k_seq_combine
      float* part = a.part + ((int64_t)row * nsplit + split) * (D + 2);
#pragma unroll
      for (int e = 0; e < EPL; ++e) part[c * EPL + e] = acc[hh][e];
      if (c == 0) {
        part[D] = l[hh] > 0.f ? m[hh] : -INFINITY;
        part[D + 1] = l[hh];
      }
      continue;
    }
    const bool has = l[hh] > 0.f;
    const float lse_seq = has ? m[hh] + logf(l[hh]) : -INFINITY;
    const float lkg = a.lse_kg[row];
    float lam;
    if (lkg == -INFINITY) lam = 0.f;
    else if (!has) lam = 1.f;
    else lam = 1.f / (1.f + __expf(lse_seq - lkg));
    const float inv = has ? 1.f / l[hh] : 0.f;
    const float* okg = a.o_kg + (int64_t)row * D;
    const int64_t ob = q_off(a.os, b, n, h);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int dim = c * EPL + e;
      const float o = lam * okg[dim] + (1.f - lam) * (acc[hh][e] * inv);
      if (a.out_dtype == kDtypeBF16) ((uint16_t*)a.out)[ob + dim] = f32_to_bf16_rne(o);
      else ((float*)a.out)[ob + dim] = o;
    }
    if (a.lse_seq_out && c == 0) a.lse_seq_out[row] = lse_seq;
  }
}

// Decode on the matrix cores (bf16): the same work items and V layout as
// k_seq_decode, with the scores S^T = K Q^T of a 16-key chunk on
// v_mfma_f32_16x16x32_bf16: the chunk's keys are the M side (lane l feeds key
// l%16 with dims 32m + 8(l/16) .. +8, m < D/32), the group's heads the N side
// (head column l%16, zero beyond the group).  Lane (r, c) then holds the
// scores of keys 4r .. 4r+3 for head c, which is also the key set of its V
// rows, so the online softmax runs in place (in-lane over four keys, across
// the four 16-lane rows by two xor shuffles) and each lane takes the
// probability of its keys under head hh, and the head's rescale factor, from
// lane (r, hh) by a DPP row broadcast; P V accumulates on VALU.
template <int D>
__device__ inline float row_bcast(float x, int hh) {
  switch (hh) {  // DPP row_newbcast:hh (lane hh of each 16-lane row)
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150, 0xf, 0xf, false));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x151, 0xf, 0xf, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x152, 0xf, 0xf, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x153, 0xf, 0xf, false));
  }
}

template <int D>
__global__ __launch_bounds__(64) void k_seq_decode_mfma(SeqArgs a) {
  typedef __bf16 Bf16x8 __attribute__((ext_vector_type(8)));
  typedef float Float4 __attribute__((ext_vector_type(4)));
  constexpr int EPL = D / 16, HG = 4, CK = 16, KM = D / 32;
  const int lane = threadIdx.x, r = lane >> 4, c = lane & 15;
  const int G = a.r.G, HGP = (G + HG - 1) / HG;
  int t = blockIdx.x;
  const int hgp = t % HGP; t /= HGP;
  const int g = t % a.Hkv; t /= a.Hkv;
  const int n = t % a.r.N, b = t / a.r.N;
  const int nh = (G - hgp * HG) < HG ? (G - hgp * HG) : HG;   // heads of this wave
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int vis = a.k ? a.S - a.r.N + n + 1 : 0;
  const int k0 = split * a.split_len;
  const int k1 = (k0 + a.split_len) < vis ? (k0 + a.split_len) : vis;
  const float scale = (float)a.r.scale;

  // B operand: head column c of the group, dims 32m + 8r .. +8 (zero past the group)
  uint4 qb[KM];
#pragma unroll
  for (int m = 0; m < KM; ++m) qb[m] = make_uint4(0, 0, 0, 0);
  if (c < nh) {
    const char* qp = (const char*)a.r.q + q_off(a.r.qs, b, n, g * G + hgp * HG + c) * 2;
#pragma unroll
    for (int m = 0; m < KM; ++m) qb[m] = *(const uint4*)(qp + (32 * m + 8 * r) * 2);
  }
  float m_run = -INFINITY, l_run = 0.f;   // head c's softmax state (same in all four rows)
  float acc[HG][EPL];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  if (k0 < k1) {
    const char* kb = (const char*)a.k + ((int64_t)b * a.ks[0] + (int64_t)g * a.ks[2]) * 2;
    const char* vb = (const char*)a.v + ((int64_t)b * a.vs[0] + (int64_t)g * a.vs[2] + c * EPL) * 2;
    const int64_t kstep = a.ks[1] * 2, vstep = a.vs[1] * 2;
    // chunk loads are issued one chunk ahead (keys past the range re-read the
    // last key and are masked): K in the MFMA layout, V rows c0 + 4r + i.  K
    // is single-buffered: the next chunk's keys load once the scores of this
    // one are on the matrix cores, while the softmax and P V run.
    uint4 kn[KM];
    RawElems<BF16, EPL> vn[CK / 4];
    auto load_k = [&](int c0) {
      const char* kp = kb + (int64_t)min(c0 + c, k1 - 1) * kstep + (8 * r) * 2;
#pragma unroll
      for (int m = 0; m < KM; ++m) kn[m] = *(const uint4*)(kp + 64 * m);
    };
    auto load_v = [&](int c0) {
#pragma unroll
      for (int i = 0; i < CK / 4; ++i) vn[i].load(vb + (int64_t)min(c0 + 4 * r + i, k1 - 1) * vstep);
    };
    load_k(k0);
    load_v(k0);
    for (int c0 = k0; c0 < k1; c0 += CK) {
      RawElems<BF16, EPL> vf[CK / 4];
#pragma unroll
      for (int i = 0; i < CK / 4; ++i) vf[i] = vn[i];
      Float4 sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KM; ++m)
        sv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(Bf16x8, kn[m]), __builtin_bit_cast(Bf16x8, qb[m]),
                                                    sv, 0, 0, 0);
      if (c0 + CK < k1) {
        load_k(c0 + CK);
        load_v(c0 + CK);
      }
      float sc[4], mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[i] = (c0 + 4 * r + i < k1) ? sv[i] * scale : -INFINITY;
        mx = fmaxf(mx, sc[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m_run, mx);   // finite: key c0 is in range
      const float alpha = __expf(m_run - mn);
      float p[4], ls = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __expf(sc[i] - mn);
        ls += p[i];
      }
      ls += __shfl_xor(ls, 16);
      ls += __shfl_xor(ls, 32);
      l_run = l_run * alpha + ls;
      m_run = mn;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float al = row_bcast<D>(alpha, hh);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] *= al;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pw = row_bcast<D>(p[i], hh);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(pw, vf[i][e], acc[hh][e]);
        }
      }
    }
  }
  // sum the four rows' partial weighted values (keys 4r .. 4r+3 of each chunk)
#pragma unroll
  for (int hh = 0; hh < HG; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[hh][e];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[hh][e] = v;
    }
  float m[HG], l[HG];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    m[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_run), hh));
    l[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_run), hh));
  }
  if (r != 0) return;
  for (int hh = 0; hh < nh; ++hh) {
    const int h = g * G + hgp * HG + hh;
    const int row = (b * a.r.N + n) * a.r.Hq + h;
    if (a.part) {  // partial (acc, m, l) for k_seq_combine
      float* part = a.part + ((int64_t)row * nsplit + split) * (D + 2);
#pragma unroll
      for (int e = 0; e < EPL; ++e) part[c * EPL + e] = acc[hh][e];
      if (c == 0) {
        part[D] = l[hh] > 0.f ? m[hh] : -INFINITY;
        part[D + 1] = l[hh];
      }
      continue;
    }
    const bool has = l[hh] > 0.f;
    const float lse_seq = has ? m[hh] + logf(l[hh]) : -INFINITY;
    const float lkg = a.lse_kg[row];
    float lam;
    if (lkg == -INFINITY) lam = 0.f;
    else if (!has) lam = 1.f;
    else lam = 1.f / (1.f + __expf(lse_seq - lkg));
    const float inv = has ? 1.f / l[hh] : 0.f;
    const float* okg = a.o_kg + (int64_t)row * D;
    const int64_t ob = q_off(a.os, b, n, h);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int dim = c * EPL + e;
      const float o = lam * okg[dim] + (1.f - lam) * (acc[hh][e] * inv);
      if (a.out_dtype == kDtypeBF16) ((uint16_t*)a.out)[ob + dim] = f32_to_bf16_rne(o);
      else ((float*)a.out)[ob + dim] = o;
    }
    if (a.lse_seq_out && c == 0) a.lse_seq_out[row] = lse_seq;
  }
}

// ---------------------------------------------------------------------------
// Prefill: flash attention on MFMA.  One workgroup per (b, KV head, 16-token
// tile); one wave per query head of the group.  Per 16-key tile: S = Q K^T on
// a 16x16 MFMA tile (rows = the tile's tokens), causal mask, online softmax
// per row, then O += P V on MFMA with the V tile transposed once in LDS and
// shared by the group's heads (P goes through a per-wave LDS tile to become
// the A operand).  bf16 inputs use bf16 MFMA (P as a hi + lo pair of bf16),
// fp32 inputs fp32 MFMA throughout.
// ---------------------------------------------------------------------------
template <class E, int D>
struct FlashSmem {
  static constexpr bool kB = E::kBytes == 2;
  static constexpr int kVp = kB ? 24 : 20;   // padded key stride of the transposed V tile
  static constexpr int kPp = kB ? 24 : 20;
  typename std::conditional<kB, uint16_t, float>::type vt[D][kVp];
  typename std::conditional<kB, uint16_t, float>::type p[4][16][kPp];
  uint16_t plo[kB ? 4 : 1][16][kPp];         // bf16 residual of P (P = hi + lo)
};

template <class E, int D>
__global__ __launch_bounds__(256) void k_seq_flash(SeqArgs a) {
  constexpr int EPV = E::kEPV, KCH = D * E::kBytes / 64, NCT = D / 16;
  constexpr bool kB = E::kBytes == 2;
  __shared__ FlashSmem<E, D> L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int quad = lane >> 4, col = lane & 15;
  const int tiles = (a.r.N + 15) / 16;
  const int g = blockIdx.x % a.Hkv;
  const int t = (blockIdx.x / a.Hkv) % tiles;
  const int b = blockIdx.x / (a.Hkv * tiles);
  const int n0 = t * 16;
  const int N = a.r.N, S = a.S, G = a.r.G;
  const int nlast = (n0 + 16 < N ? n0 + 16 : N) - 1;
  const int kseen = S - N + nlast + 1;          // keys seen by the tile's last token
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int kbeg = split * a.split_len;
  const int kmax = (kbeg + a.split_len) < kseen ? (kbeg + a.split_len) : kseen;
  const float scale = (float)a.r.scale;
  const char* kbase = (const char*)a.k + ((int64_t)b * a.ks[0] + (int64_t)g * a.ks[2]) * E::kBytes;
  const char* vbase = (const char*)a.v + ((int64_t)b * a.vs[0] + (int64_t)g * a.vs[2]) * E::kBytes;
  const int64_t kstep = a.ks[1] * E::kBytes, vstep = a.vs[1] * E::kBytes;
  const int passes = (G + nwave - 1) / nwave;

  for (int ps = 0; ps < passes; ++ps) {         // uniform over the workgroup (barriers inside)
    const int hw = ps * nwave + wave;
    const bool active = hw < G;
    const int h = g * G + (active ? hw : 0);
    // A operand: the tile's query rows (row = token n0 + col)
    uint4 afr[KCH];
    {
      const int tok = n0 + col;
      if (active && tok < N) {
        const char* qp = (const char*)a.r.q + q_off(a.r.qs, b, tok, h) * E::kBytes;
#pragma unroll
        for (int m = 0; m < KCH; ++m) afr[m] = *(const uint4*)(qp + m * 64 + quad * 16);
      } else {
#pragma unroll
        for (int m = 0; m < KCH; ++m) afr[m] = make_uint4(0, 0, 0, 0);
      }
    }
    float4_t O[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) O[c] = float4_t{0.f, 0.f, 0.f, 0.f};
    float mrow[4], lrow[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) { mrow[v] = -INFINITY; lrow[v] = 0.f; }

    for (int k0 = kbeg; k0 < kmax; k0 += 16) {
      // V tile (16 keys x D) into LDS, transposed: vt[dim][key]
      __syncthreads();
      for (int x = threadIdx.x; x < 16 * (D / EPV); x += blockDim.x) {
        const int key = x / (D / EPV), ch = x % (D / EPV);
        uint4 vv = make_uint4(0, 0, 0, 0);
        if (k0 + key < S) vv = *(const uint4*)(vbase + (int64_t)(k0 + key) * vstep + ch * 16);
        if constexpr (kB) {
          const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            L.vt[ch * 8 + 2 * e][key] = (uint16_t)(w[e] & 0xffffu);
            L.vt[ch * 8 + 2 * e + 1][key] = (uint16_t)(w[e] >> 16);
          }
        } else {
          L.vt[ch * 4 + 0][key] = __uint_as_float(vv.x);
          L.vt[ch * 4 + 1][key] = __uint_as_float(vv.y);
          L.vt[ch * 4 + 2][key] = __uint_as_float(vv.z);
          L.vt[ch * 4 + 3][key] = __uint_as_float(vv.w);
        }
      }
      __syncthreads();
      if (!active) continue;
      // S = Q K^T for 16 tokens x 16 keys
      uint4 bfr[KCH];
      {
        const int key = k0 + col;
        if (key < S) {
          const char* kp = kbase + (int64_t)key * kstep;
#pragma unroll
          for (int m = 0; m < KCH; ++m) bfr[m] = *(const uint4*)(kp + m * 64 + quad * 16);
        } else {
#pragma unroll
          for (int m = 0; m < KCH; ++m) bfr[m] = make_uint4(0, 0, 0, 0);
        }
      }
      const float4_t sacc = tile_dot<E, KCH>(afr, bfr);
      float p4[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = n0 + quad * 4 + v;
        const int vis = S - N + tok + 1;
        const bool ok = tok < N && (k0 + col) < vis;
        const float sv = ok ? sacc[v] * scale : -INFINITY;
        const float mx = group_max<16>(sv);  // the tile row's 16 keys: one DPP row
        const float mn = fmaxf(mrow[v], mx);
        const float alpha = mn == -INFINITY ? 1.f : __expf(mrow[v] - mn);
        const float pv = ok ? __expf(sv - mn) : 0.f;
        const float rs = group_sum<16>(pv);
        lrow[v] = lrow[v] * alpha + rs;
        mrow[v] = mn;
#pragma unroll
        for (int c = 0; c < NCT; ++c) O[c][v] *= alpha;
        p4[v] = pv;
      }
      // P (rows 4*quad+v, key col) -> LDS, read back as the A operand.  For
      // bf16 MFMA, P is split into two bf16 parts (hi + lo) so the product
      // keeps ~16 significant bits of P.
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if constexpr (kB) {
          const uint16_t hi = f32_to_bf16_rne(p4[v]);
          L.p[wave][quad * 4 + v][col] = hi;
          L.plo[wave][quad * 4 + v][col] = f32_to_bf16_rne(p4[v] - __uint_as_float((uint32_t)hi << 16));
        } else {
          L.p[wave][quad * 4 + v][col] = p4[v];
        }
      }
      wave_sync();
      if constexpr (kB) {
        const short4_t pa = __builtin_bit_cast(short4_t, *(const uint2*)&L.p[wave][col][quad * 4]);
        const short4_t pl = __builtin_bit_cast(short4_t, *(const uint2*)&L.plo[wave][col][quad * 4]);
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          const short4_t vb = __builtin_bit_cast(short4_t, *(const uint2*)&L.vt[c * 16 + col][quad * 4]);
          O[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, O[c], 0, 0, 0);
          O[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vb, O[c], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float pa = L.p[wave][col][st * 4 + quad];
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            O[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, L.vt[c * 16 + col][st * 4 + quad], O[c], 0, 0, 0);
        }
      }
      wave_sync();
    }
    if (!active) continue;
    // epilogue: rows 4*quad+v, dims 16c+col
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tok = n0 + quad * 4 + v;
      if (tok >= N) continue;
      const int row = (b * N + tok) * a.r.Hq + h;
      if (a.part) {  // partial (acc, m, l) for k_seq_combine
        float* part = a.part + ((int64_t)row * nsplit + split) * (D + 2);
#pragma unroll
        for (int c = 0; c < NCT; ++c) part[c * 16 + col] = O[c][v];
        if (col == 0) {
          part[D] = lrow[v] > 0.f ? mrow[v] : -INFINITY;
          part[D + 1] = lrow[v];
        }
        continue;
      }
      const bool has = lrow[v] > 0.f;
      const float lse_seq = has ? mrow[v] + logf(lrow[v]) : -INFINITY;
      const float lkg = a.lse_kg[row];
      float lam;
      if (lkg == -INFINITY) lam = 0.f;
      else if (!has) lam = 1.f;
      else lam = 1.f / (1.f + __expf(lse_seq - lkg));
      const float inv = has ? 1.f / lrow[v] : 0.f;
      const float* okg = a.o_kg + (int64_t)row * D;
      const int64_t ob = q_off(a.os, b, tok, h);
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const int dim = c * 16 + col;
        const float o = lam * okg[dim] + (1.f - lam) * (O[c][v] * inv);
        if (a.out_dtype == kDtypeBF16) ((uint16_t*)a.out)[ob + dim] = f32_to_bf16_rne(o);
        else ((float*)a.out)[ob + dim] = o;
      }
      if (a.lse_seq_out && col == 0) a.lse_seq_out[row] = lse_seq;
    }
  }
}

// Log-sum-exp combine of the key splits of one row (one wave per row), then
// the λ merge with the KG half.
template <class E, int D>
__global__ __launch_bounds__(256) void k_seq_combine(SeqArgs a, int nsplit) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int row = blockIdx.x * nwave + wave;
  if (row >= a.r.R) return;
  const int h = row % a.r.Hq;
  const int bn = row / a.r.Hq;
  const int n = bn % a.r.N, b = bn / a.r.N;
  const float* part = a.part + (int64_t)row * nsplit * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part[s * (D + 2) + D]);
  float l = 0.f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float* ps = part + s * (D + 2);
      const float ms = ps[D];
      if (ms == -INFINITY) continue;
      const float w = __expf(ms - M);
      l = fmaf(w, ps[D + 1], l);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, ps[lane * DPL + e], acc[e]);
    }
  }
  const bool has = M != -INFINITY;
  float oseq[DPL];
  const float inv_l = has ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) oseq[e] = acc[e] * inv_l;
  merge_store<E, D>(a, row, b, n, h, has ? M + logf(l) : -INFINITY, has, oseq, lane);
}

// Prefill, bf16: the matrix-core flash core with a causal mask.  A workgroup
// of two waves takes 64 rows of one (b, KV head) -- row u is token u / G,
// query head g*G + u % G -- and one key range of its causal span.  Token n
// sees positions 0 .. S - N + n.  With one key range the epilogue merges with
// the KG half and stores the output; otherwise it writes the (o, m, l)
// partial that k_seq_combine merges.
constexpr int kSeqRows = 64;
constexpr int64_t kSeqMfmaTarget = 512;  // workgroups to aim for before splitting keys

template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2)))
void k_seq_mfma(SeqArgs a, int tiles) {
  using namespace flash;
  __shared__ __attribute__((aligned(16))) uint32_t lds[2 * Lds<D>::kBufDw];
  const int nsplit = a.part ? a.nsplit : 1;
  int bid = blockIdx.x;
  const int split = bid % nsplit;
  bid /= nsplit;
  const int tile = bid % tiles;
  bid /= tiles;
  const int g = bid % a.Hkv, b = bid / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int G = a.r.G, NG = a.r.N * G;
  const int u = tile * kSeqRows + wave * 32 + col;
  const bool valid = u < NG;
  const int n = valid ? u / G : 0, h = g * G + (valid ? u % G : 0);
  const int off = a.S - a.r.N;                       // token n sees positions 0 .. off + n
  const int n_first = (tile * kSeqRows) / G;
  const int n_last = min(a.r.N - 1, (tile * kSeqRows + kSeqRows - 1) / G);
  const int64_t key_lo = (int64_t)split * a.split_len;
  const int span = off + n_last + 1;                 // keys any row of the tile sees
  const int nkeys = (int)max<int64_t>(0, min<int64_t>(span, key_lo + a.split_len) - key_lo);
  const int lim = valid ? (int)max<int64_t>(0, min<int64_t>(nkeys, off + n + 1 - key_lo)) : nkeys;
  const int lim_min = (int)max<int64_t>(0, min<int64_t>(nkeys, off + n_first + 1 - key_lo));
  u32x4 qop[D / 16];
  load_query<D>(valid ? (const uint16_t*)a.r.q + q_off(a.r.qs, b, n, h) : nullptr, half, qop);
  const uint32_t krs = (uint32_t)(a.ks[1] * 2), vrs = (uint32_t)(a.vs[1] * 2);
  const char* kbase = (const char*)a.k + ((int64_t)b * a.ks[0] + (int64_t)g * a.ks[2]) * 2 + key_lo * krs;
  const char* vbase = (const char*)a.v + ((int64_t)b * a.vs[0] + (int64_t)g * a.vs[2]) * 2 + key_lo * vrs;
  State<D> S;
  run<D, 128, true>(S, qop, kbase, krs, vbase, vrs, nkeys, lim, lim_min, (float)a.r.scale * kLog2e, lds);
  if (!valid) return;
  const int64_t row = ((int64_t)b * a.r.N + n) * a.r.Hq + h;
  constexpr float kLn2 = 0.6931471805599453f;
  const bool has = S.l > 0.f;
  if (a.part) {  // partial (o, m, l) for k_seq_combine, m in natural-log units
    float* part = a.part + (row * nsplit + split) * (D + 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store4u(part + dt * 32 + 8 * q4 + 4 * half, S.acc[dt][4 * q4], S.acc[dt][4 * q4 + 1],
                S.acc[dt][4 * q4 + 2], S.acc[dt][4 * q4 + 3]);
    if (half == 0) {
      part[D] = has ? S.m * kLn2 : -INFINITY;
      part[D + 1] = S.l;
    }
    return;
  }
  const float lse_seq = has ? (S.m + log2f(S.l)) * kLn2 : -INFINITY;
  const float lkg = a.lse_kg[row];
  float lam;
  if (lkg == -INFINITY) lam = 0.f;
  else if (!has) lam = 1.f;
  else lam = 1.f / (1.f + __expf(lse_seq - lkg));
  const float inv = has ? 1.f / S.l : 0.f;
  const float* okg = a.o_kg + row * D;
  const int64_t ob = q_off(a.os, b, n, h);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = dt * 32 + 8 * q4 + 4 * half;
      const float4 kg = *(const float4*)(okg + d0);
      const float o[4] = {lam * kg.x + (1.f - lam) * (S.acc[dt][4 * q4] * inv),
                          lam * kg.y + (1.f - lam) * (S.acc[dt][4 * q4 + 1] * inv),
                          lam * kg.z + (1.f - lam) * (S.acc[dt][4 * q4 + 2] * inv),
                          lam * kg.w + (1.f - lam) * (S.acc[dt][4 * q4 + 3] * inv)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (a.out_dtype == kDtypeBF16) ((uint16_t*)a.out)[ob + d0 + e] = f32_to_bf16_rne(o[e]);
        else ((float*)a.out)[ob + d0 + e] = o[e];
      }
    }
  if (a.lse_seq_out && half == 0) a.lse_seq_out[row] = lse_seq;
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

static bool seq_uses_mfma(int N, int dtype) { return N >= 16 && dtype == kDtypeBF16; }

static int seq_mfma_tiles(int N, int G) { return (N * G + kSeqRows - 1) / kSeqRows; }

int seq_splits(int B, int N, int Hkv, int G, int S, int dtype) {
  if (seq_uses_mfma(N, dtype)) {
    // 64-row tiles of one (b, KV head); split the keys only while there are
    // fewer tiles than a round of the chip, at least 4 blocks a range
    const int64_t items = (int64_t)B * Hkv * seq_mfma_tiles(N, G);
    if (items <= 0 || S <= 0) return 1;
    int64_t want = (kSeqMfmaTarget + items - 1) / items;
    const int64_t maxs = (S + 255) / 256;
    if (want > maxs) want = maxs;
    return want < 1 ? 1 : (int)want;
  }
  const int64_t flash = N >= 16;
  // workgroups before splitting: one per (b, n, KV head) for decode, one per
  // (b, 16-token tile, KV head) for the flash prefill
  const int64_t items = flash ? (int64_t)B * ((N + 15) / 16) * Hkv : (int64_t)B * N * Hkv;
  if (items <= 0 || S <= 0) return 1;
  // prefill: enough workgroups to fill the chip; decode: about one wave per
  // SIMD, each streaming one long key range.  More decode waves measured
  // slower alone and much slower beside the KG descent, whose kernels then
  // find no registers free on the SIMDs the decode waves hold.
  const int64_t target = flash ? 1024 : 1024;
  const int64_t min_keys = flash ? 64 : 128;    // keys per split at least
  int64_t want = (target + items - 1) / items;
  const int64_t maxs = (S + min_keys - 1) / min_keys;
  if (want > maxs) want = maxs;
  return want < 1 ? 1 : (int)want;
}

int seq_split_len(int S, int nsplit) {
  int len = (S + nsplit - 1) / nsplit;
  return (len + 63) / 64 * 64;
}

hipError_t launch_seq_attend(const SeqArgs& a, hipStream_t s) {
  if (a.r.R <= 0) return hipSuccess;
  const int nsplit = a.part ? a.nsplit : 1;
  if (a.k && seq_uses_mfma(a.r.N, a.dtype)) {
    const int tiles = seq_mfma_tiles(a.r.N, a.r.G);
    const unsigned blocks = (unsigned)(a.r.B * a.Hkv * tiles * nsplit);
    if (a.d == 128) hipLaunchKernelGGL(k_seq_mfma<128>, dim3(blocks), dim3(128), 0, s, a, tiles);
    else hipLaunchKernelGGL(k_seq_mfma<64>, dim3(blocks), dim3(128), 0, s, a, tiles);
    return hipGetLastError();
  }
  if (a.k && a.r.N >= 16) {
    // prefill: MFMA flash attention per (b, KV head, 16-token tile [, key split])
    const unsigned blocks = (unsigned)(a.r.B * ((a.r.N + 15) / 16) * a.Hkv);
    const int waves = a.r.G < 4 ? a.r.G : 4;
    HIKVP_DISPATCH(a.dtype, a.d, k_seq_flash, dim3(blocks, (unsigned)nsplit), dim3(64 * waves), 0, s, a);
    return hipGetLastError();
  }
  // decode: one wave per (b, n, KV head, group of 4 query heads [, key split])
  const unsigned blocks = (unsigned)(a.r.B * a.r.N * a.Hkv * ((a.r.G + 3) / 4));
  if (a.dtype == kDtypeBF16) {
    if (a.d == 128) hipLaunchKernelGGL(k_seq_decode_mfma<128>, dim3(blocks, (unsigned)nsplit), dim3(64), 0, s, a);
    else hipLaunchKernelGGL(k_seq_decode_mfma<64>, dim3(blocks, (unsigned)nsplit), dim3(64), 0, s, a);
    return hipGetLastError();
  }
  HIKVP_DISPATCH(a.dtype, a.d, k_seq_decode, dim3(blocks, (unsigned)nsplit), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_seq_combine(const SeqArgs& a, hipStream_t s) {
  const int nsplit = a.part ? a.nsplit : 1;
  if (a.r.R <= 0 || !a.part) return hipSuccess;  // without partials the attention kernel merged
  const unsigned cblocks = (unsigned)((a.r.R + 3) / 4);
  HIKVP_DISPATCH(a.dtype, a.d, k_seq_combine, dim3(cblocks), dim3(256), 0, s, a, nsplit);
  return hipGetLastError();
}

}  // namespace hikvp
