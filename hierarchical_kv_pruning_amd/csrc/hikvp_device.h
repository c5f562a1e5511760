// hikvp_device.h -- device helpers shared by the gfx950 kernels of
// libatlaskv.so: element unpacking, wave/block reductions, coalesced key-span
// scoring and the exact-boundary Top-K select.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "hikvp_internal.h"

namespace hikvp {

struct BF16 {
  static constexpr int kBytes = 2;
  static constexpr int kEPV = 8;  // elements per 16-byte vector
};
struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kEPV = 4;
};

template <class E>
__device__ inline void unpack(const uint4& v, float* f);
template <>
__device__ inline void unpack<BF16>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xffff0000u);
}
template <>
__device__ inline void unpack<F32>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

template <class E>
__device__ inline float load_f32(const void* base, int64_t i);
template <>
__device__ inline float load_f32<BF16>(const void* base, int64_t i) {
  return __uint_as_float(((uint32_t)((const uint16_t*)base)[i]) << 16);
}
template <>
__device__ inline float load_f32<F32>(const void* base, int64_t i) {
  return ((const float*)base)[i];
}

// DPL = D/64 consecutive elements owned by one lane (value rows, outputs)
template <class E, int DPL>
__device__ inline void load_lane(const void* row, int lane, float* f) {
  if constexpr (DPL == 2 && E::kBytes == 2) {
    const uint32_t u = ((const uint32_t*)row)[lane];
    f[0] = __uint_as_float(u << 16);
    f[1] = __uint_as_float(u & 0xffff0000u);
  } else if constexpr (DPL == 2 && E::kBytes == 4) {
    const float2 v = ((const float2*)row)[lane];
    f[0] = v.x;
    f[1] = v.y;
  } else {
#pragma unroll
    for (int e = 0; e < DPL; ++e) f[e] = load_f32<E>(row, (int64_t)lane * DPL + e);
  }
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// LDS visibility within one wave (rows handled by separate waves never meet).
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Barrier of the NT threads that cooperate on one row.
template <int NT>
__device__ inline void group_sync() {
  if constexpr (NT == 64) wave_sync();
  else __syncthreads();
}

// ---------------------------------------------------------------------------
// Cross-lane reductions and scans on DPP (data-parallel primitives: a VALU
// operand read from another lane of the same 16-lane row, a few cycles) and
// v_readlane, instead of LDS-crossbar shuffles (~100+ cycles each).
// Control words: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_shr:n =
// 0x110+n, row_mirror = 0x140, row_half_mirror = 0x141, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143.
// ---------------------------------------------------------------------------
template <int CTRL, int ROWS = 0xf, int BANKS = 0xf, bool ZERO = true>
__device__ inline int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, BANKS, ZERO);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Inclusive prefix sum over the wave's 64 lanes.
__device__ inline int wave_incl_sum(int x) {
  x += dpp_i<0x111>(0, x);
  x += dpp_i<0x112>(0, x);
  x += dpp_i<0x114>(0, x);
  x += dpp_i<0x118>(0, x);
  x += dpp_i<0x142, 0xa, 0xf, false>(0, x);  // rows 1, 3 add lane 15 of the row before
  x += dpp_i<0x143, 0xc, 0xf, false>(0, x);  // rows 2, 3 add lane 31
  return x;
}
__device__ inline int wave_sum_i(int x) { return __builtin_amdgcn_readlane(wave_incl_sum(x), 63); }

// Reduction within aligned groups of L lanes (L = 2..16): after the quad,
// half-row and row steps every lane of the group holds the result.
template <int L, class T, class Op>
__device__ inline T group_reduce16(T v, Op op) {
  if constexpr (L >= 2) v = op(v, dpp_f<0xB1>(v));
  if constexpr (L >= 4) v = op(v, dpp_f<0x4E>(v));
  if constexpr (L >= 8) v = op(v, dpp_f<0x141>(v));
  if constexpr (L >= 16) v = op(v, dpp_f<0x140>(v));
  return v;
}
struct AddF { __device__ float operator()(float a, float b) const { return a + b; } };
struct MaxF { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// Sum / max within aligned groups of L lanes (L = 1..64), every lane of the
// group getting the result.
template <int L>
__device__ inline float group_sum(float v) {
  v = group_reduce16<(L < 16 ? L : 16)>(v, AddF{});
  if constexpr (L >= 32) v += __shfl_xor(v, 16);
  if constexpr (L >= 64) v += __shfl_xor(v, 32);
  return v;
}
template <int L>
__device__ inline float group_max(float v) {
  v = group_reduce16<(L < 16 ? L : 16)>(v, MaxF{});
  if constexpr (L >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (L >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Whole-wave sum / max, uniform result (row results combined through
// v_readlane in a fixed order).
__device__ inline float wave_sum(float v) {
  v = group_reduce16<16>(v, AddF{});
  return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
}
__device__ inline float wave_max(float v) {
  v = group_reduce16<16>(v, MaxF{});
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48))));
}
__device__ inline uint32_t wave_max_u(uint32_t x) {
  x = max(x, (uint32_t)dpp_i<0xB1>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<0x4E>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<0x141>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<0x140>((int)x, (int)x));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48)));
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ inline uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float ord_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ inline int64_t q_off(const int64_t* s, int b, int n, int h) {
  return (int64_t)b * s[0] + (int64_t)n * s[1] + (int64_t)h * s[2];
}

// Rows are processed KV-head-major (all rows reading one head's tree run
// together, so shared child spans meet in the caches): block index ->
// (g, b*N + n, h within the group) -> row = (b*N + n)*Hq + g*G + hw.
__device__ inline int row_of_block(const RowsDev& r, int blk) {
  const int hw = blk % r.G;
  const int t = blk / r.G;
  const int BN = r.B * r.N;
  const int bn = t % BN;
  const int g = t / BN;
  return bn * r.Hq + g * r.G + hw;
}

// Candidate list of a row at one level: the children of its selected
// parents, in the parents' order.  pre[k] = first slot of parent k,
// base[k] = global index of parent k's first child.  One whole wave; the
// span (first0, fan0) of parent `lane` (< 64) is passed in, read early.
__device__ inline int build_candidates(const int32_t* parents, int Kp, const int64_t* off,
                                       int lane, int* pre, int64_t* base, int64_t first0, int fan0) {
  int carry = 0;
  if (lane == 0) pre[0] = 0;
  for (int k0 = 0; k0 < Kp; k0 += 64) {
    const int k = k0 + lane;
    int fan = 0;
    int64_t first = 0;
    if (k0 == 0) {
      first = first0;
      fan = fan0;
      if (k < Kp) base[k] = first;
    } else if (k < Kp) {
      const int p = parents[k];
      if (p >= 0) {
        first = off[p];
        fan = (int)(off[p + 1] - first);
      }
      base[k] = first;
    }
    const int incl = wave_incl_sum(fan);
    if (k < Kp) pre[k + 1] = carry + incl;
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  return carry;
}

// Candidate slot -> global node index.  np < 0: the slot is the node (roots).
// Entries of a select are the slots themselves (in candidate order).
struct SlotMap {
  static constexpr bool kOrdered = true;   // entry order is candidate order
  const int* pre;
  const int64_t* base;
  int np;
  __device__ int64_t operator()(int c) const {
    if (np < 0) return c;
    int lo = 0, hi = np - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return base[lo] + (c - pre[lo]);
  }
  __device__ int slot(int e) const { return e; }
};

// Entries of a compacted candidate list: entry e holds candidate slot slots[e]
// (in no particular order); nodes through the level's slot map.
struct CompactMap {
  static constexpr bool kOrdered = false;
  const int* slots;
  SlotMap inner;
  __device__ int64_t operator()(int e) const { return inner(slots[e]); }
  __device__ int slot(int e) const { return slots[e]; }
};

// Reductions and scans within each 16-lane DPP row (every lane of the row
// gets the result; rows are independent).
__device__ inline uint32_t row_max_u(uint32_t x) {
  x = max(x, (uint32_t)dpp_i<0xB1>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<0x4E>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<0x141>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<0x140>((int)x, (int)x));
  return x;
}
__device__ inline int row_sum_i(int x) {
  x += dpp_i<0xB1>(x, x);
  x += dpp_i<0x4E>(x, x);
  x += dpp_i<0x141>(x, x);
  x += dpp_i<0x140>(x, x);
  return x;
}
// Inclusive prefix sum within each 16-lane row (lane order).
__device__ inline int row_incl_sum(int x) {
  x += dpp_i<0x111>(0, x);
  x += dpp_i<0x112>(0, x);
  x += dpp_i<0x114>(0, x);
  x += dpp_i<0x118>(0, x);
  return x;
}

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles
// ---------------------------------------------------------------------------
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// One 16x16 tile of <q_member, key_child> over the head dim.  Lane l feeds
// tile row/column l%16 with the 16-byte pieces m*64 + (l/16)*16 of its row
// (m < KCH); the same element permutation on both operands leaves the dot
// products unchanged.
// tile_dot_acc adds the tile to acc (key rows scored slice by slice).
template <class E, int KCH>
__device__ inline float4_t tile_dot_acc(const uint4* a, const uint4* b, float4_t acc) {
  if constexpr (E::kBytes == 2) {
#pragma unroll
    for (int m = 0; m < KCH; ++m) {
      short4_t alo, ahi, blo, bhi;
      alo = __builtin_bit_cast(short4_t, make_uint2(a[m].x, a[m].y));
      ahi = __builtin_bit_cast(short4_t, make_uint2(a[m].z, a[m].w));
      blo = __builtin_bit_cast(short4_t, make_uint2(b[m].x, b[m].y));
      bhi = __builtin_bit_cast(short4_t, make_uint2(b[m].z, b[m].w));
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, blo, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, bhi, acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int m = 0; m < KCH; ++m) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[m].x), __uint_as_float(b[m].x), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[m].y), __uint_as_float(b[m].y), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[m].z), __uint_as_float(b[m].z), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[m].w), __uint_as_float(b[m].w), acc, 0, 0, 0);
    }
  }
  return acc;
}
template <class E, int KCH>
__device__ inline float4_t tile_dot(const uint4* a, const uint4* b) {
  return tile_dot_acc<E, KCH>(a, b, float4_t{0.f, 0.f, 0.f, 0.f});
}

// Half-split 16x16 tiles for streaming many rows: tile row (or column) i is
// item i&7 over half i>>3 of the head dimension.  Lane l holds item l&7 and,
// of that item's RB-byte row, the 16-byte pieces m*128 + ((l>>3)&1)*64 +
// (l>>4)*16 for m < RB/128, so one load instruction covers eight whole
// 128-byte lines (a 16-items-per-instruction layout touches sixteen half
// lines and streams about a quarter slower).  Of the 16x16 product only the
// two diagonal 8x8 blocks pair equal halves; their sum is the full dot
// product of each item pair.
__device__ inline int split_off(int lane, int m) {
  return m * 128 + ((lane >> 3) & 1) * 64 + (lane >> 4) * 16;
}

// Four consecutive floats to a 4-byte aligned address (one 16-byte store;
// the target permits dword-aligned vector accesses to global memory).
struct __attribute__((packed, aligned(4))) Float4U { float x, y, z, w; };

// 16-byte load marked non-temporal: data streamed once (leaf keys) then does
// not displace reused lines such as freshly written scores.
typedef unsigned int U32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 load_nt(const void* p) {
  const U32x4 v = __builtin_nontemporal_load((const U32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void store4u(float* p, float x, float y, float z, float w) {
  *(Float4U*)p = Float4U{x, y, z, w};
}
struct __attribute__((packed, aligned(4))) Float2U { float x, y; };
__device__ inline void store2u(float* p, float x, float y) { *(Float2U*)p = Float2U{x, y}; }

// Sum the two half blocks of a half-split tile.  Lanes with (l&15) < 8 and
// l < 32 then hold dot(row item 4*(l>>4)+v, column item l&7) in element v;
// other lanes hold garbage.
__device__ inline float4_t split_combine(float4_t acc, int lane) {
  float4_t s;
#pragma unroll
  for (int v = 0; v < 4; ++v) s[v] = acc[v] + __shfl(acc[v], (lane + 40) & 63);
  return s;
}

// ---------------------------------------------------------------------------
// Exact-boundary Top-K select over n fp32 candidate scores.
//
// The page ranks the candidates of each level by their attention score and
// keeps the K best (速读 › 怎么做的).  Here the ranking key is the fp64 logit
// s = scale * Σ_t q_t k_t, summed
// left to right over the exact products of the stored values, ties to the
// lower node index.  The fp32 scores f differ from the fp64 sums by at most
// E = n_e * 2^-23 * |q| * max|k| (a bound for any summation order with at
// most 2 ulp per operation; n_e = d, or 128 + d/128 for wide rows summed
// slice by slice, err_terms), plus |q_kg - q_exact| * max|k| when the stored
// query is a rounding of an exact one that the ranking is defined by.  With
// T the K-th largest fp32 score (radix select), every candidate with
// f > T + 2E is certainly selected and every candidate with f < T - 2E
// certainly is not; the candidates in between are re-scored in fp64 exactly
// as defined and the remaining places filled by rank.
// ---------------------------------------------------------------------------
constexpr int kBand = 32;        // band members handled per round
constexpr int kLoadBatch = 8;    // score loads kept in flight per lane in the select passes
constexpr int kExactGroup = 4;   // key rows staged per exact re-score group

// LDS work area of one select group (NT threads), carved from dynamic LDS.
struct SelWork {
  int* ctl;                      // [8]: 0 bin, 1 krem, 2 nsure, 3 nband, 4 chunk band count
  int* hist;                     // [NT/64][256] radix histograms (one per wave)
  int* band_slot;                // [kBand]
  int* band_node;                // [kBand]
  double* band_s;                // [kBand]
  int* sel_slot;                 // [K]
  float* sel_logit;              // [K]
  double* best_s;                // [K]
  int* best_node;                // [K]
  double* tmp_s;                 // [K + kBand] wide-band merge scratch
  int* tmp_node;                 // [K + kBand]
  int* tmp_slot;                 // [K + kBand]
  int* tmp_rank;                 // [K + kBand]
  float* kbuf;                   // [kExactGroup][W+1] staged key-row slices (W = slice width; padded)
  float* qrow;                   // [d] KG query row, fp32 (exact copy of the stored values)
  const double* qx;              // [d] exact KG query (global) when the stored one is rounded, else NULL
  int d;                         // query / key width
};

// Key rows of width d are handled in slices of W = SliceW<D> elements: the
// whole row for the head dims 64 and 128 (D = d), 128-element slices for
// wide rows (D = 0: d a multiple of 128, base-embedding trees).
template <int D>
struct SliceW {
  static constexpr int W = D == 0 ? 128 : D;
};
__host__ __device__ inline int slice_width(int d) { return d <= 128 ? d : 128; }

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Bytes of a SelWork for NT threads, Top-K K, row width d.
__host__ __device__ inline size_t selwork_bytes(int NT, int K, int d) {
  size_t b = 0;
  b += align16(8 * 4);
  b += align16((size_t)(NT / 64) * 256 * 4);
  b += align16(kBand * 4) * 2 + align16(kBand * 8);
  b += align16((size_t)K * 4) * 2 + align16((size_t)K * 8) + align16((size_t)K * 4);
  b += align16((size_t)(K + kBand) * 8) + 3 * align16((size_t)(K + kBand) * 4);
  b += align16((size_t)kExactGroup * (slice_width(d) + 1) * 4);
  b += align16((size_t)d * 4);
  return b;
}

__device__ inline SelWork carve_selwork(char*& p, int NT, int K, int d) {
  SelWork w;
  auto take = [&](size_t bytes) { char* q = p; p += align16(bytes); return q; };
  w.ctl = (int*)take(8 * 4);
  w.hist = (int*)take((size_t)(NT / 64) * 256 * 4);
  w.band_slot = (int*)take(kBand * 4);
  w.band_node = (int*)take(kBand * 4);
  w.band_s = (double*)take(kBand * 8);
  w.sel_slot = (int*)take((size_t)K * 4);
  w.sel_logit = (float*)take((size_t)K * 4);
  w.best_s = (double*)take((size_t)K * 8);
  w.best_node = (int*)take((size_t)K * 4);
  w.tmp_s = (double*)take((size_t)(K + kBand) * 8);
  w.tmp_node = (int*)take((size_t)(K + kBand) * 4);
  w.tmp_slot = (int*)take((size_t)(K + kBand) * 4);
  w.tmp_rank = (int*)take((size_t)(K + kBand) * 4);
  w.kbuf = (float*)take((size_t)kExactGroup * (slice_width(d) + 1) * 4);
  w.qrow = (float*)take((size_t)d * 4);
  w.qx = nullptr;
  w.d = d;
  return w;
}

struct KeyRows {                 // keys of one level and KV head
  const char* base;
  int64_t rsb;                   // row stride in bytes
};

// Wide rows (a base-embedding tree): 16 lanes a band member, each summing
// every 16th 16-byte piece of the member's key row against the query in
// fp64, then the 16 partial sums are added; NT / 16 members at a time.
template <class E, int NT>
__device__ inline void exact_rescore_wide(const SelWork& S, int m, const KeyRows& kr, double scale, int tid) {
  constexpr int L = 16, EPV = E::kEPV;
  const int npieces = S.d / EPV;
  for (int b0 = 0; b0 < m; b0 += NT / L) {
    const int mem = b0 + tid / L;
    double acc = 0.0;
    if (mem < m) {
      const char* row = kr.base + (int64_t)S.band_node[mem] * kr.rsb;
      for (int c = tid % L; c < npieces; c += L) {
        const uint4 v = *(const uint4*)(row + (int64_t)c * 16);
        float f[EPV];
        unpack<E>(v, f);
        if (S.qx) {
#pragma unroll
          for (int t = 0; t < EPV; ++t) acc = fma(S.qx[c * EPV + t], (double)f[t], acc);
        } else {
#pragma unroll
          for (int t = 0; t < EPV; ++t) acc = fma((double)S.qrow[c * EPV + t], (double)f[t], acc);
        }
      }
    }
#pragma unroll
    for (int x = 1; x < L; x <<= 1) acc += __shfl_xor(acc, x);
    if (mem < m && tid % L == 0) S.band_s[mem] = scale * acc;
  }
  group_sync<NT>();
}

// fp64 logits of band members [0, m): stage key-row slices of W elements in
// LDS (coalesced), then one thread per member sums the products left to
// right over the whole row (the sum runs on across slices).  The query is the
// stored one (S.qrow) or, when that is a rounding of an exact query, the exact
// one (S.qx): the ranking is then exact with respect to the exact query.
template <class E, int W, int NT>
__device__ inline void exact_rescore(const SelWork& S, int m, const KeyRows& kr, double scale,
                                     int tid) {
  constexpr int EPV = E::kEPV, CPK = W / EPV;
  const int ns = S.d / W;
  for (int b0 = 0; b0 < m; b0 += kExactGroup) {
    const int mm = (m - b0) < kExactGroup ? (m - b0) : kExactGroup;
    double acc = 0.0;
    for (int sl = 0; sl < ns; ++sl) {
      for (int idx = tid; idx < mm * CPK; idx += NT) {
        const int mem = idx / CPK, ch = idx % CPK;
        const int64_t node = S.band_node[b0 + mem];
        const uint4 v = *(const uint4*)(kr.base + node * kr.rsb + ((int64_t)sl * W + ch * EPV) * E::kBytes);
        float f[EPV];
        unpack<E>(v, f);
#pragma unroll
        for (int t = 0; t < EPV; ++t) S.kbuf[mem * (W + 1) + ch * EPV + t] = f[t];
      }
      group_sync<NT>();
      if (tid < mm) {
        const float* kr_row = S.kbuf + tid * (W + 1);
        if (S.qx) {
          const double* q = S.qx + sl * W;
#pragma unroll 4
          for (int t = 0; t < W; ++t) acc += q[t] * (double)kr_row[t];
        } else {
          const float* q = S.qrow + sl * W;
#pragma unroll 4
          for (int t = 0; t < W; ++t) acc += (double)q[t] * (double)kr_row[t];
        }
      }
      group_sync<NT>();
    }
    if (tid < mm) S.band_s[b0 + tid] = scale * acc;
    group_sync<NT>();
  }
}

template <class E, int D, int NT>
__device__ inline void exact_band(const SelWork& S, int m, const KeyRows& kr, double scale, int tid) {
  if constexpr (D == 0) exact_rescore_wide<E, NT>(S, m, kr, scale, tid);
  else exact_rescore<E, D, NT>(S, m, kr, scale, tid);
}

__device__ inline bool ranks_before(double sa, int na, double sb, int nb) {
  return sa > sb || (sa == sb && na < nb);
}

// Sources of a row's candidate scores for select_topk.  each(n, tid, f) calls
// f(i, score_i) for the candidates i owned by thread tid (i = tid + k*NT);
// at(i) reads any candidate (memory; used only by the wide-band sweep).
template <int NT>
struct MemScores {
  const float* p;
  template <class F>
  __device__ inline void each(int n, int tid, F&& f) const {
    for (int i0 = tid; i0 < n; i0 += NT * kLoadBatch) {
      float x[kLoadBatch];
#pragma unroll
      for (int b = 0; b < kLoadBatch; ++b) x[b] = (i0 + b * NT < n) ? p[i0 + b * NT] : 0.f;
#pragma unroll
      for (int b = 0; b < kLoadBatch; ++b)
        if (i0 + b * NT < n) f(i0 + b * NT, x[b]);
    }
  }
  __device__ inline float at(int i) const { return p[i]; }
};

// Up to NT*SPT scores held in registers: loaded once, then every pass of the
// select runs without memory traffic.
template <int NT, int SPT>
struct RegScores {
  float v[SPT];
  const float* p;
  __device__ inline void load(const float* src, int n, int tid) {
    p = src;
#pragma unroll
    for (int k = 0; k < SPT; ++k) v[k] = (k * NT + tid < n) ? src[k * NT + tid] : 0.f;
  }
  template <class F>
  __device__ inline void each(int n, int tid, F&& f) const {
#pragma unroll
    for (int k = 0; k < SPT; ++k)
      if (k * NT + tid < n) f(k * NT + tid, v[k]);
  }
  __device__ inline float at(int i) const { return p[i]; }
};

// Returns the count selected (min(K, n)); out_node/out_logit hold the
// selection sorted by candidate slot.  All NT threads must call it; S.qrow
// must hold the KG query row.
// The KG query row S.qrow is read only by the exact re-score of the band;
// a caller that has not staged it passes a QLoad that stages it (all NT
// threads call it, at most once, before the first re-score).
struct QueryStaged {
  __device__ void operator()() const {}
};

template <class E, int D, int NT, class Src, bool kShortLists = false, class Map = SlotMap,
          class QLoad = QueryStaged>
__device__ int select_topk(const Src& src, int n, int K, double err2, double scale,
                           const Map& map, const KeyRows& kr, const SelWork& S,
                           int* out_node, float* out_logit, int tid, const QLoad& qload = QLoad{}) {
  if (K >= n) {
    src.each(n, tid, [&](int i, float f) {
      int r = i;
      if constexpr (!Map::kOrdered) {  // output in candidate order
        const int si = map.slot(i);
        r = 0;
        for (int j = 0; j < n; ++j) r += map.slot(j) < si ? 1 : 0;
      }
      out_node[r] = (int)map(i);
      out_logit[r] = (float)(scale * (double)f);
    });
    group_sync<NT>();
    return n;
  }
  if (K <= 0) return 0;

  // 1) radix select of the K-th largest fp32 score, 8 bits per pass.
  //    The first digit (top byte of the order key) is nearly constant over a
  //    score distribution, so it is counted without LDS atomics: per-thread
  //    counters over the kWin top bytes just below the maximum, then a group
  //    reduction.  Only if the K-th key lies below that window is the first
  //    digit histogrammed like the others.
  constexpr int kWin = 4;
  constexpr int NH = NT / 64;
  uint32_t prefix = 0, mask = 0;
  int krem = K;
  int first_pass = 0;
  if (tid == 0) { S.ctl[2] = 0; S.ctl[3] = 0; }
  int* myhist = S.hist + (tid >> 6) * 256;
  if constexpr (kShortLists && NT == 64) {
    if (K <= 16 && n <= 256) {
      // short list, small K (a few scores per lane): the K-th largest key by
      // repeated maxima, each round the largest key below the previous
      // round's, its copies counted (ties leave together); no LDS, no
      // barriers.  Sets the full 32-bit prefix: the radix passes are skipped.
      uint32_t prev = 0xffffffffu;  // above every finite score's key
      int cum = 0;
      for (int r = 0; r <= K; ++r) {
        uint32_t lm = 0;
        int lc = 0;
        src.each(n, tid, [&](int, float f) {
          const uint32_t u = ord_key(f);
          lc += (u == prev) ? 1 : 0;
          if (u < prev) lm = max(lm, u);
        });
        lm = wave_max_u(lm);
        if (r > 0) {
          cum += wave_sum_i(lc);   // copies of the previous round's key
          if (cum >= K) break;     // prefix holds the K-th largest key
        }
        prefix = lm;
        prev = lm;
      }
      first_pass = 4;
      wave_sync();  // the classification counters zeroed above, before use
    }
  }
  if (first_pass == 0) {
    uint32_t tmax = 0;
    src.each(n, tid, [&](int, float f) { tmax = max(tmax, ord_key(f) >> 24); });
    tmax = wave_max_u(tmax);
    if (NH > 1) {
      if ((tid & 63) == 0) S.hist[tid >> 6] = (int)tmax;
      group_sync<NT>();
      for (int w = 0; w < NH; ++w) tmax = max(tmax, (uint32_t)S.hist[w]);
      group_sync<NT>();
    }
    int cnt[kWin];
#pragma unroll
    for (int b = 0; b < kWin; ++b) cnt[b] = 0;
    src.each(n, tid, [&](int, float f) {
      const uint32_t d = tmax - (ord_key(f) >> 24);
#pragma unroll
      for (int c = 0; c < kWin; ++c) cnt[c] += (d == (uint32_t)c) ? 1 : 0;
    });
#pragma unroll
    for (int c = 0; c < kWin; ++c) cnt[c] = wave_sum_i(cnt[c]);
    if (NH > 1) {
      if ((tid & 63) < kWin) {
        int mine = 0;
#pragma unroll
        for (int c = 0; c < kWin; ++c) mine = ((tid & 63) == c) ? cnt[c] : mine;
        S.hist[(tid >> 6) * kWin + (tid & 63)] = mine;
      }
      group_sync<NT>();
#pragma unroll
      for (int c = 0; c < kWin; ++c) {
        int v = 0;
        for (int w = 0; w < NH; ++w) v += S.hist[w * kWin + c];
        cnt[c] = v;
      }
      group_sync<NT>();
    }
    int cum = 0, found = -1;
#pragma unroll
    for (int c = 0; c < kWin; ++c) {
      if (found < 0 && cum + cnt[c] >= K) { found = c; krem = K - cum; }
      cum += cnt[c];
    }
    if (found >= 0) {
      prefix = (tmax - (uint32_t)found) << 24;
      mask = 0xff000000u;
      first_pass = 1;
    }
  }
  for (int pass = first_pass; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256 * NH; i += NT) S.hist[i] = 0;
    group_sync<NT>();
    src.each(n, tid, [&](int, float f) {
      const uint32_t u = ord_key(f);
      if ((u & mask) == prefix) atomicAdd(&myhist[(u >> shift) & 255u], 1);
    });
    group_sync<NT>();
    if (tid < 64) {
      const int lane = tid;
      int c0 = 0, c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
      for (int w = 0; w < NH; ++w) {
        const int* hw = S.hist + w * 256 + 4 * lane;
        c0 += hw[0];
        c1 += hw[1];
        c2 += hw[2];
        c3 += hw[3];
      }
      const int tot = c0 + c1 + c2 + c3;
      // inclusive suffix sum over lanes (higher lanes hold higher bins)
      const int incl = wave_incl_sum(tot);
      const int suf = __builtin_amdgcn_readlane(incl, 63) - incl + tot;
      const int above = suf - tot;
      const unsigned long long hit = __ballot(above < krem && krem <= suf);
      const int src_lane = __ffsll((long long)hit) - 1;
      if (lane == src_lane) {
        int cum = above, bin = 4 * lane, newk = krem - cum;
        const int cnt4[4] = {c0, c1, c2, c3};
        for (int q = 3; q >= 0; --q) {
          if (cum + cnt4[q] >= krem) { bin = 4 * lane + q; newk = krem - cum; break; }
          cum += cnt4[q];
        }
        S.ctl[0] = bin;
        S.ctl[1] = newk;
      }
    }
    group_sync<NT>();
    prefix |= (uint32_t)S.ctl[0] << shift;
    mask |= 0xffu << shift;
    krem = S.ctl[1];
  }
  const double T = (double)ord_float(prefix);
  // err2 = 2E; the extra terms are slack for the fp64 threshold arithmetic
  const double W = err2 * 1.01 + 4.0 * fabs(T) * (1.0 / 8388608.0) + 1e-37;

  // 2) classify: above the band (selected) or inside it.  fp32 thresholds,
  //    each widened beyond T +- W by far more than its own rounding, so the
  //    band can only grow (it is resolved exactly below).
  const float hi = (float)(T + W * 1.0001);
  const float lo = (float)(T - W * 1.0001);
  const float fscale = (float)scale;
  src.each(n, tid, [&](int i, float f) {
    if (f > hi) {
      const int p = atomicAdd(&S.ctl[2], 1);
      S.sel_slot[p] = i;
      S.sel_logit[p] = fscale * f;
    } else if (f >= lo) {
      const int p = atomicAdd(&S.ctl[3], 1);
      if (p < kBand) S.band_slot[p] = i;
    }
  });
  group_sync<NT>();
  const int nsure = S.ctl[2], nband = S.ctl[3];
  const int need = K - nsure;

  if (nband == need && nband <= kBand) {
    // 3) the band holds exactly the remaining places: all of it is selected,
    //    whatever the exact order inside it (its fp32 logits are kept)
    for (int i = tid; i < nband; i += NT) {
      const int slot = S.band_slot[i];
      S.sel_slot[nsure + i] = slot;
      S.sel_logit[nsure + i] = (float)(scale * (double)src.at(slot));
    }
    group_sync<NT>();
  } else if (nband <= kBand) {
    // 3) exact logits of the band, then the top `need` by (logit desc, index asc)
    for (int i = tid; i < nband; i += NT) S.band_node[i] = (int)map(S.band_slot[i]);
    qload();
    group_sync<NT>();
    exact_band<E, D, NT>(S, nband, kr, scale, tid);
    for (int i = tid; i < nband; i += NT) {
      const double si = S.band_s[i];
      const int ni = S.band_node[i];
      int rank = 0;
      for (int j = 0; j < nband; ++j) rank += ranks_before(S.band_s[j], S.band_node[j], si, ni) ? 1 : 0;
      if (rank < need) {
        S.sel_slot[nsure + rank] = S.band_slot[i];
        S.sel_logit[nsure + rank] = (float)si;
      }
    }
    group_sync<NT>();
  } else {
    // 3') a wide band (many near-equal scores): sweep the candidates in
    //     chunks, keeping the best `need` exact logits seen so far
    qload();
    int nbest = 0;
    for (int c0 = 0; c0 < n; c0 += kBand) {
      if (tid == 0) S.ctl[4] = 0;
      group_sync<NT>();
      if (tid < kBand) {
        const int i = c0 + tid;
        if (i < n) {
          const float f = src.at(i);
          if (f <= hi && f >= lo) {
            const int p = atomicAdd(&S.ctl[4], 1);
            S.band_slot[p] = i;
            S.band_node[p] = (int)map(i);
          }
        }
      }
      group_sync<NT>();
      const int m = S.ctl[4];
      if (m == 0) continue;
      exact_band<E, D, NT>(S, m, kr, scale, tid);
      const int tot = nbest + m;
      // rank every element of (best so far) + (this chunk's band) in LDS
      for (int e = tid; e < tot; e += NT) {
        double es;
        int en, eslot;
        if (e < nbest) { es = S.best_s[e]; en = S.best_node[e]; eslot = S.sel_slot[nsure + e]; }
        else { es = S.band_s[e - nbest]; en = S.band_node[e - nbest]; eslot = S.band_slot[e - nbest]; }
        int rank = 0;
        for (int x = 0; x < nbest; ++x) rank += ranks_before(S.best_s[x], S.best_node[x], es, en) ? 1 : 0;
        for (int x = 0; x < m; ++x) rank += ranks_before(S.band_s[x], S.band_node[x], es, en) ? 1 : 0;
        S.tmp_s[e] = es;
        S.tmp_node[e] = en;
        S.tmp_slot[e] = eslot;
        S.tmp_rank[e] = rank;
      }
      group_sync<NT>();
      for (int e = tid; e < tot; e += NT) {
        const int r = S.tmp_rank[e];
        if (r < need) {
          S.best_s[r] = S.tmp_s[e];
          S.best_node[r] = S.tmp_node[e];
          S.sel_slot[nsure + r] = S.tmp_slot[e];
        }
      }
      nbest = tot < need ? tot : need;
      group_sync<NT>();
    }
    for (int i = tid; i < need; i += NT) S.sel_logit[nsure + i] = (float)S.best_s[i];
    group_sync<NT>();
  }

  // 4) output sorted by candidate slot (deterministic order)
  for (int i = tid; i < K; i += NT) {
    const int s = map.slot(S.sel_slot[i]);
    int r = 0;
    for (int j = 0; j < K; ++j) r += map.slot(S.sel_slot[j]) < s ? 1 : 0;
    out_node[r] = (int)map(S.sel_slot[i]);
    out_logit[r] = S.sel_logit[i];
  }
  group_sync<NT>();
  return K;
}

// Factor that turns the square root of an fp32 sum of d squares into an
// upper bound of the 2-norm (the sum's rounding is below d * 2^-24 relative).
__host__ __device__ inline float norm_slack(int d) { return 1.0001f + (float)d * 6.0e-8f; }

// Sum over the wave's 64 lanes, fp64.
__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Rounding steps the error bound of a score over d elements counts: d for
// rows of up to 128 (one fp32 accumulation), 128 + d/128 for wide rows, whose
// 128-element slices are accumulated from zero each and then added (the
// slice sums' bounds add up to 128 * 2^-23 |q||k| by Cauchy-Schwarz, the
// d/128 additions another d/128 * 2^-23 |q||k|).
__host__ __device__ inline int err_terms(int d) { return d <= 128 ? d : 128 + d / 128; }

// 2E for a query of norm qnorm against keys of norm <= knorm over d
// elements; qdelta > 0 bounds |q_stored - q_exact| when the stored query is a
// rounding of an exact one, whose score differs by at most qdelta * knorm.
__device__ inline double twice_err_bound(double qnorm, double knorm, int d, double qdelta = 0.0) {
  return 2.0 * qnorm * knorm * (double)err_terms(d) * (1.0 / 8388608.0) + 2.0 * qdelta * knorm * 1.0001;
}

}  // namespace hikvp
