// hikvp_tree.hip -- tree-view set-up kernels (gfx950): validation of the
// child offsets (方法细节 › KGKVs的层次化聚类 of the AtlasKV digest page gives
// the three levels; the offsets encode parent -> children) and per-level
// key-norm bounds used by the exact-boundary Top-K.
#include <hip/hip_runtime.h>

#include "hikvp_device.h"

namespace hikvp {
namespace {

// Selections computed with a K clamped below the caller's: copied into the
// caller's rows of Kd entries, -1 past the computed ones.
__global__ void k_expand_sel(const int32_t* src, int Ks, int32_t* dst, int Kd, int64_t total) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / Kd;
    const int c = (int)(i % Kd);
    dst[i] = c < Ks ? src[r * Ks + c] : -1;
  }
}

// ---------------------------------------------------------------------------
// tree-view set-up
// ---------------------------------------------------------------------------
__global__ void k_validate(const int64_t* off, int64_t count, int64_t children, int which,
                           BuildStats* st) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i <= count;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t v = off[i];
    bool bad = v < 0 || v > children;
    if (i == 0 && v != 0) bad = true;
    if (i == count && v != children) bad = true;
    if (i < count) {
      const int64_t w = off[i + 1];
      if (w < v) bad = true;
      else atomicMax(&st->maxfan[which], (unsigned long long)(w - v));
    }
    if (bad) atomicOr(&st->bad, 1 << which);
  }
}

// Upper bound of the 2-norms of `rows` key rows of width d per KV head.  The
// rows of width 64 / 128 are read LPK lanes a row; wide rows (D = 0, a
// base-embedding tree) one wave a row.
template <class E, int D>
__global__ __launch_bounds__(256) void k_key_norms(const void* key, int64_t rows, int64_t hs,
                                                   int64_t rs, int d, unsigned int* out_bits) {
  constexpr int EPV = E::kEPV, LPK = D ? D / EPV : 64, KPW = 64 / LPK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int g = blockIdx.y;
  const int j = lane % LPK;
  const char* kb = (const char*)key + (int64_t)g * hs * E::kBytes;
  float mx = 0.f;
  for (int64_t r0 = ((int64_t)blockIdx.x * nwave + wave) * KPW; r0 < rows;
       r0 += (int64_t)gridDim.x * nwave * KPW) {
    const int64_t r = r0 + lane / LPK;
    float s = 0.f;
    if (r < rows) {
      for (int c = j; c < (D ? D : d) / EPV; c += LPK) {
        const uint4 kv = *(const uint4*)(kb + r * rs * E::kBytes + c * 16);
        float kf[EPV];
        unpack<E>(kv, kf);
#pragma unroll
        for (int t = 0; t < EPV; ++t) s = fmaf(kf[t], kf[t], s);
      }
    }
    s = group_sum<LPK>(s);
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (lane == 0) atomicMax(&out_bits[g], __float_as_uint(sqrtf(mx) * norm_slack(D ? D : d)));
}


}  // namespace

#define HIKVP_DISPATCH(dtype, d, KERNEL, ...)                                                        \
  do {                                                                                               \
    const bool wide_ = (d) > 128 && (d) <= kMaxWideD && (d) % 128 == 0;                              \
    if ((dtype) == kDtypeBF16 && (d) == 128) hipLaunchKernelGGL((KERNEL<BF16, 128>), __VA_ARGS__);   \
    else if ((dtype) == kDtypeBF16 && (d) == 64) hipLaunchKernelGGL((KERNEL<BF16, 64>), __VA_ARGS__); \
    else if ((dtype) == kDtypeBF16 && wide_) hipLaunchKernelGGL((KERNEL<BF16, 0>), __VA_ARGS__);     \
    else if ((dtype) == kDtypeF32 && (d) == 128) hipLaunchKernelGGL((KERNEL<F32, 128>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 64) hipLaunchKernelGGL((KERNEL<F32, 64>), __VA_ARGS__);  \
    else if ((dtype) == kDtypeF32 && wide_) hipLaunchKernelGGL((KERNEL<F32, 0>), __VA_ARGS__);       \
    else return hipErrorInvalidValue;                                                                \
  } while (0)

hipError_t launch_validate(const int64_t* off, int64_t count, int64_t children, int which,
                           BuildStats* stats, hipStream_t s) {
  int64_t blocks = (count + 1 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_validate, dim3((unsigned)blocks), dim3(256), 0, s, off, count, children,
                     which, stats);
  return hipGetLastError();
}

hipError_t launch_key_norms(const void* key, int dtype, int d, int Hkv, int64_t rows, int64_t hs,
                            int64_t rs, unsigned int* out_bits, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  int64_t blocks = (rows + 63) / 64;
  if (blocks > 2048) blocks = 2048;
  HIKVP_DISPATCH(dtype, d, k_key_norms, dim3((unsigned)blocks, (unsigned)Hkv), dim3(256), 0, s, key,
                 rows, hs, rs, d, out_bits);
  return hipGetLastError();
}

hipError_t launch_expand_sel(const int32_t* src, int Ks, int32_t* dst, int Kd, int R, hipStream_t s) {
  const int64_t total = (int64_t)R * Kd;
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_expand_sel, dim3((unsigned)blocks), dim3(256), 0, s, src, Ks, dst, Kd, total);
  return hipGetLastError();
}

}  // namespace hikvp
