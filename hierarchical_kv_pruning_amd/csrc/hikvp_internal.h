// hikvp_internal.h -- argument blocks shared by the C-ABI layer and the HIP
// kernels of libatlaskv.so.  Internal: not installed, not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hikvp {

constexpr int kMaxK = 256;        // largest Top-K per level
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;

// A three-level key tree in device memory.  Levels: 0 root, 1 mid, 2 leaf.
// Element strides: hs = per KV head, rs = per node (innermost stride 1).
struct TreeDev {
  const void* key[3];         // root_k, mid_k, leaf_k
  const void* leaf_v;
  int64_t hs[4], rs[4];       // [0..2] keys of each level, [3] leaf values
  const int64_t* off[2];      // child offsets of roots (into mids) and mids (into leaves)
  int64_t count[3];           // M_R, M_I, M
  const float* norm;          // [3][Hkv] upper bounds of the key 2-norms per level and head
  int Hkv, d, dtype;
};

// The query rows of one call: row r = (b*N + n)*Hq + h.
struct RowsDev {
  const void* q;              // sequence query [B,N,Hq,d]
  const void* q_kg;           // KG query (== q when not given)
  int64_t qs[3], qks[3];      // strides of b, n, h for q and q_kg
  int B, N, Hq, G;            // G = Hq / Hkv
  int R;                      // B*N*Hq
  double scale;               // logit scale (the fp64 ranking uses exactly this value)
};

struct LevelArgs {
  TreeDev t;
  RowsDev r;
  int level;                  // 0, 1, 2
  const int32_t* parent_sel;  // [R, Kp] selection of level-1 (unused at level 0)
  int Kp;
  int K;                      // this level's K (before clamping)
  float* scores;              // [R, cmax] unscaled fp32 dot products, candidate order
  int64_t cmax;
  int32_t* band_slot;         // [R, cmax] workspace for near-boundary candidates
  double* band_s;             // [R, cmax]
  int32_t* sel;               // [R, K] output selection (-1 padded)
  float* o_kg;                // leaf level: [R, d] softmax-weighted values (fp32)
  float* lse_kg;              // leaf level: [R]
  int stage_lds;              // 1: the Top-K kernel stages a row's scores in LDS
};

struct SeqArgs {
  RowsDev r;
  const void* k;              // [B, S, Hkv, d] (NULL: no sequence half)
  const void* v;
  int64_t ks[3], vs[3];       // strides of b, position, KV head
  int S, Hkv, d, dtype;
  const float* o_kg;          // [R, d]
  const float* lse_kg;        // [R]
  void* out;                  // [B, N, Hq, d]
  int64_t os[3];
  int out_dtype;
  float* lse_seq_out;         // optional [R]
};

struct BuildStats {           // device-side result of tree validation
  int bad;                    // non-zero: malformed offsets
  int pad;
  unsigned long long maxfan[2];
  unsigned int norm_bits[1];  // [3*Hkv] float bits of the norm bounds (flexible)
};

hipError_t launch_validate(const int64_t* off, int64_t count, int64_t children, int which,
                           BuildStats* stats, hipStream_t s);
hipError_t launch_key_norms(const void* key, int dtype, int d, int Hkv, int64_t rows,
                            int64_t hs, int64_t rs, unsigned int* out_bits, hipStream_t s);
hipError_t launch_score_rows(const LevelArgs& a, hipStream_t s);
hipError_t launch_topk(const LevelArgs& a, hipStream_t s);
hipError_t launch_seq_merge(const SeqArgs& a, hipStream_t s);

}  // namespace hikvp
