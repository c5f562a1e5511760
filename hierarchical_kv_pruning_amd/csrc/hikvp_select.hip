// hikvp_select.hip -- the tree-descent kernels of HiKVP attention on gfx950.
//
// Page: "AtlasKV: Augmenting LLMs with Billion-Scale Knowledge Graphs in 20GB
// VRAM" (digest of arXiv 2510.17934), 速读 › 怎么做的: score the query against
// the root keys and keep the Top-K branches, score the children of those
// branches and keep the Top-K, and so on down to the leaves; the selected
// leaves' softmax then forms the KG half of the merged output.
//
//   k_root_mfma zeroes the group and bucket counters of the part's KV heads,
//               then, one wave per 16 rows of one KV head: their scores
//               against all M_R root keys of the head on MFMA 16x16 tiles (a
//               root key is read once per 16 rows).
//   k_root      one wave per row: exact-boundary Top-K_R over the row's root
//               scores; each selection is counted in its (KV head, root)
//               group.  The per-row select kernels keep a few KB of LDS per
//               wave so many rows are in flight per CU.
//   k_root_scan / k_root_fill  lay the groups out in tiles of 64 rows; the
//               fill also records where each selected root's children start
//               in the row's mid candidate list.
//   k_mid_gemm  one workgroup (four waves of 16 rows) per tile: the tile's
//               rows against the root's child span on bf16 (or fp32) MFMA
//               16x16 tiles, the span staged in LDS and read once per tile
//               instead of once per row.  Only the children that can still be
//               among a row's K_I best are written, as (score, child) pairs.
//   k_mid_select   one wave per row: Top-K_I over the row's surviving mid
//               candidates (held in registers, or read from the workspace in
//               every pass when there are more than the register list holds).
//   k_bucket_link  registers each selection in its (KV head, mid) bucket,
//               with where the mid's children start in the row's leaf
//               candidate list.
//   k_leaf_score   one wave per bucket: streams the mid's leaf span once (it is
//               contiguous in the head-major layout) and writes the scores of
//               every member row into that row's candidate slots; then the
//               members past a bucket's fixed slots, from its list.
//   k_leaf_select  one wave (or workgroup) per row: Top-K_L, then the KG softmax over the
//               selected leaves and the weighted sum of their values.
//   k_leaf_score_filtered / k_leaf_select_pairs  the same two steps when mids
//               have at least 4 K_L children: the stream keeps, per member
//               and span, only the leaves that can still be among the row's
//               K_L best, and the select reads just those.
#include <hip/hip_runtime.h>

#include "hikvp_device.h"

namespace hikvp {
namespace {

__device__ inline void decode_row(const RowsDev& r, int row, int& b, int& n, int& h) {
  h = row % r.Hq;
  const int bn = row / r.Hq;
  n = bn % r.N;
  b = bn / r.N;
}

__device__ inline const char* key_base(const TreeDev& t, int lev, int g, int64_t& rsb, int eb) {
  rsb = t.rs[lev] * eb;
  return (const char*)t.key[lev] + (int64_t)g * t.hs[lev] * eb;
}

// ---------------------------------------------------------------------------
// per-row select kernels: one wave per row, LDS work area carved per wave
// ---------------------------------------------------------------------------
constexpr int kStageMax = 0;     // mid/leaf scores are not staged in LDS (registers instead)

struct RowWork {
  SelWork sel;
  int* out_node;                 // [K]
  float* out_logit;              // [K]
  int* pre;                      // [Kp + 1]
  int64_t* base;                 // [Kp]
  float* stage;                  // [stage] staged scores (or unused)
};

__host__ __device__ inline size_t rowwork_bytes(int K, int Kp, int d, int stage, int NT = 64) {
  return selwork_bytes(NT, K, d) + 2 * align16((size_t)K * 4) + align16((size_t)(Kp + 1) * 4) +
         align16((size_t)Kp * 8) + align16((size_t)stage * 4);
}

__device__ inline RowWork carve_rowwork(char* p, int K, int Kp, int d, int stage, int NT = 64) {
  RowWork w;
  w.sel = carve_selwork(p, NT, K, d);
  auto take = [&](size_t bytes) { char* q = p; p += align16(bytes); return q; };
  w.out_node = (int*)take((size_t)K * 4);
  w.out_logit = (float*)take((size_t)K * 4);
  w.pre = (int*)take((size_t)(Kp + 1) * 4);
  w.base = (int64_t*)take((size_t)Kp * 8);
  w.stage = (float*)take((size_t)stage * 4);
  return w;
}

// One MFMA tile of a key-row slice added to acc: the query fragment's
// products (plus its bf16 residual's, LO) accumulated onto acc, or, for the
// slices of a wide row (SLICED), accumulated from zero and then added, which
// keeps the score's error bound at that of 128 + d/128 rounding steps.
template <class E, int KCH, bool LO, bool SLICED>
__device__ inline float4_t slice_tile(const uint4 (&afr)[KCH], const uint4 (&alo)[KCH], const uint4 (&bfr)[KCH],
                                      float4_t acc) {
  if constexpr (SLICED) {
    float4_t t = tile_dot<E, KCH>(afr, bfr);
    if constexpr (LO) t = tile_dot_acc<E, KCH>(alo, bfr, t);
    return acc + t;
  } else {
    acc = tile_dot_acc<E, KCH>(afr, bfr, acc);
    if constexpr (LO) acc = tile_dot_acc<E, KCH>(alo, bfr, acc);
    return acc;
  }
}

// With a bf16 residual row lo beside the rounded query q (|lo| <= 2^-8 |q|
// (1 + 2^-8)^2), the scores sum the products of q and of lo: their error
// bound takes |q| + |lo| <= |q| * kLoNorm, the filter's squared form
// kLoNorm2.
constexpr float kLoNorm = 1.004f;
constexpr float kLoNorm2 = kLoNorm * kLoNorm;

// The row's KG query (exact fp32 copy in LDS) and its 2-norm (rounded up).
template <class E>
__device__ inline double load_query(const RowsDev& r, int b, int n, int h, int d, float* qrow, int lane) {
  const char* qp = (const char*)r.q_kg + q_off(r.qks, b, n, h) * E::kBytes;
  float qq = 0.f;
  for (int t = lane; t < d; t += 64) {
    const float v = load_f32<E>(qp, t);
    qrow[t] = v;
    qq = fmaf(v, v, qq);
  }
  qq = wave_sum(qq);
  return sqrt((double)qq) * norm_slack(d) * (r.q_lo ? kLoNorm : 1.f);
}

// The exact query of a row and the bound on its rounding, when the stored
// KG query is a rounding of one (else NULL and 0).
__device__ inline const double* exact_query(const RowsDev& r, int row, int d) {
  return r.q_exact ? r.q_exact + (int64_t)row * d : nullptr;
}
__device__ inline double query_delta(const RowsDev& r, int row) {
  return r.q_delta ? (double)r.q_delta[row] : 0.0;
}

// The 16-byte pieces m*64 of a query row from qp (NULL: zeros) for an MFMA
// fragment, and the sum of their squares.
template <class E, int KCH>
__device__ inline float load_frag(uint4 (&afr)[KCH], const char* qp) {
  float qq = 0.f;
#pragma unroll
  for (int m = 0; m < KCH; ++m) {
    afr[m] = qp ? *(const uint4*)(qp + m * 64) : make_uint4(0, 0, 0, 0);
    float f[E::kEPV];
    unpack<E>(afr[m], f);
#pragma unroll
    for (int e = 0; e < E::kEPV; ++e) qq = fmaf(f[e], f[e], qq);
  }
  return qq;
}

// The root scores of a row, between k_root_mfma and k_root: the first M_R
// floats of the row's mid-candidate region (c1max >= M_R pairs).
__device__ inline float* root_score_row(const StepArgs& a, int row) {
  return (float*)(a.mid_pairs + (int64_t)row * a.c1max);
}

// The part's group and bucket counters zeroed (its keys of the (head, root)
// sub-counters and (head, mid) buckets, the descriptor counts), by thread
// tid of nthreads: done by k_root_mfma, whose grid every part launches
// first, so that no launch of its own is spent on it.
__device__ inline void clear_counters(const StepArgs& a, int64_t tid, int64_t nthreads) {
  const int64_t MI = a.t.count[1], MR = a.t.count[0];
  const int64_t nk1 = (a.g1 - a.g0) * MI, nk0 = (a.g1 - a.g0) * MR;  // the part's keys
  const int64_t nall = (int64_t)a.t.Hkv * MR;
  if (a.g0 == 0 && a.g1 == a.t.Hkv) {  // all heads: the whole arrays, in order
    for (int64_t i = tid; i < (int64_t)a.bucket_q * 64; i += nthreads) {
      a.bucket_cnt[i] = 0;
      a.bucket_head[i] = -1;
    }
  } else {
    for (int64_t i = tid; i < nk1; i += nthreads) {
      const int64_t bix = bucket_index(a, a.g0 * MI + i);
      a.bucket_cnt[bix] = 0;
      a.bucket_head[bix] = -1;
    }
  }
  for (int64_t i = tid; i < nk0 * kRootSub; i += nthreads)
    a.root_cnt[(i / nk0) * nall + a.g0 * MR + i % nk0] = 0;
  if (tid <= kDescSub) a.bucket_count[tid] = 0;
}

// Root scores on MFMA: one wave per 16 consecutive rows of one KV head and
// kRootChunk of its roots (the rows are the M side, 16 roots the N side of
// each 16x16 tile, the chunk's tiles loaded at once), so a root key is read
// once per 16 rows instead of once per row.  The raw dot products (the
// select applies the scale) land in each row's mid-candidate region (indexed
// by row, like the mid level's candidates, so concurrent descent parts touch
// disjoint rows), which k_root reads before the mid level reuses it.
constexpr int kRootChunk = 64;  // roots per k_root_mfma wave

template <class E, int D, bool LO>
__global__ __launch_bounds__(256) void k_root_mfma(StepArgs a, int tph, int nrc) {
  constexpr int SW = SliceW<D>::W;          // key-row slice width (the whole row unless wide)
  constexpr int KCH = SW * E::kBytes / 64;  // 16-byte pieces per lane per row slice
  constexpr int NU = kRootChunk / 16;       // root tiles in flight
  const int lane = threadIdx.x & 63, quad = lane >> 4, col = lane & 15;
  clear_counters(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x);
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (a.g1 - a.g0) * tph * nrc) return;
  const int rc = w % nrc, t = w / nrc;     // root chunk, row tile
  const int g = a.g0 + t / tph, m0 = (t % tph) * 16;
  const int per_head = a.r.B * a.r.N * a.r.G;  // rows of one KV head
  const int hb = g * per_head;                 // its first block
  const int MR = (int)a.t.count[0];
  const int d = D ? D : a.t.d;
  const int ns = d / SW;                       // slices per row
  const char* qp = nullptr;                    // the lane's row query (+ quad * 16)
  const char* lp = nullptr;                    // its bf16 residual (LO)
  if (m0 + col < per_head) {
    int b, n, h;
    const int row = row_of_block(a.r, hb + m0 + col);
    decode_row(a.r, row, b, n, h);
    qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes + quad * 16;
    if constexpr (LO) lp = (const char*)a.r.q_lo + (int64_t)row * d * E::kBytes + quad * 16;
  }
  uint4 afr[KCH], alo[KCH];
  if constexpr (D != 0) {
    load_frag<E, KCH>(afr, qp);
    if constexpr (LO) load_frag<E, KCH>(alo, lp);
  }
  // this lane's outputs: rows m0 + 4*quad + v, root j0 + 16*u + col
  float* dst[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int mv = m0 + 4 * quad + v;
    dst[v] = mv < per_head ? root_score_row(a, row_of_block(a.r, hb + mv)) : nullptr;
  }
  int64_t rsb;
  const char* kb = key_base(a.t, 0, g, rsb, E::kBytes) + quad * 16;
  const int j1 = min(MR, (rc + 1) * kRootChunk);
  for (int j0 = rc * kRootChunk; j0 < j1; j0 += 16 * NU) {
    float4_t sc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) sc[u] = float4_t{0.f, 0.f, 0.f, 0.f};
    for (int sl = 0; sl < ns; ++sl) {
      const int64_t so = (int64_t)sl * SW * E::kBytes;
      if constexpr (D == 0) {
        load_frag<E, KCH>(afr, qp ? qp + so : nullptr);
        if constexpr (LO) load_frag<E, KCH>(alo, lp ? lp + so : nullptr);
      }
      uint4 bfr[NU][KCH];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const char* kp = kb + (int64_t)min(j0 + 16 * u + col, j1 - 1) * rsb + so;
#pragma unroll
        for (int m = 0; m < KCH; ++m) bfr[u][m] = *(const uint4*)(kp + m * 64);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) sc[u] = slice_tile<E, KCH, LO, D == 0>(afr, alo, bfr[u], sc[u]);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int j = j0 + 16 * u + col;
      if (j < j1)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (dst[v]) dst[v][j] = sc[u][v];
    }
  }
}

template <class E, int D>
__global__ __launch_bounds__(256) void k_root(StepArgs a, size_t wave_bytes, int stage) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int blk = a.blk0 + blockIdx.x * nwave + wave;
  if (blk >= a.blk1) return;  // whole wave; waves never meet at a barrier
  const int MR = (int)a.t.count[0];
  const int K = a.K[0];
  const int d = D ? D : a.t.d;
  RowWork W = carve_rowwork(smem + (size_t)wave * wave_bytes, K, 0, d, stage);
  const int row = row_of_block(a.r, blk);
  W.sel.qx = exact_query(a.r, row, d);
  // the row's scores, from k_root_mfma in the row's mid-candidate region (by
  // row, as the mid level uses it: concurrent parts own disjoint rows),
  // staged in LDS when they fit
  const float* gsc = root_score_row(a, row);
  float* sc = stage ? W.stage : root_score_row(a, row);
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  const int g = h / a.r.G;
  if (stage)
    for (int j = lane; j < MR; j += 64) sc[j] = gsc[j];
  const double qnorm = load_query<E>(a.r, b, n, h, d, W.sel.qrow, lane);
  wave_sync();

  int64_t rsb;
  const char* kb = key_base(a.t, 0, g, rsb, E::kBytes);
  const SlotMap ident{nullptr, nullptr, -1};
  const double err2 = twice_err_bound(qnorm, a.t.norm[g], d, query_delta(a.r, row));
  const int k = select_topk<E, D, 64, MemScores<64>, true>(MemScores<64>{sc}, MR, K, err2, a.r.scale, ident,
                                                           KeyRows{kb, rsb}, W.sel, W.out_node, W.out_logit,
                                                           lane);
  int32_t* out = a.sel[0] + (int64_t)row * K;
  for (int i = lane; i < K; i += 64) out[i] = i < k ? W.out_node[i] : -1;
  // count the row in each selected (head, root) group, on the row's
  // sub-counter (by token): spreading a group over kRootSub counters keeps
  // the atomics on one address few.  Nothing waits for these atomics; the
  // row's rank in the group is taken when k_root_fill places it.
  const int sub = (row / a.r.Hq) % kRootSub;
  for (int i = lane; i < k; i += 64)
    atomicAdd(&a.root_cnt[(int64_t)sub * a.t.Hkv * MR + g * MR + W.out_node[i]], 1);
}

// Exclusive scan of the (head, root) group sizes in tiles of kRootTile rows:
// first tile of each group and the group of each tile.  One workgroup.
__global__ __launch_bounds__(1024) void k_root_scan(StepArgs a) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int MR = (int)a.t.count[0];
  const int nall = a.t.Hkv * MR;                 // sub-counter stride
  const int nkeys = (a.g1 - a.g0) * MR, kb = a.g0 * MR;  // the part's groups
  int carry = 0;
  for (int k0 = 0; k0 < nkeys; k0 += 1024) {
    const int key = kb + k0 + tid;
    int tot = 0;
    if (k0 + tid < nkeys) {
      // sub-counts -> first rank of each sub-counter; all loads are issued
      // before the first store, so they take one memory round trip
      int c[kRootSub];
#pragma unroll
      for (int sb = 0; sb < kRootSub; ++sb) c[sb] = a.root_cnt[(int64_t)sb * nall + key];
#pragma unroll
      for (int sb = 0; sb < kRootSub; ++sb) {
        a.root_cnt[(int64_t)sb * nall + key] = tot;
        tot += c[sb];
      }
      a.root_tot[key] = tot;
    }
    const int pc = (tot + kRootTile - 1) / kRootTile;
    const int incl = wave_incl_sum(pc);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int woff = 0, total = 0;
    for (int w = 0; w < 16; ++w) {
      woff += w < wave ? wsum[w] : 0;
      total += wsum[w];
    }
    const int first = carry + woff + incl - pc;
    if (k0 + tid < nkeys) {
      a.root_tile_off[key] = first;
      for (int i = 0; i < pc; ++i) a.root_tile_key[first + i] = key;
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) *a.root_ntiles = carry;
}

// Place the selections e of lanes `ok` (one wave; s0 the start lane of each
// lane's row, carry the fanouts of the row's selections before this part) in
// their groups' tile rows: the rank comes from the row's sub-counter, which
// k_root_scan turned into the sub-counter's first rank; the first
// mid-candidate slot of the root's children is the sum of the fanouts of the
// row's earlier selected roots (children of the selected roots, in selection
// order, form the row's mid candidate list), an in-wave segmented scan.
__device__ inline int fill_part(const StepArgs& a, bool ok, int64_t e, int row, int s0, int carry, int lane) {
  const int MR = (int)a.t.count[0];
  const int64_t* off0 = a.t.off[0];
  const int node = ok ? a.sel[0][e] : -1;
  const int fan = node >= 0 ? (int)(off0[node + 1] - off0[node]) : 0;
  const int incl = wave_incl_sum(fan);
  const int excl = incl - fan;
  const int base = carry + excl - __shfl(excl, s0);
  if (node >= 0) {
    const int key = ((row % a.r.Hq) / a.r.G) * MR + node;
    const int sub = (row / a.r.Hq) % kRootSub;
    const int rank = atomicAdd(&a.root_cnt[(int64_t)sub * a.t.Hkv * MR + key], 1);
    const int k = (int)(e - (int64_t)row * a.K[0]);   // the root's place in the row's selection
    a.root_members[(int64_t)a.root_tile_off[key] * kRootTile + rank] = make_int2(row, base | (k << 24));
  }
  return carry + __builtin_amdgcn_readlane(incl, 63);
}

// One wave per row-aligned chunk of the root selections.
__global__ void k_root_fill(StepArgs a) {
  const int K0 = a.K[0];
  const int lane = threadIdx.x & 63;
  const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int nwaves = (int)((gridDim.x * blockDim.x) >> 6);
  const int nch = row_chunks(a.blk1 - a.blk0, K0);
  for (int c = wave; c < nch; c += nwaves) {
    if (K0 <= 64) {
      const int rpc = 64 / K0, rr = lane / K0, blk = a.blk0 + c * rpc + rr;
      const bool ok = rr < rpc && blk < a.blk1;
      const int row = ok ? row_of_block(a.r, blk) : 0;
      fill_part(a, ok, (int64_t)row * K0 + lane % K0, row, rr < rpc ? rr * K0 : lane, 0, lane);
    } else {
      const int row = row_of_block(a.r, a.blk0 + c);
      int carry = 0;
      for (int i0 = 0; i0 < K0; i0 += 64)
        carry = fill_part(a, i0 + lane < K0, (int64_t)row * K0 + i0 + lane, row, 0, carry, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// mid level: one workgroup of kMidWaves waves per tile of kRootTile rows of a
// (head, root) group, 16 rows a wave.  The root's children are staged 32 at a
// time in LDS (double-buffered: the next round is loaded while this one is
// scored), so the child span is read from L2 once per 64 rows; each wave
// scores its rows (the M side of 16x16 MFMA tiles) against them (the N side).
//
// Only candidates that can still be among the row's K_I best are written.
// The children are scored in chunks of 128; the 16 lanes holding a row each
// keep the kLaneTop largest scores they have seen, and after each chunk the
// row's threshold T becomes the K_I-th largest score of the union of those
// lane lists (a subset of the scores seen, so T never exceeds the K_I-th
// largest score of the row's whole candidate list).  The chunk keeps its
// children with f >= T - Wf, Wf being twice the band half-width the select
// uses: every candidate the select could take -- above its band or inside it
// -- survives, so the select over the survivors takes exactly what it would
// take over all candidates.  The survivors of the row's k-th selected root go
// to the row's pairs from that root's first candidate slot on, as (score
// bits, child index); mid_meta[row, k] records their count, that slot, the
// root's first child and the row's query-norm bound.
// ---------------------------------------------------------------------------
constexpr int kMidWaves = kRootTile / 16;  // waves per mid workgroup
constexpr int kLaneTop = 2;                // largest scores each lane keeps per row
constexpr int kChunkRounds = 4;            // rounds of 32 children between threshold updates
constexpr int kMidPad = 16;                // LDS row padding (bytes) against bank conflicts

// K-th largest order key of the union of the lane lists top[v][0..kLaneTop)
// of each row v (the 16 lanes of this lane's DPP row hold the row; 0 = empty
// entry), 0 while fewer than K keys exist.  Each entry counts the entries
// greater than it (the lane's others, and every entry of the other 15 lanes
// through 15 DPP row rotations); the K-th largest is the smallest entry with
// fewer than K greater.  Branch-free.
template <int N>
__device__ inline uint32_t row_ror_n(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x120 + N, 0xf, 0xf, false);
}
template <int N>
__device__ inline void rank_step(const uint32_t (&top)[4][kLaneTop], int (&gt)[4][kLaneTop]) {
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int j = 0; j < kLaneTop; ++j) {
      const uint32_t o = row_ror_n<N>(top[v][j]);
#pragma unroll
      for (int i = 0; i < kLaneTop; ++i) gt[v][i] += o > top[v][i] ? 1 : 0;
    }
}
__device__ inline void rows_union_kth(const uint32_t (&top)[4][kLaneTop], int K, uint32_t (&kth)[4]) {
  int gt[4][kLaneTop];
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int i = 0; i < kLaneTop; ++i) {
      int c = 0;
#pragma unroll
      for (int j = 0; j < kLaneTop; ++j) c += top[v][j] > top[v][i] ? 1 : 0;
      gt[v][i] = c;
    }
  rank_step<1>(top, gt);  rank_step<2>(top, gt);  rank_step<3>(top, gt);  rank_step<4>(top, gt);
  rank_step<5>(top, gt);  rank_step<6>(top, gt);  rank_step<7>(top, gt);  rank_step<8>(top, gt);
  rank_step<9>(top, gt);  rank_step<10>(top, gt); rank_step<11>(top, gt); rank_step<12>(top, gt);
  rank_step<13>(top, gt); rank_step<14>(top, gt); rank_step<15>(top, gt);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    uint32_t m = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < kLaneTop; ++i) m = gt[v][i] < K ? min(m, top[v][i]) : m;
    kth[v] = ~row_max_u(~m);               // the row's minimum; 0 if an empty entry ranks below K
  }
}

// A round's children staged by the workgroup: thread tid's 16-byte pieces
// p = tid + i*NT, piece p being part p % (RB/16) of child c0 + p / (RB/16)
// (clamped into the span), loaded to registers then put in LDS rows of LRB.
// (Native 4 x u32 vectors: copies of the HIP vector struct through a private
// array were lowered to memcpy through scratch.)
template <int RB, int NT, int PPT>
__device__ inline void stage_round(U32x4 (&stg)[PPT], const char* kb, int64_t rsb, int c0, int F, int tid) {
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = tid + i * NT, c = p / (RB / 16), o = p % (RB / 16);
    stg[i] = *(const U32x4*)(kb + (int64_t)min(c0 + c, F - 1) * rsb + o * 16);
  }
}
template <int RB, int LRB, int NT, int PPT>
__device__ inline void stage_put(const U32x4 (&stg)[PPT], char* buf, int tid) {
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = tid + i * NT, c = p / (RB / 16), o = p % (RB / 16);
    *(U32x4*)(buf + c * LRB + o * 16) = stg[i];
  }
}

template <class E, int D, bool LO>
__global__ __launch_bounds__(64 * kMidWaves) void k_mid_gemm(StepArgs a) {
  constexpr int SW = SliceW<D>::W;         // key-row slice width (the whole row unless wide)
  constexpr int KCH = SW * E::kBytes / 64; // 16-byte pieces per lane per row slice
  constexpr int RB = SW * E::kBytes;       // bytes per staged key-row slice
  constexpr int LRB = RB + kMidPad;        // LDS bytes per staged child
  constexpr int TU = 2;                    // child tiles per round = consecutive children per lane
  constexpr int RC = 16 * TU;              // children per round
  constexpr int CR = kChunkRounds;         // rounds per chunk
  constexpr int NV = CR * TU;              // keys per lane per row in a chunk
  constexpr int NT = 64 * kMidWaves;
  constexpr int PPT = RC * RB / 16 / NT;   // 16-byte pieces each thread stages per round slice
  static_assert(PPT >= 1 && RC * RB / 16 == PPT * NT, "a round's children split evenly over the threads");
  __shared__ __align__(16) char lds[2][RC * LRB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int quad = lane >> 4, col = lane & 15;
  const int ntiles = *a.root_ntiles;
  const int MR = (int)a.t.count[0];
  const int K0 = a.K[0], K1 = a.K[1];
  const int d = D ? D : a.t.d;
  const int ns = d / SW;                   // slices per key row; a stage is one (round, slice)
  const bool filt = K1 <= kFilterK;
  const int64_t* off0 = a.t.off[0];
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {  // uniform over the workgroup
    const int key = a.root_tile_key[t];
    const int toff = a.root_tile_off[key];
    const int cnt = a.root_tot[key];
    const int g = key / MR, j = key % MR;
    const int64_t first = off0[j];
    const int F = (int)(off0[j + 1] - first);
    const int m0 = (t - toff) * kRootTile + 16 * wave;  // the wave's first member
    const bool active = m0 < cnt;                       // wave-uniform
    const float knorm = a.t.norm[a.t.Hkv + g];
    int64_t rsb;
    const char* kb = key_base(a.t, 1, g, rsb, E::kBytes) + first * rsb;
    if (F > 0) {  // stage 0 staged
      U32x4 stg[PPT];
      stage_round<RB, NT, PPT>(stg, kb, rsb, 0, F, tid);
      stage_put<RB, LRB, NT, PPT>(stg, lds[0], tid);
    }
    // A fragment (members) and this lane's output rows (member 4*quad + v):
    // row, first slot | selection index << 24 (row -1: none)
    uint4 afr[KCH], alo[KCH];
    const char* qp = nullptr;                  // this lane's member query (+ quad * 16), NULL past the members
    const char* lp = nullptr;                  // its bf16 residual (LO)
    int orow[4], obk[4];
    float qnv[4], wf[4];                       // query-norm bound, filter margin
    {
      const int mi = m0 + col;
      const int2 mem = active && mi < cnt ? a.root_members[(int64_t)toff * kRootTile + mi] : make_int2(-1, 0);
      if (mem.x >= 0) {
        int b, n, h;
        decode_row(a.r, mem.x, b, n, h);
        qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes + quad * 16;
        if constexpr (LO) lp = (const char*)a.r.q_lo + (int64_t)mem.x * d * E::kBytes + quad * 16;
      }
      float qq = 0.f;
      for (int sl = 0; sl < ns; ++sl) qq += load_frag<E, KCH>(afr, qp ? qp + (int64_t)sl * RB : nullptr);
      if constexpr (D != 0 && LO) load_frag<E, KCH>(alo, lp);
      qq += __shfl_xor(qq, 16);
      qq += __shfl_xor(qq, 32);                // member col's |q|^2 (every quad)
      if constexpr (LO) qq *= kLoNorm2;        // |q + lo|^2 <= |q|^2 * kLoNorm2
      const float qd = mem.x >= 0 && a.r.q_delta ? a.r.q_delta[mem.x] : 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ms = 4 * quad + v;
        orow[v] = __shfl(mem.x, ms);           // -1 past the members
        obk[v] = __shfl(mem.y, ms);
        // the row's |q| bound (fp32 sum of squares in any order) and twice
        // the select's band half-width for it (its error bound 2E, with the
        // rounding of an exact query if any, and its slack on T, |T| <= |q| max|k|)
        qnv[v] = sqrtf(__shfl(qq, ms)) * norm_slack(d) * 1.001f;
        const float e2 = 2.f * qnv[v] * knorm * (float)err_terms(d) * (1.f / 8388608.f) +
                         2.f * __shfl(qd, ms) * knorm * 1.001f;
        wf[v] = 2.f * (e2 * 1.01f + 4.f * qnv[v] * knorm * (1.f / 8388608.f)) + 1e-30f;
      }
    }
    uint32_t top[4][kLaneTop], kth[4];
    int run[4];                                // survivors written per output row
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      run[v] = 0;
      kth[v] = 0;
#pragma unroll
      for (int i = 0; i < kLaneTop; ++i) top[v][i] = 0;
    }
    __syncthreads();                           // stage 0 staged
    const int nr = (F + RC - 1) / RC;
    // Stages go chunk by chunk, within a chunk slice by slice and within a
    // slice round by round (one slice for rows of up to 128: stage = round),
    // so a wide row's query slice is read once per chunk and slice rather
    // than once per round; the chunk's rounds accumulate side by side.
    int st = 0;                                // the current stage (its buffer: st & 1)
    uint4 anx[KCH], lnx[KCH];                  // wide rows: the next query slice, loaded a slice ahead
    if constexpr (D == 0) {
      if (active) {
        load_frag<E, KCH>(anx, qp);
        if constexpr (LO) load_frag<E, KCH>(lnx, lp);
      }
    }
    for (int cc = 0; cc < nr; cc += CR) {      // chunks of CR rounds
      const int nrc = min(CR, nr - cc);        // rounds in this chunk
      float4_t p[CR][TU];
#pragma unroll
      for (int r = 0; r < CR; ++r)
#pragma unroll
        for (int u = 0; u < TU; ++u) p[r][u] = float4_t{0.f, 0.f, 0.f, 0.f};
      for (int sl = 0; sl < ns; ++sl) {
        if constexpr (D == 0) {
          if (active) {
#pragma unroll
            for (int m = 0; m < KCH; ++m) {
              afr[m] = anx[m];
              if constexpr (LO) alo[m] = lnx[m];
            }
            // the next (chunk, slice)'s query slice, in flight during this slice's rounds
            if (sl + 1 < ns || cc + CR < nr) {
              const int64_t no = (int64_t)(sl + 1 < ns ? sl + 1 : 0) * RB;
              load_frag<E, KCH>(anx, qp ? qp + no : nullptr);
              if constexpr (LO) load_frag<E, KCH>(lnx, lp ? lp + no : nullptr);
            }
          }
        }
#pragma unroll
        for (int r = 0; r < CR; ++r) {
          if (r < nrc) {                       // uniform over the workgroup
            // the next stage: the chunk's next round, else the next slice's
            // first round, else the next chunk's first stage
            int nrr = -1, nsl = 0;
            if (r + 1 < nrc) nrr = cc + r + 1, nsl = sl;
            else if (sl + 1 < ns) nrr = cc, nsl = sl + 1;
            else if (cc + CR < nr) nrr = cc + CR, nsl = 0;
            const bool more = nrr >= 0;
            U32x4 stg[PPT];                    // the next stage, in flight while this one is scored
            if (more) stage_round<RB, NT, PPT>(stg, kb + (int64_t)nsl * RB, rsb, nrr * RC, F, tid);
            if (active) {
              // in tile u, lane column col is child (cc+r)*RC + col*TU + u
              const char* lb = lds[st & 1] + quad * 16;
#pragma unroll
              for (int u = 0; u < TU; ++u) {
                uint4 bfr[KCH];
#pragma unroll
                for (int m = 0; m < KCH; ++m) bfr[m] = *(const uint4*)(lb + (col * TU + u) * LRB + m * 64);
                p[r][u] = slice_tile<E, KCH, LO, D == 0>(afr, alo, bfr, p[r][u]);
              }
            }
            if (more) stage_put<RB, LRB, NT, PPT>(stg, lds[(st + 1) & 1], tid);
            __syncthreads();
            ++st;
          }
        }
      }
      uint32_t x[4][NV];                       // the chunk's keys (0: past the span)
#pragma unroll
      for (int r = 0; r < CR; ++r)
#pragma unroll
        for (int u = 0; u < TU; ++u) {
          const bool valid = r < nrc && (cc + r) * RC + col * TU + u < F;
#pragma unroll
          for (int v = 0; v < 4; ++v) x[v][r * TU + u] = valid ? ord_key(p[r][u][v]) : 0u;
        }
      if (!active) continue;
      uint32_t lo[4] = {0u, 0u, 0u, 0u};       // keep every valid child
      if (filt) {
        // the lane lists take the new keys, then the row threshold moves up
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int q = 0; q < NV; ++q) {
            uint32_t y = x[v][q];
#pragma unroll
            for (int i = 0; i < kLaneTop; ++i) {
              const uint32_t hi = max(y, top[v][i]);
              y = min(y, top[v][i]);
              top[v][i] = hi;
            }
          }
        rows_union_kth(top, K1, kth);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (kth[v]) lo[v] = ord_key(ord_float(kth[v]) - wf[v]);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int nk = 0;
#pragma unroll
        for (int q = 0; q < NV; ++q) nk += (x[v][q] != 0u && x[v][q] >= lo[v]) ? 1 : 0;
        const int incl = row_incl_sum(nk);
        if (orow[v] >= 0) {
          uint2* dp = a.mid_pairs + (int64_t)orow[v] * a.c1max + (obk[v] & 0xffffff);
          int pos = run[v] + incl - nk;
#pragma unroll
          for (int q = 0; q < NV; ++q)
            if (x[v][q] != 0u && x[v][q] >= lo[v])
              dp[pos++] = make_uint2(__float_as_uint(ord_float(x[v][q])),
                                     (uint32_t)(cc * RC + RC * (q / TU) + col * TU + (q % TU)));
        }
        run[v] += __shfl(incl, (lane & 48) | 15);   // the row's total: the DPP row's last lane
      }
    }
    if (active && col == 0)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (orow[v] >= 0)
          a.mid_meta[(int64_t)orow[v] * K0 + (int)((uint32_t)obk[v] >> 24)] =
              make_int4(run[v], obk[v] & 0xffffff, (int)first, (int)__float_as_uint(qnv[v]));
    __syncthreads();                           // the staging buffers are free for the next tile
  }
}

// ---------------------------------------------------------------------------
// mid-level Top-K, one wave per row
// ---------------------------------------------------------------------------
// First parent of a select prologue, read by the caller before anything
// else so that the parents' spans are on their way while the row's scores
// and query arrive: parent gtid (< 64) of the row at level lev - 1, or -1.
__device__ inline int first_parent(const StepArgs& a, int row, int lev, int gtid) {
  const int Kp = a.K[lev - 1];
  return gtid < Kp && gtid < 64 ? a.sel[lev - 1][(int64_t)row * Kp + gtid] : -1;
}

// Prologue of the mid/leaf select kernels (NT threads per row): query row
// in LDS, its norm, the candidate list of level `lev` (children of the row's
// level-1 selection; p0 from first_parent).  Returns the candidate count.
template <class E, int D, int NT>
__device__ inline int select_prologue(const StepArgs& a, const RowWork& W, int row, int lev, int& g,
                                      double& qnorm, int gtid, int p0) {
  constexpr int QPT = D ? (D + NT - 1) / NT : 1;  // query elements per thread held (fixed widths)
  const int d = D ? D : a.t.d;
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  g = h / a.r.G;
  const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes;
  float qv[QPT];
  if constexpr (D != 0) {
#pragma unroll
    for (int j = 0; j < QPT; ++j) qv[j] = gtid + j * NT < D ? load_f32<E>(qp, gtid + j * NT) : 0.f;
  }
  const int64_t* off = a.t.off[lev - 1];
  int64_t first0 = 0;
  int fan0 = 0;
  if (p0 >= 0) {
    first0 = off[p0];
    fan0 = (int)(off[p0 + 1] - first0);
  }
  if constexpr (D != 0) {
#pragma unroll
    for (int j = 0; j < QPT; ++j)
      if (gtid + j * NT < D) W.sel.qrow[gtid + j * NT] = qv[j];
  } else {
    for (int t = gtid; t < d; t += NT) W.sel.qrow[t] = load_f32<E>(qp, t);
  }
  group_sync<NT>();
  const int Kp = a.K[lev - 1];
  if (gtid < 64) {
    float qq = 0.f;
    for (int t = gtid; t < d; t += 64) qq = fmaf(W.sel.qrow[t], W.sel.qrow[t], qq);
    qq = wave_sum(qq);
    if (gtid == 0)
      W.sel.ctl[7] = __float_as_int((float)(sqrt((double)qq) * norm_slack(d) * (a.r.q_lo ? kLoNorm : 1.f)));
    build_candidates(a.sel[lev - 1] + (int64_t)row * Kp, Kp, off, gtid, W.pre, W.base, first0, fan0);
  }
  group_sync<NT>();
  qnorm = (double)__int_as_float(W.sel.ctl[7]);
  return W.pre[Kp];
}

// The row's candidate scores: in registers (SPT per thread, loaded once) or,
// for very long candidate lists, read from the workspace in every pass.
template <int NT, int SPT>
struct RowScores {
  using type = RegScores<NT, SPT>;
  __device__ static inline type make(const float* p, int cap, int tid) {
    type r;
    r.load(p, cap, tid);
    return r;
  }
};
template <int NT>
struct RowScores<NT, 0> {
  using type = MemScores<NT>;
  __device__ static inline type make(const float* p, int, int) { return type{p}; }
};

// Mid-level Top-K over the row's surviving candidates (k_mid_gemm): entry e
// is the e-th survivor in (selected root k, position) order; its candidate
// slot is pre[k] + j and its node base[k] + j, for the child index j stored
// with its score.
struct MidEntries {
  const uint2* pairs;         // the row's mid-candidate region
  const int* cpre;            // [K0 + 1] first entry of each selected root's survivors (LDS)
  const int* pre;             // [K0 + 1] first candidate slot of each selected root (LDS)
  const int64_t* base;        // [K0] first child node of each selected root (LDS)
  int K0;
  __device__ inline int root_of(int e) const {  // the k with cpre[k] <= e < cpre[k + 1]
    int lo = 0, hi = K0 - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cpre[mid] <= e) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  __device__ inline uint2 pair(int e, int& k) const {
    k = root_of(e);
    return pairs[pre[k] + (e - cpre[k])];
  }
};

// Up to 64 * SPT entries loaded once: scores in registers, (k, j) packed in LDS.
template <int SPT>
struct MidRegScores {
  float v[SPT];
  MidEntries m;
  template <class F>
  __device__ inline void each(int n, int tid, F&& f) const {
#pragma unroll
    for (int k = 0; k < SPT; ++k)
      if (k * 64 + tid < n) f(k * 64 + tid, v[k]);
  }
  __device__ inline float at(int e) const {
    int k;
    return __uint_as_float(m.pair(e, k).x);
  }
};
struct MidRegMap {
  static constexpr bool kOrdered = false;
  const int* kj;              // [n] (k << 24) | j per entry (LDS)
  const int* pre;
  const int64_t* base;
  __device__ int64_t operator()(int e) const { return base[(uint32_t)kj[e] >> 24] + (kj[e] & 0xffffff); }
  __device__ int slot(int e) const { return pre[(uint32_t)kj[e] >> 24] + (kj[e] & 0xffffff); }
};

// Longer lists: every pass reads the entries from the workspace.
struct MidMemScores {
  MidEntries m;
  template <class F>
  __device__ inline void each(int n, int tid, F&& f) const {
    for (int e = tid; e < n; e += 64) {
      int k;
      f(e, __uint_as_float(m.pair(e, k).x));
    }
  }
  __device__ inline float at(int e) const {
    int k;
    return __uint_as_float(m.pair(e, k).x);
  }
};
struct MidMemMap {
  static constexpr bool kOrdered = false;
  MidEntries m;
  __device__ int64_t operator()(int e) const {
    int k;
    const uint2 p = m.pair(e, k);
    return m.base[k] + p.y;
  }
  __device__ int slot(int e) const {
    int k;
    const uint2 p = m.pair(e, k);
    return m.pre[k] + (int)p.y;
  }
};

// The entries of a survivor list into registers (scores) and LDS (k, j):
// every entry's search and load first, the LDS stores after them, so the
// loads are in flight together (a store between two entries' loads, which
// might alias the next search's LDS reads, kept one load in flight: 26 of
// the 72 us of the leaf select at 4 096 rows x 1 030 survivors).
template <int SPT>
__device__ inline void load_entries(MidRegScores<SPT>& src, const MidEntries& me, int* kj, int cnt, int lane) {
  uint2 pr[SPT];
  int kk[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int e = i * 64 + lane;
    kk[i] = 0;
    pr[i] = make_uint2(0u, 0u);
    if (e < cnt) pr[i] = me.pair(e, kk[i]);
  }
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int e = i * 64 + lane;
    src.v[i] = 0.f;
    if (e < cnt) {
      src.v[i] = __uint_as_float(pr[i].x);
      kj[e] = (kk[i] << 24) | (int)pr[i].y;
    }
  }
  wave_sync();
}

// LDS of one k_mid_select wave: the select's work area, cpre, (k, j) of the
// register-held entries.
__host__ __device__ inline size_t mid_select_wave_bytes(int K1, int K0, int d, int SPT) {
  return rowwork_bytes(K1, K0, d, 0) + align16((size_t)(K0 + 1) * 4) + align16((size_t)64 * SPT * 4);
}

// Stages the row's KG query in the select's work area (exact fp32 copy), for
// the exact re-score of a band, which needs it (unless it re-scores with the
// exact query).
template <class E>
struct StageQuery {
  const char* qp;
  float* qrow;
  int d;
  int lane;
  __device__ void operator()() const {
    for (int t = lane; t < d; t += 64) qrow[t] = load_f32<E>(qp, t);
    wave_sync();
  }
};

// One wave per row: the row's survivors from mid_meta (no parent or offset
// lookups: the mid tiles recorded each selected root's first slot and first
// child), Top-K_I over them.
template <class E, int D, int SPT>
__device__ inline void mid_select_row(StepArgs a, size_t wave_bytes) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int blk = a.blk0 + blockIdx.x * nwave + wave;
  if (blk >= a.blk1) return;  // whole wave; waves never meet at a barrier
  const int K0 = a.K[0], K1 = a.K[1];
  const int d = D ? D : a.t.d;
  char* p = smem + (size_t)wave * wave_bytes;
  RowWork W = carve_rowwork(p, K1, K0, d, 0);
  p += rowwork_bytes(K1, K0, d, 0);
  int* cpre = (int*)p;
  p += align16((size_t)(K0 + 1) * 4);
  int* kj = (int*)p;
  const int row = row_of_block(a.r, blk);
  W.sel.qx = exact_query(a.r, row, d);
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  const int g = h / a.r.G;
  // survivors, first slot and first child of each selected root
  int carry = 0;
  float qn = 0.f;
  if (lane == 0) cpre[0] = 0;
  for (int k0 = 0; k0 < K0; k0 += 64) {
    const int k = k0 + lane;
    const int4 m = k < K0 ? a.mid_meta[(int64_t)row * K0 + k] : make_int4(0, 0, 0, 0);
    if (k < K0) {
      W.pre[k] = m.y;
      W.base[k] = m.z;
    }
    if (k0 == 0) qn = __int_as_float(__builtin_amdgcn_readlane(m.w, 0));
    const int incl = wave_incl_sum(m.x);
    if (k < K0) cpre[k + 1] = carry + incl;
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  wave_sync();
  const int cnt = carry;
  const MidEntries me{a.mid_pairs + (int64_t)row * a.c1max, cpre, W.pre, W.base, K0};
  int64_t rsb;
  const char* kb = key_base(a.t, 1, g, rsb, E::kBytes);
  const double err2 = twice_err_bound((double)qn, a.t.norm[a.t.Hkv + g], d, query_delta(a.r, row));
  const StageQuery<E> ql{(const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes, W.sel.qrow, d, lane};
  int k1;
  if (cnt <= 64 * SPT) {
    MidRegScores<SPT> src;
    src.m = me;
    load_entries<SPT>(src, me, kj, cnt, lane);
    k1 = select_topk<E, D, 64, MidRegScores<SPT>, true, MidRegMap, StageQuery<E>>(
        src, cnt, K1, err2, a.r.scale, MidRegMap{kj, W.pre, W.base}, KeyRows{kb, rsb}, W.sel, W.out_node,
        W.out_logit, lane, ql);
  } else {
    k1 = select_topk<E, D, 64, MidMemScores, false, MidMemMap, StageQuery<E>>(
        MidMemScores{me}, cnt, K1, err2, a.r.scale, MidMemMap{me}, KeyRows{kb, rsb}, W.sel, W.out_node,
        W.out_logit, lane, ql);
  }
  int32_t* o1 = a.sel[1] + (int64_t)row * K1;
  for (int i = lane; i < K1; i += 64) o1[i] = i < k1 ? W.out_node[i] : -1;
}

// Survivors a lane holds in registers: 4 (256 a row) or 16 (1024).  The
// smaller list keeps less LDS a wave (its (k, j) index), so more rows are in
// flight; rows with more survivors read them from the workspace instead.
template <class E, int D, int SPT>
__global__ __launch_bounds__(256) void k_mid_select(StepArgs a, size_t wave_bytes) {
  mid_select_row<E, D, SPT>(a, wave_bytes);
}

// ---------------------------------------------------------------------------
// leaf scoring, deduplicated: every distinct (KV head, mid) selected by any
// row is one bucket.  The link kernel writes one 16-byte descriptor per bucket
// (key, fanout, element offset of the span) and stores the first
// bslots member rows as (row, first leaf slot) pairs; later members go
// to a linked list, scored at the end of the same kernel.  One wave per bucket
// streams the mid's leaf span (contiguous in the head-major layout) once and
// scores it for every member row, prefetching its next bucket's descriptor.
// Each member's dot products are computed independently, so results do not
// depend on the (atomic) member or bucket order.
// ---------------------------------------------------------------------------
// Register selection e = (row, mid) in its (KV head, mid) bucket, given its
// rank from the bucket's counter (-1: nothing to register): the first
// bslots members in fixed slots (row, first leaf slot), later ones in
// the bucket's list; a new bucket appends its 16-byte descriptor (bucket
// index, fanout, first leaf element) to descriptor sub-list `sub`, one atomic
// per wave.  All lanes of a wave call it.
__device__ inline void register_in_bucket(const StepArgs& a, int64_t e, int row, int sub, int g, int64_t key,
                                          int rank, int64_t f0, int fan, int slot_base, int lane) {
  const uint64_t fresh = __ballot(rank == 0);
  if (fresh) {
    int got = 0;
    const int leader = __builtin_ctzll(fresh);
    if (lane == leader) got = atomicAdd(&a.bucket_count[sub], __popcll(fresh));
    const int64_t base = (int64_t)sub * a.desc_per_sub + __builtin_amdgcn_readlane(got, leader);
    if (rank == 0) {
      const int below = __popcll(fresh & ((1ull << lane) - 1ull));
      const int64_t first = (int64_t)g * a.t.hs[2] + f0 * a.t.rs[2];
      a.bucket_desc[base + below] = make_int4((int)bucket_index(a, key), fan, (int)(uint32_t)first,
                                              (int)(first >> 32));
    }
  }
  if (rank < 0) return;
  const int64_t bix = bucket_index(a, key);
  if (rank < a.bslots) {
    a.bucket_slot[bix * a.bslots + rank] = make_int2(row, slot_base);
  } else {
    a.bucket_next[e] = atomicExch(&a.bucket_head[bix], (int)e);
    if (rank == a.bslots) a.bucket_ovf[atomicAdd(&a.bucket_count[kDescSub], 1)] = (int)key;
  }
}

// Link the selections e of lanes `ok` (one wave; row start lane `s0` of each
// lane's row, `carry` the fanouts of the row's selections before this part):
// the first leaf-candidate slot of selection e is the sum of the fanouts of
// the row's earlier selections (children of the selected mids, in selection
// order, form the row's leaf candidate list), an in-wave segmented scan.
// Returns carry plus this part's fanouts (for parts holding one row).
__device__ inline int link_part(const StepArgs& a, bool ok, int64_t e, int row, int s0, int sub, int carry,
                                int lane) {
  const int64_t* off1 = a.t.off[1];
  const int mid = ok ? a.sel[1][e] : -1;
  const int g = (row % a.r.Hq) / a.r.G;
  const int64_t key = (int64_t)g * a.t.count[1] + (mid >= 0 ? mid : 0);
  const int rank = mid >= 0 ? atomicAdd(&a.bucket_cnt[bucket_index(a, key)], 1) : -1;
  const int64_t f0 = mid >= 0 ? off1[mid] : 0;
  const int fan = mid >= 0 ? (int)(off1[mid + 1] - f0) : 0;
  const int incl = wave_incl_sum(fan);
  const int excl = incl - fan;
  const int base = carry + excl - __shfl(excl, s0);
  if (ok) a.mid_base[e] = base;
  // filtered leaf scoring also needs the mid's place k in the row's selection
  const int tag = a.leaf_nst > 0 ? (int)(e - (int64_t)row * a.K[1]) << 24 : 0;
  register_in_bucket(a, e, row, sub, g, key, rank, f0, fan, base | tag, lane);
  return carry + __builtin_amdgcn_readlane(incl, 63);
}

// One wave per chunk of whole rows' selections: floor(64 / K_I) rows when
// K_I <= 64, else one row in ceil(K_I / 64) parts.  Chunk c appends its new
// descriptors to sub-list c mod kDescSub (one counter for all chunks would
// serialise one atomic per chunk on one address), so a sub-list receives at
// most ceil(chunks / kDescSub) chunks of at most row_chunk_entries(K_I)
// entries each.
__global__ void k_bucket_link(StepArgs a) {
  const int K1 = a.K[1];
  const int lane = threadIdx.x & 63;
  const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int nwaves = (int)((gridDim.x * blockDim.x) >> 6);
  const int nch = row_chunks(a.blk1 - a.blk0, K1);
  for (int c = wave; c < nch; c += nwaves) {
    const int sub = c % kDescSub;
    if (K1 <= 64) {
      const int rpc = 64 / K1, rr = lane / K1, blk = a.blk0 + c * rpc + rr;
      const bool ok = rr < rpc && blk < a.blk1;
      const int row = ok ? row_of_block(a.r, blk) : 0;
      link_part(a, ok, (int64_t)row * K1 + lane % K1, row, rr < rpc ? rr * K1 : lane, sub, 0, lane);
    } else {
      const int row = row_of_block(a.r, a.blk0 + c);
      int carry = 0;
      for (int i0 = 0; i0 < K1; i0 += 64)
        carry = link_part(a, i0 + lane < K1, (int64_t)row * K1 + i0 + lane, row, 0, sub, carry, lane);
    }
  }
}

// One tile of member scores: the query fragment's products, plus those of
// its bf16 residual (LO) on the same keys.
template <class E, int KP, bool LO>
__device__ inline float4_t member_tile(const uint4 (&afr)[KP], const uint4 (&alo)[KP], const uint4 (&bfr)[KP]) {
  float4_t t = tile_dot<E, KP>(afr, bfr);
  if constexpr (LO) t = tile_dot_acc<E, KP>(alo, bfr, t);
  return t;
}

// Scores of one group of up to 8 member rows of a bucket over its leaf span,
// on half-split MFMA tiles: the group is the M side and the span's keys the N
// side.  Lanes g0 .. g0+7 of mem hold the members (row, first leaf slot),
// gcnt of them valid.  A round covers 8*TU keys; in its tile u, item i is key
// t0 + i*TU + u, so every load instruction reads eight whole 128-byte lines
// and each lane ends the round holding TU consecutive scores per member,
// written with one 16-byte store.  Every member's scores go through exactly
// this arithmetic, whichever group or kernel it lands in, so they do not
// depend on the (atomic) order in which members joined the bucket.
template <class E, int D, bool LO>
__device__ inline void score_member_group(const StepArgs& a, const char* kp, int64_t rsb, int F, int2 mem,
                                          int g0, int gcnt, int lane) {
  constexpr int RB = D * E::kBytes;        // bytes per key row
  constexpr int KP = RB / 128;             // 16-byte pieces per lane per tile
  constexpr int TU = 4;                    // tiles per round = consecutive keys per lane
  const int quad = lane >> 4, item = lane & 7;
  const bool owner = lane < 32 && (lane & 15) < 8;   // holds combined scores
  // A fragment: member `item` (and its bf16 residual, LO), zeros past the members
  uint4 afr[KP], alo[KP];
  const int row = __shfl(mem.x, g0 + item);
  if (item < gcnt) {
    int b, n, h;
    decode_row(a.r, row, b, n, h);
    const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes + split_off(lane, 0);
#pragma unroll
    for (int m = 0; m < KP; ++m) afr[m] = *(const uint4*)(qp + m * 128);
    if constexpr (LO) {
      const char* lp = (const char*)a.r.q_lo + (int64_t)row * D * E::kBytes + split_off(lane, 0);
#pragma unroll
      for (int m = 0; m < KP; ++m) alo[m] = *(const uint4*)(lp + m * 128);
    }
  } else {
#pragma unroll
    for (int m = 0; m < KP; ++m) afr[m] = alo[m] = make_uint4(0, 0, 0, 0);
  }
  // owners store members 4*quad + vv, keys t0 + item*TU .. + TU-1
  float* dst[4];
#pragma unroll
  for (int vv = 0; vv < 4; ++vv) {
    const int ms = 4 * (quad & 1) + vv;
    const int srow = __shfl(mem.x, g0 + ms), sbase = __shfl(mem.y, g0 + ms);
    dst[vv] = (owner && ms < gcnt) ? a.leaf_scores + (int64_t)srow * a.c2max + sbase + item * TU : nullptr;
  }
  // Each round issues its loads, then writes the previous round's scores,
  // then waits for the loads; loads are unconditional (keys past the span
  // re-read its last row).  Score stores are predicated per lane: sending the
  // idle lanes to a junk slot instead, so that every round issues the same
  // stores, measured ~2 % slower.
  float4_t prev[TU];
#pragma unroll
  for (int u = 0; u < TU; ++u) prev[u] = float4_t{0.f, 0.f, 0.f, 0.f};
  int pt0 = -1;                        // round held in prev, -1 none
  auto load_round = [&](int t0, uint4 (&bfr)[TU][KP]) {
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const int c = min(t0 + item * TU + u, F - 1);
      const char* p = kp + (int64_t)c * rsb;
#pragma unroll
      for (int m = 0; m < KP; ++m) bfr[u][m] = load_nt(p + m * 128);
    }
  };
  auto store_full = [&]() {            // prev holds a full round (or none)
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      float* d = (pt0 >= 0 && dst[vv]) ? dst[vv] + pt0 : nullptr;
#pragma unroll
      for (int u = 0; u < TU; u += 4)
        if (d) store4u(d + u, prev[u][vv], prev[u + 1][vv], prev[u + 2][vv], prev[u + 3][vv]);
    }
  };
  int t0 = 0;
  for (; t0 + 8 * TU <= F; t0 += 8 * TU) {
    uint4 bfr[TU][KP];
    load_round(t0, bfr);
    store_full();
#pragma unroll
    for (int u = 0; u < TU; ++u) prev[u] = split_combine(member_tile<E, KP, LO>(afr, alo, bfr[u]), lane);
    pt0 = t0;
  }
  if (t0 < F) {  // last, partial round
    uint4 bfr[TU][KP];
    load_round(t0, bfr);
    store_full();
#pragma unroll
    for (int u = 0; u < TU; ++u) prev[u] = split_combine(member_tile<E, KP, LO>(afr, alo, bfr[u]), lane);
    const int c0 = t0 + item * TU;
#pragma unroll
    for (int vv = 0; vv < 4; ++vv)
#pragma unroll
      for (int u = 0; u < TU; ++u)
        if (dst[vv] && c0 + u < F) dst[vv][t0 + u] = prev[u][vv];
  } else {
    store_full();
  }
}

// Filtered scoring (per-head trees, leaf_nst > 0): a group of up to leaf_nst
// members is scored with exactly the arithmetic of score_member_group, but
// the scores go to the wave's LDS stage [leaf_nst][leaf_fpad] instead of the
// workspace.  Then, member by member: T_b, the K_L-th largest score of the
// span cut to the top 16 bits of its order key (two 8-bit radix passes over
// the staged keys; a lower bound of that score), is at most the K_L-th
// largest score of the member's whole leaf candidate list (the span's K_L
// best are candidates of that list), so every candidate the row's select can
// take -- above its band or inside it, i.e. f >= T - W with T >= T_b -- has
// f >= T_b - Wf, Wf >= 2 W being the mid tiles' filter margin; those are
// written as (score bits, index in the span) pairs from the mid's first
// slot on, in span order, and their number to leaf_cnt[row, k].  A span of
// at most K_L leaves keeps every leaf.
template <class E, int D, bool LO>
__device__ inline void score_member_group_filtered(const StepArgs& a, const char* kp, int64_t rsb, int F,
                                                   int2 mem, int g0, int gcnt, int lane, float* stage) {
  int* hist = (int*)(stage + a.leaf_nst * a.leaf_fpad);  // [256] radix histogram of the wave
  constexpr int RB = D * E::kBytes;        // bytes per key row
  constexpr int KP = RB / 128;             // 16-byte pieces per lane per tile
  constexpr int TU = 4;                    // tiles per round = consecutive keys per lane
  const int quad = lane >> 4, item = lane & 7;
  const bool owner = lane < 32 && (lane & 15) < 8;   // holds combined scores
  const int fpad = a.leaf_fpad;
  // A fragment: member `item` (and its bf16 residual, LO), zeros past the
  // members; qq: the sum of squares of this lane's pieces of member item
  uint4 afr[KP], alo[KP];
  const int row = __shfl(mem.x, g0 + item);
  float qq = 0.f;
  if (item < gcnt) {
    int b, n, h;
    decode_row(a.r, row, b, n, h);
    const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes + split_off(lane, 0);
#pragma unroll
    for (int m = 0; m < KP; ++m) {
      afr[m] = *(const uint4*)(qp + m * 128);
      float f[E::kEPV];
      unpack<E>(afr[m], f);
#pragma unroll
      for (int e = 0; e < E::kEPV; ++e) qq = fmaf(f[e], f[e], qq);
    }
    if constexpr (LO) {
      const char* lp = (const char*)a.r.q_lo + (int64_t)row * D * E::kBytes + split_off(lane, 0);
#pragma unroll
      for (int m = 0; m < KP; ++m) alo[m] = *(const uint4*)(lp + m * 128);
    }
  } else {
#pragma unroll
    for (int m = 0; m < KP; ++m) afr[m] = alo[m] = make_uint4(0, 0, 0, 0);
  }
  // the 8 lanes item, item + 8, ..., item + 56 hold member item's pieces
  qq += __shfl_xor(qq, 8);
  qq += __shfl_xor(qq, 16);
  qq += __shfl_xor(qq, 32);
  // owners stage members 4*quad + vv, keys t0 + item*TU .. + TU-1
  float* sdst[4];
#pragma unroll
  for (int vv = 0; vv < 4; ++vv) {
    const int ms = 4 * (quad & 1) + vv;
    sdst[vv] = (owner && ms < gcnt) ? stage + ms * fpad + item * TU : nullptr;
  }
  for (int t0 = 0; t0 < F; t0 += 8 * TU) {
    uint4 bfr[TU][KP];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const char* p = kp + (int64_t)min(t0 + item * TU + u, F - 1) * rsb;
#pragma unroll
      for (int m = 0; m < KP; ++m) bfr[u][m] = load_nt(p + m * 128);
    }
    float4_t sc[TU];
#pragma unroll
    for (int u = 0; u < TU; ++u) sc[u] = split_combine(member_tile<E, KP, LO>(afr, alo, bfr[u]), lane);
    const bool full = t0 + 8 * TU <= F;
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      if (!sdst[vv]) continue;
      if (full) {
        *(float4*)(sdst[vv] + t0) = make_float4(sc[0][vv], sc[1][vv], sc[2][vv], sc[3][vv]);
      } else {
#pragma unroll
        for (int u = 0; u < TU; ++u)
          if (t0 + item * TU + u < F) sdst[vv][t0 + u] = sc[u][vv];
      }
    }
  }
  wave_sync();
  const int K2 = a.K[2], K1 = a.K[1];
  const int nv = (F + 63) >> 6;                      // wave-uniform
  for (int ms = 0; ms < gcnt; ++ms) {                // wave-uniform
    const int srow = __shfl(mem.x, g0 + ms);
    const uint32_t sy = (uint32_t)__shfl(mem.y, g0 + ms);
    const float* sp = stage + ms * fpad;
    // order key of staged score lane + 64 j (0 past the span)
    auto key_at = [&](int j) { return lane + 64 * j < F ? ord_key(sp[lane + 64 * j]) : 0u; };
    uint32_t lo = 0u;                                // keep keys >= lo (0: every leaf)
    if (F > K2) {
      // the K_L-th largest key's top two bytes: two 8-bit radix passes with
      // an LDS histogram (pass 2 over the keys in pass 1's bin)
      uint32_t pre = 0u;
      int krem = K2;
      for (int pass = 0; pass < 2; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t mask = pass ? 0xff000000u : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[lane + 64 * i] = 0;
        wave_sync();
        for (int j = 0; j < nv; ++j) {
          const uint32_t x = key_at(j);
          if (x != 0u && (x & mask) == pre) atomicAdd(&hist[(x >> shift) & 255u], 1);
        }
        wave_sync();
        // lane l holds bins 4l .. 4l+3; the bin where the count from the top reaches krem
        const int c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
        const int tot = c0 + c1 + c2 + c3;
        const int incl = wave_incl_sum(tot);
        const int suf = __builtin_amdgcn_readlane(incl, 63) - incl + tot;
        const int above = suf - tot;
        const uint64_t hit = __ballot(above < krem && krem <= suf);
        const int src = (int)__builtin_ctzll(hit);   // one lane holds the crossing (krem <= the bins' total)
        int bin = 0, nk = 0;
        if (lane == src) {
          int cum = above;
          const int c4[4] = {c0, c1, c2, c3};
          bin = 4 * lane;
          nk = krem - cum;
          for (int q = 3; q >= 0; --q) {
            if (cum + c4[q] >= krem) { bin = 4 * lane + q; nk = krem - cum; break; }
            cum += c4[q];
          }
        }
        pre |= (uint32_t)__builtin_amdgcn_readlane(bin, src) << shift;
        krem = __builtin_amdgcn_readlane(nk, src);
        wave_sync();                                   // the histogram is read before the next pass clears it
      }
      // the select's band for this row, doubled (the mid tiles' margin)
      const int g = (srow % a.r.Hq) / a.r.G;
      const float knorm = a.t.norm[2 * a.t.Hkv + g];
      const float qsq = __shfl(qq, ms) * (LO ? kLoNorm2 : 1.f);
      const float qnv = sqrtf(qsq) * norm_slack(D) * 1.001f;
      const float qd = a.r.q_delta ? a.r.q_delta[srow] : 0.f;
      const float e2 = 2.f * qnv * knorm * (float)err_terms(D) * (1.f / 8388608.f) + 2.f * qd * knorm * 1.001f;
      const float wf = 2.f * (e2 * 1.01f + 4.f * qnv * knorm * (1.f / 8388608.f)) + 1e-30f;
      if (pre >= 0x00800000u) lo = ord_key(ord_float(pre) - wf);  // (finite scores have keys above it)
    }
    uint2* dp = a.leaf_pairs + (int64_t)srow * a.c2max + (sy & 0xffffffu);
    int cnt = 0;
    for (int j = 0; j < nv; ++j) {
      const uint32_t x = key_at(j);
      const bool keep = x != 0u && x >= lo;
      const uint64_t bal = __ballot(keep);
      if (keep) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        dp[cnt + below] = make_uint2(__float_as_uint(ord_float(x)), (uint32_t)(lane + 64 * j));
      }
      cnt += __popcll(bal);
    }
    if (lane == 0) a.leaf_cnt[(int64_t)srow * K1 + (sy >> 24)] = cnt;
  }
  wave_sync();                                       // the stage is free for the next group
}

// Wide key rows (base-embedding trees): the same tiles and item layout over
// 128-element slices of the row, each round's tiles accumulated over the
// slices before the two halves are combined.  Up to NG groups of 8 members
// (members g0 .. g0 + cnt - 1) are scored together: each round's key slices
// are loaded once for all of them, so a bucket's span is read once per 8*NG
// members rather than once per 8 (with base-embedding trees every query head
// selects from the one tree, and a bucket holds ~13 rows when 32 heads x 512
// tokens select 8 of 10 000 mids).
template <class E, bool LO, int NG, int TU>
__device__ inline void score_members_wide(const StepArgs& a, const char* kp, int64_t rsb, int F, int2 mem,
                                          int g0, int cnt, int lane) {
  constexpr int SW = 128;
  constexpr int RB = SW * E::kBytes;       // bytes per key-row slice
  constexpr int KP = RB / 128;             // 16-byte pieces per lane per tile and slice
  // TU: tiles per round = consecutive keys per lane
  const int ns = a.t.d / SW;
  const int quad = lane >> 4, item = lane & 7;
  const bool owner = lane < 32 && (lane & 15) < 8;   // holds combined scores
  const char* qp[NG];                      // group g's member `item`: its query (+ this lane's piece offset)
  const char* lp[NG];                      // its bf16 residual (LO)
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int mi = 8 * g + item;
    const int row = __shfl(mem.x, g0 + mi);
    qp[g] = nullptr;
    lp[g] = nullptr;
    if (mi < cnt) {
      int b, n, h;
      decode_row(a.r, row, b, n, h);
      qp[g] = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes + split_off(lane, 0);
      if constexpr (LO) lp[g] = (const char*)a.r.q_lo + (int64_t)row * a.t.d * E::kBytes + split_off(lane, 0);
    }
  }
  for (int t0 = 0; t0 < F; t0 += 8 * TU) {
    float4_t acc[NG][TU];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int u = 0; u < TU; ++u) acc[g][u] = float4_t{0.f, 0.f, 0.f, 0.f};
    for (int sl = 0; sl < ns; ++sl) {
      const int64_t so = (int64_t)sl * RB;
      uint4 bfr[TU][KP];
#pragma unroll
      for (int u = 0; u < TU; ++u) {
        const char* p = kp + (int64_t)min(t0 + item * TU + u, F - 1) * rsb + so;
#pragma unroll
        for (int m = 0; m < KP; ++m) bfr[u][m] = load_nt(p + m * 128);
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (8 * g < cnt) {                 // uniform over the wave
          uint4 afr[KP], alo[KP];
#pragma unroll
          for (int m = 0; m < KP; ++m) {
            afr[m] = qp[g] ? *(const uint4*)(qp[g] + so + m * 128) : make_uint4(0, 0, 0, 0);
            if constexpr (LO) alo[m] = lp[g] ? *(const uint4*)(lp[g] + so + m * 128) : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < TU; ++u) acc[g][u] = slice_tile<E, KP, LO, true>(afr, alo, bfr[u], acc[g][u]);
        }
      }
    }
    const int c0 = t0 + item * TU;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (8 * g < cnt) {                   // uniform over the wave
        float4_t sc[TU];
#pragma unroll
        for (int u = 0; u < TU; ++u) sc[u] = split_combine(acc[g][u], lane);
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          const int mi = 8 * g + 4 * (quad & 1) + vv;
          const int srow = __shfl(mem.x, g0 + mi), sbase = __shfl(mem.y, g0 + mi);
          if (owner && mi < cnt) {
            float* d = a.leaf_scores + (int64_t)srow * a.c2max + sbase + c0;
#pragma unroll
            for (int u = 0; u < TU; ++u)
              if (c0 + u < F) d[u] = sc[u][vv];
          }
        }
      }
    }
  }
}

template <class E, int D, bool LO>
__device__ inline void score_members(const StepArgs& a, const char* kp, int64_t rsb, int F, int2 mem, int g0,
                                     int gcnt, int lane) {
  if constexpr (D == 0) score_members_wide<E, LO, 1, 4>(a, kp, rsb, F, mem, g0, gcnt, lane);
  else score_member_group<E, D, LO>(a, kp, rsb, F, mem, g0, gcnt, lane);
}

// Members per scoring group, and one group scored: filtered (staged in the
// wave's LDS `stage`) when the call filters leaf candidates, else written
// whole to the workspace.
template <bool FILT>
__device__ inline int group_size(const StepArgs& a) {
  return FILT ? a.leaf_nst : 8;
}
template <class E, int D, bool LO, bool FILT>
__device__ inline void score_group(const StepArgs& a, const char* kp, int64_t rsb, int F, int2 mem, int g0,
                                   int gcnt, int lane, float* stage) {
  if constexpr (FILT && D != 0) score_member_group_filtered<E, D, LO>(a, kp, rsb, F, mem, g0, gcnt, lane, stage);
  else score_members<E, D, LO>(a, kp, rsb, F, mem, g0, gcnt, lane);
}

// Members of buckets with more than bslots rows: wave `wave0` of `nwaves`
// takes every nwaves-th listed bucket, walks its list and scores the members
// a group at a time with the same group arithmetic as the fixed slots.
template <class E, int D, bool LO, bool FILT>
__device__ inline void score_overflow(const StepArgs& a, int wave0, int nwaves, int lane, float* stage) {
  const int nov = a.bucket_count[kDescSub];
  const int K1 = a.K[1];
  const int MI = (int)a.t.count[1];
  const char* kbase = (const char*)a.t.key[2];
  const int64_t rsb = a.t.rs[2] * E::kBytes;
  for (int v = wave0; v < nov; v += nwaves) {
    const int key = a.bucket_ovf[v];
    const int g = key / MI, mid = key % MI;
    const int64_t bix = bucket_index(a, key);
    const int64_t f0 = a.t.off[1][mid];
    const int F = (int)(a.t.off[1][mid + 1] - f0);
    const char* kp = kbase + ((int64_t)g * a.t.hs[2] + f0 * a.t.rs[2]) * E::kBytes + split_off(lane, 0);
    const int gsz = group_size<FILT>(a);
    int e = a.bucket_head[bix];
    while (e != -1) {  // wave-uniform walk: lane i takes the group's i-th entry
      int mine = -1, gcnt = 0;
      for (; gcnt < gsz && e != -1; ++gcnt) {
        if (lane == gcnt) mine = e;
        e = a.bucket_next[e];
      }
      // (row, first slot), with the mid's place in the row's selection when filtered
      const int2 gm = (lane < gcnt) ? make_int2(mine / K1, a.mid_base[mine] | (FILT ? (mine % K1) << 24 : 0))
                                    : make_int2(-1, 0);
      score_group<E, D, LO, FILT>(a, kp, rsb, F, gm, 0, gcnt, lane, stage);
    }
  }
}

// One wave per bucket: its first bslots members (32, or 64 in a folded
// call), 8 at a time (a bucket with more than 8 members makes further passes
// over its span, mostly L2 hits; wide rows take 24 a pass).  Then the
// members past bslots (score_overflow; the lists are complete once the link
// kernel has run): a separate launch for them cost ~5 us a step.
template <class E, int D, bool LO, bool FILT>
__device__ inline void leaf_score_body(const StepArgs& a) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  // this wave's score stage (filtered calls)
  float* stage = (float*)smem + (size_t)wave * (FILT ? a.leaf_nst * a.leaf_fpad + 256 : 0);
  // descriptor v of the concatenated sub-lists: lane s holds sub-list s's
  // count and its inclusive prefix
  const int scnt = a.bucket_count[lane];  // lane < kDescSub = 64
  const int sincl = wave_incl_sum(scnt);
  const int nb = __builtin_amdgcn_readlane(sincl, 63);
  auto desc_at = [&](int v) {
    const int sub = __popcll(__ballot(sincl <= v));
    const int first = __builtin_amdgcn_readlane(sincl - scnt, sub);
    return a.bucket_desc[(int64_t)sub * a.desc_per_sub + (v - first)];
  };
  const char* kbase = (const char*)a.t.key[2];
  const int64_t rsb = a.t.rs[2] * E::kBytes;
  const int stride = gridDim.x * nwave;
  int v = blockIdx.x * nwave + wave;
  int4 cur = v < nb ? desc_at(v) : make_int4(0, 0, 0, 0);
  while (v < nb) {
    const int vn = v + stride;
    const int4 nxt = vn < nb ? desc_at(vn) : make_int4(0, 0, 0, 0);  // prefetch
    const int key = cur.x, F = cur.y;   // key: bucket array index
    const int64_t first = (int64_t)(uint32_t)cur.z | ((int64_t)cur.w << 32);
    const char* kp = (const char*)kbase + first * E::kBytes + split_off(lane, 0);  // + key * rsb
    int cnt = a.bucket_cnt[key];
    cnt = cnt < a.bslots ? cnt : a.bslots;
    const int2 mem = lane < a.bslots ? a.bucket_slot[(int64_t)key * a.bslots + lane] : make_int2(-1, 0);
    if constexpr (D == 0) {
      // three groups (24 members) a pass, four keys a lane a round: at one
      // group a pass the span is read once a group, and fewer keys a round
      // keep too few bytes in flight (measured)
      for (int g0 = 0; g0 < cnt; g0 += 24)
        score_members_wide<E, LO, 3, 4>(a, kp, rsb, F, mem, g0, min(24, cnt - g0), lane);
    } else {
      const int gsz = group_size<FILT>(a);
      for (int g0 = 0; g0 < cnt; g0 += gsz)
        score_group<E, D, LO, FILT>(a, kp, rsb, F, mem, g0, min(gsz, cnt - g0), lane, stage);
    }
    cur = nxt;
    v = vn;
  }
  score_overflow<E, D, LO, FILT>(a, blockIdx.x * nwave + wave, stride, lane, stage);
}
template <class E, int D, bool LO>
__global__ __launch_bounds__(256) void k_leaf_score(StepArgs a) {
  leaf_score_body<E, D, LO, false>(a);
}
// Filtered calls (per-head trees, D = 64 or 128; the wide instances are
// never launched)
template <class E, int D, bool LO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_leaf_score_filtered(StepArgs a) {
  if constexpr (D != 0) leaf_score_body<E, D, LO, true>(a);
}

// ---------------------------------------------------------------------------
// leaf Top-K and the KG softmax over the selected leaves, one wave per row
// ---------------------------------------------------------------------------
// KG half of one row (one wave): softmax over the selected leaves' logits
// (W.out_node / W.out_logit, k2 of them) and the weighted sum of their values
// into o_kg, the log-sum-exp into lse_kg.
template <class E, int D>
__device__ inline void kg_half(const StepArgs& a, const RowWork& W, int row, int g, int k2, const char* kb,
                               int64_t rsb, int lane) {
  constexpr int SW = SliceW<D>::W;  // value-row slice width (the whole row unless wide)
  const int d = D ? D : a.t.d;
  float* okg = a.o_kg + (int64_t)row * d;
  if (k2 == 0) {
    for (int e = lane; e < d; e += 64) okg[e] = 0.f;
    if (lane == 0) a.lse_kg[row] = -INFINITY;
    return;
  }
  if (a.exact_logits && W.sel.qx) {
    // the logits of an exact query: fp64 dot products of it with the
    // selected keys (the scores are those of its rounding).  L lanes a key
    // (as many keys at once as fit the wave), each summing every L-th
    // 16-byte piece of the key row, then the L partial sums are added.
    int p2 = 1;
    while (p2 < k2 && p2 < 64) p2 <<= 1;
    const int L = 64 / p2;
    const int npieces = d / E::kEPV;
    for (int i0 = 0; i0 < k2; i0 += p2) {
      const int i = i0 + lane / L;
      double acc = 0.0;
      if (i < k2) {
        const char* kr = kb + (int64_t)W.out_node[i] * rsb;
        for (int c = lane % L; c < npieces; c += L) {
          const uint4 v = *(const uint4*)(kr + c * 16);
          float f[E::kEPV];
          unpack<E>(v, f);
          const double* q = W.sel.qx + c * E::kEPV;
#pragma unroll
          for (int t = 0; t < E::kEPV; ++t) acc = fma(q[t], (double)f[t], acc);
        }
      }
      for (int m = 1; m < L; m <<= 1) acc += __shfl_xor(acc, m);
      if (i < k2 && lane % L == 0) W.out_logit[i] = (float)(a.r.scale * acc);
    }
    wave_sync();
  }
  float mx = -INFINITY;
  for (int i = lane; i < k2; i += 64) mx = fmaxf(mx, W.out_logit[i]);
  mx = wave_max(mx);
  float sum = 0.f;
  for (int i = lane; i < k2; i += 64) {
    const float p = __expf(W.out_logit[i] - mx);
    W.out_logit[i] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  wave_sync();
  // Value rows are read 16 bytes a lane, LPK lanes a row (slice), so one
  // load instruction covers KPW rows and VU instructions in flight cover the
  // K_L rows of a row in one or two memory round trips; each lane sums its
  // dims over the rows of its lane group, then the KPW groups are added.
  // Wide rows take their 128-element slices one after the other.
  constexpr int EPV = E::kEPV, LPK = SW / EPV, KPW = 64 / LPK;
  constexpr int VU = 8;
  const int sub = lane / LPK, ch = lane % LPK;
  const int64_t vrs = a.t.rs[3] * E::kBytes;
  const float inv = 1.f / sum;
  for (int s0 = 0; s0 < d; s0 += SW) {
    const char* vb = (const char*)a.t.leaf_v + ((int64_t)g * a.t.hs[3] + s0) * E::kBytes + ch * 16;
    float acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
    for (int i0 = 0; i0 < k2; i0 += KPW * VU) {
      uint4 raw[VU];
#pragma unroll
      for (int u = 0; u < VU; ++u) {
        const int i = i0 + u * KPW + sub;
        raw[u] = i < k2 ? *(const uint4*)(vb + (int64_t)W.out_node[i] * vrs) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < VU; ++u) {
        const int i = i0 + u * KPW + sub;
        const float w = i < k2 ? W.out_logit[i] : 0.f;
        float v[EPV];
        unpack<E>(raw[u], v);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] = fmaf(w, v[e], acc[e]);
      }
    }
#pragma unroll
    for (int m = LPK; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] += __shfl_xor(acc[e], m);
    if (sub == 0) {
      float4* dst = (float4*)(okg + s0 + ch * EPV);
#pragma unroll
      for (int e = 0; e < EPV; e += 4)
        dst[e / 4] = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    }
  }
  if (lane == 0) a.lse_kg[row] = mx + logf(sum);
}

template <class E, int D, int NT, int SPT>
__device__ inline void leaf_select_body(const StepArgs& a, size_t group_bytes) {
  extern __shared__ __align__(16) char smem[];
  const int groups = blockDim.x / NT, grp = threadIdx.x / NT, gtid = threadIdx.x % NT;
  const int blk = a.blk0 + blockIdx.x * groups + grp;
  if (blk >= a.blk1) return;
  const int K2 = a.K[2];
  const int d = D ? D : a.t.d;
  RowWork W = carve_rowwork(smem + (size_t)grp * group_bytes, K2, a.K[1], d, 0, NT);
  const int row = row_of_block(a.r, blk);
  W.sel.qx = exact_query(a.r, row, d);
  const int p0 = first_parent(a, row, 2, gtid);
  const auto sc = RowScores<NT, SPT>::make(a.leaf_scores + (int64_t)row * a.c2max, (int)a.c2max, gtid);
  int g;
  double qnorm;
  const int n2 = select_prologue<E, D, NT>(a, W, row, 2, g, qnorm, gtid, p0);
  int64_t rsb;
  const char* kb = key_base(a.t, 2, g, rsb, E::kBytes);
  const double err2 = twice_err_bound(qnorm, a.t.norm[2 * a.t.Hkv + g], d, query_delta(a.r, row));
  const int k2 = select_topk<E, D, NT>(sc, n2, K2, err2, a.r.scale, SlotMap{W.pre, W.base, a.K[1]},
                                       KeyRows{kb, rsb}, W.sel, W.out_node, W.out_logit, gtid);
  int32_t* o2 = a.sel[2] + (int64_t)row * K2;
  for (int i = gtid; i < K2; i += NT) o2[i] = i < k2 ? W.out_node[i] : -1;
  if (gtid >= 64) return;  // the KG half is formed by the group's first wave
  const int lane = gtid;
  kg_half<E, D>(a, W, row, g, k2, kb, rsb, lane);
}

template <class E, int D, int NT, int SPT>
__global__ __launch_bounds__(256) void k_leaf_select(StepArgs a, size_t gb) {
  leaf_select_body<E, D, NT, SPT>(a, gb);
}

// LDS of one k_leaf_select_pairs wave: the select's work area, cpre, (k, j)
// of the register-held survivors.
__host__ __device__ inline size_t leaf_pairs_wave_bytes(int K2, int K1, int d, int SPT) {
  return rowwork_bytes(K2, K1, d, 0) + align16((size_t)(K1 + 1) * 4) + align16((size_t)64 * SPT * 4);
}

// Leaf Top-K over the survivors of the filtered leaf stream, one wave per
// row, then the KG half.  The survivors of the row's k-th selected mid sit
// from its first candidate slot pre[k] on (leaf_cnt of them), so the mid
// select's entry machinery serves: entry e of mid k is slot pre[k] + j and
// node base[k] + j for the span index j stored with its score.
template <class E, int D, int SPT>
__global__ __launch_bounds__(256) void k_leaf_select_pairs(StepArgs a, size_t wave_bytes) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int blk = a.blk0 + blockIdx.x * nwave + wave;
  if (blk >= a.blk1) return;  // whole wave; waves never meet at a barrier
  const int K1 = a.K[1], K2 = a.K[2];
  const int d = D ? D : a.t.d;
  char* p = smem + (size_t)wave * wave_bytes;
  RowWork W = carve_rowwork(p, K2, K1, d, 0);
  p += rowwork_bytes(K2, K1, d, 0);
  int* cpre = (int*)p;
  p += align16((size_t)(K1 + 1) * 4);
  int* kj = (int*)p;
  const int row = row_of_block(a.r, blk);
  W.sel.qx = exact_query(a.r, row, d);
  const int p0 = first_parent(a, row, 2, lane);
  int g;
  double qnorm;
  select_prologue<E, D, 64>(a, W, row, 2, g, qnorm, lane, p0);  // query, its norm, pre[] and base[]
  // survivors of each selected mid (a mid without children has none: its
  // count is never written)
  int carry = 0;
  if (lane == 0) cpre[0] = 0;
  for (int k0 = 0; k0 < K1; k0 += 64) {
    const int k = k0 + lane;
    const int c = (k < K1 && W.pre[k + 1] > W.pre[k]) ? a.leaf_cnt[(int64_t)row * K1 + k] : 0;
    const int incl = wave_incl_sum(c);
    if (k < K1) cpre[k + 1] = carry + incl;
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  wave_sync();
  const int cnt = carry;
  const MidEntries me{a.leaf_pairs + (int64_t)row * a.c2max, cpre, W.pre, W.base, K1};
  int64_t rsb;
  const char* kb = key_base(a.t, 2, g, rsb, E::kBytes);
  const double err2 = twice_err_bound(qnorm, a.t.norm[2 * a.t.Hkv + g], d, query_delta(a.r, row));
  int k2;
  if (cnt <= 64 * SPT) {
    MidRegScores<SPT> src;
    src.m = me;
    load_entries<SPT>(src, me, kj, cnt, lane);
    k2 = select_topk<E, D, 64, MidRegScores<SPT>, false, MidRegMap>(
        src, cnt, K2, err2, a.r.scale, MidRegMap{kj, W.pre, W.base}, KeyRows{kb, rsb}, W.sel, W.out_node,
        W.out_logit, lane);
  } else {
    k2 = select_topk<E, D, 64, MidMemScores, false, MidMemMap>(
        MidMemScores{me}, cnt, K2, err2, a.r.scale, MidMemMap{me}, KeyRows{kb, rsb}, W.sel, W.out_node,
        W.out_logit, lane);
  }
  int32_t* o2 = a.sel[2] + (int64_t)row * K2;
  for (int i = lane; i < K2; i += 64) o2[i] = i < k2 ? W.out_node[i] : -1;
  kg_half<E, D>(a, W, row, g, k2, kb, rsb, lane);
}

}  // namespace

// Width template argument: 64 and 128 as such, 0 for the wide rows of a
// base-embedding tree (a multiple of 128, handled in 128-element slices).
__host__ inline bool wide_width(int d) { return d > 128 && d <= kMaxWideD && d % 128 == 0; }

#define HIKVP_DISPATCH(dtype, d, KERNEL, ...)                                                        \
  do {                                                                                               \
    if ((dtype) == kDtypeBF16 && (d) == 128) hipLaunchKernelGGL((KERNEL<BF16, 128>), __VA_ARGS__);   \
    else if ((dtype) == kDtypeBF16 && (d) == 64) hipLaunchKernelGGL((KERNEL<BF16, 64>), __VA_ARGS__); \
    else if ((dtype) == kDtypeBF16 && wide_width(d)) hipLaunchKernelGGL((KERNEL<BF16, 0>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 128) hipLaunchKernelGGL((KERNEL<F32, 128>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 64) hipLaunchKernelGGL((KERNEL<F32, 64>), __VA_ARGS__);  \
    else if ((dtype) == kDtypeF32 && wide_width(d)) hipLaunchKernelGGL((KERNEL<F32, 0>), __VA_ARGS__); \
    else return hipErrorInvalidValue;                                                                \
  } while (0)

#define HIKVP_DISPATCH_SEL(dtype, d, KERNEL, NT, SPT, ...)                                          \
  do {                                                                                               \
    if ((dtype) == kDtypeBF16 && (d) == 128) hipLaunchKernelGGL((KERNEL<BF16, 128, NT, SPT>), __VA_ARGS__); \
    else if ((dtype) == kDtypeBF16 && (d) == 64) hipLaunchKernelGGL((KERNEL<BF16, 64, NT, SPT>), __VA_ARGS__); \
    else if ((dtype) == kDtypeBF16 && wide_width(d)) hipLaunchKernelGGL((KERNEL<BF16, 0, NT, SPT>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 128) hipLaunchKernelGGL((KERNEL<F32, 128, NT, SPT>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 64) hipLaunchKernelGGL((KERNEL<F32, 64, NT, SPT>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && wide_width(d)) hipLaunchKernelGGL((KERNEL<F32, 0, NT, SPT>), __VA_ARGS__); \
    else return hipErrorInvalidValue;                                                                \
  } while (0)

// Scoring kernels: KERNEL<E, D, LO>, LO when the rows carry a bf16 residual
// query (rows of an exact query in bf16).
#define HIKVP_DISPATCH_LO(a, KERNEL, ...)                                                            \
  do {                                                                                               \
    const int dt_ = (a).t.dtype, d_ = (a).t.d;                                                       \
    if ((a).r.q_lo) {                                                                                \
      if (dt_ == kDtypeBF16 && d_ == 128) hipLaunchKernelGGL((KERNEL<BF16, 128, true>), __VA_ARGS__); \
      else if (dt_ == kDtypeBF16 && d_ == 64) hipLaunchKernelGGL((KERNEL<BF16, 64, true>), __VA_ARGS__); \
      else if (dt_ == kDtypeBF16 && wide_width(d_)) hipLaunchKernelGGL((KERNEL<BF16, 0, true>), __VA_ARGS__); \
      else return hipErrorInvalidValue;                                                              \
    } else {                                                                                         \
      if (dt_ == kDtypeBF16 && d_ == 128) hipLaunchKernelGGL((KERNEL<BF16, 128, false>), __VA_ARGS__); \
      else if (dt_ == kDtypeBF16 && d_ == 64) hipLaunchKernelGGL((KERNEL<BF16, 64, false>), __VA_ARGS__); \
      else if (dt_ == kDtypeBF16 && wide_width(d_)) hipLaunchKernelGGL((KERNEL<BF16, 0, false>), __VA_ARGS__); \
      else if (dt_ == kDtypeF32 && d_ == 128) hipLaunchKernelGGL((KERNEL<F32, 128, false>), __VA_ARGS__); \
      else if (dt_ == kDtypeF32 && d_ == 64) hipLaunchKernelGGL((KERNEL<F32, 64, false>), __VA_ARGS__); \
      else if (dt_ == kDtypeF32 && wide_width(d_)) hipLaunchKernelGGL((KERNEL<F32, 0, false>), __VA_ARGS__); \
      else return hipErrorInvalidValue;                                                              \
    }                                                                                                \
  } while (0)

// Per-row select shape: one wave per row while the list fits 16 scores per
// lane, else a 256-thread workgroup; a wave holds 8, 13 or 16 scores a lane,
// a workgroup 8, 16 or 32 a thread, in registers (the fewest that cover the
// list: fewer registers held means more rows in flight, which these
// latency-bound kernels need; 13 for the 800-candidate lists of 8 mids x 100
// leaves takes 98 -> 89 registers, 4 -> 5 waves a SIMD: leaf Top-K + KG 72 ->
// 64 us at 16384 rows); lists above 8192 are re-read from the workspace in
// every pass.
#define HIKVP_SELECT_LAUNCH(a, cap, KERNEL, Kc, Kp, s)                                               \
  do {                                                                                               \
    const int64_t cap_ = (cap);                                                                      \
    if (cap_ <= 64 * 16) {                                                                           \
      int wpb, stage;                                                                                \
      size_t wb;                                                                                     \
      if (!row_launch_shape((Kc), (Kp), (a).t.d, 0, wpb, wb, stage)) return hipErrorInvalidValue;   \
      const unsigned blocks = (unsigned)(((a).blk1 - (a).blk0 + wpb - 1) / wpb);                     \
      if (cap_ <= 64 * 8)                                                                            \
        HIKVP_DISPATCH_SEL((a).t.dtype, (a).t.d, KERNEL, 64, 8, dim3(blocks), dim3(64 * wpb), wb * wpb, s, a, wb); \
      else if (cap_ <= 64 * 13)                                                                      \
        HIKVP_DISPATCH_SEL((a).t.dtype, (a).t.d, KERNEL, 64, 13, dim3(blocks), dim3(64 * wpb), wb * wpb, s, a, wb); \
      else                                                                                           \
        HIKVP_DISPATCH_SEL((a).t.dtype, (a).t.d, KERNEL, 64, 16, dim3(blocks), dim3(64 * wpb), wb * wpb, s, a, wb); \
    } else {                                                                                         \
      const size_t gb = rowwork_bytes((Kc), (Kp), (a).t.d, 0, 256);                                  \
      const dim3 grid((unsigned)((a).blk1 - (a).blk0));                                              \
      if (cap_ <= 256 * 8)                                                                           \
        HIKVP_DISPATCH_SEL((a).t.dtype, (a).t.d, KERNEL, 256, 8, grid, dim3(256), gb, s, a, gb);      \
      else if (cap_ <= 256 * 16)                                                                     \
        HIKVP_DISPATCH_SEL((a).t.dtype, (a).t.d, KERNEL, 256, 16, grid, dim3(256), gb, s, a, gb);     \
      else if (cap_ <= 256 * 32)                                                                     \
        HIKVP_DISPATCH_SEL((a).t.dtype, (a).t.d, KERNEL, 256, 32, grid, dim3(256), gb, s, a, gb);     \
      else                                                                                           \
        HIKVP_DISPATCH_SEL((a).t.dtype, (a).t.d, KERNEL, 256, 0, grid, dim3(256), gb, s, a, gb);      \
    }                                                                                                \
  } while (0)

// Waves per block and per-wave LDS of a per-row select kernel.
static bool row_launch_shape(int K, int Kp, int D, int64_t cands, int& wpb, size_t& wave_bytes,
                             int& stage, bool must_stage = false) {
  stage = (must_stage || cands <= kStageMax) ? (int)cands : 0;
  wave_bytes = rowwork_bytes(K, Kp, D, stage);
  const size_t limit = 64 * 1024;
  wpb = 4;
  while (wpb > 1 && wave_bytes * wpb > limit) --wpb;
  return wave_bytes * wpb <= limit;
}

hipError_t launch_root(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0) return hipSuccess;
  int wpb, stage;
  size_t wb;
  // the root scores come from k_root_mfma through the mid-score buffer (which
  // holds at least M_R slots a row); k_root stages them in LDS when they fit
  if (!row_launch_shape(a.K[0], 0, a.t.d, a.t.count[0], wpb, wb, stage, a.t.count[0] <= 2048))
    return hipErrorInvalidValue;
  if (a.t.count[0] > a.c1max) return hipErrorInvalidValue;  // score buffer too small
  const int64_t per_head = (int64_t)a.r.B * a.r.N * a.r.G;
  const int tph = (int)((per_head + 15) / 16);
  const int nrc = (int)((a.t.count[0] + kRootChunk - 1) / kRootChunk);
  const int64_t waves = (int64_t)(a.g1 - a.g0) * tph * nrc;
  // at least one block: the kernel also clears the part's counters
  const unsigned mblocks = (unsigned)(waves > 0 ? (waves + 3) / 4 : 1);
  HIKVP_DISPATCH_LO(a, k_root_mfma, dim3(mblocks), dim3(256), 0, s, a, tph, nrc);
  const unsigned blocks = (unsigned)((a.blk1 - a.blk0 + wpb - 1) / wpb);
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_root, dim3(blocks), dim3(64 * wpb), wb * wpb, s, a, wb, stage);
  return hipGetLastError();
}

hipError_t launch_root_groups(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0 || a.K[0] <= 0 || a.t.count[0] <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_root_scan, dim3(1), dim3(1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t blocks = ((int64_t)row_chunks(a.blk1 - a.blk0, a.K[0]) + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_root_fill, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mid_gemm(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0 || a.t.count[0] <= 0 || a.K[0] <= 0) return hipSuccess;
  int64_t blocks = a.root_tiles_max;       // one workgroup per tile (grid-stride past 8192)
  if (blocks > 8192) blocks = 8192;
  HIKVP_DISPATCH_LO(a, k_mid_gemm, dim3((unsigned)blocks), dim3(64 * kMidWaves), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mid_select(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0) return hipSuccess;
  // one wave per row
  const int spt = a.mid_spt;
  if (spt != 4 && spt != 16) return hipErrorInvalidValue;
  const size_t wb = mid_select_wave_bytes(a.K[1], a.K[0], a.t.d, spt);
  int wpb = 4;
  while (wpb > 1 && wb * wpb > 64 * 1024) --wpb;
  if (wb * wpb > 64 * 1024) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((a.blk1 - a.blk0 + wpb - 1) / wpb);
#define HIKVP_MID_SEL(SPT_)                                                                          \
  do {                                                                                               \
    const dim3 g_(blocks), b_(64 * wpb);                                                             \
    if (a.t.dtype == kDtypeBF16 && a.t.d == 128) hipLaunchKernelGGL((k_mid_select<BF16, 128, SPT_>), g_, b_, wb * wpb, s, a, wb); \
    else if (a.t.dtype == kDtypeBF16 && a.t.d == 64) hipLaunchKernelGGL((k_mid_select<BF16, 64, SPT_>), g_, b_, wb * wpb, s, a, wb); \
    else if (a.t.dtype == kDtypeBF16 && wide_width(a.t.d)) hipLaunchKernelGGL((k_mid_select<BF16, 0, SPT_>), g_, b_, wb * wpb, s, a, wb); \
    else if (a.t.dtype == kDtypeF32 && a.t.d == 128) hipLaunchKernelGGL((k_mid_select<F32, 128, SPT_>), g_, b_, wb * wpb, s, a, wb); \
    else if (a.t.dtype == kDtypeF32 && a.t.d == 64) hipLaunchKernelGGL((k_mid_select<F32, 64, SPT_>), g_, b_, wb * wpb, s, a, wb); \
    else if (a.t.dtype == kDtypeF32 && wide_width(a.t.d)) hipLaunchKernelGGL((k_mid_select<F32, 0, SPT_>), g_, b_, wb * wpb, s, a, wb); \
    else return hipErrorInvalidValue;                                                                \
  } while (0)
  if (spt == 4) HIKVP_MID_SEL(4);
  else HIKVP_MID_SEL(16);
#undef HIKVP_MID_SEL
  return hipGetLastError();
}

hipError_t launch_leaf_link(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0 || a.K[1] <= 0) return hipSuccess;
  int64_t blocks = ((int64_t)row_chunks(a.blk1 - a.blk0, a.K[1]) + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_bucket_link, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_leaf_score(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0 || a.K[1] <= 0) return hipSuccess;
  // at most rows * K_I distinct (head, mid) buckets
  const int64_t nb_max = (int64_t)(a.blk1 - a.blk0) * a.K[1];
  int64_t blocks = (nb_max + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  // filtered calls: each of the 4 waves stages leaf_nst members' scores
  if (a.leaf_nst > 0) {
    const size_t lds = (size_t)4 * (a.leaf_nst * a.leaf_fpad + 256) * 4;
    if (lds > 64 * 1024 || (a.t.d != 64 && a.t.d != 128)) return hipErrorInvalidValue;
    HIKVP_DISPATCH_LO(a, k_leaf_score_filtered, dim3((unsigned)blocks), dim3(256), lds, s, a);
  } else {
    HIKVP_DISPATCH_LO(a, k_leaf_score, dim3((unsigned)blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_leaf_select(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0) return hipSuccess;
  if (a.leaf_nst > 0) {
    // the filtered stream's survivors: one wave per row
    const int spt = a.leaf_spt;
    if ((spt != 8 && spt != 16 && spt != 24 && spt != 40) || (a.t.d != 64 && a.t.d != 128))
      return hipErrorInvalidValue;
    const size_t wb = leaf_pairs_wave_bytes(a.K[2], a.K[1], a.t.d, spt);
    // waves a workgroup: the most waves a CU can hold by LDS (160 KB; 13.6 KB
    // a wave at K_I = 16, K_L = 64 takes 11 as single waves, 8 as groups of 4)
    int wpb = 0, best = -1;
    for (int w = 4; w >= 1; --w) {
      if (wb * w > 64 * 1024) continue;
      const int fit = w * (int)((size_t)160 * 1024 / (wb * w));
      if (fit > best) { best = fit; wpb = w; }
    }
    if (wpb == 0) return hipErrorInvalidValue;
    const dim3 g_((unsigned)((a.blk1 - a.blk0 + wpb - 1) / wpb)), b_(64 * wpb);
    const bool bf = a.t.dtype == kDtypeBF16, d128 = a.t.d == 128;
#define HIKVP_LEAF_PAIRS(SPT_)                                                                          \
    do {                                                                                               \
      if (bf && d128) hipLaunchKernelGGL((k_leaf_select_pairs<BF16, 128, SPT_>), g_, b_, wb * wpb, s, a, wb); \
      else if (bf) hipLaunchKernelGGL((k_leaf_select_pairs<BF16, 64, SPT_>), g_, b_, wb * wpb, s, a, wb); \
      else if (d128) hipLaunchKernelGGL((k_leaf_select_pairs<F32, 128, SPT_>), g_, b_, wb * wpb, s, a, wb); \
      else hipLaunchKernelGGL((k_leaf_select_pairs<F32, 64, SPT_>), g_, b_, wb * wpb, s, a, wb);    \
    } while (0)
    if (spt == 8) HIKVP_LEAF_PAIRS(8);
    else if (spt == 16) HIKVP_LEAF_PAIRS(16);
    else if (spt == 24) HIKVP_LEAF_PAIRS(24);
    else HIKVP_LEAF_PAIRS(40);
#undef HIKVP_LEAF_PAIRS
    return hipGetLastError();
  }
  HIKVP_SELECT_LAUNCH(a, a.c2max, k_leaf_select, a.K[2], a.K[1], s);
  return hipGetLastError();
}

}  // namespace hikvp
