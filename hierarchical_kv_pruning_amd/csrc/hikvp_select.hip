// hikvp_select.hip -- the tree-descent kernels of HiKVP attention on gfx950.
//
// Page: "AtlasKV: Augmenting LLMs with Billion-Scale Knowledge Graphs in 20GB
// VRAM" (digest of arXiv 2510.17934), 速读 › 怎么做的: score the query against
// the root keys and keep the Top-K branches, score the children of those
// branches and keep the Top-K, and so on down to the leaves; the selected
// leaves' softmax then forms the KG half of the merged output.
//
//   k_clear     zeroes the group and bucket counters of the part's KV heads.
//   k_root_mfma one wave per 16 rows of one KV head: their scores against all
//               M_R root keys of the head on MFMA 16x16 tiles (a root key is
//               read once per 16 rows).
//   k_root      one wave per row: exact-boundary Top-K_R over the row's root
//               scores; each selection is counted in its (KV head, root)
//               group.  The per-row select kernels keep a few KB of LDS per
//               wave so many rows are in flight per CU.
//   k_root_scan / k_root_fill  lay the groups out in tiles of 32 rows; the
//               fill also records where each selected root's children start
//               in the row's mid candidate list.
//   k_mid_gemm  one wave per tile: the tile's rows against the root's child
//               span on bf16 (or fp32) MFMA 16x16 tiles; the span is read once
//               per tile instead of once per row.  Scores land in each row's
//               candidate slots of the workspace.
//   k_mid_select   one wave per row (a workgroup per row for long candidate
//               lists): Top-K_I over the row's mid scores.
//   k_bucket_link  registers each selection in its (KV head, mid) bucket,
//               with where the mid's children start in the row's leaf
//               candidate list.
//   k_leaf_score   one wave per bucket: streams the mid's leaf span once (it is
//               contiguous in the head-major layout) and writes the scores of
//               every member row into that row's candidate slots.
//   k_leaf_select  one wave (or workgroup) per row: Top-K_L, then the KG softmax over the
//               selected leaves and the weighted sum of their values.
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

__host__ __device__ inline size_t rowwork_bytes(int K, int Kp, int D, int stage, int NT = 64) {
  return selwork_bytes(NT, K, D) + 2 * align16((size_t)K * 4) + align16((size_t)(Kp + 1) * 4) +
         align16((size_t)Kp * 8) + align16((size_t)stage * 4);
}

__device__ inline RowWork carve_rowwork(char* p, int K, int Kp, int D, int stage, int NT = 64) {
  RowWork w;
  w.sel = carve_selwork(p, NT, K, D);
  auto take = [&](size_t bytes) { char* q = p; p += align16(bytes); return q; };
  w.out_node = (int*)take((size_t)K * 4);
  w.out_logit = (float*)take((size_t)K * 4);
  w.pre = (int*)take((size_t)(Kp + 1) * 4);
  w.base = (int64_t*)take((size_t)Kp * 8);
  w.stage = (float*)take((size_t)stage * 4);
  return w;
}

// The row's KG query (exact fp32 copy in LDS) and its 2-norm (rounded up).
template <class E, int D>
__device__ inline double load_query(const RowsDev& r, int b, int n, int h, float* qrow, int lane) {
  const char* qp = (const char*)r.q_kg + q_off(r.qks, b, n, h) * E::kBytes;
  float qq = 0.f;
  for (int t = lane; t < D; t += 64) {
    const float v = load_f32<E>(qp, t);
    qrow[t] = v;
    qq = fmaf(v, v, qq);
  }
  qq = wave_sum(qq);
  return sqrt((double)qq) * 1.0001;
}

// Root scores on MFMA: one wave per 16 consecutive rows of one KV head and
// kRootChunk of its roots (the rows are the M side, 16 roots the N side of
// each 16x16 tile, the chunk's tiles loaded at once), so a root key is read
// once per 16 rows instead of once per row.  The raw dot products (the
// select applies the scale) land in each row's slots of the mid-score buffer
// (indexed by row, like the mid level's scores, so concurrent descent parts
// touch disjoint slots), which k_root reads before the mid level reuses them.
constexpr int kRootChunk = 64;  // roots per k_root_mfma wave

template <class E, int D>
__global__ __launch_bounds__(256) void k_root_mfma(StepArgs a, int tph, int nrc) {
  constexpr int KCH = D * E::kBytes / 64;  // 16-byte pieces per lane per row
  constexpr int NU = kRootChunk / 16;      // root tiles in flight
  const int lane = threadIdx.x & 63, quad = lane >> 4, col = lane & 15;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (a.g1 - a.g0) * tph * nrc) return;
  const int rc = w % nrc, t = w / nrc;     // root chunk, row tile
  const int g = a.g0 + t / tph, m0 = (t % tph) * 16;
  const int per_head = a.r.B * a.r.N * a.r.G;  // rows of one KV head
  const int hb = g * per_head;                 // its first block
  const int MR = (int)a.t.count[0];
  uint4 afr[KCH];
  if (m0 + col < per_head) {
    int b, n, h;
    decode_row(a.r, row_of_block(a.r, hb + m0 + col), b, n, h);
    const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes + quad * 16;
#pragma unroll
    for (int m = 0; m < KCH; ++m) afr[m] = *(const uint4*)(qp + m * 64);
  } else {
#pragma unroll
    for (int m = 0; m < KCH; ++m) afr[m] = make_uint4(0, 0, 0, 0);
  }
  // this lane's outputs: rows m0 + 4*quad + v, root j0 + 16*u + col
  float* dst[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int mv = m0 + 4 * quad + v;
    dst[v] = mv < per_head ? a.mid_scores + (int64_t)row_of_block(a.r, hb + mv) * a.c1max : nullptr;
  }
  int64_t rsb;
  const char* kb = key_base(a.t, 0, g, rsb, E::kBytes) + quad * 16;
  const int j1 = min(MR, (rc + 1) * kRootChunk);
  for (int j0 = rc * kRootChunk; j0 < j1; j0 += 16 * NU) {
    uint4 bfr[NU][KCH];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const char* kp = kb + (int64_t)min(j0 + 16 * u + col, j1 - 1) * rsb;
#pragma unroll
      for (int m = 0; m < KCH; ++m) bfr[u][m] = *(const uint4*)(kp + m * 64);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const float4_t sc = tile_dot<E, KCH>(afr, bfr[u]);
      const int j = j0 + 16 * u + col;
      if (j < j1)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (dst[v]) dst[v][j] = sc[v];
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
  RowWork W = carve_rowwork(smem + (size_t)wave * wave_bytes, K, 0, D, stage);
  const int row = row_of_block(a.r, blk);
  // the row's scores, from k_root_mfma in the row's slots of the mid-score
  // buffer (by row, as the mid level uses it: concurrent parts own disjoint
  // rows), staged in LDS when they fit
  const float* gsc = a.mid_scores + (int64_t)row * a.c1max;
  float* sc = stage ? W.stage : a.mid_scores + (int64_t)row * a.c1max;
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  const int g = h / a.r.G;
  if (stage)
    for (int j = lane; j < MR; j += 64) sc[j] = gsc[j];
  const double qnorm = load_query<E, D>(a.r, b, n, h, W.sel.qrow, lane);
  wave_sync();

  int64_t rsb;
  const char* kb = key_base(a.t, 0, g, rsb, E::kBytes);
  const SlotMap ident{nullptr, nullptr, -1};
  const int k = select_topk<E, D, 64, MemScores<64>, true>(MemScores<64>{sc}, MR, K, twice_err_bound<D>(qnorm, a.t.norm[g]),
                                      a.r.scale, ident, KeyRows{kb, rsb}, W.sel, W.out_node, W.out_logit,
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
    a.root_members[(int64_t)a.root_tile_off[key] * kRootTile + rank] = make_int2(row, base);
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
// mid level: one wave per tile of kRootTile (32) rows of a (head, root)
// group, as two 16-row halves.  The rows are the M side and the root's
// children the N side of 16x16 MFMA tiles; each child fragment loaded serves
// both halves, so the child span is read once per 32 rows (from L2 after the
// group's first tile).
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(256) void k_mid_gemm(StepArgs a) {
  constexpr int KCH = D * E::kBytes / 64;  // 16-byte pieces per lane per row
  constexpr int TU = 2;                    // child tiles per round = consecutive children per lane
  constexpr int HR = kRootTile / 16;       // 16-row halves per tile
  static_assert(kRootTile == 32, "two 16-row halves per tile");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int quad = lane >> 4, col = lane & 15;
  float* const junk = a.junk + ((blockIdx.x * nwave + wave) % kJunkSlots) * 16;
  const int ntiles = *a.root_ntiles;
  const int MR = (int)a.t.count[0];
  const int64_t* off0 = a.t.off[0];
  for (int t = blockIdx.x * nwave + wave; t < ntiles; t += gridDim.x * nwave) {
    const int key = a.root_tile_key[t];
    const int toff = a.root_tile_off[key];
    const int cnt = a.root_tot[key];
    const int g = key / MR, j = key % MR;
    const int64_t first = off0[j];
    const int F = (int)(off0[j + 1] - first);
    const int m0 = (t - toff) * kRootTile;     // first member of the tile
    const bool two = m0 + 16 < cnt;            // wave-uniform: the second half has members
    uint4 afr[HR][KCH];
    float* dst[HR][4];
#pragma unroll
    for (int hh = 0; hh < HR; ++hh) {
      const int mi = m0 + 16 * hh + col;
      const int2 mem = mi < cnt ? a.root_members[(int64_t)toff * kRootTile + mi] : make_int2(-1, 0);
      if (mi < cnt) {
        int b, n, h;
        decode_row(a.r, mem.x, b, n, h);
        const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes;
#pragma unroll
        for (int m = 0; m < KCH; ++m) afr[hh][m] = *(const uint4*)(qp + m * 64 + quad * 16);
      } else {
#pragma unroll
        for (int m = 0; m < KCH; ++m) afr[hh][m] = make_uint4(0, 0, 0, 0);
      }
      // Rounds of TU child tiles; in tile u, column col is child c0 + col*TU
      // + u, so a lane ends the round with TU consecutive scores of each of
      // its 4 rows (half rows 4*quad + v), written with one 8-byte store.
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ms = 4 * quad + v;
        const int srow = __shfl(mem.x, ms), sbase = __shfl(mem.y, ms);
        dst[hh][v] = m0 + 16 * hh + ms < cnt ? a.mid_scores + (int64_t)srow * a.c1max + sbase + col * TU : nullptr;
      }
    }
    // Loads and stores are unconditional (clamped child, junk slot) and a
    // round's stores follow the next round's loads, so the wait for the loads
    // never covers the stores.
    int64_t rsb;
    const char* kb = key_base(a.t, 1, g, rsb, E::kBytes) + first * rsb + quad * 16;
    float4_t prev[HR][TU];
#pragma unroll
    for (int hh = 0; hh < HR; ++hh)
#pragma unroll
      for (int u = 0; u < TU; ++u) prev[hh][u] = float4_t{0.f, 0.f, 0.f, 0.f};
    int pc0 = -1;
    auto load_round = [&](int c0, uint4 (&bfr)[TU][KCH]) {
#pragma unroll
      for (int u = 0; u < TU; ++u) {
        const char* kp = kb + (int64_t)min(c0 + col * TU + u, F - 1) * rsb;
#pragma unroll
        for (int m = 0; m < KCH; ++m) bfr[u][m] = *(const uint4*)(kp + m * 64);
      }
    };
    auto store_full = [&]() {
#pragma unroll
      for (int hh = 0; hh < HR; ++hh)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          store2u((pc0 >= 0 && dst[hh][v]) ? dst[hh][v] + pc0 : junk, prev[hh][0][v], prev[hh][1][v]);
    };
    auto compute = [&](const uint4 (&bfr)[TU][KCH]) {
#pragma unroll
      for (int u = 0; u < TU; ++u) prev[0][u] = tile_dot<E, KCH>(afr[0], bfr[u]);
      if (two) {
#pragma unroll
        for (int u = 0; u < TU; ++u) prev[1][u] = tile_dot<E, KCH>(afr[1], bfr[u]);
      }
    };
    int c0 = 0;
    for (; c0 + 16 * TU <= F; c0 += 16 * TU) {
      uint4 bfr[TU][KCH];
      load_round(c0, bfr);
      store_full();
      compute(bfr);
      pc0 = c0;
    }
    if (c0 < F) {  // last, partial round
      uint4 bfr[TU][KCH];
      load_round(c0, bfr);
      store_full();
      compute(bfr);
      const int cl = c0 + col * TU;
#pragma unroll
      for (int hh = 0; hh < HR; ++hh)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int u = 0; u < TU; ++u)
            if (dst[hh][v] && cl + u < F) dst[hh][v][c0 + u] = prev[hh][u][v];
    } else {
      store_full();
    }
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
  constexpr int QPT = (D + NT - 1) / NT;
  int b, n, h;
  decode_row(a.r, row, b, n, h);
  g = h / a.r.G;
  const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes;
  float qv[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) qv[j] = gtid + j * NT < D ? load_f32<E>(qp, gtid + j * NT) : 0.f;
  const int64_t* off = a.t.off[lev - 1];
  int64_t first0 = 0;
  int fan0 = 0;
  if (p0 >= 0) {
    first0 = off[p0];
    fan0 = (int)(off[p0 + 1] - first0);
  }
#pragma unroll
  for (int j = 0; j < QPT; ++j)
    if (gtid + j * NT < D) W.sel.qrow[gtid + j * NT] = qv[j];
  group_sync<NT>();
  const int Kp = a.K[lev - 1];
  if (gtid < 64) {
    float qq = 0.f;
    for (int t = gtid; t < D; t += 64) qq = fmaf(W.sel.qrow[t], W.sel.qrow[t], qq);
    qq = wave_sum(qq);
    if (gtid == 0) W.sel.ctl[7] = __float_as_int((float)(sqrt((double)qq) * 1.0001));
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

template <class E, int D, int NT, int SPT>
__device__ inline void mid_select_body(const StepArgs& a, size_t group_bytes) {
  extern __shared__ __align__(16) char smem[];
  const int groups = blockDim.x / NT, grp = threadIdx.x / NT, gtid = threadIdx.x % NT;
  const int blk = a.blk0 + blockIdx.x * groups + grp;
  if (blk >= a.blk1) return;  // whole group (whole waves) leaves together
  const int K1 = a.K[1];
  RowWork W = carve_rowwork(smem + (size_t)grp * group_bytes, K1, a.K[0], D, 0, NT);
  const int row = row_of_block(a.r, blk);
  const int p0 = first_parent(a, row, 1, gtid);
  // the scores do not depend on the candidate list: load them next
  const auto sc = RowScores<NT, SPT>::make(a.mid_scores + (int64_t)row * a.c1max, (int)a.c1max, gtid);
  int g;
  double qnorm;
  const int n1 = select_prologue<E, D, NT>(a, W, row, 1, g, qnorm, gtid, p0);
  int64_t rsb;
  const char* kb = key_base(a.t, 1, g, rsb, E::kBytes);
  const int k1 = select_topk<E, D, NT>(sc, n1, K1,
                                       twice_err_bound<D>(qnorm, a.t.norm[a.t.Hkv + g]), a.r.scale,
                                       SlotMap{W.pre, W.base, a.K[0]}, KeyRows{kb, rsb}, W.sel,
                                       W.out_node, W.out_logit, gtid);
  int32_t* o1 = a.sel[1] + (int64_t)row * K1;
  for (int i = gtid; i < K1; i += NT) o1[i] = i < k1 ? W.out_node[i] : -1;
}

// One wave per row (short candidate lists) or one workgroup per row; the
// scores are held in registers (SPT per thread, sized to the list at launch)
// or re-read from the workspace in every pass (SPT = 0, long lists).
template <class E, int D, int NT, int SPT>
__global__ __launch_bounds__(256) void k_mid_select(StepArgs a, size_t gb) {
  mid_select_body<E, D, NT, SPT>(a, gb);
}

// ---------------------------------------------------------------------------
// leaf scoring, deduplicated: every distinct (KV head, mid) selected by any
// row is one bucket.  The link kernel writes one 16-byte descriptor per bucket
// (key, fanout, element offset of the span) and stores the first
// kBucketSlots member rows as (row, first leaf slot) pairs; later members go
// to a linked list scored by k_leaf_score_overflow.  One wave per bucket
// streams the mid's leaf span (contiguous in the head-major layout) once and
// scores it for every member row, prefetching its next bucket's descriptor.
// Each member's dot products are computed independently, so results do not
// depend on the (atomic) member or bucket order.
// ---------------------------------------------------------------------------
__global__ void k_clear(StepArgs a) {
  const int64_t MI = a.t.count[1], MR = a.t.count[0];
  const int64_t nk1 = (a.g1 - a.g0) * MI, nk0 = (a.g1 - a.g0) * MR;  // the part's keys
  const int64_t nall = (int64_t)a.t.Hkv * MR;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (a.g0 == 0 && a.g1 == a.t.Hkv) {  // all heads: the whole arrays, in order
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < (int64_t)a.bucket_q * 64; i += stride) {
      a.bucket_cnt[i] = 0;
      a.bucket_head[i] = -1;
    }
  } else {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nk1; i += stride) {
      const int64_t bix = bucket_index(a, a.g0 * MI + i);
      a.bucket_cnt[bix] = 0;
      a.bucket_head[bix] = -1;
    }
  }
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nk0 * kRootSub; i += stride)
    a.root_cnt[(i / nk0) * nall + a.g0 * MR + i % nk0] = 0;
  if (blockIdx.x == 0 && threadIdx.x <= kDescSub) a.bucket_count[threadIdx.x] = 0;
}

// Register selection e = (row, mid) in its (KV head, mid) bucket, given its
// rank from the bucket's counter (-1: nothing to register): the first
// kBucketSlots members in fixed slots (row, first leaf slot), later ones in
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
  if (rank < kBucketSlots) {
    a.bucket_slot[bix * kBucketSlots + rank] = make_int2(row, slot_base);
  } else {
    a.bucket_next[e] = atomicExch(&a.bucket_head[bix], (int)e);
    if (rank == kBucketSlots) a.bucket_ovf[atomicAdd(&a.bucket_count[kDescSub], 1)] = (int)key;
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
  register_in_bucket(a, e, row, sub, g, key, rank, f0, fan, base, lane);
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

// Scores of one group of up to 8 member rows of a bucket over its leaf span,
// on half-split MFMA tiles: the group is the M side and the span's keys the N
// side.  Lanes g0 .. g0+7 of mem hold the members (row, first leaf slot),
// gcnt of them valid.  A round covers 8*TU keys; in its tile u, item i is key
// t0 + i*TU + u, so every load instruction reads eight whole 128-byte lines
// and each lane ends the round holding TU consecutive scores per member,
// written with one 16-byte store.  Every member's scores go through exactly
// this arithmetic, whichever group or kernel it lands in, so they do not
// depend on the (atomic) order in which members joined the bucket.
template <class E, int D>
__device__ inline void score_member_group(const StepArgs& a, const char* kp, int64_t rsb, int F, int2 mem,
                                          int g0, int gcnt, int lane) {
  constexpr int RB = D * E::kBytes;        // bytes per key row
  constexpr int KP = RB / 128;             // 16-byte pieces per lane per tile
  constexpr int TU = 4;                    // tiles per round = consecutive keys per lane
  const int quad = lane >> 4, item = lane & 7;
  const bool owner = lane < 32 && (lane & 15) < 8;   // holds combined scores
  // A fragment: member `item`, zeros past the members
  uint4 afr[KP];
  const int row = __shfl(mem.x, g0 + item);
  if (item < gcnt) {
    int b, n, h;
    decode_row(a.r, row, b, n, h);
    const char* qp = (const char*)a.r.q_kg + q_off(a.r.qks, b, n, h) * E::kBytes + split_off(lane, 0);
#pragma unroll
    for (int m = 0; m < KP; ++m) afr[m] = *(const uint4*)(qp + m * 128);
  } else {
#pragma unroll
    for (int m = 0; m < KP; ++m) afr[m] = make_uint4(0, 0, 0, 0);
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
    for (int u = 0; u < TU; ++u) prev[u] = split_combine(tile_dot<E, KP>(afr, bfr[u]), lane);
    pt0 = t0;
  }
  if (t0 < F) {  // last, partial round
    uint4 bfr[TU][KP];
    load_round(t0, bfr);
    store_full();
#pragma unroll
    for (int u = 0; u < TU; ++u) prev[u] = split_combine(tile_dot<E, KP>(afr, bfr[u]), lane);
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

// One wave per bucket: its first kBucketSlots members, 8 at a time (a bucket
// with more than 8 members makes further passes over its span, mostly L2
// hits); members past kBucketSlots are left to k_leaf_score_overflow.
template <class E, int D>
__global__ __launch_bounds__(256) void k_leaf_score(StepArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
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
    cnt = cnt < kBucketSlots ? cnt : kBucketSlots;
    const int2 mem = lane < kBucketSlots ? a.bucket_slot[(int64_t)key * kBucketSlots + lane] : make_int2(-1, 0);
    for (int g0 = 0; g0 < cnt; g0 += 8)
      score_member_group<E, D>(a, kp, rsb, F, mem, g0, min(8, cnt - g0), lane);
    cur = nxt;
    v = vn;
  }
}

// Members of buckets with more than kBucketSlots rows: one wave per listed
// bucket walks its overflow list and scores the members 8 at a time with the
// same group arithmetic as k_leaf_score.
template <class E, int D>
__global__ __launch_bounds__(256) void k_leaf_score_overflow(StepArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  const int nov = a.bucket_count[kDescSub];
  const int K1 = a.K[1];
  const int MI = (int)a.t.count[1];
  const char* kbase = (const char*)a.t.key[2];
  const int64_t rsb = a.t.rs[2] * E::kBytes;
  for (int v = blockIdx.x * nwave + wave; v < nov; v += gridDim.x * nwave) {
    const int key = a.bucket_ovf[v];
    const int g = key / MI, mid = key % MI;
    const int64_t bix = bucket_index(a, key);
    const int64_t f0 = a.t.off[1][mid];
    const int F = (int)(a.t.off[1][mid + 1] - f0);
    const char* kp = kbase + ((int64_t)g * a.t.hs[2] + f0 * a.t.rs[2]) * E::kBytes + split_off(lane, 0);
    int e = a.bucket_head[bix];
    while (e != -1) {  // wave-uniform walk: lane i takes the group's i-th entry
      int mine = -1, gcnt = 0;
      for (; gcnt < 8 && e != -1; ++gcnt) {
        if (lane == gcnt) mine = e;
        e = a.bucket_next[e];
      }
      const int2 gm = (lane < gcnt) ? make_int2(mine / K1, a.mid_base[mine]) : make_int2(-1, 0);
      score_member_group<E, D>(a, kp, rsb, F, gm, 0, gcnt, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// leaf Top-K and the KG softmax over the selected leaves, one wave per row
// ---------------------------------------------------------------------------
template <class E, int D, int NT, int SPT>
__device__ inline void leaf_select_body(const StepArgs& a, size_t group_bytes) {
  constexpr int DPL = D / 64;
  extern __shared__ __align__(16) char smem[];
  const int groups = blockDim.x / NT, grp = threadIdx.x / NT, gtid = threadIdx.x % NT;
  const int blk = a.blk0 + blockIdx.x * groups + grp;
  if (blk >= a.blk1) return;
  const int K2 = a.K[2];
  RowWork W = carve_rowwork(smem + (size_t)grp * group_bytes, K2, a.K[1], D, 0, NT);
  const int row = row_of_block(a.r, blk);
  const int p0 = first_parent(a, row, 2, gtid);
  const auto sc = RowScores<NT, SPT>::make(a.leaf_scores + (int64_t)row * a.c2max, (int)a.c2max, gtid);
  int g;
  double qnorm;
  const int n2 = select_prologue<E, D, NT>(a, W, row, 2, g, qnorm, gtid, p0);
  int64_t rsb;
  const char* kb = key_base(a.t, 2, g, rsb, E::kBytes);
  const int k2 = select_topk<E, D, NT>(sc, n2, K2,
                                       twice_err_bound<D>(qnorm, a.t.norm[2 * a.t.Hkv + g]), a.r.scale,
                                       SlotMap{W.pre, W.base, a.K[1]}, KeyRows{kb, rsb}, W.sel,
                                       W.out_node, W.out_logit, gtid);
  int32_t* o2 = a.sel[2] + (int64_t)row * K2;
  for (int i = gtid; i < K2; i += NT) o2[i] = i < k2 ? W.out_node[i] : -1;
  if (gtid >= 64) return;  // the KG half is formed by the group's first wave
  const int lane = gtid;

  // KG half: softmax over the selected leaves' logits, weighted values
  float* okg = a.o_kg + (int64_t)row * D;
  if (k2 == 0) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) okg[lane * DPL + e] = 0.f;
    if (lane == 0) a.lse_kg[row] = -INFINITY;
    return;
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
  // Value rows are read 16 bytes a lane, LPK lanes a row, so one load
  // instruction covers KPW rows and VU instructions in flight cover the
  // K_L rows of a row in one or two memory round trips; each lane sums its
  // dims over the rows of its lane group, then the KPW groups are added.
  constexpr int EPV = E::kEPV, LPK = D / EPV, KPW = 64 / LPK;
  constexpr int VU = 8;
  const int sub = lane / LPK, ch = lane % LPK;
  const char* vb = (const char*)a.t.leaf_v + (int64_t)g * a.t.hs[3] * E::kBytes + ch * 16;
  const int64_t vrs = a.t.rs[3] * E::kBytes;
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
  const float inv = 1.f / sum;
  if (sub == 0) {
    float4* dst = (float4*)(okg + ch * EPV);
#pragma unroll
    for (int e = 0; e < EPV; e += 4)
      dst[e / 4] = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
  }
  if (lane == 0) a.lse_kg[row] = mx + logf(sum);
}

template <class E, int D, int NT, int SPT>
__global__ __launch_bounds__(256) void k_leaf_select(StepArgs a, size_t gb) {
  leaf_select_body<E, D, NT, SPT>(a, gb);
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

#define HIKVP_DISPATCH_SEL(dtype, d, KERNEL, NT, SPT, ...)                                          \
  do {                                                                                               \
    if ((dtype) == kDtypeBF16 && (d) == 128) hipLaunchKernelGGL((KERNEL<BF16, 128, NT, SPT>), __VA_ARGS__); \
    else if ((dtype) == kDtypeBF16 && (d) == 64) hipLaunchKernelGGL((KERNEL<BF16, 64, NT, SPT>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 128) hipLaunchKernelGGL((KERNEL<F32, 128, NT, SPT>), __VA_ARGS__); \
    else if ((dtype) == kDtypeF32 && (d) == 64) hipLaunchKernelGGL((KERNEL<F32, 64, NT, SPT>), __VA_ARGS__); \
    else return hipErrorInvalidValue;                                                                \
  } while (0)

// Per-row select shape: one wave per row while the list fits 16 scores per
// lane, else a 256-thread workgroup with 8, 16 or 32 scores per thread held
// in registers (the fewest that cover the list: fewer registers held means
// more rows in flight, which these latency-bound kernels need); lists above
// 8192 are re-read from the workspace in every pass.
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
  if (waves > 0)
    HIKVP_DISPATCH(a.t.dtype, a.t.d, k_root_mfma, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a, tph, nrc);
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
  int64_t blocks = (a.root_tiles_max + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_mid_gemm, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mid_select(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0) return hipSuccess;
  HIKVP_SELECT_LAUNCH(a, a.c1max, k_mid_select, a.K[1], a.K[0], s);
  return hipGetLastError();
}

hipError_t launch_clear(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0) return hipSuccess;
  const int64_t nk1 = (a.g0 == 0 && a.g1 == a.t.Hkv) ? (int64_t)a.bucket_q * 64 : (int64_t)(a.g1 - a.g0) * a.t.count[1];
  const int64_t nk0 = (int64_t)(a.g1 - a.g0) * a.t.count[0] * kRootSub;
  int64_t blocks = ((nk1 > nk0 ? nk1 : nk0) + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_clear, dim3((unsigned)blocks), dim3(256), 0, s, a);
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
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_leaf_score, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_leaf_overflow(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0 || a.K[1] <= 0) return hipSuccess;
  // at most rows * K_I / (kBucketSlots + 1) buckets overflow
  const int64_t nb_max = (int64_t)(a.blk1 - a.blk0) * a.K[1];
  int64_t blocks = (nb_max / (kBucketSlots + 1) + 4) / 4;
  if (blocks > 1024) blocks = 1024;
  HIKVP_DISPATCH(a.t.dtype, a.t.d, k_leaf_score_overflow, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_leaf_select(const StepArgs& a, hipStream_t s) {
  if (a.blk1 <= a.blk0) return hipSuccess;
  HIKVP_SELECT_LAUNCH(a, a.c2max, k_leaf_select, a.K[2], a.K[1], s);
  return hipGetLastError();
}

}  // namespace hikvp
