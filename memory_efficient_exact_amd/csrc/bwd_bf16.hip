// Backward attention for bf16 inputs on gfx950, by recomputation.
//
// "Self-attention Does Not Need O(n^2) Memory" (abstract; 方法详解; English
// digest method bullets) differentiates the chunked forward by recomputing
// each chunk's intermediates instead of storing them. Here the forward saves
// only two fp32 numbers per query row (row max m_i and row sum l_i); the
// kernels below rebuild the probability tile
//     P_ij = exp(s_ij - m_i) / l_i = exp2(x_ij * log2(e)/sqrt(d) - lse2_i),
//     lse2_i = m_i * log2(e) + log2(l_i),   x_ij = q_i . k_j,
// from Q and K on the fly. The pages print no gradient formulas; the textbook
// softmax Jacobian is used: dV = P^T dO, dP = dO V^T, D_i = dO_i . O_i,
// dS = P * (dP - D), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).
//
// Two launches on the caller's stream:
//  1. bwd_rows: -D_i and lse2_i for every row, into the workspace (reads O,
//     dO, m, l once; a few microseconds).
//  2. bwd_main: one grid holding two kinds of workgroup of W waves, two waves
//     per SIMD: W = 8 (one workgroup per CU) when that grid covers every CU,
//     else W = 4 (two per CU).
//     * dK/dV workgroups own R*W keys (R per wave, K and V of those keys in
//       registers) and sweep every query tile of 64 rows (Q, dO, lse2, D
//       copied into LDS by DMA, double-buffered), accumulating dV^T and dK^T
//       in registers: per tile S = Q K^T, dP = dO V^T (lane = key), then
//       dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T from transposed LDS
//       reads.
//     * dQ workgroups own R*W queries (R per wave, Q and dO in registers)
//       and sweep every key tile of 64 keys (K, V in LDS), accumulating dQ^T:
//       S^T = K Q^T, dP^T = V dO^T (lane = query), dQ^T += K^T dS^T.
//     d = 64 takes R = 32 rows per wave on 32x32x16 MFMAs and padded LDS
//     tiles (bwd_main_kernel); d = 128 takes R = 16 on 16x16x32 MFMAs and
//     swizzled tiles (bwd_main128_kernel), which halves the accumulators so
//     that two waves still fit per SIMD.
//     The dK/dV workgroups come first in the grid (they carry more work), the
//     dQ workgroups fill the machine behind them.
// No probability or score array is written to memory; dQ, dK and dV are each
// written once by one workgroup, so results do not depend on scheduling.
//
// Split mode (grids of at most 256 workgroups, when the caller's workspace
// holds it): each workgroup position repeats for several ranges of the tiles
// it sweeps, each range writing fp32 partial sums to the workspace, and a
// reduce pass (bwd_reduce.hip) adds the ranges in a fixed order; results are
// again independent of scheduling.
//
// Grouped-query heads: the query heads sharing one key/value head arrive
// stacked as the rows of one problem (see mea_launch.h), so a dK/dV workgroup
// sweeps the query rows of the whole group and its dK, dV are the sums over
// that group that the chain rule asks for, still written once.
#include <type_traits>

#include "mea_device.h"
#include "mea_launch.h"

namespace mea {
namespace {

#if MEA_SYNC_TIMERS
// per role: the SyncTimer counters (mea_device.h); roles: d = 64 dK/dV,
// d = 64 dQ, d = 128 dK/dV, d = 128 dQ
__device__ unsigned long long g_sync[4][kSyncCounters];
#define MEA_SYNC_COUNTERS(role) (g_sync[role])
#else
#define MEA_SYNC_COUNTERS(role) nullptr
#endif

constexpr int kThreads = 256;     // row-term kernel
constexpr int kWaves = 4;         // waves per main-kernel workgroup on small grids
constexpr int kWideWaves = 8;     // waves per main-kernel workgroup on grids that fill the chip
constexpr int64_t kComputeUnits = 256;
constexpr int kTileQ = 64;            // query rows per staged tile (dK/dV role)
constexpr int kTileK = 64;            // key rows per staged tile (dQ role)

// ------------------------------------------------------------ 1. row terms
// One wave per 8 rows (d=64) / 4 rows (d=128): lanes read 16 bytes of O and
// dO each and reduce over the lanes of a row.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_rows_kernel(
    const bf16* __restrict__ O, const bf16* __restrict__ dO, const float* __restrict__ Mx,
    const float* __restrict__ Ls, float* __restrict__ Dv, float* __restrict__ Lse2,
    int64_t rows) {
  constexpr int LPR = D / 8;  // lanes per row
  constexpr int RPB = kThreads / LPR;  // rows per workgroup and pass
  const int part = threadIdx.x % LPR;
  // workgroup-uniform stride over the rows (the grid may be capped)
  for (int64_t r0 = (int64_t)blockIdx.x * RPB; r0 < rows; r0 += (int64_t)gridDim.x * RPB) {
    const int64_t row = r0 + threadIdx.x / LPR;
    float acc = 0.f;
    if (row < rows) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(O + row * D + part * 8);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(dO + row * D + part * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && part == 0) {
      Dv[row] = -acc;  // stored negated: it seeds the dP accumulators below
      Lse2[row] = Mx[row] * kLog2e + __builtin_log2f(Ls[row]);
    }
  }
}

// ------------------------------------------------------------ 2. main kernel
struct BwdArgs {
  const bf16* Q;
  const bf16* K;
  const bf16* V;
  const bf16* dO;
  const float* Dv;    // -D per row
  const float* Lse2;
  bf16* dQ;
  bf16* dK;
  bf16* dV;
  int n_q;        // query rows per head (the query heads of a group, stacked)
  int n_k;        // keys per head
  int tiles_kv;   // dK/dV workgroups per head
  int tiles_q;    // dQ workgroups per head
  int total_kv;   // dK/dV workgroups in the grid
  int total_q;    // dQ workgroups in the grid
  float C;        // log2(e) / sqrt(d)
  float scale;    // 1 / sqrt(d)
  // split backward (small grids): each dK/dV workgroup position repeats for s_kv
  // ranges of len_q staged query tiles, each dQ position for s_q ranges of len_k
  // key tiles; a split side writes fp32 partials (before the 1/sqrt(d) factor)
  // to Pdk, Pdv ([s_kv][kv_rows][D]) or Pdq ([s_q][q_rows][D]), else they are null
  int s_kv;
  int len_q;
  int s_q;
  int len_k;
  float* Pdk;
  float* Pdv;
  float* Pdq;
  int64_t kv_rows;  // heads * n_k
  int64_t q_rows;   // heads * n_q
};

template <int D>
struct BwdShared {
  using TQ = TileDma<D, kTileQ, kWaves>;  // (tile sizes do not depend on the wave count)
  using TK = TileDma<D, kTileK, kWaves>;
  static_assert(TQ::kElems == TK::kElems, "both roles share the LDS arrays");
  static constexpr int kElems = TQ::kElems;
};

// --- dK / dV role -----------------------------------------------------------
template <int D, int W>
__device__ __forceinline__ void dkdv_role(const BwdArgs& a, int wg, bf16* s0, bf16* s1, bf16* s2,
                                          bf16* s3, float* f0, float* f1) {
  using L = Padded<D>;
  using TQ = TileDma<D, kTileQ, W>;
  constexpr int RS = L::kRowElems;
  constexpr int DK = D / 16;
  constexpr int DB = D / 32;
  constexpr int NC = kTileQ / 16;  // 16-query chunks per tile
  constexpr int QBT = kTileQ / 32; // 32-query blocks per tile

  const int n_q = a.n_q, n_k = a.n_k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int l32 = lane & 31, hi = lane >> 5;
  const int tile = xcd_remap(wg, a.total_kv);  // ((bh * s_kv) + sp) * tiles_kv + kt
  const int bh = tile / (a.tiles_kv * a.s_kv);
  const int sp = (tile - bh * a.tiles_kv * a.s_kv) / a.tiles_kv;  // range of query tiles
  const int kt = tile - (bh * a.s_kv + sp) * a.tiles_kv;
  const int64_t qbase = (int64_t)bh * n_q * D;  // Q, dO (all query rows of the head)
  const int64_t kbase = (int64_t)bh * n_k * D;  // K, V, dK, dV
  const int64_t rbase = (int64_t)bh * n_q;
  const int key = kt * (32 * W) + wave * 32 + l32;  // this lane's key (column of S)

  // K and V of this wave's 32 keys: B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[DK], vf[DK];
  const int krow = min(key, n_k - 1);
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    kf[dk] = *reinterpret_cast<const bf16x8*>(a.K + kbase + (int64_t)krow * D + dk * 16 + 8 * hi);
    vf[dk] = *reinterpret_cast<const bf16x8*>(a.V + kbase + (int64_t)krow * D + dk * 16 + 8 * hi);
  }
  f32x16 accV[DB], accK[DB];  // dV^T, dK^T: register r -> column 32*db + 8*(r/4) + 4*hi + r%4
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    accV[db] = f32x16{};
    accK[db] = f32x16{};
  }

  TQ dma;
  dma.init(wave, lane);
  // lse2 and D of a query tile: 64 floats each, one 4-byte DMA per lane
  auto issue = [&](bf16* qdst, bf16* odst, float* fdst, int i0) {
    dma.issue(a.Q + qbase, i0, n_q, qdst);
    dma.issue(a.dO + qbase, i0, n_q, odst);
    if (wave == W - 1) {
      const int r = min(i0 + lane, n_q - 1);
      dma4_untracked(a.Lse2 + rbase + r, fdst);
      dma4_untracked(a.Dv + rbase + r, fdst + kTileQ);
    }
  };

  const int g = lane >> 4, jj = lane & 15;
  const int a_lane = L::off(l32, 8 * hi);  // 16-byte row reads (A operands of S, dP)
  const int t_lane = L::off(4 * hi + (jj >> 2), (g & 1) * 16 + 4 * (jj & 3));  // transposed reads

  auto tile_body = [&](const bf16* qs, const bf16* os, const float* fs, int i0, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    bf16x8 pf[NC], sf[NC];  // P and dS: chunk c element e <-> query 16c + 8(e/4) + 4hi + e%4
#pragma unroll
    for (int qb = 0; qb < QBT; ++qb) {
      // lane holds key `key`; register r holds query row i0 + 32*qb + 8*(r/4) + 4*hi + r%4.
      // The dP accumulator starts at -D of its query row, so it ends at dP - D.
      f32x16 s = f32x16{}, dp;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 nd = *reinterpret_cast<const f32x4*>(fs + kTileQ + qb * 32 + 8 * r4 + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * r4 + e] = nd[e];
      }
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) {
        const int off = a_lane + L::off(qb * 32, dk * 16);
        s = mfma32x32x16(lds_read_b128(qs + off), kf[dk], s);
        dp = mfma32x32x16(lds_read_b128(os + off), vf[dk], dp);
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 lse = *reinterpret_cast<const f32x4*>(fs + qb * 32 + 8 * r4 + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          float p = fast_exp2(__builtin_fmaf(s[r], a.C, -lse[e]));
          if constexpr (kMasked) {
            if (i0 + qb * 32 + 8 * r4 + 4 * hi + e >= n_q) p = 0.f;  // padding query rows
          }
          pf[2 * qb + (r >> 3)][r & 7] = (bf16)p;
          sf[2 * qb + (r >> 3)][r & 7] = (bf16)(p * dp[r]);
        }
      }
    }
    // dV^T += dO^T P,  dK^T += Q^T dS   (A operands by transposed LDS reads)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int off = t_lane + L::off(c * 16, db * 32);
        const bf16x8 ao = cat(lds_read_tr16(os + off), lds_read_tr16(os + off + 8 * RS));
        const bf16x8 aq = cat(lds_read_tr16(qs + off), lds_read_tr16(qs + off + 8 * RS));
        accV[db] = mfma32x32x16(ao, pf[c], accV[db]);
        accK[db] = mfma32x32x16(aq, sf[c], accK[db]);
      }
    }
  };

  // this workgroup's query tiles [t0, t1): all of them unless the backward is split
  const int t0 = sp * a.len_q;
  const int t1 = min(t0 + a.len_q, (n_q + kTileQ - 1) / kTileQ);
  SyncTimer tim;
  auto step = [&](const bf16* qs, const bf16* os, const float* fs, bf16* qn, bf16* on, float* fn,
                  int t, auto full_tag) {
    const int i0 = t * kTileQ;
    if (t + 1 < t1) issue(qn, on, fn, i0 + kTileQ);
    if constexpr (decltype(full_tag)::value) tile_body(qs, os, fs, i0, std::false_type{});
    else tile_body(qs, os, fs, i0, std::true_type{});
    tim.end_of_tile();
  };
  if (t1 > t0) {  // no query rows at all: dK = dV = 0
    issue(s0, s1, f0, t0 * kTileQ);
    wait_all();
    __syncthreads();
  }
  tim.start(wave, W);
  // Full tiles in pairs, then at most one more and the ragged last tile: with the
  // ragged tile outside the loop, the loop body has one path and its running state
  // is not copied between register sets at every tile. Identical results; with the
  // same in the dQ role, 1.4-2% faster at d = 64, 7% at d = 128 (1 x 16 x 8192 x 128).
  {
    const int tf = min(t1, n_q / kTileQ);
    int t = t0;
    for (; t + 1 < tf; t += 2) {
      step(s0, s1, f0, s2, s3, f1, t, std::true_type{});
      step(s2, s3, f1, s0, s1, f0, t + 1, std::true_type{});
    }
    if (t < tf) {
      step(s0, s1, f0, s2, s3, f1, t, std::true_type{});
      ++t;
    }
    if (t < t1) {
      if ((t - t0) & 1) step(s2, s3, f1, s0, s1, f0, t, std::false_type{});
      else step(s0, s1, f0, s2, s3, f1, t, std::false_type{});
    }
  }
  tim.flush(MEA_SYNC_COUNTERS(0), lane);

  if (a.Pdk != nullptr) {  // split: this range's fp32 partials, dK before its factor
    if (key < n_k) {
      const int64_t prow = (int64_t)sp * a.kv_rows * D + kbase + (int64_t)key * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int col = db * 32 + 8 * r4 + 4 * hi;
          f32x4 pv, pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pv[e] = accV[db][4 * r4 + e];
            pk[e] = accK[db][4 * r4 + e];
          }
          *reinterpret_cast<f32x4*>(a.Pdv + prow + col) = pv;
          *reinterpret_cast<f32x4*>(a.Pdk + prow + col) = pk;
        }
    }
    return;
  }
  if (key < n_k) {
    bf16* vrow = a.dV + kbase + (int64_t)key * D;
    bf16* krow_out = a.dK + kbase + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 wv, wk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wv[e] = (bf16)accV[db][4 * r4 + e];
          wk[e] = (bf16)(accK[db][4 * r4 + e] * a.scale);
        }
        *reinterpret_cast<bf16x4*>(vrow + db * 32 + 8 * r4 + 4 * hi) = wv;
        *reinterpret_cast<bf16x4*>(krow_out + db * 32 + 8 * r4 + 4 * hi) = wk;
      }
  }
}

// --- dQ role ------------------------------------------------------------------
template <int D, int W>
__device__ __forceinline__ void dq_role(const BwdArgs& a, int wg, bf16* s0, bf16* s1, bf16* s2,
                                        bf16* s3) {
  using L = Padded<D>;
  using TK = TileDma<D, kTileK, W>;
  constexpr int RS = L::kRowElems;
  constexpr int DK = D / 16;
  constexpr int DB = D / 32;
  constexpr int KB = kTileK / 32;
  constexpr int NC = kTileK / 16;

  const int n_q = a.n_q, n_k = a.n_k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int l32 = lane & 31, hi = lane >> 5;
  const int tile = xcd_remap(wg, a.total_q);  // ((bh * s_q) + sp) * tiles_q + qt
  const int bh = tile / (a.tiles_q * a.s_q);
  const int sp = (tile - bh * a.tiles_q * a.s_q) / a.tiles_q;  // range of key tiles
  const int qt = tile - (bh * a.s_q + sp) * a.tiles_q;
  const int64_t qbase = (int64_t)bh * n_q * D;  // Q, dO, dQ
  const int64_t kbase = (int64_t)bh * n_k * D;  // K, V
  const int row = qt * (32 * W) + wave * 32 + l32;  // this lane's query
  const int qrow = min(row, n_q - 1);

  bf16x8 qf[DK], of[DK];  // B operands of S^T = K Q^T and dP^T = V dO^T
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    qf[dk] = *reinterpret_cast<const bf16x8*>(a.Q + qbase + (int64_t)qrow * D + dk * 16 + 8 * hi);
    of[dk] = *reinterpret_cast<const bf16x8*>(a.dO + qbase + (int64_t)qrow * D + dk * 16 + 8 * hi);
  }
  const float lse = a.Lse2[(int64_t)bh * n_q + qrow];
  // -D of this query row, in every register: the first dP^T product reads it
  // as its accumulator input, so dP^T comes out as dP^T - D with no extra VALU.
  f32x16 ndv;
  {
    const float nd = a.Dv[(int64_t)bh * n_q + qrow];
#pragma unroll
    for (int r = 0; r < 16; ++r) ndv[r] = nd;
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  TK dma;
  dma.init(wave, lane);
  const int g = lane >> 4, jj = lane & 15;
  const int a_lane = L::off(l32, 8 * hi);
  const int t_lane = L::off(4 * hi + (jj >> 2), (g & 1) * 16 + 4 * (jj & 3));

  auto tile_body = [&](const bf16* ks, const bf16* vs, int j0, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    bf16x8 sf[NC];  // dS^T as B operand, same chunking as P^T in the forward
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16 s = f32x16{}, dp = ndv;
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) {
        const int off = a_lane + L::off(kb * 32, dk * 16);
        s = mfma32x32x16(lds_read_b128(ks + off), qf[dk], s);
        dp = mfma32x32x16(lds_read_b128(vs + off), of[dk], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[r], a.C, -lse));
        if constexpr (kMasked) {
          if (j0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3) >= n_k) p = 0.f;  // padding keys
        }
        sf[2 * kb + (r >> 3)][r & 7] = (bf16)(p * dp[r]);
      }
    }
    // dQ^T += K^T dS^T (A operand by transposed reads of the K tile)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int off = t_lane + L::off(c * 16, db * 32);
        const bf16x8 ak = cat(lds_read_tr16(ks + off), lds_read_tr16(ks + off + 8 * RS));
        acc[db] = mfma32x32x16(ak, sf[c], acc[db]);
      }
    }
  };

  // this workgroup's key tiles [t0, t1): all of them unless the backward is split
  const int t0 = sp * a.len_k;
  const int t1 = min(t0 + a.len_k, (n_k + kTileK - 1) / kTileK);
  SyncTimer tim;
  auto step = [&](const bf16* ks, const bf16* vs, bf16* kn, bf16* vn, int t, auto full_tag) {
    const int j0 = t * kTileK;
    if (t + 1 < t1) {
      dma.issue(a.K + kbase, j0 + kTileK, n_k, kn);
      dma.issue(a.V + kbase, j0 + kTileK, n_k, vn);
    }
    if constexpr (decltype(full_tag)::value) tile_body(ks, vs, j0, std::false_type{});
    else tile_body(ks, vs, j0, std::true_type{});
    tim.end_of_tile();
  };
  dma.issue(a.K + kbase, t0 * kTileK, n_k, s0);
  dma.issue(a.V + kbase, t0 * kTileK, n_k, s1);
  wait_all();
  __syncthreads();
  tim.start(wave, W);
  {  // full tiles in pairs, then at most one more and the ragged last tile
    const int tf = min(t1, n_k / kTileK);
    int t = t0;
    for (; t + 1 < tf; t += 2) {
      step(s0, s1, s2, s3, t, std::true_type{});
      step(s2, s3, s0, s1, t + 1, std::true_type{});
    }
    if (t < tf) {
      step(s0, s1, s2, s3, t, std::true_type{});
      ++t;
    }
    if (t < t1) {
      if ((t - t0) & 1) step(s2, s3, s0, s1, t, std::false_type{});
      else step(s0, s1, s2, s3, t, std::false_type{});
    }
  }
  tim.flush(MEA_SYNC_COUNTERS(1), lane);

  if (a.Pdq != nullptr) {  // split: this range's fp32 partial, before the 1/sqrt(d) factor
    if (row < n_q) {
      const int64_t prow = (int64_t)sp * a.q_rows * D + qbase + (int64_t)row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 pq;
#pragma unroll
          for (int e = 0; e < 4; ++e) pq[e] = acc[db][4 * r4 + e];
          *reinterpret_cast<f32x4*>(a.Pdq + prow + db * 32 + 8 * r4 + 4 * hi) = pq;
        }
    }
    return;
  }
  if (row < n_q) {
    bf16* qout = a.dQ + qbase + (int64_t)row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[db][4 * r4 + e] * a.scale);
        *reinterpret_cast<bf16x4*>(qout + db * 32 + 8 * r4 + 4 * hi) = w;
      }
  }
}

// two waves per SIMD (<= 256 registers): 8-wave workgroups one per CU, or
// 4-wave workgroups two per CU (d = 64; d = 128 has its own kernel above)
template <int D, int W>
__global__ __launch_bounds__(64 * W, 2) void bwd_main_kernel(BwdArgs a) {
  static_assert(D == 64, "d = 128 uses bwd_main128_kernel");
  // two named buffers per staged operand (see the forward kernel)
  __shared__ __attribute__((aligned(1024))) bf16 s0[BwdShared<D>::kElems];
  __shared__ __attribute__((aligned(1024))) bf16 s1[BwdShared<D>::kElems];
  __shared__ __attribute__((aligned(1024))) bf16 s2[BwdShared<D>::kElems];
  __shared__ __attribute__((aligned(1024))) bf16 s3[BwdShared<D>::kElems];
  __shared__ __attribute__((aligned(256))) float f0[2 * kTileQ];
  __shared__ __attribute__((aligned(256))) float f1[2 * kTileQ];
  const int wg = blockIdx.x;
  if (wg < a.total_kv) dkdv_role<D, W>(a, wg, s0, s1, s2, s3, f0, f1);
  else dq_role<D, W>(a, wg - a.total_kv, s0, s1, s2, s3);
}

// ------------------------------------------------------------ d = 128 roles
// 16 keys (dK/dV) or 16 queries (dQ) per wave on v_mfma_f32_16x16x32_bf16:
//   A: lane l holds A[l%16][8*(l/16) + e];  B: lane l holds B[8*(l/16) + e][l%16]
//   D: lane l, register r holds D[4*(l/16) + r][l%16]
// A wave's dV^T and dK^T (or dQ^T) for 16 rows take 64 (32) registers instead
// of 128 (64), so two waves fit per SIMD. Tiles are staged with their 16-byte
// chunks XOR-permuted by 2*row mod 16 (Layout128 below). The bank-conflict
// counter measured that layout conflict-free for both read patterns used here:
// 16-byte reads of 16 rows x 4 chunks, and transposed reads of 4 rows x 32 bytes
// per 16 lanes. The forward's layout (XOR by the bit-reversed row) costs these
// 16-byte reads four extra cycles each.
//
// The products dV^T += dO^T P and dK^T += Q^T dS contract over 32 query rows per
// MFMA; their k index 8*(l/16) + e stands for row 4*(l/16) + e (e < 4) or
// 16 + 4*(l/16) + e - 4 (e >= 4) of the 32-row chunk, which is the order in which
// a lane holds P and dS from two 16-row score blocks, and the order in which two
// transposed reads of 4 rows each deliver dO^T and Q^T.

// row-major 128-column bf16 tile, 16-byte chunk c of row r at position c ^ (2r mod 16);
// row offsets that are multiples of 8 keep the permutation
struct Layout128 {
  static constexpr int kChunks = 16;
  __device__ static constexpr int swz(int r) { return (2 * r) & 15; }
  __device__ static constexpr int off(int row, int col) {
    return row * 128 + (((col >> 3) ^ swz(row)) << 3) + (col & 7);
  }
};

// U: copies issued out of sight of the compiler's wait-count pass (dma16_untracked),
// used by the d = 128 dQ role (1.2-1.6% faster, identical results; the dK/dV role
// spills with them)
template <int ROWS, int WAVES, bool U = false>
struct SwzDma128 {
  using L = Layout128;
  static constexpr int kBlocks = ROWS * L::kChunks / 64;
  static constexpr int kPerWave = (kBlocks + WAVES - 1) / WAVES;
  static_assert(kBlocks * 64 == ROWS * L::kChunks, "tile must be whole DMA blocks");
  static constexpr int kElems = ROWS * 128;
  int row[kPerWave];
  int col[kPerWave];
  int wave;
  __device__ void init(int wave_, int lane) {
    wave = wave_;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int slot = (wave + WAVES * i) * 64 + lane;
      const int r = slot / L::kChunks;
      const int pc = slot - r * L::kChunks;
      row[i] = r;
      col[i] = (pc ^ L::swz(r)) * 8;
    }
  }
  // rows r0 .. r0+ROWS-1 of src (row stride 128) into dst; rows past n repeat row n-1
  __device__ void issue(const bf16* src, int r0, int n, bf16* dst) const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int b = wave + WAVES * i;
      if (b < kBlocks) {
        const int sr = min(r0 + row[i], n - 1);
        if constexpr (U) dma16_untracked(src + (int64_t)sr * 128 + col[i], dst + b * 512);
        else dma16(src + (int64_t)sr * 128 + col[i], dst + b * 512);
      }
    }
  }
};

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int W>
__device__ __forceinline__ void dkdv_role128(const BwdArgs& a, int wg, bf16* s0, bf16* s1,
                                             bf16* s2, bf16* s3, float* f0, float* f1) {
  constexpr int D = 128;
  using L = Layout128;
  using TQ = SwzDma128<kTileQ, W>;
  constexpr int DK = D / 32;        // k-steps of the score products
  constexpr int DB = D / 16;        // 16-row blocks of dV^T, dK^T
  constexpr int NC = kTileQ / 32;   // 32-row chunks (k-steps of dV, dK products)

  const int n_q = a.n_q, n_k = a.n_k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int l16 = lane & 15, g = lane >> 4;
  const int tile = xcd_remap(wg, a.total_kv);  // ((bh * s_kv) + sp) * tiles_kv + kt
  const int bh = tile / (a.tiles_kv * a.s_kv);
  const int sp = (tile - bh * a.tiles_kv * a.s_kv) / a.tiles_kv;  // range of query tiles
  const int kt = tile - (bh * a.s_kv + sp) * a.tiles_kv;
  const int64_t qbase = (int64_t)bh * n_q * D;
  const int64_t kbase = (int64_t)bh * n_k * D;
  const int64_t rbase = (int64_t)bh * n_q;
  const int key = kt * (16 * W) + wave * 16 + l16;  // this lane's key (column of S)

  // K and V of this wave's 16 keys: B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[DK], vf[DK];
  const int krow = min(key, n_k - 1);
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    kf[dk] = *reinterpret_cast<const bf16x8*>(a.K + kbase + (int64_t)krow * D + dk * 32 + 8 * g);
    vf[dk] = *reinterpret_cast<const bf16x8*>(a.V + kbase + (int64_t)krow * D + dk * 32 + 8 * g);
  }
  f32x4 accV[DB], accK[DB];  // dV^T, dK^T: register r of block db -> column 16*db + 4*g + r
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    accV[db] = f32x4{};
    accK[db] = f32x4{};
  }

  TQ dma;
  dma.init(wave, lane);
  auto issue = [&](bf16* qdst, bf16* odst, float* fdst, int i0) {
    dma.issue(a.Q + qbase, i0, n_q, qdst);
    dma.issue(a.dO + qbase, i0, n_q, odst);
    if (wave == W - 1) {
      const int r = min(i0 + lane, n_q - 1);
      dma4(a.Lse2 + rbase + r, fdst);
      dma4(a.Dv + rbase + r, fdst + kTileQ);
    }
  };

  // per-lane element offsets (row blocks of 16 rows keep the swizzle):
  // row reads of row l16, columns 32*dk + 8*g; transposed reads of rows
  // 4*g + l16/4 (and 16 below), columns 16*db + 4*(l16%4)
  int a_off[DK], t_off[DB];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) a_off[dk] = L::off(l16, dk * 32 + 8 * g);
#pragma unroll
  for (int db = 0; db < DB; ++db) t_off[db] = L::off(4 * g + (l16 >> 2), db * 16 + 4 * (l16 & 3));

  auto tile_body = [&](const bf16* qs, const bf16* os, const float* fs, int i0, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 pf, sf;  // P and dS of query rows 32c + {4g .. 4g+3, 16+4g .. 16+4g+3}
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qb = 2 * c + h;
        // lane holds key `key`; register r holds query row i0 + 16*qb + 4*g + r.
        // The dP accumulator starts at -D of its row, so it ends at dP - D.
        f32x4 s = f32x4{};
        f32x4 dp = *reinterpret_cast<const f32x4*>(fs + kTileQ + qb * 16 + 4 * g);
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
          const int off = a_off[dk] + qb * 16 * D;
          s = mfma16x16x32(lds_read_b128(qs + off), kf[dk], s);
          dp = mfma16x16x32(lds_read_b128(os + off), vf[dk], dp);
        }
        const f32x4 lse = *reinterpret_cast<const f32x4*>(fs + qb * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], a.C, -lse[r]));
          if constexpr (kMasked) {
            if (i0 + qb * 16 + 4 * g + r >= n_q) p = 0.f;  // padding query rows
          }
          pf[4 * h + r] = (bf16)p;
          sf[4 * h + r] = (bf16)(p * dp[r]);
        }
      }
      // dV^T += dO^T P,  dK^T += Q^T dS over the 32 rows of chunk c
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int o0 = t_off[db] + c * 32 * D, o1 = o0 + 16 * D;
        const bf16x8 ao = cat(lds_read_tr16(os + o0), lds_read_tr16(os + o1));
        const bf16x8 aq = cat(lds_read_tr16(qs + o0), lds_read_tr16(qs + o1));
        accV[db] = mfma16x16x32(ao, pf, accV[db]);
        accK[db] = mfma16x16x32(aq, sf, accK[db]);
      }
    }
  };

  // this workgroup's query tiles [t0, t1): all of them unless the backward is split
  const int t0 = sp * a.len_q;
  const int t1 = min(t0 + a.len_q, (n_q + kTileQ - 1) / kTileQ);
  SyncTimer tim;
  auto step = [&](const bf16* qs, const bf16* os, const float* fs, bf16* qn, bf16* on, float* fn,
                  int t, auto full_tag) {
    const int i0 = t * kTileQ;
    if (t + 1 < t1) issue(qn, on, fn, i0 + kTileQ);
    if constexpr (decltype(full_tag)::value) tile_body(qs, os, fs, i0, std::false_type{});
    else tile_body(qs, os, fs, i0, std::true_type{});
    tim.end_of_tile();
  };
  if (t1 > t0) {  // no query rows at all: dK = dV = 0
    issue(s0, s1, f0, t0 * kTileQ);
    wait_all();
    __syncthreads();
  }
  tim.start(wave, W);
  {  // full tiles in pairs, then at most one more and the ragged last tile (as above)
    const int tf = min(t1, n_q / kTileQ);
    int t = t0;
    for (; t + 1 < tf; t += 2) {
      step(s0, s1, f0, s2, s3, f1, t, std::true_type{});
      step(s2, s3, f1, s0, s1, f0, t + 1, std::true_type{});
    }
    if (t < tf) {
      step(s0, s1, f0, s2, s3, f1, t, std::true_type{});
      ++t;
    }
    if (t < t1) {
      if ((t - t0) & 1) step(s2, s3, f1, s0, s1, f0, t, std::false_type{});
      else step(s0, s1, f0, s2, s3, f1, t, std::false_type{});
    }
  }
  tim.flush(MEA_SYNC_COUNTERS(2), lane);

  if (a.Pdk != nullptr) {  // split: this range's fp32 partials, dK before its factor
    if (key < n_k) {
      const int64_t prow = (int64_t)sp * a.kv_rows * D + kbase + (int64_t)key * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        *reinterpret_cast<f32x4*>(a.Pdv + prow + db * 16 + 4 * g) = accV[db];
        *reinterpret_cast<f32x4*>(a.Pdk + prow + db * 16 + 4 * g) = accK[db];
      }
    }
    return;
  }
  if (key < n_k) {
    bf16* vrow = a.dV + kbase + (int64_t)key * D;
    bf16* krow_out = a.dK + kbase + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x4 wv, wk;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wv[r] = (bf16)accV[db][r];
        wk[r] = (bf16)(accK[db][r] * a.scale);
      }
      *reinterpret_cast<bf16x4*>(vrow + db * 16 + 4 * g) = wv;
      *reinterpret_cast<bf16x4*>(krow_out + db * 16 + 4 * g) = wk;
    }
  }
}

template <int W>
__device__ __forceinline__ void dq_role128(const BwdArgs& a, int wg, bf16* s0, bf16* s1, bf16* s2,
                                           bf16* s3) {
  constexpr int D = 128;
  using L = Layout128;
  using TK = SwzDma128<kTileK, W, true>;
  constexpr int DK = D / 32;
  constexpr int DB = D / 16;
  constexpr int NC = kTileK / 32;  // 32-key chunks (k-steps of the dQ product)

  const int n_q = a.n_q, n_k = a.n_k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int l16 = lane & 15, g = lane >> 4;
  const int tile = xcd_remap(wg, a.total_q);  // ((bh * s_q) + sp) * tiles_q + qt
  const int bh = tile / (a.tiles_q * a.s_q);
  const int sp = (tile - bh * a.tiles_q * a.s_q) / a.tiles_q;  // range of key tiles
  const int qt = tile - (bh * a.s_q + sp) * a.tiles_q;
  const int64_t qbase = (int64_t)bh * n_q * D;
  const int64_t kbase = (int64_t)bh * n_k * D;
  const int row = qt * (16 * W) + wave * 16 + l16;  // this lane's query
  const int qrow = min(row, n_q - 1);

  bf16x8 qf[DK], of[DK];  // B operands of S^T = K Q^T and dP^T = V dO^T
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    qf[dk] = *reinterpret_cast<const bf16x8*>(a.Q + qbase + (int64_t)qrow * D + dk * 32 + 8 * g);
    of[dk] = *reinterpret_cast<const bf16x8*>(a.dO + qbase + (int64_t)qrow * D + dk * 32 + 8 * g);
  }
  const float lse = a.Lse2[(int64_t)bh * n_q + qrow];
  const float nd = a.Dv[(int64_t)bh * n_q + qrow];
  const f32x4 ndv = f32x4{nd, nd, nd, nd};  // -D: the first dP^T product's accumulator

  f32x4 acc[DB];  // dQ^T: register r of block db -> column 16*db + 4*g + r
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4{};

  TK dma;
  dma.init(wave, lane);
  int a_off[DK], t_off[DB];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) a_off[dk] = L::off(l16, dk * 32 + 8 * g);
#pragma unroll
  for (int db = 0; db < DB; ++db) t_off[db] = L::off(4 * g + (l16 >> 2), db * 16 + 4 * (l16 & 3));

  auto tile_body = [&](const bf16* ks, const bf16* vs, int j0, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 sf;  // dS^T of keys 32c + {4g .. 4g+3, 16+4g .. 16+4g+3}
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = 2 * c + h;
        f32x4 s = f32x4{}, dp = ndv;
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
          const int off = a_off[dk] + kb * 16 * D;
          s = mfma16x16x32(lds_read_b128(ks + off), qf[dk], s);
          dp = mfma16x16x32(lds_read_b128(vs + off), of[dk], dp);
        }
        // the exponentials and dS of a block at raised issue priority in 8-wave
        // workgroups: the wave in them wins VALU issue over the other wave of its
        // SIMD, whose MFMAs keep the matrix pipe busy meanwhile (1% faster at
        // 1 x 16 x 8192 x 128 and 2 x 32 x 2048 x 128 with identical results; 1%
        // slower with 4-wave workgroups; the dK/dV role spills with it)
        if constexpr (W == 8) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], a.C, -lse));
          if constexpr (kMasked) {
            if (j0 + kb * 16 + 4 * g + r >= n_k) p = 0.f;  // padding keys
          }
          sf[4 * h + r] = (bf16)(p * dp[r]);
        }
        if constexpr (W == 8) __builtin_amdgcn_s_setprio(0);
      }
      // dQ^T += K^T dS^T over the 32 keys of chunk c
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int o0 = t_off[db] + c * 32 * D, o1 = o0 + 16 * D;
        const bf16x8 ak = cat(lds_read_tr16(ks + o0), lds_read_tr16(ks + o1));
        acc[db] = mfma16x16x32(ak, sf, acc[db]);
      }
    }
  };

  // this workgroup's key tiles [t0, t1): all of them unless the backward is split
  const int t0 = sp * a.len_k;
  const int t1 = min(t0 + a.len_k, (n_k + kTileK - 1) / kTileK);
  SyncTimer tim;
  auto step = [&](const bf16* ks, const bf16* vs, bf16* kn, bf16* vn, int t, auto full_tag) {
    const int j0 = t * kTileK;
    if (t + 1 < t1) {
      dma.issue(a.K + kbase, j0 + kTileK, n_k, kn);
      dma.issue(a.V + kbase, j0 + kTileK, n_k, vn);
    }
    if constexpr (decltype(full_tag)::value) tile_body(ks, vs, j0, std::false_type{});
    else tile_body(ks, vs, j0, std::true_type{});
    tim.end_of_tile();
  };
  dma.issue(a.K + kbase, t0 * kTileK, n_k, s0);
  dma.issue(a.V + kbase, t0 * kTileK, n_k, s1);
  wait_all();
  __syncthreads();
  tim.start(wave, W);
  {  // full tiles in pairs, then at most one more and the ragged last tile
    const int tf = min(t1, n_k / kTileK);
    int t = t0;
    for (; t + 1 < tf; t += 2) {
      step(s0, s1, s2, s3, t, std::true_type{});
      step(s2, s3, s0, s1, t + 1, std::true_type{});
    }
    if (t < tf) {
      step(s0, s1, s2, s3, t, std::true_type{});
      ++t;
    }
    if (t < t1) {
      if ((t - t0) & 1) step(s2, s3, s0, s1, t, std::false_type{});
      else step(s0, s1, s2, s3, t, std::false_type{});
    }
  }
  tim.flush(MEA_SYNC_COUNTERS(3), lane);

  if (a.Pdq != nullptr) {  // split: this range's fp32 partial, before the 1/sqrt(d) factor
    if (row < n_q) {
      const int64_t prow = (int64_t)sp * a.q_rows * D + qbase + (int64_t)row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(a.Pdq + prow + db * 16 + 4 * g) = acc[db];
    }
    return;
  }
  if (row < n_q) {
    bf16* qout = a.dQ + qbase + (int64_t)row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (bf16)(acc[db][r] * a.scale);
      *reinterpret_cast<bf16x4*>(qout + db * 16 + 4 * g) = w;
    }
  }
}

template <int W>
__global__ __launch_bounds__(64 * W, 2) void bwd_main128_kernel(BwdArgs a) {
  constexpr int kElems = SwzDma128<kTileQ, W>::kElems;
  static_assert(SwzDma128<kTileK, W>::kElems == kElems, "both roles share the LDS arrays");
  __shared__ __attribute__((aligned(1024))) bf16 s0[kElems];
  __shared__ __attribute__((aligned(1024))) bf16 s1[kElems];
  __shared__ __attribute__((aligned(1024))) bf16 s2[kElems];
  __shared__ __attribute__((aligned(1024))) bf16 s3[kElems];
  __shared__ __attribute__((aligned(256))) float f0[2 * kTileQ];
  __shared__ __attribute__((aligned(256))) float f1[2 * kTileQ];
  const int wg = blockIdx.x;
  if (wg < a.total_kv) dkdv_role128<W>(a, wg, s0, s1, s2, s3, f0, f1);
  else dq_role128<W>(a, wg - a.total_kv, s0, s1, s2, s3);
}

// Split fields of the kernel arguments; an unsplit side sweeps every tile.
void set_split(BwdArgs& a, const BwdProblem& p) {
  const bool kv = p.split.kv > 1, q = p.split.q > 1;
  a.s_kv = kv ? p.split.kv : 1;
  a.len_q = kv ? p.split.len_q : (p.rows_q + kTileQ - 1) / kTileQ;
  a.s_q = q ? p.split.q : 1;
  a.len_k = q ? p.split.len_k : (p.n_k + kTileK - 1) / kTileK;
  a.Pdk = kv ? p.part_dk : nullptr;
  a.Pdv = kv ? p.part_dv : nullptr;
  a.Pdq = q ? p.part_dq : nullptr;
  a.kv_rows = p.heads * p.n_k;
  a.q_rows = p.heads * p.rows_q;
  a.total_kv = (int)(p.heads * a.tiles_kv * a.s_kv);
  a.total_q = (int)(p.heads * a.tiles_q * a.s_q);
}

template <int D, int W>
hipError_t launch(const BwdProblem& p, hipStream_t stream) {
  const int64_t rows = p.heads * p.rows_q;
  float* Dv = p.ws;
  float* Lse2 = p.ws + rows;
  if (rows > 0) {
    const unsigned blocks = row_blocks(rows, kThreads / (D / 8));
    hipLaunchKernelGGL((bwd_rows_kernel<D>), dim3(blocks), dim3(kThreads), 0, stream,
                       (const bf16*)p.o, (const bf16*)p.dO, p.m, p.l, Dv, Lse2, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs a;
  a.Q = (const bf16*)p.q;
  a.K = (const bf16*)p.k;
  a.V = (const bf16*)p.v;
  a.dO = (const bf16*)p.dO;
  a.Dv = Dv;
  a.Lse2 = Lse2;
  a.dQ = (bf16*)p.dq;
  a.dK = (bf16*)p.dk;
  a.dV = (bf16*)p.dv;
  a.n_q = p.rows_q;
  a.n_k = p.n_k;
  a.tiles_kv = (p.n_k + 32 * W - 1) / (32 * W);
  a.tiles_q = (p.rows_q + 32 * W - 1) / (32 * W);
  set_split(a, p);
  a.scale = 1.0f / sqrtf((float)D);
  a.C = kLog2e * a.scale;
  hipLaunchKernelGGL((bwd_main_kernel<D, W>), dim3((unsigned)(a.total_kv + a.total_q)), dim3(64 * W),
                     0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_bwd_reduce(true, D, p, stream);
}

}  // namespace

template <int W>
hipError_t launch128(const BwdProblem& p, hipStream_t stream) {
  constexpr int D = 128;
  const int64_t rows = p.heads * p.rows_q;
  float* Dv = p.ws;
  float* Lse2 = p.ws + rows;
  if (rows > 0) {
    const unsigned blocks = row_blocks(rows, kThreads / (D / 8));
    hipLaunchKernelGGL((bwd_rows_kernel<D>), dim3(blocks), dim3(kThreads), 0, stream,
                       (const bf16*)p.o, (const bf16*)p.dO, p.m, p.l, Dv, Lse2, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs a;
  a.Q = (const bf16*)p.q;
  a.K = (const bf16*)p.k;
  a.V = (const bf16*)p.v;
  a.dO = (const bf16*)p.dO;
  a.Dv = Dv;
  a.Lse2 = Lse2;
  a.dQ = (bf16*)p.dq;
  a.dK = (bf16*)p.dk;
  a.dV = (bf16*)p.dv;
  a.n_q = p.rows_q;
  a.n_k = p.n_k;
  a.tiles_kv = (p.n_k + 16 * W - 1) / (16 * W);
  a.tiles_q = (p.rows_q + 16 * W - 1) / (16 * W);
  set_split(a, p);
  a.scale = 1.0f / sqrtf((float)D);
  a.C = kLog2e * a.scale;
  hipLaunchKernelGGL((bwd_main128_kernel<W>), dim3((unsigned)(a.total_kv + a.total_q)),
                     dim3(64 * W), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_bwd_reduce(true, D, p, stream);
}

static_assert(kTileQ == kTileK, "one staged tile size for both roles");
BwdGeometry bwd_geometry_bf16(int d) {
  return BwdGeometry{(d == 64 ? 32 : 16) * kWaves, kTileQ};
}

hipError_t launch_bwd_bf16(int d, const BwdProblem& p, hipStream_t stream) {
  // 8-wave workgroups serve each staged tile to twice the rows (measured 3-4%
  // faster at d = 64) but halve the workgroup count: only on grids that still
  // give every CU one
  const int64_t rows = (d == 64 ? 32 : 16) * kWideWaves;
  const int64_t wide_grid = p.heads * ((p.n_k + rows - 1) / rows + (p.rows_q + rows - 1) / rows);
  const bool wide = wide_grid >= kComputeUnits;
  if (d == 128) return wide ? launch128<kWideWaves>(p, stream) : launch128<kWaves>(p, stream);
  return wide ? launch<64, kWideWaves>(p, stream) : launch<64, kWaves>(p, stream);
}

}  // namespace mea

#if MEA_SYNC_TIMERS
// Timing library only: copies the backward's 4 x 7 synchronisation counters to
// `out` (host memory) after a device synchronisation, and clears them if
// `reset`. Returns 0 or the failing hipError_t.
extern "C" __attribute__((visibility("default"))) int mea_sync_timers_bwd(unsigned long long* out,
                                                                        int reset) {
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpyFromSymbol(out, HIP_SYMBOL(mea::g_sync), sizeof(mea::g_sync));
  if (e == hipSuccess && reset) {
    const unsigned long long zero[4][mea::kSyncCounters] = {};
    e = hipMemcpyToSymbol(HIP_SYMBOL(mea::g_sync), zero, sizeof(zero));
    if (e == hipSuccess) e = hipDeviceSynchronize();
  }
  return (int)e;
}
#endif
