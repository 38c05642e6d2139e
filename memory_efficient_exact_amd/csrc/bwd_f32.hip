// Backward attention for fp32 inputs on gfx950, by recomputation, with scores
// formed in fp64.
//
// Method and formulas as in the bf16 backward (bwd_bf16.hip): the forward
// keeps two numbers per query row, the probability tiles are rebuilt from
// them ("Self-attention Does Not Need O(n^2) Memory": abstract; 方法详解;
// English digest method bullets), and the gradients are the textbook softmax
// Jacobian: dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij, dS = P * (dP - D),
// dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).
//
// Precision (the 1e-5 bar of fp32 inputs). As in the fp32 forward, an fp32
// product is exact in fp64, so S runs on fp64 MFMA (16x16x4) and the exponent
// x * log2(e)/sqrt(d) - lse2 is formed in fp64 (at scores of ~1e4 an fp32
// exponent would carry errors of ~1e-3). dP also runs on fp64 MFMA and D is
// kept in fp64: dP - D cancels wherever P is concentrated (with a single key
// it is exactly 0), and in fp32 the residue of that cancellation, summed over
// many query rows into dK, reaches the tolerance. For the same reason D is not
// taken from the caller's O (dO_i . O_i) but formed from the probabilities this
// backward itself rebuilds, D_i = sum_j P_ij dP_ij / sum_j P_ij in fp64 (the D
// pass below), so that every row of dS sums to zero; with D from an fp32 O the
// rounding of O alone moved dQ by up to 7e-6 at the x30 stress scale. The
// weights, dS and the three gradient products are fp32 (fp32 MFMA 16x16x4).
// lse2 = m*log2(e) + log2(l) is formed per row in fp64 from the forward's
// statistics; the fp32 forward reports l relative to its reported (rounded)
// m, so the pair reproduces the row's log-sum-exp to fp32 rounding of l alone.
//
// Launches on the caller's stream (the caller's O is not read):
//  1. bwd_dterm_f32: the row terms {lse2, -D} (fp64), D by a sweep over all
//     keys of the row's head that forms S, dP and P as the main kernel does.
//     On a split grid (below) the sweep is cut into the dQ workgroups' key
//     ranges; each range leaves its fp64 sums of P and P*dP, and
//     bwd_dterm_merge_f32 adds them per row in range order.
//  2. bwd_main_f32: dK/dV workgroups (64 keys, 16 per wave, K and V of the
//     wave's keys in registers) sweeping 32-row query tiles of Q, dO and the
//     row terms staged in LDS; then dQ workgroups (64 queries, Q and dO in
//     registers) sweeping 32-key tiles of K, V. Every output element is
//     written once by one workgroup. On grids of at most 256 workgroups, when
//     the caller's workspace holds them, each workgroup position repeats for
//     several ranges of its sweep and writes fp32 partial sums that a reduce
//     pass (bwd_reduce.hip) adds in a fixed order.
//
// Occupancy. The register operands are held in fp32 and widened to fp64 at
// each use (exact), and each tile goes through one LDS buffer, written
// between two barriers, with no copy of the next tile kept in flight. That
// brings d = 128 to 256 registers (two waves per SIMD, against one when the
// operands were held in fp64 and the next tile was staged during compute)
// and d = 64 to three waves: 11% and 8% faster, with identical results.
//
// Lane layouts (mea_device.h): S and dP (fp64 products) leave lane l,
// register r at row 4r + l/16 of a 16-row block and column l%16; that
// register is exactly the B operand lane l supplies for k-step r of the fp32
// gradient products, whose k-step r covers rows 4r .. 4r + 3.
#include "mea_device.h"
#include "mea_launch.h"

namespace mea {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16 * kWaves;  // keys per dK/dV workgroup = queries per dQ workgroup
constexpr int kTile = 32;           // staged rows per tile (two 16-row blocks)

// per query row: lse2 = m*log2(e) + log2(l) and -D, both fp64; 16 bytes
struct RowTerm {
  double lse2;
  double neg_d;
};
static_assert(sizeof(RowTerm) == 16, "row term layout");

// ------------------------------------------------------------ 1. row terms
// lse2 = m*log2(e) + log2(l) in fp64 from the forward's statistics. The D pass
// and the merge of its split ranges both form it with this one function, so
// the two paths store the same value.
__device__ __forceinline__ double row_lse2(float m, float l) {
  return (double)m * 1.4426950408889634 + log2((double)l);
}

// ------------------------------------------------------------ 2. main kernel
struct BwdArgs32 {
  const float* Q;   // [heads, n_q, D]
  const float* K;   // [heads, n_k, D]
  const float* V;
  const float* dO;  // [heads, n_q, D]
  const RowTerm* T; // [heads, n_q]
  float* dQ;
  float* dK;
  float* dV;
  int n_q;
  int n_k;
  int tiles_kv;  // dK/dV workgroups per head
  int tiles_q;   // dQ workgroups per head
  int total_kv;
  int total_q;
  double C64;      // log2(e) / sqrt(D)
  double scale64;  // 1 / sqrt(D)
  // split backward (small grids), as in the bf16 kernels: s_kv ranges of len_q
  // query tiles per dK/dV position, s_q ranges of len_k key tiles per dQ
  // position; a split side writes fp32 partials (before the 1/sqrt(d) factor)
  int s_kv;
  int len_q;
  int s_q;
  int len_k;
  float* Pdk;      // [s_kv][kv_rows][D] or null
  float* Pdv;
  float* Pdq;      // [s_q][q_rows][D] or null
  int64_t kv_rows;  // heads * n_k
  int64_t q_rows;   // heads * n_q
};

template <int D>
struct Shared32 {
  static constexpr int kStride = D + 4;          // row stride (floats): 16-byte pad
  static constexpr int kElems = kTile * kStride;  // floats per staged tile
  static constexpr int kLoads = kTile * D / 4 / kThreads;  // 16-byte loads per thread per tile
  static_assert(kLoads * 4 * kThreads == kTile * D, "tile split");
};

// Register-staged copy of a kTile x D fp32 tile (rows past `rows` read as 0).
template <int D>
struct Stage {
  u32x4 r[Shared32<D>::kLoads];
  __device__ __forceinline__ void load(const float* src, int row0, int rows, int tid) {
    constexpr int kCPR = D / 4;
#pragma unroll
    for (int i = 0; i < Shared32<D>::kLoads; ++i) {
      const int c = tid + i * kThreads;
      const int rr = c / kCPR;
      const int ch = c - rr * kCPR;
      r[i] = row0 + rr < rows ? *reinterpret_cast<const u32x4*>(src + (int64_t)(row0 + rr) * D + ch * 4)
                              : u32x4{};
    }
  }
  __device__ __forceinline__ void store(float* dst, int tid) const {
    constexpr int kCPR = D / 4;
#pragma unroll
    for (int i = 0; i < Shared32<D>::kLoads; ++i) {
      const int c = tid + i * kThreads;
      const int rr = c / kCPR;
      const int ch = c - rr * kCPR;
      *reinterpret_cast<u32x4*>(dst + rr * Shared32<D>::kStride + ch * 4) = r[i];
    }
  }
};

// --- dK / dV role -------------------------------------------------------------
template <int D>
__device__ __forceinline__ void dkdv_role32(const BwdArgs32& a, int wg, float* sQ, float* sO,
                                            RowTerm* sT) {
  constexpr int S = Shared32<D>::kStride;
  constexpr int KK = D / 4;   // k-steps over the head dimension
  constexpr int CB = D / 16;  // 16-column output blocks
  const int n_k = a.n_k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int tile = xcd_remap(wg, a.total_kv);  // ((bh * s_kv) + sp) * tiles_kv + kt
  const int bh = tile / (a.tiles_kv * a.s_kv);
  const int sp = (tile - bh * a.tiles_kv * a.s_kv) / a.tiles_kv;  // range of query tiles
  const int kt = tile - (bh * a.s_kv + sp) * a.tiles_kv;
  // this workgroup's query rows start at q_off (0 unless the backward is split); the
  // sweep addresses them from there, so its loop keeps the unsplit form
  const int q_off = sp * a.len_q * kTile;
  const int n_q = a.n_q - q_off;  // query rows from the range's first on
  const float* Qh = a.Q + ((int64_t)bh * a.n_q + q_off) * D;
  const float* dOh = a.dO + ((int64_t)bh * a.n_q + q_off) * D;
  const RowTerm* Th = a.T + (int64_t)bh * a.n_q + q_off;
  const int64_t kbase = (int64_t)bh * n_k * D;
  const int key = kt * kRows + wave * 16 + l16;  // this lane's key (column of S)
  const int krow = min(key, n_k - 1);

  // B operands: K^T for S = Q K^T, V^T for dP = dO V^T, widened to fp64 at each use
  float kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    kf[kk] = a.K[kbase + (int64_t)krow * D + 4 * kk + g4];
    vf[kk] = a.V[kbase + (int64_t)krow * D + 4 * kk + g4];
  }
  // dV^T, dK^T accumulated in fp64 (fp64 MFMA): register r <-> column 16*cb + 4*r + g4
  f64x4 accV[CB], accK[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    accV[cb] = f64x4{};
    accK[cb] = f64x4{};
  }

  const int ntiles = min(a.len_q, (n_q + kTile - 1) / kTile);  // tiles of this range
  Stage<D> stQ, stO;
  RowTerm stT;
  auto gload = [&](int i0) {
    stQ.load(Qh, i0, n_q, tid);
    stO.load(dOh, i0, n_q, tid);
    if (tid < kTile) stT = i0 + tid < n_q ? Th[i0 + tid] : RowTerm{0.0, 0.0};
  };
  auto swrite = [&]() {
    stQ.store(sQ, tid);
    stO.store(sO, tid);
    if (tid < kTile) sT[tid] = stT;
  };
  if (ntiles > 0) {  // no query rows at all: dK = dV = 0
    gload(0);
    swrite();
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int i0 = t * kTile;
    const float* qs = sQ;
    const float* os = sO;
    const RowTerm* ts = sT;
#pragma unroll
    for (int qb = 0; qb < kTile / 16; ++qb) {
      // S[q][key] and dP[q][key] (fp64): lane holds key l16, register r <-> query 16qb + 4r + g4
      f64x4 s = f64x4{}, dp = f64x4{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int off = (16 * qb + l16) * S + 4 * kk + g4;
        s = mfma_f64_16x16x4((double)qs[off], (double)kf[kk], s);
        dp = mfma_f64_16x16x4((double)os[off], (double)vf[kk], dp);
      }
      float p[4], ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = 16 * qb + 4 * r + g4;
        const RowTerm rt = ts[q];
        p[r] = fast_exp2((float)(s[r] * a.C64 - rt.lse2));
        if (i0 + q >= n_q) p[r] = 0.f;  // padding query rows
        ds[r] = p[r] * (float)(dp[r] + rt.neg_d);
      }
      // dV^T += dO^T P, dK^T += Q^T dS: k-step r covers queries 16qb + 4r .. + 3
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = 16 * qb + 4 * r + g4;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          accV[cb] = mfma_f64_16x16x4((double)os[q * S + 16 * cb + l16], (double)p[r], accV[cb]);
          accK[cb] = mfma_f64_16x16x4((double)qs[q * S + 16 * cb + l16], (double)ds[r], accK[cb]);
        }
      }
    }
    if (t + 1 < ntiles) {
      __syncthreads();
      gload(i0 + kTile);
      swrite();
    }
    __syncthreads();
  }

  // outputs, or (split) this range's fp32 partials with dK before its factor: the
  // same stores into other rows, chosen by workgroup-uniform values
  const bool part = a.Pdk != nullptr;
  float* vout_base = part ? a.Pdv + (int64_t)sp * a.kv_rows * D : a.dV;
  float* kout_base = part ? a.Pdk + (int64_t)sp * a.kv_rows * D : a.dK;
  const double kscale = part ? 1.0 : a.scale64;
  if (key < n_k) {
    float* vrow = vout_base + kbase + (int64_t)key * D;
    float* krow_out = kout_base + kbase + (int64_t)key * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vrow[16 * cb + 4 * r + g4] = (float)accV[cb][r];
        krow_out[16 * cb + 4 * r + g4] = (float)(accK[cb][r] * kscale);
      }
  }
}

// --- dQ role --------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void dq_role32(const BwdArgs32& a, int wg, float* sK, float* sV) {
  constexpr int S = Shared32<D>::kStride;
  constexpr int KK = D / 4;
  constexpr int CB = D / 16;
  const int n_q = a.n_q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int tile = xcd_remap(wg, a.total_q);  // ((bh * s_q) + sp) * tiles_q + qt
  const int bh = tile / (a.tiles_q * a.s_q);
  const int sp = (tile - bh * a.tiles_q * a.s_q) / a.tiles_q;  // range of key tiles
  const int qt = tile - (bh * a.s_q + sp) * a.tiles_q;
  const int64_t qbase = (int64_t)bh * n_q * D;
  // this workgroup's keys start at k_off (0 unless the backward is split); the sweep
  // addresses them from there, so its loop keeps the unsplit form
  const int k_off = sp * a.len_k * kTile;
  const int n_k = a.n_k - k_off;  // keys from the range's first on
  const float* Kh = a.K + ((int64_t)bh * a.n_k + k_off) * D;
  const float* Vh = a.V + ((int64_t)bh * a.n_k + k_off) * D;
  const int row = qt * kRows + wave * 16 + l16;  // this lane's query
  const int qrow = min(row, n_q - 1);

  // B operands: Q^T for S^T = K Q^T, dO^T for dP^T = V dO^T, widened to fp64 at each use
  float qf[KK], of[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qf[kk] = a.Q[qbase + (int64_t)qrow * D + 4 * kk + g4];
    of[kk] = a.dO[qbase + (int64_t)qrow * D + 4 * kk + g4];
  }
  const RowTerm rt = a.T[(int64_t)bh * n_q + qrow];
  f64x4 acc[CB];  // dQ^T in fp64 (fp64 MFMA): register r <-> column 16*cb + 4*r + g4
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f64x4{};

  const int ntiles = min(a.len_k, (n_k + kTile - 1) / kTile);  // tiles of this range
  Stage<D> stK, stV;
  auto gload = [&](int j0) {
    stK.load(Kh, j0, n_k, tid);
    stV.load(Vh, j0, n_k, tid);
  };
  auto swrite = [&]() {
    stK.store(sK, tid);
    stV.store(sV, tid);
  };
  gload(0);
  swrite();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kTile;
    const float* ks = sK;
    const float* vs = sV;
#pragma unroll
    for (int kb = 0; kb < kTile / 16; ++kb) {
      // S^T[key][q] and dP^T (fp64): lane holds query l16, register r <-> key 16kb + 4r + g4
      f64x4 s = f64x4{}, dp = f64x4{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int off = (16 * kb + l16) * S + 4 * kk + g4;
        s = mfma_f64_16x16x4((double)ks[off], (double)qf[kk], s);
        dp = mfma_f64_16x16x4((double)vs[off], (double)of[kk], dp);
      }
      float ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = fast_exp2((float)(s[r] * a.C64 - rt.lse2));
        if (j0 + 16 * kb + 4 * r + g4 >= n_k) p = 0.f;  // padding keys
        ds[r] = p * (float)(dp[r] + rt.neg_d);
      }
      // dQ^T += K^T dS^T: k-step r covers keys 16kb + 4r .. + 3
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kr = 16 * kb + 4 * r + g4;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[cb] = mfma_f64_16x16x4((double)ks[kr * S + 16 * cb + l16], (double)ds[r], acc[cb]);
      }
    }
    if (t + 1 < ntiles) {
      __syncthreads();
      gload(j0 + kTile);
      swrite();
    }
    __syncthreads();
  }

  // the output, or (split) this range's fp32 partial before the 1/sqrt(d) factor
  const bool part = a.Pdq != nullptr;
  float* qout_base = part ? a.Pdq + (int64_t)sp * a.q_rows * D : a.dQ;
  const double qscale = part ? 1.0 : a.scale64;
  if (row < n_q) {
    float* qout = qout_base + qbase + (int64_t)row * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) qout[16 * cb + 4 * r + g4] = (float)(acc[cb][r] * qscale);
  }
}

// ------------------------------------------------------------ 3. D pass
// D_i = sum_j P_ij dP_ij / sum_j P_ij, with P_ij formed exactly as the main kernel
// forms it (the same fp32 exp2 of the same fp64 exponent), accumulated in fp64.
// Both sums run over every key of the row's head, so the main kernel's
// dS_ij = P_ij (dP_ij - D_i) sums to zero over each row up to the fp32 rounding
// of its terms. With D taken from the caller's O instead (dO_i . O_i, the same
// number in exact arithmetic), the rounding of O enters dS through D alone:
// where one key dominates a row (scores in the thousands), dS is a small
// difference and dQ = dS K / sqrt(d) scales that error by |k| / sqrt(d)
// (about 9 at the x30 stress scale, where even a correctly rounded fp32 O
// costs 7e-6). Grid and sweep as the dQ role: 64 query rows per workgroup
// (lane = query), 32-key tiles of K and V staged in LDS.
// fp64 sums of one key range's P and P*dP for one query row (split D pass)
struct DPart {
  double sum_p;
  double sum_pdp;
};
static_assert(sizeof(DPart) == 16, "D partial layout");

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dterm_f32_kernel(const BwdArgs32 a,
                                                                     const float* __restrict__ Mx,
                                                                     const float* __restrict__ Ls,
                                                                     RowTerm* __restrict__ terms,
                                                                     DPart* __restrict__ part) {
  constexpr int S = Shared32<D>::kStride;
  constexpr int KK = D / 4;
  __shared__ __attribute__((aligned(16))) float sK[Shared32<D>::kElems];
  __shared__ __attribute__((aligned(16))) float sV[Shared32<D>::kElems];
  const int n_q = a.n_q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  // ((bh * s_q) + sp) * tiles_q + qt: the dQ workgroups' ranges of key tiles
  const int tile = xcd_remap(blockIdx.x, (int)gridDim.x);
  const int bh = tile / (a.tiles_q * a.s_q);
  const int sp = (tile - bh * a.tiles_q * a.s_q) / a.tiles_q;
  const int qt = tile - (bh * a.s_q + sp) * a.tiles_q;
  const int64_t qbase = (int64_t)bh * n_q * D;
  const int k_off = sp * a.len_k * kTile;
  const int n_k = a.n_k - k_off;  // keys from the range's first on
  const float* Kh = a.K + ((int64_t)bh * a.n_k + k_off) * D;
  const float* Vh = a.V + ((int64_t)bh * a.n_k + k_off) * D;
  const int row = qt * kRows + wave * 16 + l16;  // this lane's query
  const int qrow = min(row, n_q - 1);
  const int64_t trow = (int64_t)bh * n_q + qrow;
  float qf[KK], of[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qf[kk] = a.Q[qbase + (int64_t)qrow * D + 4 * kk + g4];
    of[kk] = a.dO[qbase + (int64_t)qrow * D + 4 * kk + g4];
  }
  const double lse2 = row_lse2(Mx[trow], Ls[trow]);
  double sum_p = 0.0, sum_pdp = 0.0;

  const int ntiles = min(a.len_k, (n_k + kTile - 1) / kTile);  // tiles of this range
  Stage<D> stK, stV;
  stK.load(Kh, 0, n_k, tid);
  stV.load(Vh, 0, n_k, tid);
  stK.store(sK, tid);
  stV.store(sV, tid);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kTile;
#pragma unroll
    for (int kb = 0; kb < kTile / 16; ++kb) {
      // S^T[key][q] and dP^T (fp64): lane holds query l16, register r <-> key 16kb + 4r + g4
      f64x4 s = f64x4{}, dp = f64x4{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int off = (16 * kb + l16) * S + 4 * kk + g4;
        s = mfma_f64_16x16x4((double)sK[off], (double)qf[kk], s);
        dp = mfma_f64_16x16x4((double)sV[off], (double)of[kk], dp);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = fast_exp2((float)(s[r] * a.C64 - lse2));
        if (j0 + 16 * kb + 4 * r + g4 >= n_k) p = 0.f;  // padding keys
        sum_p += (double)p;
        sum_pdp = __builtin_fma((double)p, dp[r], sum_pdp);
      }
    }
    if (t + 1 < ntiles) {
      __syncthreads();
      stK.load(Kh, j0 + kTile, n_k, tid);
      stV.load(Vh, j0 + kTile, n_k, tid);
      stK.store(sK, tid);
      stV.store(sV, tid);
    }
    __syncthreads();
  }
  // the four lane groups g4 hold different keys of the same query
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    sum_p += __shfl_xor(sum_p, off, 64);
    sum_pdp += __shfl_xor(sum_pdp, off, 64);
  }
  if (row < n_q && g4 == 0) {
    if (a.s_q > 1) part[sp * a.q_rows + trow] = DPart{sum_p, sum_pdp};
    else terms[trow] = RowTerm{lse2, -(sum_pdp / sum_p)};
  }
}

// Split D pass: one thread per query row adds the ranges' sums in range order.
__global__ __launch_bounds__(kThreads) void bwd_dterm_merge_f32_kernel(
    const float* __restrict__ Mx, const float* __restrict__ Ls, const DPart* __restrict__ part,
    int ranges, RowTerm* __restrict__ terms, int64_t rows) {
  for (int64_t row = (int64_t)blockIdx.x * kThreads + threadIdx.x; row < rows;
       row += (int64_t)gridDim.x * kThreads) {
    double sum_p = 0.0, sum_pdp = 0.0;
    for (int r = 0; r < ranges; ++r) {
      const DPart d = part[r * rows + row];
      sum_p += d.sum_p;
      sum_pdp += d.sum_pdp;
    }
    terms[row] = RowTerm{row_lse2(Mx[row], Ls[row]), -(sum_pdp / sum_p)};
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, D == 128 ? 1 : 2) void bwd_main_f32_kernel(const BwdArgs32 a) {
  __shared__ __attribute__((aligned(16))) float s0[Shared32<D>::kElems];
  __shared__ __attribute__((aligned(16))) float s1[Shared32<D>::kElems];
  __shared__ __attribute__((aligned(16))) RowTerm sT[kTile];
  const int wg = blockIdx.x;
  if (wg < a.total_kv) dkdv_role32<D>(a, wg, s0, s1, sT);
  else dq_role32<D>(a, wg - a.total_kv, s0, s1);
}

template <int D>
hipError_t launch(const BwdProblem& p, hipStream_t stream) {
  const int64_t rows = p.heads * p.rows_q;
  RowTerm* terms = reinterpret_cast<RowTerm*>(p.ws);
  BwdArgs32 a;
  a.Q = (const float*)p.q;
  a.K = (const float*)p.k;
  a.V = (const float*)p.v;
  a.dO = (const float*)p.dO;
  a.T = terms;
  a.dQ = (float*)p.dq;
  a.dK = (float*)p.dk;
  a.dV = (float*)p.dv;
  a.n_q = p.rows_q;
  a.n_k = p.n_k;
  a.tiles_kv = (p.n_k + kRows - 1) / kRows;
  a.tiles_q = (p.rows_q + kRows - 1) / kRows;
  // split fields; an unsplit side sweeps every tile
  const bool kv = p.split.kv > 1, q = p.split.q > 1;
  a.s_kv = kv ? p.split.kv : 1;
  a.len_q = kv ? p.split.len_q : (p.rows_q + kTile - 1) / kTile;
  a.s_q = q ? p.split.q : 1;
  a.len_k = q ? p.split.len_k : (p.n_k + kTile - 1) / kTile;
  a.Pdk = kv ? p.part_dk : nullptr;
  a.Pdv = kv ? p.part_dv : nullptr;
  a.Pdq = q ? p.part_dq : nullptr;
  a.kv_rows = p.heads * p.n_k;
  a.q_rows = p.heads * p.rows_q;
  a.total_kv = (int)(p.heads * a.tiles_kv * a.s_kv);
  a.total_q = (int)(p.heads * a.tiles_q * a.s_q);
  a.scale64 = 1.0 / sqrt((double)D);
  a.C64 = 1.4426950408889634 / sqrt((double)D);
  if (rows > 0) {
    // row terms; split: the D pass's range sums go where the dQ partials will
    // later be written (16 bytes per row and range, against 4 * D)
    DPart* part = q ? reinterpret_cast<DPart*>(p.part_dq) : nullptr;
    hipLaunchKernelGGL((bwd_dterm_f32_kernel<D>), dim3((unsigned)a.total_q), dim3(kThreads), 0,
                       stream, a, p.m, p.l, terms, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (q) {
      hipLaunchKernelGGL(bwd_dterm_merge_f32_kernel, dim3(row_blocks(rows, kThreads)),
                         dim3(kThreads), 0, stream, p.m, p.l, part, a.s_q, terms, rows);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL((bwd_main_f32_kernel<D>), dim3((unsigned)(a.total_kv + a.total_q)),
                     dim3(kThreads), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_bwd_reduce(false, D, p, stream);
}

}  // namespace

BwdGeometry bwd_geometry_f32(int) { return BwdGeometry{kRows, kTile}; }

hipError_t launch_bwd_f32(int d, const BwdProblem& p, hipStream_t stream) {
  if (d == 64) return launch<64>(p, stream);
  return launch<128>(p, stream);
}

}  // namespace mea
