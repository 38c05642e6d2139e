// Backward attention for bf16 inputs on gfx950, by recomputation.
//
// "Self-attention Does Not Need O(n^2) Memory" (abstract; 方法详解; English
// digest method bullets) differentiates the chunked forward by recomputing
// each chunk's intermediates instead of storing them. Here the forward saves
// only two fp32 numbers per query row (row max m_i and row sum l_i); every
// kernel below rebuilds the probability tile
//     P_ij = exp(s_ij - m_i) / l_i = exp2(x_ij * log2(e)/sqrt(d) - lse2_i),
//     lse2_i = m_i * log2(e) + log2(l_i),   x_ij = q_i . k_j,
// from Q and K on the fly. The pages print no gradient formulas; the textbook
// softmax Jacobian is used: dV = P^T dO, dP = dO V^T, D_i = dO_i . O_i,
// dS = P * (dP - D), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).
//
// Three kernels on the caller's stream:
//  1. bwd_rows:  D_i and lse2_i for every row, into the workspace.
//  2. bwd_dkdv:  one workgroup per 128-key tile (32 keys per wave, K and V of
//     those keys in registers); sweeps all query tiles (Q, dO, lse2, D staged
//     in LDS, double-buffered) accumulating dV^T and dK^T in registers.
//  3. bwd_dq:    one workgroup per query tile (32 queries per wave, Q and dO
//     in registers); sweeps all key tiles (K, V in LDS) accumulating dQ^T.
// No probability or score array is written to memory; dQ, dK and dV are each
// written once, so the result does not depend on scheduling (deterministic).
#include "mea_device.h"
#include "mea_launch.h"

namespace mea {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// ------------------------------------------------------------ 1. row terms
// One wave per 8 rows (d=64) / 4 rows (d=128): lanes read 16 bytes of O and
// dO each and reduce over the lanes of a row.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_rows_kernel(
    const bf16* __restrict__ O, const bf16* __restrict__ dO, const float* __restrict__ Mx,
    const float* __restrict__ Ls, float* __restrict__ Dv, float* __restrict__ Lse2,
    int64_t rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t gtid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = gtid / LPR;
  const int part = (int)(gtid - row * LPR);
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
    Dv[row] = acc;
    Lse2[row] = Mx[row] * kLog2e + __builtin_log2f(Ls[row]);
  }
}

// ------------------------------------------------------------ 2. dK and dV
constexpr int kBQ2 = 64;  // query rows per staged tile

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ Dv, const float* __restrict__ Lse2,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int n, int ktiles, int total, float C,
    float scale) {
  constexpr int kBK = kWaves * 32;  // keys per workgroup
  constexpr int DK = D / 16;
  constexpr int DB = D / 32;
  constexpr int NC = kBQ2 / 16;   // 16-query chunks per staged tile
  constexpr int QBT = kBQ2 / 32;  // 32-query blocks per staged tile
  constexpr int kTile = kBQ2 * D;
  constexpr int kCPR = D / 8;
  constexpr int kLoads = kTile / 8 / kThreads;
  static_assert(kLoads * 8 * kThreads == kTile, "tile split");

  __shared__ __attribute__((aligned(16))) bf16 sQ[2][kTile];
  __shared__ __attribute__((aligned(16))) bf16 sO[2][kTile];  // dO tile
  __shared__ __attribute__((aligned(16))) float sL[2][kBQ2];  // lse2
  __shared__ __attribute__((aligned(16))) float sD[2][kBQ2];  // D

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / ktiles;
  const int kt = tile - bh * ktiles;
  const int64_t base = (int64_t)bh * n * D;
  const int64_t rbase = (int64_t)bh * n;
  const int key = kt * kBK + wave * 32 + l32;  // this lane's key (column of S)

  // K and V of this wave's 32 keys: B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[DK], vf[DK];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    if (key < n) {
      kf[dk] = *reinterpret_cast<const bf16x8*>(K + base + (int64_t)key * D + dk * 16 + 8 * hi);
      vf[dk] = *reinterpret_cast<const bf16x8*>(V + base + (int64_t)key * D + dk * 16 + 8 * hi);
    } else {
      kf[dk] = bf16x8{};
      vf[dk] = bf16x8{};
    }
  }
  f32x16 accV[DB], accK[DB];  // dV^T, dK^T: register r -> column 32*db + 8*(r/4) + 4*hi + r%4
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    accV[db] = f32x16{};
    accK[db] = f32x16{};
  }

  u32x4 qreg[kLoads], oreg[kLoads];
  float lreg = 0.f, dreg = 0.f;
  auto gload = [&](int i0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / kCPR;
      const int ch = c - r * kCPR;
      if (i0 + r < n) {
        const int64_t off = base + (int64_t)(i0 + r) * D + ch * 8;
        qreg[i] = *reinterpret_cast<const u32x4*>(Q + off);
        oreg[i] = *reinterpret_cast<const u32x4*>(dO + off);
      } else {
        qreg[i] = u32x4{};
        oreg[i] = u32x4{};
      }
    }
    if (tid < kBQ2) {
      const bool ok = i0 + tid < n;
      lreg = ok ? Lse2[rbase + i0 + tid] : INFINITY;  // padding rows get P = 0
      dreg = ok ? Dv[rbase + i0 + tid] : 0.f;
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / kCPR;
      const int ch = c - r * kCPR;
      const int off = r * D + swz_chunk<D>(r, ch) * 8;
      *reinterpret_cast<u32x4*>(&sQ[buf][off]) = qreg[i];
      *reinterpret_cast<u32x4*>(&sO[buf][off]) = oreg[i];
    }
    if (tid < kBQ2) {
      sL[buf][tid] = lreg;
      sD[buf][tid] = dreg;
    }
  };

  const int g = lane >> 4;
  const int jj = lane & 15;
  const int tr_row = 4 * hi + (jj >> 2);
  const int tr_col = (g & 1) * 16 + 4 * (jj & 3);

  const int ntiles = (n + kBQ2 - 1) / kBQ2;
  gload(0);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload((t + 1) * kBQ2);
    const bf16* qs = sQ[buf];
    const bf16* os = sO[buf];
    const float* ls = sL[buf];
    const float* dsv = sD[buf];

    bf16x8 pf[NC], sf[NC];  // P and dS as B operands: chunk c element e <-> query 16c + 8(e/4) + 4hi + e%4
#pragma unroll
    for (int qb = 0; qb < QBT; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) {
        const int off = swz_off<D>(qb * 32 + l32, dk * 16 + 8 * hi);
        s = mfma32x32x16(lds_read_b128(qs + off), kf[dk], s);
        dp = mfma32x32x16(lds_read_b128(os + off), vf[dk], dp);
      }
      // lane holds key `key`; register r holds query row 32*qb + 8*(r/4) + 4*hi + r%4
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 lse = *reinterpret_cast<const f32x4*>(ls + qb * 32 + 8 * r4 + 4 * hi);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(dsv + qb * 32 + 8 * r4 + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float p = fast_exp2(__builtin_fmaf(s[r], C, -lse[e]));
          const float dsc = p * (dp[r] - dd[e]);
          pf[2 * qb + (r >> 3)][r & 7] = (bf16)p;
          sf[2 * qb + (r >> 3)][r & 7] = (bf16)dsc;
        }
      }
    }
    // dV^T += dO^T P,  dK^T += Q^T dS   (A operands by transposed LDS reads)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 32 + tr_col;
        const int o0 = swz_off<D>(c * 16 + tr_row, col);
        const int o1 = swz_off<D>(c * 16 + 8 + tr_row, col);
        const bf16x8 ao = cat(lds_read_tr16(os + o0), lds_read_tr16(os + o1));
        const bf16x8 aq = cat(lds_read_tr16(qs + o0), lds_read_tr16(qs + o1));
        accV[db] = mfma32x32x16(ao, pf[c], accV[db]);
        accK[db] = mfma32x32x16(aq, sf[c], accK[db]);
      }
    }
    if (t + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

  if (key < n) {
    bf16* vrow = dV + base + (int64_t)key * D;
    bf16* krow = dK + base + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 wv, wk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wv[e] = (bf16)accV[db][4 * r4 + e];
          wk[e] = (bf16)(accK[db][4 * r4 + e] * scale);
        }
        *reinterpret_cast<bf16x4*>(vrow + db * 32 + 8 * r4 + 4 * hi) = wv;
        *reinterpret_cast<bf16x4*>(krow + db * 32 + 8 * r4 + 4 * hi) = wk;
      }
  }
}

// ------------------------------------------------------------ 3. dQ
constexpr int kBC3 = 64;  // keys per staged tile

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ Dv, const float* __restrict__ Lse2,
    bf16* __restrict__ dQ, int n, int qtiles, int total, float C, float scale) {
  constexpr int kBQ = kWaves * 32;
  constexpr int DK = D / 16;
  constexpr int DB = D / 32;
  constexpr int KB = kBC3 / 32;
  constexpr int NC = kBC3 / 16;
  constexpr int kTile = kBC3 * D;
  constexpr int kCPR = D / 8;
  constexpr int kLoads = kTile / 8 / kThreads;
  static_assert(kLoads * 8 * kThreads == kTile, "tile split");

  __shared__ __attribute__((aligned(16))) bf16 sK[2][kTile];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / qtiles;
  const int qt = tile - bh * qtiles;
  const int64_t base = (int64_t)bh * n * D;
  const int row = qt * kBQ + wave * 32 + l32;  // this lane's query

  bf16x8 qf[DK], of[DK];  // B operands of S^T = K Q^T and dP^T = V dO^T
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    if (row < n) {
      qf[dk] = *reinterpret_cast<const bf16x8*>(Q + base + (int64_t)row * D + dk * 16 + 8 * hi);
      of[dk] = *reinterpret_cast<const bf16x8*>(dO + base + (int64_t)row * D + dk * 16 + 8 * hi);
    } else {
      qf[dk] = bf16x8{};
      of[dk] = bf16x8{};
    }
  }
  const float lse = row < n ? Lse2[(int64_t)bh * n + row] : INFINITY;
  const float dd = row < n ? Dv[(int64_t)bh * n + row] : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  u32x4 kreg[kLoads], vreg[kLoads];
  auto gload = [&](int j0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / kCPR;
      const int ch = c - r * kCPR;
      if (j0 + r < n) {
        const int64_t off = base + (int64_t)(j0 + r) * D + ch * 8;
        kreg[i] = *reinterpret_cast<const u32x4*>(K + off);
        vreg[i] = *reinterpret_cast<const u32x4*>(V + off);
      } else {
        kreg[i] = u32x4{};
        vreg[i] = u32x4{};
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / kCPR;
      const int ch = c - r * kCPR;
      const int off = r * D + swz_chunk<D>(r, ch) * 8;
      *reinterpret_cast<u32x4*>(&sK[buf][off]) = kreg[i];
      *reinterpret_cast<u32x4*>(&sV[buf][off]) = vreg[i];
    }
  };

  const int g = lane >> 4;
  const int jj = lane & 15;
  const int tr_row = 4 * hi + (jj >> 2);
  const int tr_col = (g & 1) * 16 + 4 * (jj & 3);

  const int ntiles = (n + kBC3 - 1) / kBC3;
  gload(0);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int j0 = t * kBC3;
    if (t + 1 < ntiles) gload(j0 + kBC3);
    const bf16* ks = sK[buf];
    const bf16* vs = sV[buf];

    bf16x8 sf[NC];  // dS^T as B operand, same chunking as P^T in the forward
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) {
        const int off = swz_off<D>(kb * 32 + l32, dk * 16 + 8 * hi);
        s = mfma32x32x16(lds_read_b128(ks + off), qf[dk], s);
        dp = mfma32x32x16(lds_read_b128(vs + off), of[dk], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = j0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        float p = fast_exp2(__builtin_fmaf(s[r], C, -lse));
        if (kj >= n) p = 0.f;
        sf[2 * kb + (r >> 3)][r & 7] = (bf16)(p * (dp[r] - dd));
      }
    }
    // dQ^T += K^T dS^T (A operand by transposed reads of the K tile)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 32 + tr_col;
        const bf16x8 a = cat(lds_read_tr16(ks + swz_off<D>(c * 16 + tr_row, col)),
                             lds_read_tr16(ks + swz_off<D>(c * 16 + 8 + tr_row, col)));
        acc[db] = mfma32x32x16(a, sf[c], acc[db]);
      }
    }
    if (t + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

  if (row < n) {
    bf16* qrow = dQ + base + (int64_t)row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[db][4 * r4 + e] * scale);
        *reinterpret_cast<bf16x4*>(qrow + db * 32 + 8 * r4 + 4 * hi) = w;
      }
  }
}

template <int D>
hipError_t launch(int64_t BH, int n, const void* q, const void* k, const void* v, const void* o,
                  const void* dO, const float* m, const float* l, void* dq, void* dk, void* dv,
                  float* ws, hipStream_t stream) {
  const float scale = 1.0f / sqrtf((float)D);
  const float C = kLog2e * scale;
  const int64_t rows = BH * n;
  float* Dv = ws;
  float* Lse2 = ws + rows;
  {
    const int64_t threads = rows * (D / 8);
    const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
    hipLaunchKernelGGL((bwd_rows_kernel<D>), dim3(blocks), dim3(kThreads), 0, stream,
                       (const bf16*)o, (const bf16*)dO, m, l, Dv, Lse2, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int ktiles = (n + kWaves * 32 - 1) / (kWaves * 32);
    const int total = (int)(BH * ktiles);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3(total), dim3(kThreads), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dO, Dv, Lse2,
                       (bf16*)dk, (bf16*)dv, n, ktiles, total, C, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int qtiles = (n + kWaves * 32 - 1) / (kWaves * 32);
    const int total = (int)(BH * qtiles);
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3(total), dim3(kThreads), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dO, Dv, Lse2,
                       (bf16*)dq, n, qtiles, total, C, scale);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(int d, int64_t BH, int n, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* m, const float* l,
                           void* dq, void* dk, void* dv, float* ws, hipStream_t stream) {
  if (d == 64) return launch<64>(BH, n, q, k, v, o, dO, m, l, dq, dk, dv, ws, stream);
  return launch<128>(BH, n, q, k, v, o, dO, m, l, dq, dk, dv, ws, stream);
}

}  // namespace mea
