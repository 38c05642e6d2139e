// Forward attention for bf16 inputs on gfx950: one workgroup per tile of
// query rows, a sweep over key/value tiles with a running maximum and running
// sum per query row, normalisation once at the end.
//
// Method: "Self-attention Does Not Need O(n^2) Memory" (abstract; method
// sections of both digests): postpone the softmax division to the end, keep
// a weighted value sum and a weight sum per query, track the maximum score
// for stability, and visit keys/values in chunks. The per-tile update is the
// two-block merge of "当注意力成为瓶颈…", section IO感知, applied once per tile.
//
// Layout of the work (per workgroup of 4 waves):
//  * each wave owns QB blocks of 32 query rows; the workgroup owns 4*QB*32;
//  * K and V tiles of 64 keys are staged in LDS, double-buffered, with the
//    16-byte chunks of each row swizzled (see mea_device.h);
//  * scores are formed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA, so
//    that each lane holds one query's scores for 16 keys per 32-key block:
//    the row maximum is a register reduction plus one exchange with lane
//    l^32, and the per-row rescale factor is a per-lane scalar;
//  * the output is accumulated transposed, O^T += V^T P^T: P^T comes straight
//    from the S^T accumulators (rounded to bf16), V^T from transposed LDS
//    reads of the row-major V tile;
//  * exponentials are base 2 with log2(e)/sqrt(d) folded into one FMA.
#include "mea_device.h"
#include "mea_launch.h"

namespace mea {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBC = 64;  // keys per tile

template <int D, int QB>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ Mx, float* __restrict__ Ls,
    int n, int qtiles, int total, float C, float scale) {
  constexpr int kBQ = kWaves * QB * 32;   // query rows per workgroup
  constexpr int DK = D / 16;              // k-steps of the score MFMA
  constexpr int DB = D / 32;              // 32-wide output column blocks
  constexpr int KB = kBC / 32;            // 32-key blocks per tile
  constexpr int NC = kBC / 16;            // 16-key chunks per tile (PV k-steps)
  constexpr int kTile = kBC * D;          // elements per K or V tile
  constexpr int kCPR = D / 8;             // 16-byte chunks per row
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
  const bf16* Qh = Q + base;
  const bf16* Kh = K + base;
  const bf16* Vh = V + base;
  const int q0 = qt * kBQ + wave * QB * 32;

  // Q fragments: B operand of S^T = K Q^T (lane: query l32, 8 columns at 16*dk + 8*hi)
  bf16x8 qf[QB][DK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q0 + qb * 32 + l32;
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      if (row < n) {
        qf[qb][dk] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)row * D + dk * 16 + 8 * hi);
      } else {
        qf[qb][dk] = bf16x8{};
      }
    }
  }

  // Per query row: the running max m of the raw scores q.k, its rounded
  // product mC = fl(m * C) (every weight is formed as exp2(fl(x*C - mC)) with
  // one FMA), and this lane's share of the running sum of those weights.
  float m_run[QB];
  float mC_run[QB];
  float l_run[QB];
  f32x16 acc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    mC_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
  }

  u32x4 kreg[kLoads], vreg[kLoads];
  auto gload = [&](int j0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / kCPR;
      const int ch = c - r * kCPR;
      if (j0 + r < n) {
        const int64_t off = (int64_t)(j0 + r) * D + ch * 8;
        kreg[i] = *reinterpret_cast<const u32x4*>(Kh + off);
        vreg[i] = *reinterpret_cast<const u32x4*>(Vh + off);
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

  const int ntiles = (n + kBC - 1) / kBC;
  gload(0);
  swrite(0);
  __syncthreads();

  // transposed-read addressing for V^T fragments (fixed per lane)
  const int g = lane >> 4;
  const int jj = lane & 15;
  const int tr_row = 4 * hi + (jj >> 2);
  const int tr_col = (g & 1) * 16 + 4 * (jj & 3);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int j0 = t * kBC;
    if (t + 1 < ntiles) gload(j0 + kBC);
    const bf16* ks = sK[buf];
    const bf16* vs = sV[buf];

    // S^T = K Q^T: lane holds query l32 and, in register r of block kb,
    // key j0 + 32*kb + 8*(r/4) + 4*hi + r%4
    f32x16 s[QB][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x16{};
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) {
        const bf16x8 a = lds_read_b128(ks + swz_off<D>(kb * 32 + l32, dk * 16 + 8 * hi));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32x32x16(a, qf[qb][dk], s[qb][kb]);
      }
    }
    if (j0 + kBC > n) {  // ragged last tile: keys beyond n get no weight
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= n) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][kb][r] = -INFINITY;
          }
        }
    }

    // online softmax; P^T fragments for the PV MFMA: chunk c, element e is
    // register 8*(c%2) + e of block c/2
    bf16x8 pf[QB][NC];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run[qb], mx);
      const float mC = m_new * C;
      // rescale by the ratio of the rounded references, so that all weights in
      // l and acc stay relative to the same mC
      const float alpha = fast_exp2(mC_run[qb] - mC);
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[qb][kb][r], C, -mC));
          ls += p;
          pf[qb][2 * kb + (r >> 3)][r & 7] = (bf16)p;
        }
      l_run[qb] = l_run[qb] * alpha + ls;
      m_run[qb] = m_new;
      mC_run[qb] = mC;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 32 + tr_col;
        const bf16x4 lo = lds_read_tr16(vs + swz_off<D>(c * 16 + tr_row, col));
        const bf16x4 up = lds_read_tr16(vs + swz_off<D>(c * 16 + 8 + tr_row, col));
        const bf16x8 a = cat(lo, up);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32x32x16(a, pf[qb][c], acc[qb][db]);
      }
    }

    if (t + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

  // epilogue: O = acc / l, written once; statistics in natural units
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q0 + qb * 32 + l32;
    const float l_tot = l_run[qb] + xor32(l_run[qb]);
    const float inv = 1.f / l_tot;
    if (row < n) {
      bf16* orow = O + base + (int64_t)row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[qb][db][4 * r4 + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * r4 + 4 * hi) = w;
        }
      if (Mx != nullptr && hi == 0) {
        // The weights summed in l_tot are 2^eps times exp(s - m), where
        // eps = m*C - fl(m*C) is the rounding residual of the reference
        // (exact through one FMA); report l for the exact maximum.
        const float eps = __builtin_fmaf(m_run[qb], C, -mC_run[qb]);
        Mx[(int64_t)bh * n + row] = m_run[qb] * scale;
        Ls[(int64_t)bh * n + row] = l_tot * fast_exp2(-eps);
      }
    }
  }
}

template <int D, int QB>
hipError_t launch(int64_t BH, int n, const void* q, const void* k, const void* v, void* o,
                  float* m, float* l, hipStream_t stream) {
  constexpr int kBQ = kWaves * QB * 32;
  const int qtiles = (n + kBQ - 1) / kBQ;
  const int64_t total = BH * qtiles;
  const float scale = 1.0f / sqrtf((float)D);
  const float C = kLog2e * scale;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QB>), dim3((unsigned)total), dim3(kThreads), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, m, l, n, qtiles,
                     (int)total, C, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(int d, int64_t BH, int n, const void* q, const void* k, const void* v,
                           void* o, float* m, float* l, hipStream_t stream) {
  if (d == 64) return launch<64, 2>(BH, n, q, k, v, o, m, l, stream);
  return launch<128, 1>(BH, n, q, k, v, o, m, l, stream);
}

}  // namespace mea
