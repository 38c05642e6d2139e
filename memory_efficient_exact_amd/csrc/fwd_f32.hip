// Forward attention for fp32 inputs on gfx950, with scores formed in fp64.
//
// Same method as the bf16 kernel ("Self-attention Does Not Need O(n^2)
// Memory": running maximum and running sums per query, one division at the
// end; "当注意力成为瓶颈…", section IO感知: per-tile merge). Precision: an
// fp32 product is exact in fp64, so S^T = K Q^T runs on fp64 MFMA
// (16x16x4) and the row maximum is subtracted in fp64. Only the difference
// s - m (<= 0) is rounded to fp32 before the base-2 exponential; the weights,
// their sum and P V (fp32 MFMA 16x16x4) are fp32. With scores of magnitude
// ~1e4 an fp32 score would carry an absolute error near 1e-3, enough to move
// the weights of near-tied keys by far more than the 1e-5 output tolerance.
//
// Work split: 4 waves, 16 query rows per wave; K/V tiles of 32 keys in LDS,
// rows padded so the column reads of both MFMA operands hit distinct banks.
// The tile is single-buffered: after every wave is done with it, the next one
// is loaded and stored between two barriers. The small LDS footprint and
// register budget (Q held in fp32 and widened at each use) let three
// workgroups share a CU at d = 128, four at d = 64, and the other workgroups
// cover the load (measured 10% faster than double buffering with the next
// tile held in registers, at two workgroups per CU). Decoding grids are too
// small for that, so the decoding layout below keeps the double buffer with
// the next tile loaded into registers during the current one. The score tile
// is transposed (lane = query), so the per-row state lives in registers; four
// lanes (l, l^16, l^32, l^48) share a query.
//
// Decoding mode (at most 32 query rows per head): the four waves share one
// 16-row query block and each takes a different 16-key block of every 64-key
// tile, so no fp64 MFMA work goes to padding query rows; their partial
// results merge through LDS after the sweep.
//
// Key ranges (split-key mode): a workgroup may cover only keys
// [key0, key0 + split_len) of its head and then writes that range's summary, the
// fp32 row acc / l, the fp64 maximum m and l (relative to m), for the merge
// pass (merge.hip).
#include "mea_device.h"
#include "mea_launch.h"

namespace mea {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 16 * kWaves;  // query rows per workgroup
constexpr int kBC = 32;           // keys per tile
constexpr int kBQDecode = 16;     // decoding: query rows per workgroup
constexpr int kBCDecode = 64;     // decoding: keys per tile (one 16-key block per wave)
constexpr int kDecodeRows = 32;   // heads with at most this many query rows decode
constexpr int64_t kComputeUnits = 256;

// The decoding layout also serves every grid of row tiles that would occupy
// at most half of the compute units: it launches four times the workgroups,
// each wave sweeping a quarter of the keys (measured 1.3-2.4x faster at
// 16-128 workgroups; from about 200 on the row-tiled layout is as fast or
// faster).
bool decode_grid(int64_t heads, int64_t rows_q) {
  return rows_q <= kDecodeRows || 2 * heads * ((rows_q + kBQ - 1) / kBQ) <= kComputeUnits;
}

__device__ __forceinline__ float xor16f(float x) { return __shfl_xor(x, 16, 64); }
__device__ __forceinline__ double xor16d(double x) { return __shfl_xor(x, 16, 64); }
__device__ __forceinline__ double xor32d(double x) { return __shfl_xor(x, 32, 64); }

struct FwdArgs32 {
  const float* Q;  // [heads, n_q, D]
  const float* K;  // [heads, n_k, D]
  const float* V;
  float* O;        // final mode: [heads, n_q, D]
  float* Mx;       // final mode: [heads, n_q] or null
  float* Ls;
  float* Po;       // split mode: [splits, rows, D] normalised partial rows (else null)
  float* Ps;       // split mode: [splits, rows] records {m (fp64, two words), l, 0}
  int64_t rows;    // heads * n_q
  int n_q;
  int n_k;
  int qtiles;
  int splits;
  int split_len;
  int total;
  double C64;      // log2(e) / sqrt(D)
  double scale64;  // 1 / sqrt(D)
};

// at least three waves per SIMD (<= 168 registers) outside decoding
template <int D, bool kDecode>
__global__ __launch_bounds__(kThreads, kDecode ? 1 : 3) void fwd_f32_kernel(const FwdArgs32 a) {
  constexpr int KS = D + 4;   // K row stride (floats): 16-byte pad
  constexpr int VS = D + 16;  // V row stride (floats): 64-byte pad
  constexpr int KK = D / 4;   // k-steps of the fp64 score MFMA
  constexpr int DB = D / 16;  // 16-wide output column blocks
  constexpr int BC = kDecode ? kBCDecode : kBC;  // keys per tile
  constexpr int BQ = kDecode ? kBQDecode : kBQ;  // query rows per workgroup
  constexpr int KB = kDecode ? 1 : BC / 16;      // 16-key blocks per wave per tile
  constexpr int kCPR = D / 4;  // 16-byte chunks per row
  constexpr int kLoads = BC * D / 4 / kThreads;
  static_assert(kLoads * 4 * kThreads == BC * D, "tile split");

  constexpr int NB = kDecode ? 2 : 1;  // LDS buffers per operand
  __shared__ __attribute__((aligned(16))) float sK[NB][BC * KS];
  __shared__ __attribute__((aligned(16))) float sV[NB][BC * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // workgroup -> (head, key range, query tile)
  const int tile = xcd_remap(blockIdx.x, a.total);
  const int hs = tile / a.qtiles;
  const int qt = tile - hs * a.qtiles;
  const int bh = hs / a.splits;
  const int sp = hs - bh * a.splits;
  const int key0 = sp * a.split_len;            // first key of this range
  const int n = min(a.n_k - key0, a.split_len);  // keys of this range
  const int n_q = a.n_q;
  const double C64 = a.C64;
  const float* Kh = a.K + ((int64_t)bh * a.n_k + key0) * D;
  const float* Vh = a.V + ((int64_t)bh * a.n_k + key0) * D;
  const int row = kDecode ? qt * BQ + l16 : qt * BQ + wave * 16 + l16;  // this lane's query row
  const int blk0 = kDecode ? wave : 0;  // first 16-key block of a tile this wave takes
  const int64_t grow = (int64_t)bh * n_q + row;

  // B operand of S^T = K Q^T: Q[row][4*kk + g4], widened to fp64 (exactly) at each use
  float qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = row < n_q ? a.Q[grow * D + 4 * kk + g4] : 0.f;

  double m_run = -INFINITY;  // running max of raw scores (fp64)
  float l_run = 0.f;         // this lane's share of the running sum
  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4{};

  u32x4 kreg[kLoads], vreg[kLoads];
  auto gload = [&](int j0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / kCPR;
      const int ch = c - r * kCPR;
      if (j0 + r < n) {
        const int64_t off = (int64_t)(j0 + r) * D + ch * 4;
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
      *reinterpret_cast<u32x4*>(&sK[buf][r * KS + ch * 4]) = kreg[i];
      *reinterpret_cast<u32x4*>(&sV[buf][r * VS + ch * 4]) = vreg[i];
    }
  };

  const int ntiles = (n + BC - 1) / BC;
  gload(0);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = NB == 2 ? (t & 1) : 0;
    const int j0 = t * BC;
    if constexpr (NB == 2) {
      if (t + 1 < ntiles) gload(j0 + BC);
    }
    const float* ks = sK[buf];
    const float* vs = sV[buf];

    // S^T block kb: lane holds query l16 and, in register r, key 16*(blk0+kb) + 4*r + g4
    f64x4 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f64x4{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const double a = (double)ks[((blk0 + kb) * 16 + l16) * KS + 4 * kk + g4];
        s[kb] = mfma_f64_16x16x4(a, (double)qf[kk], s[kb]);
      }
    }
    if (j0 + BC > n) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j0 + (blk0 + kb) * 16 + 4 * r + g4 >= n) s[kb][r] = -INFINITY;
    }

    double mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmax(mx, s[kb][r]);
    mx = fmax(mx, xor16d(mx));
    mx = fmax(mx, xor32d(mx));
    const double m_new = fmax(m_run, mx);
    // a wave that has seen no valid key yet (possible when decoding, where each
    // wave covers one block of the tile) keeps weights and rescale at exactly 0
    const double m_base = m_new == -INFINITY ? 0.0 : m_new;
    const float alpha = fast_exp2((float)((m_run - m_base) * C64));
    float p[KB][4];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kb][r] = fast_exp2((float)((s[kb][r] - m_base) * C64));
        ls += p[kb][r];
      }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;

    // O^T += V^T P^T: k-step (kb, c) covers keys 16*kb + 4*c + 0..3;
    // B = P^T[key 16*kb + 4*c + g4][query l16] is register c of block kb
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float* vrow = vs + ((blk0 + kb) * 16 + 4 * c + g4) * VS + l16;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma_f32_16x16x4(vrow[db * 16], p[kb][c], acc[db]);
      }

    if constexpr (NB == 2) {
      if (t + 1 < ntiles) swrite(buf ^ 1);
    } else if (t + 1 < ntiles) {
      __syncthreads();  // every wave is done with this tile
      gload(j0 + BC);
      swrite(0);
    }
    __syncthreads();
  }

  // lanes l, l^16, l^32, l^48 share query l16: combine their partial sums
  float l_tot = l_run + xor16f(l_run);
  l_tot = l_tot + xor32(l_tot);

  if constexpr (kDecode) {
    // Merge the four waves (same 16 query rows, different keys). The loop ended
    // with a barrier, so the tile buffers are free: per-wave maxima and sums go
    // to sK[0], each wave's re-based accumulator (16 rows x D) to sV[0].
    constexpr int AS = D + 4;
    static_assert(kWaves * 16 * AS <= BC * VS, "accumulators fit the V buffer");
    double* sm = reinterpret_cast<double*>(sK[0]);
    float* sl = sK[0] + 2 * kWaves * 16;
    float* sacc = sV[0];
    if (g4 == 0) {
      sm[wave * 16 + l16] = m_run;
      sl[wave * 16 + l16] = l_tot;
    }
    __syncthreads();
    double M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmax(M, sm[w * 16 + l16]);
    const float f = m_run == -INFINITY ? 0.f : fast_exp2((float)((m_run - M) * C64));
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<f32x4*>(sacc + (wave * 16 + l16) * AS + db * 16 + 4 * g4) = acc[db] * f;
    __syncthreads();
    // this lane: query row lane / 4 of the block, D/16 columns of the wave's quarter
    constexpr int CPL = D / 16;
    const int qr = lane >> 2;
    const int col0 = wave * (D / 4) + (lane & 3) * CPL;
    const int qrow = qt * BQ + qr;
    float L = 0.f;
    double Mq = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Mq = fmax(Mq, sm[w * 16 + qr]);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const double mw = sm[w * 16 + qr];
      L += mw == -INFINITY ? 0.f : sl[w * 16 + qr] * fast_exp2((float)((mw - Mq) * C64));
    }
    if (qrow < n_q) {
      const int64_t gq = (int64_t)bh * n_q + qrow;
      const int64_t oq = a.Po == nullptr ? gq : (int64_t)sp * a.rows + gq;
      float* orow = (a.Po == nullptr ? a.O : a.Po) + oq * D;
      const float inv = 1.f / L;
#pragma unroll
      for (int c = 0; c < CPL; c += 4) {
        f32x4 sum = f32x4{};
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          sum += *reinterpret_cast<const f32x4*>(sacc + (w * 16 + qr) * AS + col0 + c);
        *reinterpret_cast<f32x4*>(orow + col0 + c) = sum * inv;
      }
      if (wave == 0 && (lane & 3) == 0) {
        if (a.Po != nullptr) {
          float* rec = a.Ps + oq * 4;
          *reinterpret_cast<double*>(rec) = Mq;
          rec[2] = L;
          rec[3] = 0.f;
        } else if (a.Mx != nullptr) {
          const double m_nat = Mq * a.scale64;
          const float m_st = (float)m_nat;
          a.Mx[gq] = m_st;
          a.Ls[gq] = (float)((double)L * exp(m_nat - (double)m_st));
        }
      }
    }
    return;
  }

  const float inv = 1.f / l_tot;
  if (row < n_q) {
    // acc[db] register r holds O[row][16*db + 4*g4 + r]
    const int64_t orow_idx = a.Po == nullptr ? grow : (int64_t)sp * a.rows + grow;
    float* orow = (a.Po == nullptr ? a.O : a.Po) + orow_idx * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f32x4 w = acc[db] * inv;
      *reinterpret_cast<f32x4*>(orow + db * 16 + 4 * g4) = w;
    }
    if (g4 == 0) {
      if (a.Po != nullptr) {
        float* rec = a.Ps + orow_idx * 4;
        *reinterpret_cast<double*>(rec) = m_run;
        rec[2] = l_tot;
        rec[3] = 0.f;
      } else if (a.Mx != nullptr) {
        // report l against the reported (fp32-rounded) maximum, so that the pair
        // satisfies l = sum_j exp(s_j - m) as stored: l_tot * exp(m - fl(m))
        const double m_nat = m_run * a.scale64;
        const float m_st = (float)m_nat;
        a.Mx[grow] = m_st;
        a.Ls[grow] = (float)((double)l_tot * exp(m_nat - (double)m_st));
      }
    }
  }
}

template <int D, bool kDecode>
hipError_t launch(const FwdProblem& p, hipStream_t stream) {
  constexpr int BQ = kDecode ? kBQDecode : kBQ;
  FwdArgs32 a;
  a.Q = static_cast<const float*>(p.q);
  a.K = static_cast<const float*>(p.k);
  a.V = static_cast<const float*>(p.v);
  a.O = static_cast<float*>(p.o);
  a.Mx = p.m;
  a.Ls = p.l;
  a.rows = p.heads * p.rows_q;
  a.n_q = p.rows_q;
  a.n_k = p.n_k;
  a.qtiles = (p.rows_q + BQ - 1) / BQ;
  a.splits = p.splits > 1 ? p.splits : 1;
  a.split_len = p.splits > 1 ? p.split_len : p.n_k;
  a.Po = p.splits > 1 ? p.part : nullptr;
  a.Ps = p.splits > 1 ? p.part + (int64_t)a.splits * a.rows * D : nullptr;
  const int64_t total = p.heads * a.splits * a.qtiles;
  a.total = (int)total;
  a.scale64 = 1.0 / sqrt((double)D);
  a.C64 = 1.4426950408889634 * a.scale64;
  hipLaunchKernelGGL((fwd_f32_kernel<D, kDecode>), dim3((unsigned)total), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

FwdGeometry fwd_geometry_f32(int d, int64_t heads, int64_t rows_q) {
  // workgroups per CU: decoding double-buffers 64-key tiles (at d = 128 in 141 KiB
  // of LDS, one workgroup per CU); otherwise as the register budgets allow, four
  // at d = 64 and three at d = 128
  if (decode_grid(heads, rows_q)) return FwdGeometry{kBQDecode, kBCDecode, d == 64 ? 2 : 1};
  return FwdGeometry{kBQ, kBC, d == 64 ? 4 : 3};
}

hipError_t launch_fwd_f32(int d, const FwdProblem& p, hipStream_t stream) {
  if (decode_grid(p.heads, p.rows_q)) return d == 64 ? launch<64, true>(p, stream) : launch<128, true>(p, stream);
  return d == 64 ? launch<64, false>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace mea
