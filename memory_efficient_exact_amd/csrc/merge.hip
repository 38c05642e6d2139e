// Merge of split-key partial results into the attention output.
//
// "Self-attention Does Not Need O(n^2) Memory" (方法详解; English digest
// method bullets) processes key blocks independently and combines their
// summaries; "当注意力成为瓶颈…", section IO感知, gives the combination for
// two blocks: the merged maximum is the larger block maximum, and the sums
// and outputs of both blocks are re-based on it before they are added. Here
// it is applied to all S key ranges of a row at once:
//     M   = max_s ref_s
//     w_s = l_s * 2^(ref_s - M)          (the range's weight on the common base)
//     L   = sum_s w_s,   O = (sum_s w_s * o_s) / L
// where o_s = acc_s / l_s is the range's normalised partial row and ref_s the
// base its l_s and acc_s were formed against, both written by the forward
// kernels in split-key mode:
//  * bf16 inputs: record {m_s (raw max of q.k), R_s (log2 reference), l_s};
//    ref_s = R_s, already in log2 units. The row statistics follow as in the
//    unsplit kernel: m = (max_s m_s) / sqrt(d), l = L * 2^(M - m_raw * C).
//  * fp32 inputs: record {m_s (fp64 raw max), l_s}; the exponent
//    (m_s - M) * log2(e)/sqrt(d) is formed in fp64 and rounded once, as in the
//    kernel's own rescale; m = fl(M / sqrt(d)), l = L * exp(M / sqrt(d) - m).
//
// HBM-bound in bytes (each row reads S * (d + 4) floats and writes d
// outputs), latency-bound in practice when a few rows carry many ranges
// (decoding). So a row is spread over CL = D/4 column lanes (16 bytes each)
// times SL split lanes; split lane j takes ranges j, j + SL, ... and the SL
// partial results of a row are combined through LDS.
#include "mea_device.h"
#include "mea_launch.h"

namespace mea {
namespace {

constexpr int kThreads = 256;

struct MergeArgs {
  const float* Po;  // [splits, rows, D]
  const float* Ps;  // [splits, rows, 4]
  void* O;          // [rows, D] in the output type
  float* Mx;        // [rows] or null
  float* Ls;
  int64_t rows;
  int splits;
  float C;          // log2(e) / sqrt(D)
  float scale;      // 1 / sqrt(D)
  double C64;
  double scale64;
};

template <int D, bool kBf16, int SL>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeArgs a) {
  constexpr int CL = D / 4;        // column lanes per row
  constexpr int TPR = CL * SL;     // threads per row
  constexpr int RPW = kThreads / TPR;
  static_assert(RPW * TPR == kThreads, "rows must tile the workgroup");
  __shared__ double s_ref[RPW][SL];   // per split lane: max reference (R or fp64 m)
  __shared__ float s_raw[RPW][SL];    // bf16: max raw score
  __shared__ f32x4 s_acc[RPW][SL][CL];
  __shared__ float s_sum[RPW][SL];

  const int t = threadIdx.x;
  const int rl = t / TPR;
  const int j = (t - rl * TPR) / CL;
  const int c = t - rl * TPR - j * CL;
  const int64_t rstride = a.rows * 4;
  const int64_t pstride = a.rows * D;

  // workgroup-uniform stride over the rows (the grid may be capped). The two
  // barriers of a pass also order it against the next: a pass writes s_ref
  // only after every thread has read the previous pass's values (before its
  // second barrier), and s_acc only after every thread has finished the
  // previous pass (its first barrier).
  for (int64_t r0 = (int64_t)blockIdx.x * RPW; r0 < a.rows; r0 += (int64_t)gridDim.x * RPW) {
    const int64_t row = r0 + rl;
    const bool live = row < a.rows;  // every thread reaches both barriers
    const float* rec0 = a.Ps + row * 4;
    const float* po0 = a.Po + row * D + c * 4;

    // 1. largest reference (and, for bf16, largest raw score) over this lane's ranges
    double ref = -INFINITY;
    float raw = -INFINITY;
    if (live) {
      for (int s = j; s < a.splits; s += SL) {
        const float* r = rec0 + s * rstride;
        if constexpr (kBf16) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(r);
          raw = fmaxf(raw, v[0]);
          ref = fmax(ref, (double)v[1]);
        } else {
          ref = fmax(ref, *reinterpret_cast<const double*>(r));
        }
      }
    }
    if (c == 0) {
      s_ref[rl][j] = ref;
      s_raw[rl][j] = raw;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      ref = fmax(ref, s_ref[rl][i]);
      raw = fmaxf(raw, s_raw[rl][i]);
    }

    // 2. this lane's ranges, re-based on the common reference
    f32x4 acc = f32x4{};
    float L = 0.f;
    if (live) {
      const float refb = (float)ref;  // bf16: an fp32 value already
      for (int s = j; s < a.splits; s += SL) {
        const float* r = rec0 + s * rstride;
        float w;
        if constexpr (kBf16) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(r);
          w = v[2] * fast_exp2(v[1] - refb);
        } else {
          w = r[2] * fast_exp2((float)((*reinterpret_cast<const double*>(r) - ref) * a.C64));
        }
        L += w;
        acc += w * *reinterpret_cast<const f32x4*>(po0 + s * pstride);
      }
    }
    s_acc[rl][j][c] = acc;
    if (c == 0) s_sum[rl][j] = L;
    __syncthreads();
    if (!live || j != 0) continue;
#pragma unroll
    for (int i = 1; i < SL; ++i) {
      acc += s_acc[rl][i][c];
      L += s_sum[rl][i];
    }
    const float inv = 1.f / L;
    if constexpr (kBf16) {
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc[e] * inv);
      *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.O) + row * D + c * 4) = o;
      if (a.Mx != nullptr && c == 0) {
        a.Mx[row] = raw * a.scale;
        a.Ls[row] = L * fast_exp2(-__builtin_fmaf(raw, a.C, -(float)ref));
      }
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.O) + row * D + c * 4) = acc * inv;
      if (a.Mx != nullptr && c == 0) {
        // as in the unsplit kernel: l against the reported (rounded) maximum
        const double m_nat = ref * a.scale64;
        const float m_st = (float)m_nat;
        a.Mx[row] = m_st;
        a.Ls[row] = (float)((double)L * exp(m_nat - (double)m_st));
      }
    }
  }
}

template <int D, bool kBf16, int SL>
hipError_t launch_sl(const MergeArgs& a, hipStream_t stream) {
  constexpr int RPW = kThreads / (D / 4 * SL);
  hipLaunchKernelGGL((merge_kernel<D, kBf16, SL>), dim3(row_blocks(a.rows, RPW)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool kBf16>
hipError_t launch(const FwdProblem& p, hipStream_t stream) {
  MergeArgs a;
  a.rows = p.heads * p.rows_q;
  a.splits = p.splits;
  a.Po = p.part;
  a.Ps = p.part + (int64_t)p.splits * a.rows * D;
  a.O = p.o;
  a.Mx = p.m;
  a.Ls = p.l;
  a.scale = 1.0f / sqrtf((float)D);
  a.C = kLog2e * a.scale;
  a.scale64 = 1.0 / sqrt((double)D);
  a.C64 = 1.4426950408889634 * a.scale64;
  // more split lanes while there are ranges to share and the grid is small
  constexpr int kMaxSL = kThreads / (D / 4);
  int sl = 1;
  while (sl * 2 <= kMaxSL && sl * 2 <= a.splits && a.rows * (D / 4) * sl < (int64_t)512 * kThreads)
    sl *= 2;
  switch (sl) {
    case 1: return launch_sl<D, kBf16, 1>(a, stream);
    case 2: return launch_sl<D, kBf16, 2>(a, stream);
    case 4: return launch_sl<D, kBf16, 4>(a, stream);
    case 8: return launch_sl<D, kBf16, 8>(a, stream);
    default:
      if constexpr (kMaxSL >= 16) return launch_sl<D, kBf16, 16>(a, stream);
      return launch_sl<D, kBf16, 8>(a, stream);
  }
}

}  // namespace

hipError_t launch_merge(bool bf16, int d, const FwdProblem& p, hipStream_t stream) {
  if (bf16) return d == 64 ? launch<64, true>(p, stream) : launch<128, true>(p, stream);
  return d == 64 ? launch<64, false>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace mea
