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
//    kernel's own rescale; m = M / sqrt(d), l = L.
//
// HBM-bound: each row reads S * (d + 4) floats and writes d outputs. D/4 lanes
// per row, 16 bytes each, so a wave reads whole rows of every partial.
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

template <int D, bool kBf16>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeArgs a) {
  constexpr int LPR = D / 4;  // lanes per row
  const int64_t gtid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = gtid / LPR;
  const int col = (int)(gtid - row * LPR) * 4;
  if (row >= a.rows) return;  // no barriers below

  const float* rec0 = a.Ps + row * 4;
  const int64_t rstride = a.rows * 4;
  const float* po0 = a.Po + row * D + col;
  const int64_t pstride = a.rows * D;

  f32x4 acc = f32x4{};
  float L = 0.f;
  if constexpr (kBf16) {
    float m_raw = -INFINITY, M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) {
      const f32x4 r = *reinterpret_cast<const f32x4*>(rec0 + s * rstride);
      m_raw = fmaxf(m_raw, r[0]);
      M = fmaxf(M, r[1]);
    }
    for (int s = 0; s < a.splits; ++s) {
      const f32x4 r = *reinterpret_cast<const f32x4*>(rec0 + s * rstride);
      const float w = r[2] * fast_exp2(r[1] - M);
      L += w;
      acc += w * *reinterpret_cast<const f32x4*>(po0 + s * pstride);
    }
    const float inv = 1.f / L;
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.O) + row * D + col) = o;
    if (a.Mx != nullptr && col == 0) {
      a.Mx[row] = m_raw * a.scale;
      a.Ls[row] = L * fast_exp2(-__builtin_fmaf(m_raw, a.C, -M));
    }
  } else {
    double M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmax(M, *reinterpret_cast<const double*>(rec0 + s * rstride));
    for (int s = 0; s < a.splits; ++s) {
      const float* r = rec0 + s * rstride;
      const double m_s = *reinterpret_cast<const double*>(r);
      const float w = r[2] * fast_exp2((float)((m_s - M) * a.C64));
      L += w;
      acc += w * *reinterpret_cast<const f32x4*>(po0 + s * pstride);
    }
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.O) + row * D + col) = acc * (1.f / L);
    if (a.Mx != nullptr && col == 0) {
      a.Mx[row] = (float)(M * a.scale64);
      a.Ls[row] = L;
    }
  }
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
  const int64_t threads = a.rows * (D / 4);
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((merge_kernel<D, kBf16>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(bool bf16, int d, const FwdProblem& p, hipStream_t stream) {
  if (bf16) return d == 64 ? launch<64, true>(p, stream) : launch<128, true>(p, stream);
  return d == 64 ? launch<64, false>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace mea
