// Reduce pass of the split backward: sums the fp32 partial gradients that the
// key ranges (dQ) or query-tile ranges (dK, dV) of a small grid wrote to the
// workspace, applies the 1/sqrt(d) factor of dK and dQ, and writes the
// outputs in the input type. The gradients are sums over keys (dQ) or over
// query rows (dK, dV), so splitting those sums into ranges and adding the
// range totals gives the same result up to rounding. The range totals are
// added and scaled in fp64 and rounded once to the output type: where many
// query rows share few keys, a key's dV or dK is a sum of hundreds of terms of
// one sign (|dV| ~ 65 for 600 rows on one key) and fp32 additions of the range
// totals alone would cost about one fp32 ulp of that magnitude (7.6e-6).
//
// HBM-bound: per output row S * d * 4 bytes read and d * sizeof(T) written.
// One thread per 4 columns; the grid is capped and strides over the rows.
#include <type_traits>

#include "mea_device.h"
#include "mea_launch.h"

namespace mea {
namespace {

constexpr int kThreads = 256;

struct ReduceJob {
  const float* part;  // [splits][rows][D]
  void* out;          // [rows][D] in the output type
  int64_t rows;
  int splits;
  float scale;
};

struct ReduceArgs {
  ReduceJob job[3];
  int jobs;
};

template <int D, typename T>
__global__ __launch_bounds__(kThreads) void bwd_reduce_kernel(const ReduceArgs a) {
  constexpr int CPR = D / 4;              // threads per row
  constexpr int RPB = kThreads / CPR;     // rows per workgroup and pass
  const int c = threadIdx.x % CPR;
  for (int j = 0; j < a.jobs; ++j) {
    const ReduceJob& jb = a.job[j];
    const int64_t stride = jb.rows * D;  // floats between two splits' partials
    for (int64_t r0 = (int64_t)blockIdx.x * RPB; r0 < jb.rows; r0 += (int64_t)gridDim.x * RPB) {
      const int64_t row = r0 + threadIdx.x / CPR;
      if (row >= jb.rows) continue;
      const float* src = jb.part + row * D + c * 4;
      double sum[4] = {0.0, 0.0, 0.0, 0.0};
      for (int s = 0; s < jb.splits; ++s) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(src + s * stride);
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[e] += (double)x[e];
      }
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (float)(sum[e] * (double)jb.scale);
      if constexpr (std::is_same<T, float>::value) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(jb.out) + row * D + c * 4) = r;
      } else {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)r[e];
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(jb.out) + row * D + c * 4) = o;
      }
    }
  }
}

template <int D, typename T>
hipError_t launch(const BwdProblem& p, hipStream_t stream) {
  ReduceArgs a;
  a.jobs = 0;
  const float scale = 1.0f / sqrtf((float)D);
  int64_t rows_max = 0;
  auto add = [&](const float* part, void* out, int64_t rows, int splits, float sc) {
    a.job[a.jobs++] = ReduceJob{part, out, rows, splits, sc};
    rows_max = rows > rows_max ? rows : rows_max;
  };
  if (p.split.kv > 1) {
    add(p.part_dk, p.dk, p.heads * p.n_k, p.split.kv, scale);
    add(p.part_dv, p.dv, p.heads * p.n_k, p.split.kv, 1.0f);
  }
  if (p.split.q > 1) add(p.part_dq, p.dq, p.heads * p.rows_q, p.split.q, scale);
  if (a.jobs == 0 || rows_max == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_reduce_kernel<D, T>), dim3(row_blocks(rows_max, kThreads / (D / 4))),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_reduce(bool is_bf16, int d, const BwdProblem& p, hipStream_t stream) {
  if (is_bf16) return d == 64 ? launch<64, bf16>(p, stream) : launch<128, bf16>(p, stream);
  return d == 64 ? launch<64, float>(p, stream) : launch<128, float>(p, stream);
}

}  // namespace mea
