// Issue-cost probes for gfx950: the measurements behind the roofline reading of
// the attention kernels (how much MFMA work and how much VALU work one SIMD can
// issue, alone and together, what fp32 atomic adds in the pattern of a
// single-pass backward sustain, and what plain 16-byte streams read, write and
// copy from and to HBM: the bandwidth the decoding kernels can reach). Register-only loops of one instruction kind,
// timed per wave with the core-clock counter (s_memtime) and the 100 MHz
// real-time counter (s_memrealtime), whose ratio gives the clock the loop ran
// at. Prints one JSON object on stdout.
//
// Every probe writes only its own output arrays, sized from the launch shape
// checked on the host. Built by memory_efficient_exact_amd/build.py into
// memory_efficient_exact_amd/probes/mea_probe; run by `bench.py --mode probe`.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kCUs = 256;
constexpr int kIters = 2048;  // a multiple of 4 (the register-only loops run four iterations per pass)
static_assert(kIters % 4 == 0, "run_loop is unrolled by four");

enum Kind : int {
  kMfma = 0,    // 4 independent v_mfma_f32_32x32x16_bf16 chains
  kFma,         // 8 independent v_fma_f32 chains
  kAdd,         // 8 v_add_f32
  kMul,         // 8 v_mul_f32
  kExp,         // 8 v_exp_f32
  kMax3,        // 8 v_max3_f32
  kCvtPk,       // 8 v_cvt_pk_bf16_f32
  kPkFmaF16,    // 8 v_pk_fma_f16 (two fp16 values each)
  kMixTwoWaves,  // per SIMD: one wave runs the MFMA loop, another the FMA loop
  kMix1Fma8,     // one wave: 4 MFMAs and 8 independent FMAs per iteration
  kMix1Fma16,    // one wave: 4 MFMAs and 16 FMAs
  kMix1Fma32,    // one wave: 4 MFMAs and 32 FMAs
  kMix1Exp8,     // one wave: 4 MFMAs and 8 v_exp_f32
  kMix2Fma8,     // two waves per SIMD, each 4 MFMAs and 8 FMAs per iteration
  kMfmaLds,      // 4 MFMAs whose A operands come from 4 ds_read_b128 of LDS
  kMfmaLdsTr,    // 4 MFMAs whose A operands come from 8 ds_read_b64_tr_b16 of LDS
  kMfmaLdsPre,   // as kMfmaLds, each iteration's operands read one iteration ahead
  kMfmaLdsTrPre, // as kMfmaLdsTr, read one iteration ahead
  kExpAdd,       // 4 v_exp_f32 and 4 v_add_f32, alternating (does the exponential overlap?)
  kExpFma,       // 4 v_exp_f32 and 4 v_fma_f32, alternating
  kMixTwoWavesExp,  // per SIMD: one wave runs the MFMA loop, another the v_exp_f32 loop
  kKinds
};
const char* kNames[kKinds] = {"mfma_32x32x16_bf16", "v_fma_f32", "v_add_f32", "v_mul_f32",
                              "v_exp_f32", "v_max3_f32", "v_cvt_pk_bf16_f32", "v_pk_fma_f16",
                              "mfma_wave+fma_wave", "one_wave:4mfma+8fma", "one_wave:4mfma+16fma",
                              "one_wave:4mfma+32fma", "one_wave:4mfma+8exp", "two_waves:4mfma+8fma_each",
                              "mfma_fed_by_ds_read_b128", "mfma_fed_by_ds_read_b64_tr_b16",
                              "mfma_fed_by_ds_read_b128_read_ahead",
                              "mfma_fed_by_ds_read_b64_tr_b16_read_ahead",
                              "v_exp_f32+v_add_f32", "v_exp_f32+v_fma_f32", "mfma_wave+exp_wave"};
// MFMAs, and VALU instructions of the probed kind, per loop iteration
constexpr int kMfmaPerIter[kKinds] = {4, 0, 0, 0, 0, 0, 0, 0, 4, 4, 4, 4, 4, 4, 4, 4, 4, 4, 0, 0, 4};
constexpr int kValuPerIter[kKinds] = {0, 8, 8, 8, 8, 8, 8, 8, 8, 8, 16, 32, 8, 8, 0, 0, 0, 0, 8, 8, 8};
// LDS probes: a 32 KiB tile of bf16 per workgroup; every read stays inside it
constexpr int kLdsElems = 16384;

struct WaveTime {
  unsigned long long cycles;
  unsigned long long rt;  // 100 MHz ticks
  int role;               // 0: MFMA body, 1: VALU body
  int pad;
};

#define VALU8(INSN)                                                              \
  asm volatile(INSN : "+v"(x0) : "v"(a), "v"(b));                               \
  asm volatile(INSN : "+v"(x1) : "v"(a), "v"(b));                               \
  asm volatile(INSN : "+v"(x2) : "v"(a), "v"(b));                               \
  asm volatile(INSN : "+v"(x3) : "v"(a), "v"(b));                               \
  asm volatile(INSN : "+v"(x4) : "v"(a), "v"(b));                               \
  asm volatile(INSN : "+v"(x5) : "v"(a), "v"(b));                               \
  asm volatile(INSN : "+v"(x6) : "v"(a), "v"(b));                               \
  asm volatile(INSN : "+v"(x7) : "v"(a), "v"(b));

template <int K>
__device__ __forceinline__ void valu_body(float& x0, float& x1, float& x2, float& x3, float& x4,
                                          float& x5, float& x6, float& x7, float a, float b) {
  if constexpr (K == kFma) { VALU8("v_fma_f32 %0, %1, %2, %0") }
  if constexpr (K == kAdd) { VALU8("v_add_f32 %0, %1, %0") }
  if constexpr (K == kMul) { VALU8("v_mul_f32 %0, %1, %0") }
  if constexpr (K == kExp) { VALU8("v_exp_f32 %0, -%0") }
  if constexpr (K == kMax3) { VALU8("v_max3_f32 %0, %0, %1, %2") }
  if constexpr (K == kCvtPk) { VALU8("v_cvt_pk_bf16_f32 %0, %1, %2") }
  if constexpr (K == kPkFmaF16) { VALU8("v_pk_fma_f16 %0, %1, %2, %0") }
  if constexpr (K == kExpAdd) {
    asm volatile("v_exp_f32 %0, -%0" : "+v"(x0));
    asm volatile("v_add_f32 %0, %1, %0" : "+v"(x1) : "v"(a));
    asm volatile("v_exp_f32 %0, -%0" : "+v"(x2));
    asm volatile("v_add_f32 %0, %1, %0" : "+v"(x3) : "v"(a));
    asm volatile("v_exp_f32 %0, -%0" : "+v"(x4));
    asm volatile("v_add_f32 %0, %1, %0" : "+v"(x5) : "v"(a));
    asm volatile("v_exp_f32 %0, -%0" : "+v"(x6));
    asm volatile("v_add_f32 %0, %1, %0" : "+v"(x7) : "v"(a));
  }
  if constexpr (K == kExpFma) {
    asm volatile("v_exp_f32 %0, -%0" : "+v"(x0));
    asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x1) : "v"(a), "v"(b));
    asm volatile("v_exp_f32 %0, -%0" : "+v"(x2));
    asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x3) : "v"(a), "v"(b));
    asm volatile("v_exp_f32 %0, -%0" : "+v"(x4));
    asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x5) : "v"(a), "v"(b));
    asm volatile("v_exp_f32 %0, -%0" : "+v"(x6));
    asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x7) : "v"(a), "v"(b));
  }
}

struct Mfma4 {
  f32x16 c0, c1, c2, c3;
  bf16x8 fa, fb;
  __device__ __forceinline__ void step() {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fa, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fb, c3, 0, 0, 0);
  }
  __device__ float sum() const {
    float s = 0.f;
    for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
    return s;
  }
};

// one loop per wave; MFMA: 4 MFMAs per iteration; V: the VALU kind, N8 groups of 8.
// Unrolled by four (iters, kIters below, is a multiple of four): each scalar loop-control
// instruction costs the wave issue cycles of its own, and three of them per
// eight VALU instructions made v_add_f32 read 7.5 cycles per issue instead of ~5.
template <bool MFMA, int V, int N8>
__device__ __forceinline__ void run_loop(Mfma4& m, float* x, float a, float b, int iters) {
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (MFMA) m.step();
#pragma unroll
      for (int g = 0; g < N8; ++g) valu_body<V>(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7], a, b);
    }
  }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// 4 MFMAs per iteration with A operands read from LDS: row-wise (16 bytes per lane,
// as the score products read K or Q rows) or transposed (two 8-byte reads per
// operand, as the gradient products read dO^T, Q^T or K^T). The read offsets walk
// through the tile with the iteration (masked to its size), so every read is new.
template <bool TR>
__device__ __forceinline__ void lds_read4(bf16x8* a, const __bf16* lds, int lane, int it) {
  const int base = (it * 512) & (kLdsElems - 1);  // multiple of 512 elements, < kLdsElems
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // masked to the tile: every 16-byte read starts at a multiple of 8 elements inside it
    const int off = (base + j * 1024 + lane * 8) & (kLdsElems - 8);
    if constexpr (!TR) {
      a[j] = *reinterpret_cast<const bf16x8*>(lds + off);
    } else {
      const int off2 = (off + 256) & (kLdsElems - 8);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(lds + off));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(lds + off2));
      const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
      a[j] = bf16x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
    }
  }
}

__device__ __forceinline__ void mfma4(Mfma4& m, const bf16x8* a) {
  m.c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], m.fb, m.c0, 0, 0, 0);
  m.c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], m.fb, m.c1, 0, 0, 0);
  m.c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], m.fb, m.c2, 0, 0, 0);
  m.c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], m.fb, m.c3, 0, 0, 0);
}

// AHEAD: the reads for iteration it + 1 are issued before the MFMAs of iteration
// it (two register sets, loop unrolled by two; iters is even)
template <bool TR, bool AHEAD>
__device__ __forceinline__ void lds_loop(Mfma4& m, const __bf16* lds, int lane, int iters) {
  if constexpr (!AHEAD) {
    for (int it = 0; it < iters; ++it) {
      bf16x8 a[4];
      lds_read4<TR>(a, lds, lane, it);
      mfma4(m, a);
    }
  } else {
    // scheduling barriers keep each read group ahead of the MFMAs it overlaps (the
    // scheduler otherwise moves reads back next to their uses)
    bf16x8 a[4], b[4];
    lds_read4<TR>(a, lds, lane, 0);
    for (int it = 0; it < iters; it += 2) {
      lds_read4<TR>(b, lds, lane, it + 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma4(m, a);
      __builtin_amdgcn_sched_barrier(0);
      lds_read4<TR>(a, lds, lane, it + 2);
      __builtin_amdgcn_sched_barrier(0);
      mfma4(m, b);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int K>
__global__ __launch_bounds__(512) void probe_kernel(WaveTime* out, float* sink, int iters, int flag) {
  __shared__ __attribute__((aligned(1024))) __bf16 lds[K >= kMfmaLds ? kLdsElems : 8];
  const int lane = threadIdx.x & 63;
  // wave index made wave-uniform in a scalar register, so the role test below is a
  // scalar branch around whole loops, not a per-lane mask inside them
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * (blockDim.x >> 6) + wave;  // < gridDim.x * waves per block
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = (float)(lane + i);
  const float a = 0.999f, b = 1e-3f * (float)(lane & 7);
  Mfma4 m;
  m.c0 = m.c1 = m.c2 = m.c3 = f32x16{};
  for (int e = 0; e < 8; ++e) {
    m.fa[e] = (__bf16)(0.01f * (float)((lane + e) & 15));
    m.fb[e] = (__bf16)(0.02f * (float)((lane * 3 + e) & 15));
  }
  // in the two-wave probe the first four waves of a block (one per SIMD) run the
  // MFMA loop and the other four the FMA loop
  const int role = ((K == kMixTwoWaves || K == kMixTwoWavesExp) && wave >= 4) || (kMfmaPerIter[K] == 0) ? 1 : 0;
  if constexpr (K >= kMfmaLds) {
    for (int i = threadIdx.x; i < kLdsElems; i += blockDim.x) lds[i] = (__bf16)(0.001f * (float)(i & 255));
  }
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  if constexpr (K == kMfma) run_loop<true, kFma, 0>(m, x, a, b, iters);
  else if constexpr (K <= kPkFmaF16) run_loop<false, K, 1>(m, x, a, b, iters);
  else if constexpr (K == kMixTwoWaves) {
    if (role == 0) run_loop<true, kFma, 0>(m, x, a, b, iters);
    else run_loop<false, kFma, 1>(m, x, a, b, iters);
  } else if constexpr (K == kMix1Fma8 || K == kMix2Fma8) run_loop<true, kFma, 1>(m, x, a, b, iters);
  else if constexpr (K == kMix1Fma16) run_loop<true, kFma, 2>(m, x, a, b, iters);
  else if constexpr (K == kMix1Fma32) run_loop<true, kFma, 4>(m, x, a, b, iters);
  else if constexpr (K == kMix1Exp8) run_loop<true, kExp, 1>(m, x, a, b, iters);
  else if constexpr (K == kMfmaLds) lds_loop<false, false>(m, lds, lane, iters);
  else if constexpr (K == kMfmaLdsTr) lds_loop<true, false>(m, lds, lane, iters);
  else if constexpr (K == kMfmaLdsPre) lds_loop<false, true>(m, lds, lane, iters);
  else if constexpr (K == kMfmaLdsTrPre) lds_loop<true, true>(m, lds, lane, iters);
  else if constexpr (K == kExpAdd || K == kExpFma) run_loop<false, K, 1>(m, x, a, b, iters);
  else if constexpr (K == kMixTwoWavesExp) {
    if (role == 0) run_loop<true, kFma, 0>(m, x, a, b, iters);
    else run_loop<false, kExp, 1>(m, x, a, b, iters);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) out[gw] = WaveTime{t1 - t0, r1 - r0, role, 0};
  if (flag) {  // never set by the host: keeps every result live
    float sx = 0.f;
    for (int i = 0; i < 8; ++i) sx += x[i];
    sink[gw * 64 + lane] = sx + m.sum();
  }
}

// fp32 atomic adds in the pattern a single-pass backward would need for dQ at
// 1 x 16 x 16384 x 64 with 256-key workgroups: 16 heads x 64 key blocks = 1024
// workgroups of 512 threads, each adding one value per element of each of the
// 256 query tiles (64 rows x 64 columns) of its head into dq[head][row][col]
// (64 MiB). kind 0: atomicAdd (global_atomic_add_f32), 1: plain stores of the
// same volume, 2: atomicAdd with the key blocks of one head on one XCD.
constexpr int kH = 16, kN = 16384, kD = 64, kKB = 256, kTQ = 64;

__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total / 8;
  return (bid % 8) * per + bid / 8;
}

template <int MODE>
__global__ __launch_bounds__(512) void atomic_dq_kernel(float* __restrict__ dq) {
  const int wg = MODE == 2 ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;
  const int head = wg / (kN / kKB);  // < kH (grid = kH * kN / kKB)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* base = dq + (size_t)head * kN * kD;
  const float val = (1 + (wg & 3)) / 1024.0f;
  for (int t = 0; t < kN / kTQ; ++t) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float* p = base + (size_t)(t * kTQ + wave * 8 + r) * kD + lane;  // row < kN, lane < kD
      if constexpr (MODE == 1) *p = val;
      else atomicAdd(p, val);
    }
  }
}

// HBM streams: kStreamVecs 16-byte vectors (2 GiB) over kStreamGrid workgroups of
// 256 threads, each thread handling kStreamPerThread vectors (kStreamVecs =
// kStreamGrid * 256 * kStreamPerThread exactly, checked on the host), UNROLL loads
// in flight per step. STRIDED: thread t takes vectors t + j * (grid threads);
// otherwise workgroup b streams its own contiguous chunk of 256 * kStreamPerThread
// vectors, thread t taking vectors t + 256 * j of it. The read stream folds what
// it reads into one word per thread (written to `sink`), so no load is dropped.
constexpr int kStreamGrid = 8192;
constexpr int kStreamPerThread = 64;
constexpr size_t kStreamVecs = (size_t)kStreamGrid * 256 * kStreamPerThread;  // 2^27

template <int MODE, bool STRIDED, int UNROLL>  // MODE 0: read, 1: write, 2: copy
__global__ __launch_bounds__(256) void stream_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst,
                                                     unsigned* __restrict__ sink) {
  static_assert(kStreamPerThread % UNROLL == 0, "whole steps");
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // < grid threads
  const size_t base = STRIDED ? t : (size_t)blockIdx.x * 256 * kStreamPerThread + threadIdx.x;
  const size_t step = STRIDED ? (size_t)gridDim.x * blockDim.x : 256;
  unsigned acc = 0;
  for (int j = 0; j < kStreamPerThread; j += UNROLL) {
    uint4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const size_t i = base + (size_t)(j + u) * step;  // < kStreamVecs
      if constexpr (MODE == 1) v[u] = make_uint4((unsigned)i, 0u, 0u, 1u);
      else v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const size_t i = base + (size_t)(j + u) * step;
      if constexpr (MODE == 0) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      else dst[i] = v[u];
    }
  }
  if constexpr (MODE == 0) sink[t] = acc;
}

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
      exit(2);                                                                    \
    }                                                                             \
  } while (0)

void launch_probe(int kind, dim3 grid, dim3 block, WaveTime* out, float* sink, int iters) {
  switch (kind) {
#define CASE(K) case K: hipLaunchKernelGGL(probe_kernel<K>, grid, block, 0, 0, out, sink, iters, 0); break;
    CASE(kMfma) CASE(kFma) CASE(kAdd) CASE(kMul) CASE(kExp) CASE(kMax3) CASE(kCvtPk) CASE(kPkFmaF16)
    CASE(kMixTwoWaves) CASE(kMix1Fma8) CASE(kMix1Fma16) CASE(kMix1Fma32) CASE(kMix1Exp8) CASE(kMix2Fma8)
    CASE(kMfmaLds) CASE(kMfmaLdsTr) CASE(kMfmaLdsPre) CASE(kMfmaLdsTrPre) CASE(kExpAdd) CASE(kExpFma) CASE(kMixTwoWavesExp)
#undef CASE
  }
}

double median(std::vector<double> v) {
  std::sort(v.begin(), v.end());
  return v.empty() ? 0.0 : v[v.size() / 2];
}

}  // namespace

int main() {
  WaveTime* out = nullptr;
  float* sink = nullptr;
  const int max_waves = kCUs * 16;  // at most 4 waves per SIMD (4 blocks of 4 waves per CU)
  CHECK(hipMalloc(&out, max_waves * sizeof(WaveTime)));
  CHECK(hipMalloc(&sink, (size_t)max_waves * 64 * sizeof(float)));
  std::vector<WaveTime> host(max_waves);
  std::string json = "{\"probes\": [";
  bool first = true;
  struct Run { int kind; int waves_per_simd; };
  std::vector<Run> runs;
  // (four waves per SIMD only for the VALU kinds: four 4-wave blocks of the MFMA
  // loop per CU measured 24 cycles per MFMA, below the 32-cycle floor, so those
  // waves do not all share their SIMD for the whole loop)
  for (int k = kMfma; k <= kPkFmaF16; ++k)
    for (int w : {1, 2, 4})
      if (k != kMfma || w < 4) runs.push_back({k, w});
  runs.push_back({kMixTwoWaves, 2});
  runs.push_back({kMixTwoWavesExp, 2});
  for (int k = kMix1Fma8; k <= kMix1Exp8; ++k) runs.push_back({k, 1});
  runs.push_back({kMix2Fma8, 2});
  for (int k = kMfmaLds; k <= kMfmaLdsTrPre; ++k)
    for (int w : {1, 2}) runs.push_back({k, w});
  for (int k = kExpAdd; k <= kExpFma; ++k)
    for (int w : {1, 2, 4}) runs.push_back({k, w});
  for (const Run& r : runs) {
    // 4-wave blocks, one wave per SIMD, w blocks per CU; the two-wave probe uses
    // 8-wave blocks (one MFMA wave and one FMA wave per SIMD)
    const bool two = r.kind == kMixTwoWaves || r.kind == kMixTwoWavesExp;
    const int wpb = two ? 8 : 4;
    const int blocks = two ? kCUs : kCUs * r.waves_per_simd;
    const int waves = blocks * wpb;
    if (waves > max_waves) return 3;
    for (int rep = 0; rep < 2; ++rep) {  // the first launch warms the clock
      launch_probe(r.kind, dim3(blocks), dim3(64 * wpb), out, sink, kIters);
      CHECK(hipGetLastError());
      CHECK(hipDeviceSynchronize());
    }
    CHECK(hipMemcpy(host.data(), out, waves * sizeof(WaveTime), hipMemcpyDeviceToHost));
    std::vector<double> cyc[2], mhz;
    for (int i = 0; i < waves; ++i) {
      cyc[host[i].role].push_back((double)host[i].cycles);
      if (host[i].rt > 0) mhz.push_back(100.0 * (double)host[i].cycles / (double)host[i].rt);
    }
    const double per_it_mfma = median(cyc[0]) / kIters, per_it_valu = median(cyc[1]) / kIters;
    char buf[512];
    snprintf(buf, sizeof buf,
             "%s{\"probe\": \"%s\", \"waves_per_simd\": %d, \"clock_mhz\": %.0f, "
             "\"mfma_wave_cycles_per_iter\": %.2f, \"valu_wave_cycles_per_iter\": %.2f, "
             "\"mfma_per_iter\": %d, \"valu_per_iter\": %d}",
             first ? "" : ", ", kNames[r.kind], r.waves_per_simd, median(mhz), per_it_mfma,
             per_it_valu, kMfmaPerIter[r.kind], kValuPerIter[r.kind]);
    json += buf;
    first = false;
  }
  json += "], \"atomic_dq\": [";
  float* dq = nullptr;
  const size_t elems = (size_t)kH * kN * kD;
  CHECK(hipMalloc(&dq, elems * sizeof(float)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const int grid = kH * (kN / kKB);
  const double bytes = (double)grid * (kN / kTQ) * kTQ * kD * 4;
  const char* modes[3] = {"atomic_add_f32", "plain_store", "atomic_add_f32_xcd_local_heads"};
  for (int mode = 0; mode < 3; ++mode) {
    float best = 1e30f;
    for (int rep = 0; rep < 3; ++rep) {
      CHECK(hipMemset(dq, 0, elems * sizeof(float)));
      CHECK(hipDeviceSynchronize());
      CHECK(hipEventRecord(e0, 0));
      if (mode == 0) hipLaunchKernelGGL(atomic_dq_kernel<0>, dim3(grid), dim3(512), 0, 0, dq);
      else if (mode == 1) hipLaunchKernelGGL(atomic_dq_kernel<1>, dim3(grid), dim3(512), 0, 0, dq);
      else hipLaunchKernelGGL(atomic_dq_kernel<2>, dim3(grid), dim3(512), 0, 0, dq);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1, 0));
      CHECK(hipEventSynchronize(e1));
      float ms = 0.f;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      best = std::min(best, ms);
    }
    float v0 = 0.f;
    CHECK(hipMemcpy(&v0, dq, sizeof(float), hipMemcpyDeviceToHost));
    char buf[256];
    snprintf(buf, sizeof buf, "%s{\"mode\": \"%s\", \"ms\": %.4f, \"bytes\": %.0f, \"tb_per_s\": %.3f, \"dq0\": %.6f}",
             mode ? ", " : "", modes[mode], best, bytes, bytes / (best * 1e-3) / 1e12, v0);
    json += buf;
  }
  json += "], \"hbm_stream\": [";
  CHECK(hipFree(dq));
  {
    const int threads = kStreamGrid * 256;
    if ((size_t)threads * kStreamPerThread != kStreamVecs || kStreamPerThread % 4) return 4;
    uint4 *a = nullptr, *b = nullptr;
    unsigned* sk = nullptr;
    const size_t bytes = kStreamVecs * sizeof(uint4);
    CHECK(hipMalloc(&a, bytes));
    CHECK(hipMalloc(&b, bytes));
    CHECK(hipMalloc(&sk, (size_t)threads * sizeof(unsigned)));
    CHECK(hipMemset(a, 1, bytes));
    CHECK(hipMemset(b, 0, bytes));
    struct Stream { const char* name; int mode; void (*kernel)(const uint4*, uint4*, unsigned*); };
    const Stream streams[] = {
        {"read_strided_x4", 0, stream_kernel<0, true, 4>},
        {"read_blocked_x4", 0, stream_kernel<0, false, 4>},
        {"read_blocked_x8", 0, stream_kernel<0, false, 8>},
        {"write_blocked_x4", 1, stream_kernel<1, false, 4>},
        {"copy_blocked_x4", 2, stream_kernel<2, false, 4>},
    };
    bool first_stream = true;
    for (const Stream& st : streams) {
      float best = 1e30f;
      for (int rep = 0; rep < 4; ++rep) {  // the first launch warms the clock
        CHECK(hipDeviceSynchronize());
        CHECK(hipEventRecord(e0, 0));
        hipLaunchKernelGGL(st.kernel, dim3(kStreamGrid), dim3(256), 0, 0, a, b, sk);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e1, 0));
        CHECK(hipEventSynchronize(e1));
        float ms = 0.f;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        if (rep > 0) best = std::min(best, ms);
      }
      const double moved = (st.mode == 2 ? 2.0 : 1.0) * (double)bytes;  // copy: read + write
      char buf[256];
      snprintf(buf, sizeof buf, "%s{\"mode\": \"%s\", \"ms\": %.4f, \"bytes\": %.0f, \"tb_per_s\": %.3f}",
               first_stream ? "" : ", ", st.name, best, moved, moved / (best * 1e-3) / 1e12);
      json += buf;
      first_stream = false;
    }
    CHECK(hipFree(a));
    CHECK(hipFree(b));
    CHECK(hipFree(sk));
  }
  json += "]}";
  printf("%s\n", json.c_str());
  CHECK(hipFree(out));
  CHECK(hipFree(sink));
  return 0;
}
