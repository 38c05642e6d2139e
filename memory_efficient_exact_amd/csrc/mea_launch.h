// Internal launcher declarations shared by the C-ABI layer and the kernel
// translation units. Shapes arrive already validated; every launcher enqueues
// on `stream` and returns the hipGetLastError() code of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mea {

// bf16 forward: q, k, v, o bf16 [BH, n, d]; m, l fp32 [BH, n] or both null.
hipError_t launch_fwd_bf16(int d, int64_t BH, int n, const void* q, const void* k, const void* v,
                           void* o, float* m, float* l, hipStream_t stream);

// fp32 forward (fp64 scores): same layout with fp32 elements.
hipError_t launch_fwd_f32(int d, int64_t BH, int n, const void* q, const void* k, const void* v,
                          void* o, float* m, float* l, hipStream_t stream);

// bf16 backward: three kernels (row preprocess, dK/dV, dQ). ws holds 2*BH*n floats.
hipError_t launch_bwd_bf16(int d, int64_t BH, int n, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* m, const float* l,
                           void* dq, void* dk, void* dv, float* ws, hipStream_t stream);

}  // namespace mea
