// C ABI of the library (declared in include/mea.h): argument validation on
// the host, then dispatch to the gfx950 kernels on the caller's stream.
// Validation never calls HIP, so every error path can be exercised without a
// GPU. The library allocates nothing and keeps no state.
#include <climits>
#include <cstdint>

#include "../../include/mea.h"
#include "mea_launch.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0
// Largest grid the kernels are launched with is B*H*ceil(n/64) workgroups of
// 256 threads; keep it (and all row indices) comfortably inside 32 bits.
constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxBH = int64_t(1) << 24;
constexpr int64_t kMaxBlocks = int64_t(1) << 23;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mea_status_t check_common(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d, bool* empty) {
  if (dt != MEA_DTYPE_F32 && dt != MEA_DTYPE_BF16) return MEA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || n < 0 || d < 0) return MEA_ERR_SHAPE;
  if (n > kMaxN) return MEA_ERR_SHAPE;
  if (H != 0 && B > kMaxBH / H) return MEA_ERR_SHAPE;
  if (B != 0 && H != 0 && B * H * ((n + 63) / 64) > kMaxBlocks) return MEA_ERR_SHAPE;
  if (d != 64 && d != 128) return MEA_ERR_UNSUPPORTED;
  *empty = (B == 0 || H == 0 || n == 0);
  return MEA_OK;
}

mea_status_t check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p == nullptr) return MEA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MEA_ERR_ALIGN;
  return MEA_OK;
}

}  // namespace

extern "C" {

const char* attn_status_str(mea_status_t s) {
  switch (s) {
    case MEA_OK: return "MEA_OK";
    case MEA_ERR_NULL: return "MEA_ERR_NULL";
    case MEA_ERR_SHAPE: return "MEA_ERR_SHAPE";
    case MEA_ERR_UNSUPPORTED: return "MEA_ERR_UNSUPPORTED";
    case MEA_ERR_ALIGN: return "MEA_ERR_ALIGN";
    case MEA_ERR_WORKSPACE: return "MEA_ERR_WORKSPACE";
    case MEA_ERR_LAUNCH: return "MEA_ERR_LAUNCH";
  }
  return "MEA_UNKNOWN_STATUS";
}

int mea_version(void) { return kVersion; }

mea_status_t attn_fwd(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d,
                      const void* q, const void* k, const void* v, void* o,
                      float* row_max, float* row_sum, void* stream) {
  bool empty = false;
  mea_status_t st = check_common(dt, B, H, n, d, &empty);
  if (st != MEA_OK || empty) return st;
  if ((row_max == nullptr) != (row_sum == nullptr)) return MEA_ERR_NULL;
  st = check_ptrs({q, k, v, o});
  if (st != MEA_OK) return st;
  if (row_max != nullptr && (!aligned16(row_max) || !aligned16(row_sum))) return MEA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = dt == MEA_DTYPE_BF16
                     ? mea::launch_fwd_bf16((int)d, B * H, (int)n, q, k, v, o, row_max, row_sum, s)
                     : mea::launch_fwd_f32((int)d, B * H, (int)n, q, k, v, o, row_max, row_sum, s);
  return e == hipSuccess ? MEA_OK : MEA_ERR_LAUNCH;
}

size_t attn_bwd_workspace_bytes(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d) {
  bool empty = false;
  if (check_common(dt, B, H, n, d, &empty) != MEA_OK || empty) return 0;
  return (size_t)(8 * B * H * n);
}

mea_status_t attn_bwd(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d,
                      const void* q, const void* k, const void* v, const void* o,
                      const void* dO, const float* row_max, const float* row_sum,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream) {
  bool empty = false;
  mea_status_t st = check_common(dt, B, H, n, d, &empty);
  if (st != MEA_OK || empty) return st;
  if (dt != MEA_DTYPE_BF16) return MEA_ERR_UNSUPPORTED;
  st = check_ptrs({q, k, v, o, dO, row_max, row_sum, dq, dk, dv});
  if (st != MEA_OK) return st;
  if (workspace == nullptr || workspace_bytes < (size_t)(8 * B * H * n)) return MEA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MEA_ERR_ALIGN;
  hipError_t e = mea::launch_bwd_bf16((int)d, B * H, (int)n, q, k, v, o, dO, row_max, row_sum,
                                      dq, dk, dv, static_cast<float*>(workspace),
                                      reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MEA_OK : MEA_ERR_LAUNCH;
}

}  // extern "C"
