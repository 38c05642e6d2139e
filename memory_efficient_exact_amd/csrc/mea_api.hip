// C ABI of the library (declared in include/mea.h): argument validation on
// the host, then dispatch to the gfx950 kernels on the caller's stream.
// Validation never calls HIP, so every error path can be exercised without a
// GPU. The library allocates nothing; its only state is the per-device address
// of the scratch array that attn_bwd_noalloc uses.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <mutex>

#include "../../include/mea.h"
#include "mea_launch.h"

// Scratch memory of attn_bwd_noalloc: one array per GPU in the library's code
// object, alive until the process ends. In host code `scratch` names a host-side
// stand-in, not a device address: the address on each device comes from
// hipGetSymbolAddress, looked up once per device (see noalloc_scratch below),
// and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[MEA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kVersion = 400;  // 0.4.0
// Grid bounds. With heads * ceil(max(rows_q, n_k) / 64) <= kMaxBlocks, the
// tiled grids stay within 2^31 work-items: the largest give every 64 rows at
// most two workgroups of 256 threads (the backward's dK/dV plus dQ workgroups
// at 64 rows each, the decoding forwards' 32- or 16-row workgroups for heads
// of at most 64 or 32 rows), and a split grid is checked against the same
// bound. The per-row kernels (row terms, merge) cap their grids and stride.
// Row indices within a head stay below 2^24.
constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxBH = int64_t(1) << 24;
constexpr int64_t kMaxBlocks = int64_t(1) << 22;
// Split-key planning: at most this many key ranges per head; the automatic
// choice splits only grids smaller than one full round of resident
// workgroups (compute units x the forward kernel's workgroups per CU) and
// keeps at least two key tiles in every range.
constexpr int64_t kMaxSplits = 256;
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kAutoMinTiles = 2;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A validated problem: `heads` = B * H_kv, `rows_q` = G * n_q (see mea_launch.h).
struct Shape {
  bool bf16 = false;
  int d = 0;
  int64_t heads = 0;
  int64_t rows_q = 0;
  int64_t n_k = 0;
  int64_t q_rows_total = 0;  // B * H * n_q
  bool empty = false;        // nothing to compute
};

mea_status_t check_shape(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q,
                         int64_t n_k, int64_t d, Shape* s) {
  if (dt != MEA_DTYPE_F32 && dt != MEA_DTYPE_BF16) return MEA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || H_kv < 0 || n_q < 0 || n_k < 0 || d < 0) return MEA_ERR_SHAPE;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return MEA_ERR_SHAPE;
  if (n_q > kMaxN || n_k > kMaxN) return MEA_ERR_SHAPE;
  if (H != 0 && B > kMaxBH / H) return MEA_ERR_SHAPE;
  const int64_t G = H > 0 ? H / H_kv : 1;
  if (G * n_q > kMaxN) return MEA_ERR_SHAPE;
  const int64_t heads = B * (H > 0 ? H_kv : 0);
  if (heads != 0 && heads * std::max(cdiv(G * n_q, 64), cdiv(n_k, 64)) > kMaxBlocks)
    return MEA_ERR_SHAPE;
  if (d != 64 && d != 128) return MEA_ERR_UNSUPPORTED;
  s->bf16 = dt == MEA_DTYPE_BF16;
  s->d = (int)d;
  s->heads = heads;
  s->rows_q = G * n_q;
  s->n_k = n_k;
  s->q_rows_total = B * H * n_q;
  s->empty = heads == 0 || (n_q == 0 && n_k == 0);
  return MEA_OK;
}

// Backward workspace per query row: bf16 keeps {-D, lse2} as two floats; fp32
// keeps lse2 in fp64 (scores of ~1e4 need more than fp32 there) and -D.
size_t bwd_row_bytes(bool bf16) { return bf16 ? 8 : 16; }

// Split backward: grids of at most half the resident 4-wave workgroups (two
// per CU) cut each workgroup's sweep into ranges of at least kBwdMinTiles
// staged tiles, as many as keep the split grid within one round of resident
// workgroups, at most kMaxBwdSplits.
constexpr int64_t kMaxBwdSplits = 16;
constexpr int64_t kBwdMinTiles = 2;

mea::BwdSplit plan_bwd_split(const Shape& s) {
  mea::BwdSplit p;
  if (s.empty || s.rows_q == 0 || s.n_k == 0) return p;
  const mea::BwdGeometry g = s.bf16 ? mea::bwd_geometry_bf16(s.d) : mea::bwd_geometry_f32(s.d);
  const int64_t tiles_q = cdiv(s.rows_q, g.tile_rows), tiles_k = cdiv(s.n_k, g.tile_rows);
  p.len_q = (int)tiles_q;
  p.len_k = (int)tiles_k;
  const int64_t base = s.heads * (cdiv(s.n_k, g.wg_rows) + cdiv(s.rows_q, g.wg_rows));
  const int64_t want = std::min(kMaxBwdSplits, 2 * kComputeUnits / base);
  if (want < 2) return p;
  const int64_t len_q = std::min(tiles_q, std::max(kBwdMinTiles, cdiv(tiles_q, want)));
  const int64_t len_k = std::min(tiles_k, std::max(kBwdMinTiles, cdiv(tiles_k, want)));
  p.len_q = (int)len_q;
  p.kv = (int)cdiv(tiles_q, len_q);  // every range non-empty
  p.len_k = (int)len_k;
  p.q = (int)cdiv(tiles_k, len_k);
  return p;
}

// Backward workspace: the row terms, then (split sides only, from a 256-byte
// boundary) fp32 partials of dK and dV [kv][heads * n_k][d] and of dQ
// [q][heads * rows_q][d].
struct BwdLayout {
  mea::BwdSplit split;
  size_t part_off = 0;  // bytes
  size_t kv_part = 0;   // bytes of the dK partials (the dV partials follow)
  size_t q_part = 0;
  size_t total = 0;
};

BwdLayout bwd_layout(const Shape& s) {
  BwdLayout L;
  L.split = plan_bwd_split(s);
  const size_t rows = bwd_row_bytes(s.bf16) * (size_t)s.q_rows_total;
  L.part_off = (rows + 255) / 256 * 256;
  if (L.split.kv > 1) L.kv_part = (size_t)L.split.kv * s.heads * s.n_k * s.d * 4;
  if (L.split.q > 1) L.q_part = (size_t)L.split.q * s.heads * s.rows_q * s.d * 4;
  L.total = (L.kv_part + L.q_part) > 0 ? L.part_off + 2 * L.kv_part + L.q_part : rows;
  return L;
}

// Byte range [lo, hi) of one buffer of a call; empty ranges overlap nothing.
struct Span {
  uintptr_t lo = 0;
  uintptr_t hi = 0;
};
Span span(const void* p, int64_t bytes) {
  Span r;
  if (p != nullptr && bytes > 0) {
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + (uintptr_t)bytes;
  }
  return r;
}
bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

// Every output must be disjoint from the other outputs and from every input
// (the kernels read inputs while writing outputs); inputs may share memory.
mea_status_t check_alias(std::initializer_list<Span> outputs, std::initializer_list<Span> inputs) {
  for (auto o = outputs.begin(); o != outputs.end(); ++o) {
    for (auto p = o + 1; p != outputs.end(); ++p)
      if (overlap(*o, *p)) return MEA_ERR_ALIAS;
    for (const Span& i : inputs)
      if (overlap(*o, i)) return MEA_ERR_ALIAS;
  }
  return MEA_OK;
}

// Bytes of the query-side tensors (q, o, dO, dq), the key-side tensors (k, v,
// dk, dv) and one per-row statistics array of a validated shape.
int64_t q_bytes(const Shape& s) { return s.q_rows_total * s.d * (s.bf16 ? 2 : 4); }
int64_t kv_bytes(const Shape& s) { return s.heads * s.n_k * s.d * (s.bf16 ? 2 : 4); }
int64_t stat_bytes(const Shape& s) { return s.q_rows_total * 4; }

mea_status_t check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p == nullptr) return MEA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MEA_ERR_ALIGN;
  return MEA_OK;
}

// Forward-only shape rules: no query rows is a no-op; queries without keys
// have no softmax.
mea_status_t check_fwd_shape(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q,
                             int64_t n_k, int64_t d, Shape* s) {
  mea_status_t st = check_shape(dt, B, H, H_kv, n_q, n_k, d, s);
  if (st != MEA_OK) return st;
  if (s->rows_q == 0) s->empty = true;
  if (!s->empty && n_k == 0) return MEA_ERR_SHAPE;
  return MEA_OK;
}

struct SplitPlan {
  int64_t splits = 1;
  int64_t split_len = 0;
};

SplitPlan plan_splits(const Shape& s, int64_t requested) {
  SplitPlan p;
  p.split_len = s.n_k;
  if (s.empty || s.n_k == 0) return p;
  const mea::FwdGeometry g = mea::fwd_geometry(s.bf16, s.d, s.heads, s.rows_q);
  const int64_t tiles_k = cdiv(s.n_k, g.key_tile);
  int64_t want = requested;
  if (want <= 0) {
    const int64_t base = s.heads * cdiv(s.rows_q, g.query_rows);
    want = std::min(cdiv(kComputeUnits * g.resident, base), std::max<int64_t>(1, tiles_k / kAutoMinTiles));
  }
  want = std::max<int64_t>(1, std::min({want, tiles_k, kMaxSplits}));
  p.split_len = cdiv(tiles_k, want) * g.key_tile;  // whole key tiles per range
  p.splits = cdiv(s.n_k, p.split_len);             // every range non-empty
  if (p.splits == 1) p.split_len = s.n_k;
  return p;
}

size_t split_workspace_bytes(const Shape& s, const SplitPlan& p) {
  if (p.splits <= 1) return 0;
  return (size_t)(p.splits * s.heads * s.rows_q * (s.d + 4) * 4);
}

mea::FwdProblem fwd_problem(const Shape& s, const void* q, const void* k, const void* v, void* o,
                            float* row_max, float* row_sum) {
  mea::FwdProblem p;
  p.heads = s.heads;
  p.rows_q = (int)s.rows_q;
  p.n_k = (int)s.n_k;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.m = row_max;
  p.l = row_sum;
  return p;
}

hipError_t run_fwd(const Shape& s, const mea::FwdProblem& p, hipStream_t stream) {
  return s.bf16 ? mea::launch_fwd_bf16(s.d, p, stream) : mea::launch_fwd_f32(s.d, p, stream);
}

mea_status_t fwd_impl(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q,
                      int64_t n_k, int64_t d, const void* q, const void* k, const void* v,
                      void* o, float* row_max, float* row_sum, void* stream) {
  Shape s;
  mea_status_t st = check_fwd_shape(dt, B, H, H_kv, n_q, n_k, d, &s);
  if (st != MEA_OK || s.empty) return st;
  if ((row_max == nullptr) != (row_sum == nullptr)) return MEA_ERR_NULL;
  st = check_ptrs({q, k, v, o});
  if (st != MEA_OK) return st;
  if (row_max != nullptr && (!aligned16(row_max) || !aligned16(row_sum))) return MEA_ERR_ALIGN;
  st = check_alias({span(o, q_bytes(s)), span(row_max, stat_bytes(s)), span(row_sum, stat_bytes(s))},
                   {span(q, q_bytes(s)), span(k, kv_bytes(s)), span(v, kv_bytes(s))});
  if (st != MEA_OK) return st;
  hipError_t e = run_fwd(s, fwd_problem(s, q, k, v, o, row_max, row_sum),
                         reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MEA_OK : MEA_ERR_LAUNCH;
}

// Device address of `scratch` on the current device: looked up with
// hipGetSymbolAddress on the first call made with that device current, then
// cached (each GPU holds its own copy of the array at its own address).
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// With use_scratch the caller's workspace arguments are ignored: the call runs
// in the library's scratch array of MEA_NOALLOC_SCRATCH_BYTES (row terms, and the
// split layout of a small grid whenever it fits), after the same validation.
mea_status_t bwd_impl(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q,
                      int64_t n_k, int64_t d, const void* q, const void* k, const void* v,
                      const void* o, const void* dO, const float* row_max, const float* row_sum,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream, bool use_scratch = false) {
  Shape s;
  mea_status_t st = check_shape(dt, B, H, H_kv, n_q, n_k, d, &s);
  if (st != MEA_OK || s.empty) return st;
  if (n_k == 0) return MEA_ERR_SHAPE;  // query rows without keys have no forward
  // without query rows only the key side is touched (dk = dv = 0)
  st = s.rows_q > 0 ? check_ptrs({q, k, v, o, dO, row_max, row_sum, dq, dk, dv})
                    : check_ptrs({k, v, dk, dv});
  if (st != MEA_OK) return st;
  // The row terms are the minimum workspace. The split layout of a small grid
  // needs the larger size that the workspace query reports; a workspace that
  // holds only the row terms runs the unsplit backward.
  const BwdLayout lay = bwd_layout(s);
  const size_t min_need = bwd_row_bytes(s.bf16) * (size_t)s.q_rows_total;
  if (use_scratch) {
    // the scratch array is the workspace; it cannot overlap caller buffers
    if (min_need > (size_t)MEA_NOALLOC_SCRATCH_BYTES) return MEA_ERR_WORKSPACE;
    workspace = nullptr;
    workspace_bytes = MEA_NOALLOC_SCRATCH_BYTES;
  } else if (min_need > 0) {
    if (workspace == nullptr || workspace_bytes < min_need) return MEA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MEA_ERR_ALIGN;
  }
  const bool split = lay.total > min_need && workspace_bytes >= lay.total;
  const size_t need = split ? lay.total : min_need;  // bytes this call writes
  {
    const int64_t qb = q_bytes(s), kb = kv_bytes(s), sb = stat_bytes(s);
    st = check_alias({span(dq, qb), span(dk, kb), span(dv, kb), span(workspace, (int64_t)need)},
                     {span(q, qb), span(k, kb), span(v, kb), span(o, qb), span(dO, qb),
                      span(row_max, sb), span(row_sum, sb)});
    if (st != MEA_OK) return st;
  }
  if (use_scratch && noalloc_scratch(&workspace) != hipSuccess) return MEA_ERR_LAUNCH;
  mea::BwdProblem p;
  p.heads = s.heads;
  p.rows_q = (int)s.rows_q;
  p.n_k = (int)s.n_k;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dO = dO;
  p.m = row_max;
  p.l = row_sum;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.ws = static_cast<float*>(workspace);
  if (split) {
    p.split = lay.split;
    char* base = static_cast<char*>(workspace);
    if (lay.kv_part > 0) {
      p.part_dk = reinterpret_cast<float*>(base + lay.part_off);
      p.part_dv = reinterpret_cast<float*>(base + lay.part_off + lay.kv_part);
    }
    if (lay.q_part > 0) p.part_dq = reinterpret_cast<float*>(base + lay.part_off + 2 * lay.kv_part);
  }
  hipStream_t st_h = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = s.bf16 ? mea::launch_bwd_bf16(s.d, p, st_h) : mea::launch_bwd_f32(s.d, p, st_h);
  return e == hipSuccess ? MEA_OK : MEA_ERR_LAUNCH;
}

size_t bwd_ws_bytes(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q, int64_t n_k,
                    int64_t d) {
  Shape s;
  if (check_shape(dt, B, H, H_kv, n_q, n_k, d, &s) != MEA_OK || s.empty) return 0;
  return bwd_layout(s).total;
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
    case MEA_ERR_ALIAS: return "MEA_ERR_ALIAS";
  }
  return "MEA_UNKNOWN_STATUS";
}

int mea_version(void) { return kVersion; }

mea_status_t attn_fwd(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d,
                      const void* q, const void* k, const void* v, void* o,
                      float* row_max, float* row_sum, void* stream) {
  return fwd_impl(dt, B, H, H, n, n, d, q, k, v, o, row_max, row_sum, stream);
}

mea_status_t attn_fwd_ex(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q,
                         int64_t n_k, int64_t d, const void* q, const void* k, const void* v,
                         void* o, float* row_max, float* row_sum, void* stream) {
  return fwd_impl(dt, B, H, H_kv, n_q, n_k, d, q, k, v, o, row_max, row_sum, stream);
}

size_t attn_bwd_workspace_bytes(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d) {
  return bwd_ws_bytes(dt, B, H, H, n, n, d);
}

size_t attn_bwd_ex_workspace_bytes(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv,
                                   int64_t n_q, int64_t n_k, int64_t d) {
  return bwd_ws_bytes(dt, B, H, H_kv, n_q, n_k, d);
}

mea_status_t attn_bwd(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d,
                      const void* q, const void* k, const void* v, const void* o,
                      const void* dO, const float* row_max, const float* row_sum,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return bwd_impl(dt, B, H, H, n, n, d, q, k, v, o, dO, row_max, row_sum, dq, dk, dv, workspace,
                  workspace_bytes, stream);
}

mea_status_t attn_bwd_ex(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q,
                         int64_t n_k, int64_t d, const void* q, const void* k, const void* v,
                         const void* o, const void* dO, const float* row_max,
                         const float* row_sum, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return bwd_impl(dt, B, H, H_kv, n_q, n_k, d, q, k, v, o, dO, row_max, row_sum, dq, dk, dv,
                  workspace, workspace_bytes, stream);
}

mea_status_t attn_bwd_noalloc(mea_dtype_t dt, int64_t B, int64_t H, int64_t n, int64_t d,
                              const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* row_max, const float* row_sum,
                              void* dq, void* dk, void* dv, void* stream) {
  return bwd_impl(dt, B, H, H, n, n, d, q, k, v, o, dO, row_max, row_sum, dq, dk, dv, nullptr, 0,
                  stream, /*use_scratch=*/true);
}

int64_t attn_fwd_splitkv_num_splits(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv,
                                    int64_t n_q, int64_t n_k, int64_t d, int64_t num_splits) {
  Shape s;
  if (num_splits < 0 || check_fwd_shape(dt, B, H, H_kv, n_q, n_k, d, &s) != MEA_OK) return 0;
  if (s.empty) return 1;
  return plan_splits(s, num_splits).splits;
}

size_t attn_fwd_splitkv_workspace_bytes(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv,
                                        int64_t n_q, int64_t n_k, int64_t d, int64_t num_splits) {
  Shape s;
  if (num_splits < 0 || check_fwd_shape(dt, B, H, H_kv, n_q, n_k, d, &s) != MEA_OK || s.empty)
    return 0;
  return split_workspace_bytes(s, plan_splits(s, num_splits));
}

mea_status_t attn_fwd_splitkv(mea_dtype_t dt, int64_t B, int64_t H, int64_t H_kv, int64_t n_q,
                              int64_t n_k, int64_t d, const void* q, const void* k, const void* v,
                              void* o, float* row_max, float* row_sum, int64_t num_splits,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  mea_status_t st = check_fwd_shape(dt, B, H, H_kv, n_q, n_k, d, &s);
  if (st != MEA_OK) return st;
  if (num_splits < 0) return MEA_ERR_SHAPE;
  if (s.empty) return MEA_OK;
  if ((row_max == nullptr) != (row_sum == nullptr)) return MEA_ERR_NULL;
  st = check_ptrs({q, k, v, o});
  if (st != MEA_OK) return st;
  if (row_max != nullptr && (!aligned16(row_max) || !aligned16(row_sum))) return MEA_ERR_ALIGN;
  const SplitPlan plan = plan_splits(s, num_splits);
  if (s.heads * plan.splits * cdiv(s.rows_q, mea::fwd_geometry(s.bf16, s.d, s.heads, s.rows_q).query_rows) >
      kMaxBlocks)
    return MEA_ERR_SHAPE;
  const size_t need = split_workspace_bytes(s, plan);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return MEA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MEA_ERR_ALIGN;
  }
  st = check_alias({span(o, q_bytes(s)), span(row_max, stat_bytes(s)), span(row_sum, stat_bytes(s)),
                    span(workspace, (int64_t)need)},
                   {span(q, q_bytes(s)), span(k, kv_bytes(s)), span(v, kv_bytes(s))});
  if (st != MEA_OK) return st;
  hipStream_t stream_h = reinterpret_cast<hipStream_t>(stream);
  mea::FwdProblem p = fwd_problem(s, q, k, v, o, row_max, row_sum);
  if (plan.splits > 1) {
    p.splits = (int)plan.splits;
    p.split_len = (int)plan.split_len;
    p.part = static_cast<float*>(workspace);
  }
  hipError_t e = run_fwd(s, p, stream_h);
  if (e == hipSuccess && plan.splits > 1) e = mea::launch_merge(s.bf16, s.d, p, stream_h);
  return e == hipSuccess ? MEA_OK : MEA_ERR_LAUNCH;
}

}  // extern "C"
