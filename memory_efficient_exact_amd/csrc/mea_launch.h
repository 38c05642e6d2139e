// Internal launcher declarations shared by the C-ABI layer and the kernel
// translation units. Shapes arrive already validated; every launcher enqueues
// on `stream` and returns the hipGetLastError() code of its launches.
//
// Heads as the kernels see them. Query heads that share one key/value head
// (grouped-query attention) are adjacent in a [B, H, n_q, d] tensor, so the
// G = H / H_kv query heads of a group form one contiguous block of G * n_q
// rows. The kernels therefore work on `heads` = B * H_kv independent
// problems, each with `rows_q` = G * n_q query rows against `n_k` keys; row r
// of problem h is query row r % n_q of query head h * G + r / n_q. With
// H_kv = H this is plain multi-head attention.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mea {

struct FwdProblem {
  int64_t heads = 0;  // B * H_kv
  int rows_q = 0;     // G * n_q query rows per head
  int n_k = 0;        // keys per head
  const void* q = nullptr;  // [heads, rows_q, d]
  const void* k = nullptr;  // [heads, n_k, d]
  const void* v = nullptr;  // [heads, n_k, d]
  void* o = nullptr;        // [heads, rows_q, d]; written by the final pass
  float* m = nullptr;       // [heads, rows_q] row max (natural units) or null
  float* l = nullptr;       // [heads, rows_q] row sum or null (null iff m is)
  // Split-key mode (splits > 1): key range s = [s * split_len, min(n_k, (s+1) * split_len))
  // of every head is reduced by its own workgroups into `part`, then a merge
  // pass writes o, m, l. Layout of part (fp32): partial outputs
  // [splits][heads * rows_q][d], then one 16-byte record per (split, row).
  int splits = 1;
  int split_len = 0;
  float* part = nullptr;
};

// Tile geometry of the forward kernels, for planning the key splits.
struct FwdGeometry {
  int query_rows;  // query rows per workgroup
  int key_tile;    // keys per LDS tile (split lengths are multiples of it)
  int resident;    // workgroups that fit on one compute unit at once
};
// (both forwards pick a decoding layout for heads with few query rows and for
// grids too small to occupy half of the chip; the bf16 forward also picks
// wider workgroups on grids that fill the chip)
FwdGeometry fwd_geometry_bf16(int d, int64_t heads, int64_t rows_q);
FwdGeometry fwd_geometry_f32(int d, int64_t heads, int64_t rows_q);
inline FwdGeometry fwd_geometry(bool bf16, int d, int64_t heads, int64_t rows_q) {
  return bf16 ? fwd_geometry_bf16(d, heads, rows_q) : fwd_geometry_f32(d, heads, rows_q);
}

// Forward pass (final or, with p.splits > 1, partial) for bf16 / fp32 inputs.
hipError_t launch_fwd_bf16(int d, const FwdProblem& p, hipStream_t stream);
hipError_t launch_fwd_f32(int d, const FwdProblem& p, hipStream_t stream);
// Merge of the split partials in p.part into p.o, p.m, p.l.
hipError_t launch_merge(bool bf16, int d, const FwdProblem& p, hipStream_t stream);

// Grid of the per-row kernels (backward row terms, split merge): one pass of
// rows_per_block rows per workgroup, capped at kRowBlocks workgroups (2^21
// threads of 256, enough to keep HBM busy); the kernels stride over the
// remaining rows, so every grid stays far below the 2^32 work-item limit of
// a dispatch whatever the row count.
constexpr int64_t kRowBlocks = int64_t(1) << 13;
inline unsigned row_blocks(int64_t rows, int64_t rows_per_block) {
  const int64_t b = (rows + rows_per_block - 1) / rows_per_block;
  return (unsigned)(b < kRowBlocks ? b : kRowBlocks);
}

// Split backward, for grids too small to fill the chip: the dK/dV workgroups
// of a head are repeated for `kv` ranges of `len_q` staged query tiles each,
// the dQ workgroups for `q` ranges of `len_k` key tiles. Where a side has more
// than one range, each range writes fp32 partial sums (dK and dQ before their
// 1/sqrt(d) factor) to the workspace, and a reduce pass sums them into the
// outputs.
// Unsplit: kv = q = 1 and the lengths cover every tile.
struct BwdSplit {
  int kv = 1;
  int len_q = 0;
  int q = 1;
  int len_k = 0;
};

// Rows per 4-wave workgroup (keys of a dK/dV or queries of a dQ workgroup) and
// rows per staged tile of the backward kernels, for planning the split.
struct BwdGeometry {
  int wg_rows;
  int tile_rows;
};
BwdGeometry bwd_geometry_bf16(int d);
BwdGeometry bwd_geometry_f32(int d);

struct BwdProblem {
  int64_t heads = 0;  // B * H_kv
  int rows_q = 0;     // G * n_q
  int n_k = 0;
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const void* o = nullptr;
  const void* dO = nullptr;
  const float* m = nullptr;
  const float* l = nullptr;
  void* dq = nullptr;
  void* dk = nullptr;  // [heads, n_k, d]: sums over the query heads of each group
  void* dv = nullptr;
  float* ws = nullptr;  // row terms: 8 (bf16) or 16 (fp32) bytes per query row
  BwdSplit split;
  // with split.kv > 1: [kv][heads * n_k][d] fp32 partials of dK and of dV;
  // with split.q > 1: [q][heads * rows_q][d] fp32 partials of dQ (else null);
  // the fp32 backward's D pass first keeps its per-range sums there
  float* part_dk = nullptr;
  float* part_dv = nullptr;
  float* part_dq = nullptr;
};

// Backward: row preprocess, then one grid with dK/dV and dQ workgroups (and,
// when split, the reduce pass). bf16: ws holds 2 floats per query row; fp32:
// 16 bytes per query row.
hipError_t launch_bwd_bf16(int d, const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_f32(int d, const BwdProblem& p, hipStream_t stream);
// Sums the split partials of p into dK, dV (scaled by 1/sqrt(d)) and dQ (scaled),
// in the output type; does nothing for a side that is not split.
hipError_t launch_bwd_reduce(bool bf16, int d, const BwdProblem& p, hipStream_t stream);

}  // namespace mea
