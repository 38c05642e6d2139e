// Forward attention for bf16 inputs on gfx950: one workgroup per tile of
// query rows, a sweep over key/value tiles with a running maximum and running
// sum per query row, normalisation once at the end.
//
// Method: "Self-attention Does Not Need O(n^2) Memory" (abstract; method
// sections of both digests): postpone the softmax division to the end, keep
// a weighted value sum and a weight sum per query, track the maximum score
// for stability, and visit keys/values in chunks. The per-block update is the
// two-block merge of "当注意力成为瓶颈…", section IO感知, applied once per
// 32-key block.
//
// Layout of the work (per workgroup of W = 8 waves, one per CU, or W = 4 waves,
// two per CU, on grids too small to give every CU an 8-wave workgroup):
//  * each wave owns QB blocks of 32 query rows; the workgroup owns W*QB*32;
//  * K and V tiles of BC keys are copied straight from HBM into LDS
//    (global_load_lds, no register staging), double-buffered, in a swizzled
//    row-major layout free of bank conflicts (see Swizzled in mea_device.h);
//  * scores are formed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA, so
//    that each lane holds one query's scores for 16 keys per 32-key block:
//    the row maximum is a register reduction plus one v_permlane32_swap, and
//    every per-row factor is a per-lane scalar;
//  * the output is accumulated transposed, O^T += V^T P^T: P^T comes straight
//    from the S^T accumulators (rounded to bf16), V^T from transposed LDS
//    reads (ds_read_b64_tr_b16) of the row-major V tile;
//  * exponentials are base 2 with log2(e)/sqrt(d) folded into one FMA.
//
// Reference maximum. Weights are formed as p = exp2(x*C - R) with a per-row
// reference R that is refreshed to fl(m*C) (m = running max of the raw
// scores x = q.k) only when some row's maximum has grown past R + 8, at
// which point acc and l are multiplied by exp2(R_old - R_new). So p <= 2^8
// (no overflow, same bf16 relative precision), the output acc/l is exact as
// before, and the O(d) rescale of the accumulators is skipped for almost every
// block. The true running max m is tracked separately; the statistics are
// reported for it: l = sum_j exp(s_j - m) = l_R * exp2(R - m*C).
//
// The common path of a block is cheap: each lane folds its 16 scores per
// query block into its own running maximum and compares that with a
// precomputed raw-score threshold (R + 8) / C; one wave-wide test covers all
// query blocks. Only when it fires are the two lanes of a row combined
// (v_permlane32_swap) to rebase on the row maximum; the exact row maximum for
// the statistics is formed once, after the sweep. In the row-tiled layouts the
// weights are formed before that test, against the current reference, and
// formed again after a rebase (see kSpeculate below).
//
// Decoding mode (few query rows per head, e.g. one new token per query head of
// a group): the four waves share one 32-row query block and take different
// 32-key blocks of every 128-key tile, so no MFMA or VALU work is spent on
// padding query rows. After the sweep the waves' partial results (maximum,
// reference, sum, accumulator) are merged through LDS with the same re-basing
// rule, and each wave writes a quarter of the output columns.
//
// Key ranges. A workgroup may cover only the keys [key0, key0 + split_len) of its
// head (split-key mode, for grids too small to fill the chip). It then writes
// the summary of that range instead of the output: the normalised fp32 row
// acc / l_R, the exact raw maximum m, the reference R and l_R. The merge pass
// (merge.hip) combines the ranges of a row with the two-block merge of
// "当注意力成为瓶颈…", section IO感知.
#include <type_traits>

#include "mea_device.h"
#include "mea_launch.h"

namespace mea {
namespace {

#if MEA_SYNC_TIMERS
// the SyncTimer counters (mea_device.h) of the row-tiled layout and of the
// decoding layout
__device__ unsigned long long g_sync[2][kSyncCounters];
#define MEA_SYNC_COUNTERS(layout) (g_sync[layout])
#else
#define MEA_SYNC_COUNTERS(layout) nullptr
#endif

constexpr int kWaves = 4;       // waves per workgroup: decoding and small grids
constexpr int kWideWaves = 8;   // waves per workgroup when the grid fills the chip
constexpr float kRefSlack = 8.0f;  // log2 units a row max may exceed its reference

struct FwdArgs {
  const bf16* Q;  // [heads, n_q, D]
  const bf16* K;  // [heads, n_k, D]
  const bf16* V;
  bf16* O;        // final mode: [heads, n_q, D]
  float* Mx;      // final mode: [heads, n_q] or null
  float* Ls;
  float* Po;      // split mode: [splits, rows, D] normalised partial rows (else null)
  float* Ps;      // split mode: [splits, rows] records {m, R, l_R, 0}
  int64_t rows;   // heads * n_q
  int n_q;
  int n_k;
  int qtiles;     // query tiles per head
  int splits;     // key ranges per head
  int split_len;  // keys per range (n_k when splits == 1)
  int total;      // workgroups
  float C;        // log2(e) / sqrt(D)
  float scale;    // 1 / sqrt(D)
};

// W waves per workgroup, two waves per SIMD: W = 8 (one workgroup per CU) or
// W = 4 (two per CU); decoding at d = 128 runs one wave per SIMD, its 128-key
// tiles (128 KiB of LDS double-buffered) leaving room for one workgroup
template <int D, int QB, int BC, bool kDecode, int W>
__global__ __launch_bounds__(64 * W, (kDecode && D == 128) ? 1 : 2) void fwd_bf16_kernel(const FwdArgs a) {
  static_assert(!kDecode || (QB == 1 && BC == 32 * W), "decoding: one 32-key block per wave");
  constexpr int kBQ = kDecode ? 32 : W * QB * 32;  // query rows per workgroup
  constexpr int DK = D / 16;             // k-steps of the score MFMA
  constexpr int DB = D / 32;             // 32-wide output column blocks
  constexpr int SB = BC / 32;            // 32-key blocks per LDS tile
  using L = Swizzled<D>;
  constexpr int SPR = L::kChunks;         // 16-byte chunks per LDS row
  constexpr int kTile = BC * D;           // elements per K or V tile in LDS
  constexpr int NBLK = BC * SPR / 64;     // 1 KiB DMA blocks per tile
  constexpr int BPW = (NBLK + W - 1) / W;
  static_assert(NBLK * 64 == BC * SPR, "tile must be whole DMA blocks");

  // two named buffers per operand (not one array indexed by a loop
  // variable), so the compiler can see that reads of the current tile never
  // alias the DMA into the other one and does not wait for that DMA
  __shared__ __attribute__((aligned(1024))) bf16 sK0[kTile];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[kTile];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[kTile];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // uniform across the wave: the copies' LDS addresses then sit in scalar registers
  // (7% faster on 4-wave grids, 3.7% in the d = 64 decoding layout; the d = 128
  // decoding layout, at one wave per SIMD, ran 2% slower with it)
  const int wave = (kDecode && D == 128) ? tid >> 6 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // workgroup -> (head, key range, query tile); the query tiles of one key
  // range are adjacent, so they share an XCD and its L2 copy of K and V
  const int tile = xcd_remap(blockIdx.x, a.total);
  const int hs = tile / a.qtiles;
  const int qt = tile - hs * a.qtiles;
  const int bh = hs / a.splits;
  const int sp = hs - bh * a.splits;
  const int key0 = sp * a.split_len;            // first key of this range
  const int n = min(a.n_k - key0, a.split_len);  // keys of this range
  const int n_q = a.n_q;
  const float C = a.C;
  const bf16* Qh = a.Q + (int64_t)bh * n_q * D;
  const bf16* Kh = a.K + ((int64_t)bh * a.n_k + key0) * D;
  const bf16* Vh = a.V + ((int64_t)bh * a.n_k + key0) * D;
  const int q0 = kDecode ? qt * kBQ : qt * kBQ + wave * QB * 32;

  // Q fragments: B operand of S^T = K Q^T (lane: query l32, 8 columns at 16*dk + 8*hi)
  bf16x8 qf[QB][DK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q0 + qb * 32 + l32;
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      qf[qb][dk] = row < n_q ? *reinterpret_cast<const bf16x8*>(Qh + (int64_t)row * D + dk * 16 + 8 * hi)
                             : bf16x8{};
    }
  }

  float m_lane[QB];  // running max of the raw scores q.k this lane holds (exact);
                     // the row maximum is the max over the lane pair (l, l ^ 32)
  float ref[QB];     // reference R (see header), the same in both lanes of a row
  float thr[QB];     // raw-score threshold (R + slack) / C: a lane maximum above it
                     // calls for a new reference
  float l_run[QB];   // this lane's share of sum_j exp2(x_j*C - R)
  f32x16 acc[QB][DB];
  const float invC = 1.0f / C;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_lane[qb] = -INFINITY;
    ref[qb] = -INFINITY;
    thr[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
  }

  // DMA of the K and V tile starting at key j0. Block b of a tile covers
  // 16-byte LDS slots 64b..64b+63; slot s holds row s / SPR at chunk
  // position s % SPR, i.e. the row's chunk (s % SPR) ^ swz(row). Rows past n
  // repeat row n-1 (their scores are masked to -inf, and their weights are
  // exactly 0).
  int dma_row[BPW], dma_col[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int slot = (wave + W * i) * 64 + lane;
    const int r = slot / SPR;
    const int pc = slot - r * SPR;
    dma_row[i] = r;
    dma_col[i] = (pc ^ L::swz(r)) * 8;
  }
  auto issue = [&](bf16* kdst, bf16* vdst, int j0) {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = wave + W * i;
      if (b < NBLK) {
        const int src = min(j0 + dma_row[i], n - 1);
        const int64_t off = (int64_t)src * D + dma_col[i];
        dma16(Kh + off, kdst + b * 512);
        dma16(Vh + off, vdst + b * 512);
      }
    }
  };

  // per-lane LDS offsets: K rows for the score MFMA (row l32, columns
  // 16*dk + 8*hi), and the transposed-read pattern for V^T fragments (rows
  // 4*hi + jj/4 and 8 below it, columns 32*db + 16*(g%2) + 4*(jj%4)). Blocks
  // of 16 rows further down add 16*D, which leaves the swizzle unchanged.
  const int g = lane >> 4;
  const int jj = lane & 15;
  int k_off[DK], v_off[DB][2];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) k_off[dk] = L::off(l32, dk * 16 + 8 * hi);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      v_off[db][h] = L::off(4 * hi + (jj >> 2) + 8 * h, db * 32 + (g & 1) * 16 + 4 * (jj & 3));

  // The softmax of a block (masking, maxima, rescale, exponentials) runs at raised
  // issue priority in the d = 64 row-tiled layouts: the wave that enters it wins
  // VALU issue over the other wave of its SIMD, whose MFMAs keep the matrix pipe
  // busy meanwhile. With identical results, 4% faster at 1 x 16 x 16384 x 64 and
  // 2 x 8 x 8192 x 64 (8-wave workgroups) and 3.6-5.5% on 4-wave grids of two
  // workgroups per CU (1 x 24 x 4096 x 64); neutral at d = 128 and 2-3% slower in the
  // decoding layout, which keep the default priority. (Raising the MFMA phases
  // instead changed nothing.)
  constexpr bool kSoftmaxPrio = D == 64 && !kDecode;

  // Scores of one 32-key block, S^T = K Q^T; keys beyond n get no weight.
  auto scores = [&](f32x16 (&s)[QB], const bf16* ks, int sb, int j0, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      const bf16x8 a = lds_read_b128(ks + sb * 32 * D + k_off[dk]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb] = mfma32x32x16(a, qf[qb][dk], s[qb]);
    }
    if constexpr (kMasked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + sb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (key >= n) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][r] = -INFINITY;
        }
      }
    }
  };
  // Weights of a block against the current references: P^T fragments (chunk c
  // holds keys 16c..16c+15 of the block, element e is register 8c + e) and
  // this lane's share of their sum.
  auto weights = [&](const f32x16 (&s)[QB], bf16x8 (&pf)[QB][2], float (&ls)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float R = ref[qb];
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[qb][r], C, -R));
        sum += p;
        pf[qb][r >> 3][r & 7] = (bf16)p;
      }
      ls[qb] = sum;
    }
  };

  // Weights formed before the test of the maxima (row-tiled layouts). The
  // weights of a block are formed against the current references while the
  // lane maxima are folded in: the two are independent, so the exponentials
  // no longer wait for the maxima and the wave-wide test. They are final
  // unless some row's maximum passed its threshold, which after a row's first
  // block is rare; then the references move, acc and l are rescaled, and the
  // block's scores are formed again (the same MFMAs give the same values) for
  // weights against the new references. Results are identical to testing
  // first; 1.6-2.8% faster at d = 64 (1 x 16 x 16384, 2 x 8 x 8192, 4 x 8 x 4096)
  // and 1% at 1 x 16 x 8192 x 128. The decoding layout tests first.
  constexpr bool kSpeculate = !kDecode;

  // One 32-key block: scores, online softmax, P V.
  auto block = [&](const bf16* ks, const bf16* vs, int sb, int j0, auto masked_tag) {
    f32x16 s[QB];
    scores(s, ks, sb, j0, masked_tag);
    if constexpr (kSoftmaxPrio) __builtin_amdgcn_s_setprio(1);
    bf16x8 pf[QB][2];
    float ls[QB];
    // lane maxima; one wave-wide test covers all query blocks. With the weights
    // formed beside them, a max3 tree (maxima are exact: the order does not matter).
    bool moved = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const f32x16& x = s[qb];
      float mx = m_lane[qb];
      if constexpr (kSpeculate) {
        const float a0 = fmaxf(fmaxf(x[0], x[1]), x[2]);
        const float a1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
        const float a2 = fmaxf(fmaxf(x[6], x[7]), x[8]);
        const float a3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
        const float a4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
        const float b0 = fmaxf(fmaxf(a0, a1), a2);
        const float b1 = fmaxf(fmaxf(a3, a4), x[15]);
        mx = fmaxf(fmaxf(b0, b1), mx);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[r]);
      }
      m_lane[qb] = mx;
      moved |= mx > thr[qb];
    }
    // new references at the row maxima; acc and l follow
    auto rebase = [&]() {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float target = pair_max32(m_lane[qb]) * C;  // row maximum, log2 units
        const float alpha = fast_exp2(ref[qb] - target);  // 0 on the first block
        ref[qb] = target;
        thr[qb] = (target + kRefSlack) * invC;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
      }
    };
    if constexpr (kSpeculate) {
      weights(s, pf, ls);
      // Pin the weights here: left alone, the compiler moves them below the
      // test into the path that keeps them, behind the maxima again.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        asm volatile("" : "+v"(ls[qb]));
#pragma unroll
        for (int c = 0; c < 2; ++c) asm volatile("" : "+v"(pf[qb][c]));
      }
      if (wave_any(moved)) {
        rebase();
        scores(s, ks, sb, j0, masked_tag);
        weights(s, pf, ls);
      }
    } else {
      if (wave_any(moved)) rebase();
      weights(s, pf, ls);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += ls[qb];
    if constexpr (kSoftmaxPrio) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16* vp = vs + (sb * 32 + c * 16) * D;
        const bf16x8 a = cat(lds_read_tr16(vp + v_off[db][0]), lds_read_tr16(vp + v_off[db][1]));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32x32x16(a, pf[qb][c], acc[qb][db]);
      }
    }
  };

  const int ntiles = (n + BC - 1) / BC;
  // one tile: prefetch the next tile into (kn, vn) while computing on (ks, vs);
  // kFull: all BC keys of the tile exist
  SyncTimer tim;
  auto step = [&](const bf16* ks, const bf16* vs, bf16* kn, bf16* vn, int t, auto full_tag) {
    constexpr bool kFull = decltype(full_tag)::value;
    const int j0 = t * BC;
    if (t + 1 < ntiles) issue(kn, vn, j0 + BC);
    if constexpr (kDecode) {  // this wave's 32-key block of the tile
      if (j0 + BC <= n) block(ks, vs, wave, j0, std::false_type{});
      else if (j0 + wave * 32 < n) block(ks, vs, wave, j0, std::true_type{});
    } else if constexpr (kFull) {
      // two 32-key blocks per loop pass: 1-3% faster than one (d = 128: 3%) with
      // identical results
#pragma unroll 2
      for (int sb = 0; sb < SB; ++sb) block(ks, vs, sb, j0, std::false_type{});
    } else {  // ragged last tile
      for (int sb = 0; sb < SB; ++sb) {
        if (j0 + sb * 32 >= n) break;
        block(ks, vs, sb, j0, std::true_type{});
      }
    }
    tim.end_of_tile();
  };
  issue(sK0, sV0, 0);
  wait_all();
  __syncthreads();
  tim.start(wave, W);
  if constexpr (kDecode) {
    for (int t = 0; t < ntiles; t += 2) {
      step(sK0, sV0, sK1, sV1, t, std::true_type{});
      if (t + 1 < ntiles) step(sK1, sV1, sK0, sV0, t + 1, std::true_type{});
    }
  } else {
    // Full tiles in pairs, then at most one more full tile and the ragged one.
    // With the ragged tile outside the loop, the loop body has one path and its
    // running state is not copied between register sets at every tile (80 moves
    // per tile at d = 64): identical results, up to 1% faster at d = 64 and 6-8% at
    // d = 128 (1 x 16 x 8192 x 128).
    const int nfull = n / BC;
    int t = 0;
    for (; t + 1 < nfull; t += 2) {
      step(sK0, sV0, sK1, sV1, t, std::true_type{});
      step(sK1, sV1, sK0, sV0, t + 1, std::true_type{});
    }
    if (t < nfull) {
      step(sK0, sV0, sK1, sV1, t, std::true_type{});
      ++t;
    }
    if (t < ntiles) {  // the ragged tile, in the buffers its parity selects
      if (t & 1) step(sK1, sV1, sK0, sV0, t, std::false_type{});
      else step(sK0, sV0, sK1, sV1, t, std::false_type{});
    }
  }
  tim.flush(MEA_SYNC_COUNTERS(kDecode ? 1 : 0), lane);

  if constexpr (kDecode) {
    // Merge the four waves' partial results (same 32 query rows, different
    // keys). The last step ended with a barrier and no DMA in flight, so the
    // tile buffers are free: wave w's re-based accumulator (32 rows x D fp32,
    // rows padded) goes to tile buffer w, the per-wave statistics to st.
    constexpr int AS = D + 4;
    __shared__ float st[3 * W * 32];  // [3][W][32]: R, row max, row sum
    auto slice = [&](int w) {
      return reinterpret_cast<float*>(w == 0 ? sK0 : w == 1 ? sK1 : w == 2 ? sV0 : sV1);
    };
    float* sacc = slice(wave);
    static_assert(32 * AS * 4 <= kTile * 2, "one accumulator slice per tile buffer");
    const float m_row = pair_max32(m_lane[0]);
    const float l_row = pair_sum32(l_run[0]);
    if (hi == 0) {
      st[wave * 32 + l32] = ref[0];
      st[W * 32 + wave * 32 + l32] = m_row;
      st[2 * W * 32 + wave * 32 + l32] = l_row;
    }
    __syncthreads();
    float M = -INFINITY, mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      M = fmaxf(M, st[w * 32 + l32]);
      mm = fmaxf(mm, st[W * 32 + w * 32 + l32]);
    }
    const float f = fast_exp2(ref[0] - M);  // 0 for a wave that saw no key
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 w4;
#pragma unroll
        for (int e = 0; e < 4; ++e) w4[e] = acc[0][db][4 * r4 + e] * f;
        *reinterpret_cast<f32x4*>(sacc + l32 * AS + db * 32 + 8 * r4 + 4 * hi) = w4;
      }
    __syncthreads();
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w)
      L += st[2 * W * 32 + w * 32 + l32] * fast_exp2(st[w * 32 + l32] - M);
    const float inv = 1.f / L;
    const int row = q0 + l32;
    if (row < n_q) {
      // this lane: row l32, columns col0 .. col0 + D/8 (wave's quarter, lane half hi)
      constexpr int CPL = D / 8;
      const int col0 = wave * (D / 4) + hi * CPL;
      const int64_t grow = (int64_t)bh * n_q + row;
      const int64_t prow = (int64_t)sp * a.rows + grow;
#pragma unroll
      for (int c = 0; c < CPL; c += 4) {
        f32x4 sum = f32x4{};
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float* sl = slice(w);
          sum += *reinterpret_cast<const f32x4*>(sl + l32 * AS + col0 + c);
        }
        if (a.Po == nullptr) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)(sum[e] * inv);
          *reinterpret_cast<bf16x4*>(a.O + grow * D + col0 + c) = o;
        } else {
          *reinterpret_cast<f32x4*>(a.Po + prow * D + col0 + c) = sum * inv;
        }
      }
      if (wave == 0 && hi == 0) {
        if (a.Po == nullptr) {
          if (a.Mx != nullptr) {
            a.Mx[grow] = mm * a.scale;
            a.Ls[grow] = L * fast_exp2(-__builtin_fmaf(mm, C, -M));
          }
        } else {
          *reinterpret_cast<f32x4*>(a.Ps + prow * 4) = f32x4{mm, M, L, 0.f};
        }
      }
    }
    return;
  }

  // epilogue: O = acc / l, written once; statistics for the exact maximum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q0 + qb * 32 + l32;
    const float m_row = pair_max32(m_lane[qb]);
    const float l_tot = pair_sum32(l_run[qb]);
    const float inv = 1.f / l_tot;
    if (row >= n_q) continue;
    const int64_t grow = (int64_t)bh * n_q + row;
    if (a.Po == nullptr) {
      bf16* orow = a.O + grow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[qb][db][4 * r4 + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * r4 + 4 * hi) = w;
        }
      if (a.Mx != nullptr && hi == 0) {
        // l_tot sums exp2(x*C - R) = exp(s - m) * 2^(m*C - R); m*C - R is
        // formed exactly by one FMA
        const float shift = __builtin_fmaf(m_row, C, -ref[qb]);
        a.Mx[grow] = m_row * a.scale;
        a.Ls[grow] = l_tot * fast_exp2(-shift);
      }
    } else {
      // summary of this key range: acc / l_R in fp32 and {m, R, l_R}
      const int64_t prow = (int64_t)sp * a.rows + grow;
      float* orow = a.Po + prow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = acc[qb][db][4 * r4 + e] * inv;
          *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * r4 + 4 * hi) = w;
        }
      if (hi == 0) *reinterpret_cast<f32x4*>(a.Ps + prow * 4) = f32x4{m_row, ref[qb], l_tot, 0.f};
    }
  }
}

template <int D, int QB, int BC, bool kDecode, int W>
hipError_t launch(const FwdProblem& p, hipStream_t stream) {
  constexpr int kBQ = kDecode ? 32 : W * QB * 32;
  FwdArgs a;
  a.Q = static_cast<const bf16*>(p.q);
  a.K = static_cast<const bf16*>(p.k);
  a.V = static_cast<const bf16*>(p.v);
  a.O = static_cast<bf16*>(p.o);
  a.Mx = p.m;
  a.Ls = p.l;
  a.rows = p.heads * p.rows_q;
  a.n_q = p.rows_q;
  a.n_k = p.n_k;
  a.qtiles = (p.rows_q + kBQ - 1) / kBQ;
  a.splits = p.splits > 1 ? p.splits : 1;
  a.split_len = p.splits > 1 ? p.split_len : p.n_k;
  a.Po = p.splits > 1 ? p.part : nullptr;
  a.Ps = p.splits > 1 ? p.part + (int64_t)a.splits * a.rows * D : nullptr;
  const int64_t total = p.heads * a.splits * a.qtiles;
  a.total = (int)total;
  a.scale = 1.0f / sqrtf((float)D);
  a.C = kLog2e * a.scale;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BC, kDecode, W>), dim3((unsigned)total), dim3(64 * W), 0,
                     stream, a);
  return hipGetLastError();
}

// Each wave owns QB 32-row query blocks: d = 64 takes 64 rows per wave and
// 128-key tiles, d = 128 32 rows and 64-key tiles. A workgroup has 8 waves (one
// per CU; each K/V tile staged in LDS then serves twice the query rows, which
// measured 4-7% faster) whenever the grid of such workgroups covers every
// compute unit, else 4 waves (two per CU: twice the workgroups on small grids).
// The decoding mode (32 rows, 128-key tiles, keys split across the waves)
// serves heads with at most kDecodeRows query rows, and every grid whose
// 4-wave workgroups would occupy at most half of the compute units: there it
// launches eight times the workgroups, each wave sweeping a quarter of the
// keys (measured 1.2-3.5x faster at 16-128 workgroups; from about 200 on the
// row-tiled layout is as fast or faster).
constexpr int kQB64 = 2, kBC64 = 128, kQB128 = 1, kBC128 = 64;
constexpr int kDecodeRows = 64;
constexpr int64_t kComputeUnits = 256;

bool decode_grid(int d, int64_t heads, int64_t rows_q) {
  if (rows_q <= kDecodeRows) return true;
  const int64_t rows = kWaves * (d == 64 ? kQB64 : kQB128) * 32;
  return 2 * heads * ((rows_q + rows - 1) / rows) <= kComputeUnits;
}

bool wide_grid(int d, int64_t heads, int64_t rows_q) {
  const int64_t rows = kWideWaves * (d == 64 ? kQB64 : kQB128) * 32;
  return heads * ((rows_q + rows - 1) / rows) >= kComputeUnits;
}

}  // namespace

FwdGeometry fwd_geometry_bf16(int d, int64_t heads, int64_t rows_q) {
  if (decode_grid(d, heads, rows_q)) return FwdGeometry{32, 32 * kWaves, d == 64 ? 2 : 1};
  const bool wide = wide_grid(d, heads, rows_q);
  const int w = wide ? kWideWaves : kWaves;
  return d == 64 ? FwdGeometry{w * kQB64 * 32, kBC64, wide ? 1 : 2}
                 : FwdGeometry{w * kQB128 * 32, kBC128, wide ? 1 : 2};
}

hipError_t launch_fwd_bf16(int d, const FwdProblem& p, hipStream_t stream) {
  if (decode_grid(d, p.heads, p.rows_q)) {
    if (d == 64) return launch<64, 1, 32 * kWaves, true, kWaves>(p, stream);
    return launch<128, 1, 32 * kWaves, true, kWaves>(p, stream);
  }
  if (wide_grid(d, p.heads, p.rows_q)) {
    if (d == 64) return launch<64, kQB64, kBC64, false, kWideWaves>(p, stream);
    return launch<128, kQB128, kBC128, false, kWideWaves>(p, stream);
  }
  if (d == 64) return launch<64, kQB64, kBC64, false, kWaves>(p, stream);
  return launch<128, kQB128, kBC128, false, kWaves>(p, stream);
}

}  // namespace mea

#if MEA_SYNC_TIMERS
// Timing library only: copies the forward's 2 x 7 synchronisation counters to
// `out` (host memory) after a device synchronisation, and clears them if
// `reset`. Returns 0 or the failing hipError_t.
extern "C" __attribute__((visibility("default"))) int mea_sync_timers_fwd(unsigned long long* out,
                                                                        int reset) {
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpyFromSymbol(out, HIP_SYMBOL(mea::g_sync), sizeof(mea::g_sync));
  if (e == hipSuccess && reset) {
    const unsigned long long zero[2][mea::kSyncCounters] = {};
    e = hipMemcpyToSymbol(HIP_SYMBOL(mea::g_sync), zero, sizeof(zero));
    if (e == hipSuccess) e = hipDeviceSynchronize();
  }
  return (int)e;
}
#endif
