// Device-side building blocks for the gfx950 attention kernels: vector types,
// MFMA wrappers with their lane layouts, the padded and swizzled LDS tile layouts,
// transposed LDS reads, direct global-to-LDS copies and wave-level helpers.
// Host code never includes this file.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mea {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MEA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_32x32x16_bf16, D[32x32] += A[32x16] B[16x32], wave64.
//   A: lane l holds A[i = l%32][k = 8*(l/32) + e], e = 0..7
//   B: lane l holds B[k = 8*(l/32) + e][j = l%32]
//   D: lane l, register r holds D[i = 8*(r/4) + 4*(l/32) + r%4][j = l%32]
// (layouts checked on gfx950 hardware with exact small-integer products).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f64_16x16x4_f64, D[16x16] += A[16x4] B[4x16].
//   A: lane l holds A[i = l%16][k = l/16];  B: lane l holds B[k = l/16][j = l%16]
//   D: lane l, register r holds D[i = 4*r + l/16][j = l%16]
__device__ __forceinline__ f64x4 mfma_f64_16x16x4(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x4_f32, D[16x16] += A[16x4] B[4x16].
//   A: lane l holds A[i = l%16][k = l/16];  B: lane l holds B[k = l/16][j = l%16]
//   D: lane l, register r holds D[i = 4*(l/16) + r][j = l%16]
__device__ __forceinline__ f32x4 mfma_f32_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- LDS tiles
// Padded row-major bf16 tile (used by the d = 64 backward): each row of D elements is
// followed by 16 bytes of padding, so row r starts at byte r*(2D + 16). For
// D = 64 (144-byte rows) consecutive rows start 36 banks apart: 16 rows read
// at the same 16-byte column cover all 64 banks once. A transposed read
// serves 32 lanes (4 rows x 64 bytes) per pass, and there rows r and r + 2
// overlap by 8 banks (a 2-way conflict; 4-way for D = 128). The backward was
// measured no faster with the conflict-free layout below, so it keeps this
// one, whose addresses are a per-lane base plus compile-time offsets.
template <int D>
struct Padded {
  static constexpr int kRowElems = D + 8;           // row stride in elements
  static constexpr int kSlotsPerRow = D / 8 + 1;    // 16-byte slots per row (last = pad)
  __device__ static constexpr int off(int row, int col) { return row * kRowElems + col; }
};

// Swizzled row-major bf16 tile (used by the forward and by the d = 128
// backward): rows of D elements with no
// padding; the 16-byte chunk c of row r sits at chunk position c ^ swz(r).
// With 64 banks of 4 bytes, a 16-byte read of one chunk column by 16 lanes
// (rows r..r+15) touches every bank once, and so does a transposed read by 32
// lanes (4 rows x 64 bytes), which on the padded layout above overlaps
// 2-way (D = 64) or 4-way (D = 128). swz permutes the chunks of a row, so
// row offsets that are multiples of 16 keep it unchanged:
//   D = 64  (two rows per 64 banks): swz(r) = bit-reverse of (r/2) mod 8
//   D = 128 (one row per 64 banks):  swz(r) = bit-reverse of r mod 16
template <int D>
struct Swizzled {
  static_assert(D == 64 || D == 128, "head dimension");
  static constexpr int kChunks = D / 8;  // 16-byte chunks per row
  __device__ static constexpr int swz(int r) {
    if constexpr (D == 64) {
      const int x = (r >> 1) & 7;
      return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
    } else {
      const int x = r & 15;
      return ((x & 1) << 3) | ((x & 2) << 1) | ((x & 4) >> 1) | ((x >> 3) & 1);
    }
  }
  // element offset of (row, col); the 4 or 8 elements read from col on stay in one chunk
  __device__ static constexpr int off(int row, int col) {
    return row * D + (((col >> 3) ^ swz(row)) << 3) + (col & 7);
  }
};

__device__ __forceinline__ bf16x8 lds_read_b128(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// ds_read_b64_tr_b16: each lane supplies the address of 4 consecutive b16
// values (8 bytes). Within every group of 16 lanes, output lane i, element e
// is element i%4 of the 8 bytes addressed by lane 4*e + i/4 of its group.
// If lane j of a group addresses row (base + j/4), columns c0 + 4*(j%4)..+3
// of a row-major tile, output lane i holds rows base..base+3 of column c0 + i.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MEA_LDS i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------- wave helpers
// value from lane l ^ 32 (through LDS permute; used off the hot path)
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// v_permlane32_swap exchanges the upper half of one operand with the lower
// half of the other; swapping x with itself leaves lane l holding the pair
// {x[l % 32], x[32 + l % 32]} across the two results, whichever way round.
// Max and sum of the pair are therefore identical (bitwise) in lanes l, l^32.
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// true in every lane when the predicate holds in any lane of the wave
__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

// Direct global->LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds_base + 16*l, where lds_base is uniform across
// the wave. Completion is tracked by the vector-memory counter.
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (MEA_LDS void*)(lds_base), 16, 0, 0);
}
// Direct global->LDS copy of 4 bytes per lane (global_load_lds_dword):
// lane l's 4 bytes land at lds_base + 4*l.
__device__ __forceinline__ void dma4(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (MEA_LDS void*)(lds_base), 4, 0, 0);
}

// The same two copies issued from inline assembly, out of sight of the
// compiler's wait-count insertion. While that pass tracks a global->LDS copy
// in flight it treats outstanding LDS reads as completing out of order, and
// before using any one of them it waits for all (lgkmcnt(0)); without the
// copy in view it waits only for the reads a use needs (lgkmcnt(n); LDS reads
// return in issue order). The caller must wait for these copies itself before
// the LDS they write is read or rewritten: wait_all() (vmcnt 0) and a barrier,
// which the d = 64 backward does at the end of every staged tile. Waits the
// compiler does place can only grow stricter, since the copies also count in
// vmcnt. M0 holds the wave-uniform LDS address (one wait state after writing
// it before the copy; the copy reads it at issue). M0 is a reserved register
// whose clobber the compiler need not honour, so the asm saves it and puts it
// back after the copy. The instruction writes no vector register, so nothing
// is left in flight for the compiler to reuse.
__device__ __forceinline__ void dma16_untracked(const void* gsrc, void* lds_base) {
  const uint32_t lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MEA_LDS void*)(lds_base));
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(gsrc), "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4_untracked(const void* gsrc, void* lds_base) {
  const uint32_t lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MEA_LDS void*)(lds_base));
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
               "global_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(gsrc), "s"(lds)
               : "memory");
}

// Copies a tile of ROWS consecutive rows of a row-major [*, D] bf16 array
// into the padded LDS layout with 16-byte DMA (untracked, see above: the
// d = 64 backward, its only user, measured 3-5% faster that way with identical
// results), spread over the waves of a workgroup. DMA block b covers LDS slots 64b..64b+63; slot s is row
// s / kSlotsPerRow, chunk s % kSlotsPerRow. Pad slots fetch a duplicate of
// the row's first chunk. Source rows at or past `n` are clamped to n - 1,
// so every global read stays inside the tensor.
template <int D, int ROWS, int WAVES>
struct TileDma {
  using L = Padded<D>;
  static constexpr int kBlocks = ROWS * L::kSlotsPerRow / 64;
  static constexpr int kPerWave = (kBlocks + WAVES - 1) / WAVES;
  static_assert(kBlocks * 64 == ROWS * L::kSlotsPerRow, "tile must be whole DMA blocks");
  static constexpr int kElems = ROWS * L::kRowElems;  // LDS elements per tile

  int row[kPerWave];
  int col[kPerWave];
  int wave;

  __device__ void init(int wave_, int lane) {
    wave = wave_;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int slot = (wave + WAVES * i) * 64 + lane;
      const int r = slot / L::kSlotsPerRow;
      const int c = slot - r * L::kSlotsPerRow;
      row[i] = r;
      col[i] = (c == L::kSlotsPerRow - 1 ? 0 : c) * 8;
    }
  }
  // rows r0 .. r0+ROWS-1 of src (row stride D) into dst
  __device__ void issue(const bf16* src, int r0, int n, bf16* dst) const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int b = wave + WAVES * i;
      if (b < kBlocks) {
        const int sr = min(r0 + row[i], n - 1);
        dma16_untracked(src + (int64_t)sr * D + col[i], dst + b * 512);
      }
    }
  }
};

// wait for every outstanding memory operation of this wave
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// End of a staged tile in the tiled loops: every wave waits for its own tile
// copies (wait_all) and then for the other waves (barrier), after which the next
// tile is visible to all and the buffer just read may be refilled. Built with
// MEA_SYNC_TIMERS=1 (the separate timing library, never libmea.so) a SyncTimer
// also counts, per wave, the core cycles (s_memtime) spent in the copy wait and
// in the barrier and the cycles of the whole tile loop. In 8-wave workgroups,
// whose waves w and w + 4 share a SIMD, it also counts per tile the cycles both
// waves of a pair spend at the barrier together (the smaller of their two
// waits: the SIMD's idle time there), exchanged through 64 bytes of LDS.
// flush() adds the figures to seven device counters {copy wait, barrier, loop,
// tiles, waves, pair idle, loop cycles of the waves that count pair idle}.
// Without the switch end_of_tile() is exactly wait_all() and the barrier, and
// the rest is empty.
#ifndef MEA_SYNC_TIMERS
#define MEA_SYNC_TIMERS 0
#endif
constexpr int kSyncCounters = 7;
struct SyncTimer {
#if MEA_SYNC_TIMERS
  uint64_t wait = 0, bar = 0, t0 = 0, pair_idle = 0;
  uint32_t tiles = 0, prev_bar = 0;
  int wave = 0, waves = 0;
#endif
  __device__ __forceinline__ void start(int wave_, int waves_) {
#if MEA_SYNC_TIMERS
    // wave-uniform values, kept in scalar registers
    wave = __builtin_amdgcn_readfirstlane(wave_);
    waves = waves_;
    t0 = __builtin_amdgcn_s_memtime();
#else
    (void)wave_;
    (void)waves_;
#endif
  }
  __device__ __forceinline__ void end_of_tile() {
#if MEA_SYNC_TIMERS
    const uint64_t ta = __builtin_amdgcn_s_memtime();
    wait_all();
    const uint64_t tb = __builtin_amdgcn_s_memtime();
    __syncthreads();
    const uint64_t tc = __builtin_amdgcn_s_memtime();
    wait += tb - ta;
    bar += tc - tb;
    if (waves == 8) {
      // slot parity = tile parity: a wave writes its wait for tile t after
      // barrier t and reads its partner's wait for tile t - 1, written before
      // barrier t; the partner rewrites that slot only after barrier t + 1
      __shared__ uint32_t slots[2][8];
      const uint32_t b = (uint32_t)(tc - tb);
      slots[tiles & 1][wave] = b;
      if (tiles > 0 && wave < 4) {
        const uint32_t pb = __builtin_amdgcn_readfirstlane(slots[(tiles - 1) & 1][wave + 4]);
        pair_idle += min(prev_bar, pb);
      }
      prev_bar = b;
    }
    ++tiles;
#else
    wait_all();
    __syncthreads();
#endif
  }
  __device__ __forceinline__ void flush(unsigned long long* counters, int lane) {
#if MEA_SYNC_TIMERS
    const uint64_t loop = __builtin_amdgcn_s_memtime() - t0;
    if (lane == 0) {
      atomicAdd(counters + 0, (unsigned long long)wait);
      atomicAdd(counters + 1, (unsigned long long)bar);
      atomicAdd(counters + 2, (unsigned long long)loop);
      atomicAdd(counters + 3, (unsigned long long)tiles);
      atomicAdd(counters + 4, 1ull);
      if (waves == 8 && wave < 4) {
        atomicAdd(counters + 5, (unsigned long long)pair_idle);
        atomicAdd(counters + 6, (unsigned long long)loop);
      }
    }
#else
    (void)counters;
    (void)lane;
#endif
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup index remap. The hardware hands consecutive
// workgroup ids to the 8 XCDs in turn; remapping makes the ids that run on
// one XCD consecutive in the logical order, so the query tiles of one head
// (which stream the same K and V) share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd;  // whole rounds
  const int full = per * kXcd;
  if (bid >= full) return bid;   // ragged tail keeps its order
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace mea
