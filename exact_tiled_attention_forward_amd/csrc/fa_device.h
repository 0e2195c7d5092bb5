// Device building blocks for the gfx950 (CDNA4) attention kernels.
//
// Conventions used by every kernel in this library
// ------------------------------------------------
// * Matrix core: v_mfma_f32_32x32x16_{bf16,f16}, wave64.  For C[32x32] += A[32x16] B[16x32]
//   lane l holds A[l%32][8*(l/32) + j] and B[8*(l/32) + j][l%32] (j = 0..7, 16-bit values),
//   and C[8*(i/4) + 4*(l/32) + i%4][l%32] in accumulator register i = 0..15.
//   Any permutation of the contraction index that both operands share leaves C unchanged;
//   the kernels use this to feed a C tile straight back as the next product's operand.
// * Tiles in LDS are row-major [row][col] 16-bit, D columns (D = 64 or 128), with the
//   16-byte chunks of each row permuted by an XOR swizzle (swz below).  The swizzle is
//   chosen so that both access patterns the kernels use are free of bank conflicts:
//     - row reads: 16 consecutive lanes read the same chunk of 16 consecutive rows
//       (ds_read_b128, an MFMA operand whose contraction index runs along the row);
//     - transposing reads: a 32-lane half wave reads 4 consecutive rows x 4 consecutive
//       chunks (ds_read_b64_tr_b16, an operand whose contraction index runs down the
//       columns).
//   Tiles are filled by buffer_load ... lds (direct HBM -> LDS, 16 bytes per lane): a wave
//   instruction writes 1 KiB of LDS contiguously, and the swizzle is applied by choosing
//   which global chunk each lane fetches.  Rows past the end of the sequence fall outside
//   the buffer resource's range and arrive as zeros.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

// Race-check build (-DFA_RACE_CHECK=1, libfa_racecheck.so).  Its kernels compute exactly
// what the release build computes, on a perturbed schedule: after every workgroup barrier
// each wave sleeps for a time that grows with its index modulo 4, so that within each set
// of four waves (the two groups of the two-phase forward) the first wave runs ahead of the
// last by longer than a tile fill takes to land, and every tile fill waits for its own
// completion as soon as it is issued, so that it lands as early as it can.  A fill that
// overwrites a buffer some wave may still read, or a read that does not wait for its
// fill, then changes the result: the race-check tests compare both builds bit for bit.
// Checked against an earlier forward whose V fill was issued while waves of its own group
// could still be reading the buffer: the release and race-check builds of that kernel
// differed on every test case.
#ifndef FA_RACE_CHECK
#define FA_RACE_CHECK 0
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit dwords (gfx9 family)

// ------------------------------------------------------------------ 16-bit element types

struct bf16_t {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> two bf16 (round to nearest even), packed low/high
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
  }
  static __device__ __forceinline__ float to_f32(uint16_t u) {
    return __uint_as_float(((uint32_t)u) << 16);
  }
  // acc + lo + hi of a packed pair, in one v_dot2 against (1, 1)
  static __device__ __forceinline__ float sum2(uint32_t packed, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
  }
  static __device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  static constexpr uint32_t kOnePair = 0x3f803f80u;  // (1, 1)
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

struct f16_t {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
  }
  static __device__ __forceinline__ float to_f32(uint16_t u) {
    return (float)__builtin_bit_cast(_Float16, u);
  }
  static __device__ __forceinline__ float sum2(uint32_t packed, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), __builtin_bit_cast(f16x2, 0x3c003c00u), acc,
                                  false);
  }
  static __device__ __forceinline__ float lo_f32(uint32_t w) { return to_f32((uint16_t)(w & 0xffffu)); }
  static __device__ __forceinline__ float hi_f32(uint32_t w) { return to_f32((uint16_t)(w >> 16)); }
  static constexpr uint32_t kOnePair = 0x3c003c00u;  // (1, 1)
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// Constant A operand that turns a 16x16x32 MFMA into per-query sums of a P V step's B
// operand.  That operand (16 keys x 32 queries for v_mfma_f32_32x32x16: lane l holds query
// l % 32 and 8 of the keys, chosen by l / 32) is read by the 16x16x32 product as 32
// "keys" x 16 columns: lane l gives column l % 16 and contraction group l / 16, so column
// j mixes queries j (groups 0, 2) and j + 16 (groups 1, 3).  Output (i, j) lands in lane
// j + 16 (i / 4).  With ones on groups 0 and 2 in the rows i whose i / 4 is even and on
// groups 1 and 3 in the others (lane l of A: row l % 16, group l / 16), all four output
// registers of lane l hold the sum over the step's 16 keys for query l % 32, the lane's
// own row, so a rescale multiplies it by the lane's own factor like the O accumulators.
template <class T>
__device__ __forceinline__ u32x4 row_sum_operand(int lane) {
  const bool on = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1);
  const uint32_t w = on ? T::kOnePair : 0u;
  return (u32x4){w, w, w, w};
}

// Two fp32 values as a 16-bit pair hi plus the 16-bit pair of what hi missed, so that
// hi + lo carries about twice the input type's significand.  A product A (hi + lo),
// done as two MFMAs, then rounds only what both halves together cannot represent.
template <class T>
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = T::pack(x0, x1);
  lo = T::pack(x0 - T::lo_f32(hi), x1 - T::hi_f32(hi));
}

// ------------------------------------------------------------------ swizzled tiles

// XOR applied to the 16-byte chunk index of row r of a D-column 16-bit tile.
//  D = 128 (16 chunks = 256 B per row, a full bank sweep): f(r) = 4*(r%4) + (r/4)%4.
//  D = 64  (8 chunks = 128 B per row, two rows per bank sweep): f(r) = 4*((r/2)%2) + (r/4)%4.
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Byte offset in a swizzled tile of the 16-byte chunk c of row r.
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * (D * 2) + ((c ^ swz<D>(r)) << 4);
}

// Row read: this lane's 8 consecutive 16-bit values (one chunk) of row r.
template <int D>
__device__ __forceinline__ u32x4 lds_row16(const FA_LDS uint8_t* tile, int r, int c) {
  return *(const FA_LDS u32x4*)(tile + tile_off<D>(r, c));
}

// Transposing read (ds_read_b64_tr_b16).  Within each 16-lane group, lane i names row
// r(i) and the 4 columns col0(i)..col0(i)+3; the hardware returns to lane i the column
// (group base + i) of the 4x16 block formed by lanes 4e..4e+3 (e = 0..3) -> 4 values, one
// per row r(4e + ...).  Here each lane passes its own row and column (col multiple of 4).
template <int D>
__device__ __forceinline__ u32x2 lds_tr16(const FA_LDS uint8_t* tile, int r, int col) {
  const int off = r * (D * 2) + ((((col >> 3) ^ swz<D>(r)) << 4) | ((col & 7) << 1));
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(tile + off));
  return __builtin_bit_cast(u32x2, t);
}

// MFMA operand with the contraction index running down the columns of a tile:
// lane l gets rows {rbase + 4*(l/32) + e, rbase + 8 + 4*(l/32) + e : e = 0..3} of column
// cbase + l%32.  This matches the row order of an accumulator tile's registers 8m..8m+7
// (rows 16m + 8*(j/4) + 4*(l/32) + j%4), so an accumulator C tile converted to 16-bit can
// be paired with it directly.
template <int D>
__device__ __forceinline__ u32x4 lds_colop(const FA_LDS uint8_t* tile, int rbase, int cbase, int lane) {
  const int i = lane & 15;
  const int g = lane >> 4;              // 0..3
  const int h = g >> 1;                 // lane / 32
  const int r = rbase + 4 * h + (i >> 2);
  const int col = cbase + 16 * (g & 1) + 4 * (i & 3);
  u32x2 lo = lds_tr16<D>(tile, r, col);
  u32x2 hi = lds_tr16<D>(tile, r + 8, col);
  return (u32x4){lo.x, lo.y, hi.x, hi.y};
}

// Index of the calling wave in its workgroup as a wave-uniform (scalar) value.  The
// compiler does not infer that threadIdx.x / 64 is equal across a wave; conditions built
// from the plain quotient then count as divergent and are exec-masked on every pass
// instead of branched over.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// Race-check build only: wait for this wave's outstanding loads (a fill just issued).
__device__ __forceinline__ void race_check_fill_wait() {
#if FA_RACE_CHECK
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#endif
}

// Workgroup barrier.  In the race-check build each wave then sleeps about 4000 cycles
// per unit of its index modulo 4 (waves 0-3 and 4-7 each fan out over about 12000 cycles,
// longer than a tile fill takes to land).
__device__ __forceinline__ void fa_sync() {
  __syncthreads();
#if FA_RACE_CHECK
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) & 3;
  for (int i = 0; i < 8 * w; ++i) __builtin_amdgcn_s_sleep(8);
#endif
}

// Fill `rows` x D tile (16-bit) from global rows [row0, row0 + rows) of a head whose
// buffer resource covers exactly that head.  NT threads cooperate; each wave instruction
// moves 1 KiB.  Out-of-range rows read as zeros.
template <int D, int ROWS, int NT>
__device__ __forceinline__ void tile_load_async(FA_LDS uint8_t* tile, __amdgpu_buffer_rsrc_t rs, int row0, int tid) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int CHUNKS = ROWS * CPR;
  constexpr int PER_INSTR = 64;
  constexpr int WAVES = NT / 64;
  constexpr int NI = CHUNKS / PER_INSTR;     // wave instructions per tile
  static_assert(CHUNKS % PER_INSTR == 0 && (NI % WAVES == 0 || WAVES % NI == 0),
                "tile must split evenly over waves");
  const int wave = tid >> 6, lane = tid & 63;
  auto issue = [&](int base) {  // base: wave-uniform chunk index
    const int p = base + lane;
    const int r = p / CPR;
    const int slot = p % CPR;
    const int c = slot ^ swz<D>(r);
    const int voff = (row0 + r) * (D * 2) + (c << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(tile + base * 16), 16, voff, 0, 0, 0);
    race_check_fill_wait();
  };
  if constexpr (NI % WAVES == 0) {
#pragma unroll
    for (int t = 0; t < NI / WAVES; ++t) issue((t * WAVES + wave) * PER_INSTR);
  } else {
    if (wave < NI) issue(wave * PER_INSTR);  // fewer instructions than waves: the first NI waves
  }
}

// The same fill, with each 16-byte-per-lane load written as inline assembly, for kernels
// that keep several tiles in flight.  The compiler treats an outstanding buffer_load ...
// lds from its builtin as possibly writing whatever a later transposing LDS read
// (ds_read_b64_tr_b16) reads, and waits for every outstanding load before such a read,
// which would drain the whole ring of tiles on every tile.  Loads written as assembly
// are invisible to that analysis, so the caller owns the ordering: it waits with
// wait_vmem_upto for the loads of the tile it is about to read (they complete in issue
// order) and then synchronises the workgroup.  rs is the buffer resource as four words
// (rsrc_words), held in SGPRs.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is named as clobbered on purpose
__device__ __forceinline__ void dma16(const FA_LDS void* lds_dst, const u32x4& rs, int voff) {
  // wave-uniform LDS byte address, moved to an SGPR for the s_mov
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
#if FA_RACE_CHECK
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_waitcnt vmcnt(0)"
               :
               : "s"(m0), "v"(voff), "s"(rs)
               : "memory", "m0");
#else
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rs)
               : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

template <int D, int ROWS, int NT>
__device__ __forceinline__ void tile_load_async_asm(FA_LDS uint8_t* tile, const u32x4& rs, int row0, int tid) {
  constexpr int CPR = D / 8;
  constexpr int CHUNKS = ROWS * CPR;
  constexpr int PER_INSTR = 64;
  constexpr int WAVES = NT / 64;
  constexpr int NI = CHUNKS / PER_INSTR;
  static_assert(CHUNKS % PER_INSTR == 0 && (NI % WAVES == 0 || WAVES % NI == 0),
                "tile must split evenly over waves");
  const int wave = tid >> 6, lane = tid & 63;
  auto issue = [&](int base) {
    const int p = base + lane;
    const int r = p / CPR;
    const int c = (p % CPR) ^ swz<D>(r);
    dma16(tile + base * 16, rs, (row0 + r) * (D * 2) + (c << 4));
  };
  if constexpr (NI % WAVES == 0) {
#pragma unroll
    for (int t = 0; t < NI / WAVES; ++t) issue((t * WAVES + wave) * PER_INSTR);
  } else {
    if (wave < NI) issue(wave * PER_INSTR);
  }
}

// Buffer resource words of a raw (stride 0) buffer of `bytes` bytes at base.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return (u32x4){(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, kRsrcWord3};
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}


__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rs, int voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
}

// s_waitcnt vmcnt(0) (gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15).  A builtin, not inline
// asm: inline asm makes the compiler assume AGPRs may be in use and select the AGPR form of
// every MFMA, which then costs a copy for each accumulator the VALU touches.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): wait until at most N vector memory instructions of this wave are
// outstanding (they complete in issue order).  vmcnt is 6 bits, split over bits 3:0 and
// 15:14 of the immediate.
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Value of x held by lane l^32 (the other half of the wave): v_permlane32_swap.
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes 0..31 receive the upper half's value in the second result, lanes 32..63 the
  // lower half's value in the first result
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(a, b) with NaN propagation (IEEE 754-2019 maximum).  Chains of it lower to
// v_maximum3_f32, one instruction per two new values; fmaxf would first canonicalise
// every input (quieting signalling NaNs), which doubles the work of a row max.
__device__ __forceinline__ float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Row index (within a 32-row accumulator tile) held in register i by this lane's half.
__device__ __forceinline__ constexpr int acc_row(int i, int half) {
  return 8 * (i >> 2) + 4 * half + (i & 3);
}

}  // namespace fa
