// LDS tiles and matrix-core operand helpers shared by the bf16 kernels
// (gfx950): swizzled unpadded tiles filled straight from global memory, the
// transposing LDS load, and a barrier that waits for LDS traffic only.
#pragma once

#include "ssd_device.hpp"

namespace ssd {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Preconditions of the transposing load (ds_read_b64_tr_b16): every lane
// hands in the address of 8 bytes (4 consecutive 16-bit elements) that must be
// 8-byte aligned, and all 16 lanes of a group must be active (the load moves
// data between them).  For a row-major tile with leading dimension LD elements
// and an 8-byte aligned base, a lane's address T + k LD + r0 + 4q is aligned
// when LD and r0 are multiples of 4: LD is checked at compile time, r0 by the
// callers' tile arithmetic (multiples of 16).  The callers keep the load out of
// lane-divergent branches.
template <int LD>
__device__ constexpr bool tr_pitch_ok() {
  return LD > 0 && LD % 4 == 0;
}

// Operand fragment of M[r][k] = T[k][r], T row-major in LDS with leading
// dimension LD: lane (g = lane / 16, i = lane % 16) receives
// M[r0 + i][k0 + 4g .. 4g + 3].  Within each 16-lane group the transposing load
// hands lane i element (i % 4) of source lanes {i/4, 4 + i/4, 8 + i/4, 12 + i/4};
// source lane 4s + q therefore points at row k0 + 4g + s, columns r0 + 4q.
template <int LD>
__device__ inline bf16x4 tr_frag(const bf16* T, int r0, int k0, int lane) {
  static_assert(tr_pitch_ok<LD>(), "rows of the tile must start 8-byte aligned");
  const int g = lane >> 4, s = (lane >> 2) & 3, q = lane & 3;
  const bf16* p = T + (k0 + 4 * g + s) * LD + r0 + 4 * q;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// One 16 x 16 x 32 product where each lane brings 8 consecutive contraction
// values (used for contractions over the state dimension n: lane group g of a
// 32-wide n-block holds n = 8g .. 8g + 7 on both operands).
__device__ inline f32x4 mma8(f32x4 acc, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void;

// Unpadded row-major LDS tile with R 16-byte chunks per row: chunk c of row r
// sits in slot c ^ swz<R>(r).  For R <= 16, 16 / R rows share one 256-byte
// bank line, and consecutive groups of them get distinct slot permutations, so
// 16 rows read at one logical chunk, or 16 rows x 32 bytes read transposed,
// tile the 64 banks evenly.
template <int R>
__device__ inline int swz(int r) {
  static_assert(R == 2 || R == 4 || R == 8 || R == 16 || R == 32, "2 to 32 chunks per row");
  // a 32-chunk row spans two bank lines: permuting the low 4 bits of the slot
  // by the row spreads 16 rows read at one logical chunk over all 64 banks
  if constexpr (R == 32) return r % 16;
  else return (r / (16 / R)) % R;
}

// Element offset of (row r, element e) in such a tile.
template <int R>
__device__ inline int swz_off(int r, int e) {
  return r * 8 * R + 8 * ((e >> 3) ^ swz<R>(r)) + (e & 7);
}

// Transposed operand fragment from a swizzled tile T[k][r] (rows k): lane
// (g = lane / 16, i = lane % 16) receives M[r0 + i][k0 + 4g .. 4g + 3] of
// M = T^T.  Within each 16-lane group the transposing load hands lane i element
// (i % 4) of source lanes {i/4, 4 + i/4, 8 + i/4, 12 + i/4}; source lane 4s + q
// therefore points at row k0 + 4g + s, elements r0 + 4q .. + 3 (one chunk).
template <int R>
__device__ inline bf16x4 tr_frag_swz(const bf16* T, int r0, int k0, int lane) {
  const int g = lane >> 4, s = (lane >> 2) & 3, q = lane & 3;
  const bf16* p = T + swz_off<R>(k0 + 4 * g + s, r0 + 4 * q);
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Rows [0, Q) of a row-major global matrix (row stride ld elements, rows past
// len repeat row len - 1) into a swizzled LDS tile with R chunks per row.  Each
// instruction moves 64 chunks (1 KB): lane i fills LDS bytes 16 i of it, so
// lane i fetches the chunk that belongs in that slot.  The Q R / 64
// instructions are spread over the W waves; this issues the m-th of a wave's.
template <int R, int Q, int W>
__device__ inline void dma_tile_part(bf16* lds, const bf16* src, int ld, int len, int wave,
                                     int lane, int m) {
  constexpr int RPI = 64 / R, NINST = Q / RPI;
  static_assert(NINST % W == 0, "whole instructions per wave");
  const int k = wave + W * m;
  const int r = k * RPI + lane / R;
  const int c = (lane % R) ^ swz<R>(r);
  // 32-bit byte offset from a wave-uniform base (the tile spans < 2^31 bytes)
  const unsigned off = (unsigned)(min(r, len - 1) * ld + 8 * c) * 2u;
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src) + off,
                                   (lds_void*)(lds + k * 512), 16, 0, 0);
}

// Workgroup barrier for hand-offs through LDS: waits for this wave's LDS
// accesses only.  (__syncthreads() would also wait for every global load and
// store in flight, and for loads into LDS, which are waited for explicitly
// where their data is needed.)  The empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Instruction k of copying rows [r0, r0 + RN) of a row-major global matrix
// (row stride ld elements; rows at or past len repeat row len - 1) into a
// swizzled LDS tile of RN rows with R chunks per row; k < RN R / 64.
template <int R>
__device__ inline void dma_rows(bf16* lds, const bf16* src, int ld, int r0, int len, int lane,
                                int k) {
  constexpr int RPI = 64 / R;
  const int r = k * RPI + lane / R;
  const int c = (lane % R) ^ swz<R>(r);
  const unsigned off = (unsigned)(min(r0 + r, len - 1) * ld + 8 * c) * 2u;
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src) + off,
                                   (lds_void*)(lds + k * 512), 16, 0, 0);
}

}  // namespace ssd
