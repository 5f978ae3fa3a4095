// Device-side building blocks shared by the SSD kernels (gfx950 / CDNA4).
//
// Fragment convention (all matrix products in this library).  Products are
// done on 16 x 16 output tiles with the MFMA matrix cores, wave64.  For an
// operand with contraction index k, the k axis is cut into 16-row "k-blocks";
// lane l (g = l / 16) holds the 4 consecutive k values 4g .. 4g+3 of a k-block
// for row/column (l % 16).  An output tile comes back in exactly that shape:
// lane l holds column (l % 16) and rows 4g .. 4g+3.  So the output of one
// product can be fed, without any shuffle, as an operand of the next product
// whose contraction runs over the first product's rows.
//
//   bf16: v_mfma_f32_16x16x32_bf16 consumes two k-blocks per instruction
//         (8 values per lane: block 0 then block 1).  The instruction pairs the
//         same (lane group, slot) of A and B to the same k, so any consistent
//         assignment of k values to slots is a valid contraction.
//   fp32: v_mfma_f32_16x16x4_f32 consumes one k value per lane; a k-block is
//         four instructions (slot s of every lane group in instruction s).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Elem;

template <>
struct Elem<bf16> {
  using frag = bf16x4;  // 4 k-values of one lane, 8 bytes
  static constexpr int kBytes = 2;
  static constexpr int kStage = 64;  // tokens staged through LDS per step
  __device__ static inline frag from_f32(f32x4 v) { return __builtin_convertvector(v, bf16x4); }
  __device__ static inline f32x4 to_f32(frag v) { return __builtin_convertvector(v, f32x4); }
  __device__ static inline float to_float(bf16 v) { return (float)v; }
  __device__ static inline bf16 from_float(float v) { return (bf16)v; }
  __device__ static inline f32x4 mma2(f32x4 acc, frag a0, frag a1, frag b0, frag b1) {
    bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
};

template <>
struct Elem<float> {
  using frag = f32x4;  // 16 bytes
  static constexpr int kBytes = 4;
  static constexpr int kStage = 32;
  __device__ static inline frag from_f32(f32x4 v) { return v; }
  __device__ static inline f32x4 to_f32(frag v) { return v; }
  __device__ static inline float to_float(float v) { return v; }
  __device__ static inline float from_float(float v) { return v; }
  __device__ static inline f32x4 mma1(f32x4 acc, frag a, frag b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    return acc;
  }
  __device__ static inline f32x4 mma2(f32x4 acc, frag a0, frag a1, frag b0, frag b1) {
    return mma1(mma1(acc, a0, b0), a1, b1);
  }
};

template <typename T>
__device__ inline typename Elem<T>::frag load_frag(const T* p) {
  return *reinterpret_cast<const typename Elem<T>::frag*>(p);
}

template <typename T>
__device__ inline void store_frag(T* p, typename Elem<T>::frag v) {
  *reinterpret_cast<typename Elem<T>::frag*>(p) = v;
}

template <typename T>
__device__ inline typename Elem<T>::frag zero_frag() {
  return Elem<T>::from_f32(f32x4{0.f, 0.f, 0.f, 0.f});
}

// exp on the fast hardware path (v_exp_f32 after a log2(e) prescale).
__device__ inline float fast_exp(float v) { return __expf(v); }

// log(1 + e) for e in [0, 1] on the hardware log: u = 1 + e is rounded, and
// log(u) * e / (u - 1) cancels that rounding (u - 1 is exact); a few ulp.
// The correction is the classic one for log1p from a plain log (Goldberg,
// "What every computer scientist should know about floating-point
// arithmetic", 1991, Theorem 4).
__device__ inline float log1p_unit(float e) {
  const float u = 1.f + e;
  return u == 1.f ? e : __logf(u) * __fdividef(e, u - 1.f);
}

// softplus(v) = log(1 + e^v), evaluated as max(v, 0) + log1p(e^-|v|).
__device__ inline float softplus_f32(float v) {
  return fmaxf(v, 0.f) + log1p_unit(__expf(-fabsf(v)));
}

// Shape and options shared by every kernel of one call.
struct Shape {
  int64_t L;        // tokens per batch row (total tokens with cu_seqlens)
  int32_t batch;    // rows (1 with cu_seqlens)
  int32_t H;        // heads
  int32_t G;        // B groups
  int32_t hpg;      // heads per B group = H / G
  int32_t Gc;       // C groups
  int32_t hpgc;     // heads per C group = H / Gc
  int32_t nc;       // chunks per row = ceil(L / Q)
  int32_t nseqs;    // sequences (batch, or packed sequences)
  uint32_t flags;   // bit 0 softplus, bit 1 input scaled by dt'
  float dt_min, dt_max;
  int32_t varlen;   // cu_seqlens given
  int32_t has_init; // initial states given
};

constexpr uint32_t kFlagSoftplus = 1u;
constexpr uint32_t kFlagScalesInput = 2u;

// Per-chunk sequence bookkeeping (positions are token indices within the row).
struct ChunkInfo {
  int32_t seq_first;    // sequence of the chunk's first token
  int32_t seq_last;     // sequence of the chunk's last token
  int32_t start_first;  // first token of seq_first
  int32_t start_last;   // first token of seq_last
};

// v combined with the value that DPP control `ctrl` moves into this lane (rows
// outside `rows` keep v)
template <int ctrl, int rows>
__device__ inline float dpp_max(float v) {
  const int u = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), ctrl, rows, 0xF, false);
  return fmaxf(v, __int_as_float(u));
}

// Largest v over the wave, wave-uniform: within each quad (xor 1, xor 2), each
// half row and each row of 16 (mirrors), then row 0 into row 1, row 2 into row
// 3 (broadcast of lane 15 of the row in front) and rows 0-1 into rows 2-3
// (broadcast of lane 31); lane 63 then holds the maximum.  All in registers.
__device__ inline float wave_max(float v) {
  v = dpp_max<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_max<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_max<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max<0x140, 0xF>(v);  // row_mirror
  v = dpp_max<0x142, 0xA>(v);  // row_bcast:15
  v = dpp_max<0x143, 0xC>(v);  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

}  // namespace ssd
