// Stream-resident schedule of the SSD forward pass for gfx950 (bf16 storage,
// P = 64).
//
// Same block decomposition as the other schedules ("Transformers are SSMs"
// section 6: diagonal blocks in the quadratic dual form, section 6.1; chunk
// states, the scan across chunks and the left factors, section 6.2), arranged
// so that the N x P state of a head never leaves the chip inside a segment:
//
// * A workgroup owns one segment (a run of K consecutive chunks) of one
//   (batch row, head) stream and walks its chunks in order with the fp32 state
//   in registers.  The state entering the segment is the associative
//   composition of the segments before it (section 8.2's hand-off between
//   workers, appendix B's associative scan): the workgroup first forms the
//   aggregate of the segment in front of it from zero (chunk states only) and
//   composes it with the state that segment's workgroup received,
//   (a1, S1) o (a2, S2) = (a1 a2, a2 S1 + S2).  Only segment-entry states move
//   through memory, one per segment.
// * C B^T of a chunk does not depend on the head (section 7.1: heads of a group
//   share B and C), so a preparation kernel forms it once per (row, chunk,
//   group), causally masked, and every head applies its own decay mask
//   L[i,j] = exp(cs_i - cs_j) to it.
// * Matrix-core operands are fp16 (11-bit significand) rather than bf16, each
//   block scaled by a power of two into fp16 range (x per head and chunk, the
//   state per chunk, B, C and C B^T per row, chunk and group); products
//   accumulate in fp32 and the scales are undone exactly with ldexp.  With
//   bf16 operands the rounding of the masked C B^T tile alone puts the largest
//   relative error of y near 2e-2 on the 130M-shaped layer without D; with
//   fp16 operands it stays near 5e-3.
//
// Inside a chunk (Q = 256, 4 waves) wave w owns the 16-token output tiles
// {w, 7 - w, 8 + w, 15 - w} (equal causal work) and a quarter of the state
// tiles.  Per chunk: tables and the chunk's x (fp16, swizzled LDS tile) and
// the incoming state (fp16, p-major) go to LDS; each wave then forms its output
// tiles (left factors from the incoming state, then the masked diagonal
// blocks, then D x) and its share of the chunk state with no further barrier.
#include <algorithm>
#include <cstdlib>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"
#include "ssd_lds.hpp"

namespace ssd {

typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ inline f32x4 mma_h(f32x4 acc, f16x8 a, f16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}

// 2^v (the prefix sums of dt' A are kept in log2 units, so every decay factor
// is one hardware exp2)
__device__ inline float exp2_(float v) { return __builtin_amdgcn_exp2f(v); }

__device__ inline f16x8 cat_h(f16x4 a, f16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposed fp16 operand from a swizzled tile T[k][r] with R 16-byte chunks per
// row: lane (g, i) receives T[k0 + 4g .. + 3][r0 + i] (see tr_frag_swz).
template <int R>
__device__ inline f16x4 tr_h(const f16* T, int r0, int k0, int lane) {
  const int g = lane >> 4, s = (lane >> 2) & 3, q = lane & 3;
  const f16* p = T + swz_off<R>(k0 + 4 * g + s, r0 + 4 * q);
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(f16x4, v);
}

// Block scale of a block whose largest magnitude is m: 0 when m lies in
// [2^-6, 2^14) (fp16 holds the block as it is: every element at least 2^-24
// of m relative to it is a normal fp16 number), else e such that m 2^-e lies
// in [2^13, 2^14) (clamped to [-100, 100]); 0 for m = 0 or a non-finite m.
__device__ inline int scale_exp(float m) {
  if (!(m > 0.f) || !(m <= 3.0e38f)) return 0;
  const int ex = (int)((__float_as_uint(m) >> 23) & 0xFFu) - 127;
  if (ex >= -6 && ex < 14) return 0;
  return min(max(ex - 13, -100), 100);
}

__device__ inline float ldx(float v, int e) { return __builtin_amdgcn_ldexpf(v, e); }

// Value of lane src (a lane index computed from the caller's lane, so that the
// compiler does not derive its own copy outside the loops and keep it alive).
__device__ inline float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

// Waves per workgroup: eight for long chunks with large states (the state and
// the output tiles of a chunk spread over more waves), else four.
__host__ __device__ constexpr int stream_waves(int N, int Q) {
  return ((Q == 256 && N >= 64) || (N == 256 && Q >= 128)) ? 8 : 4;
}

template <int N, int Q, int W>
struct StreamCfg {
  static constexpr int P = 64;
  static constexpr int NI = Q / 16;               // 16-token tiles per chunk
  static constexpr int NTHR = 64 * W;
  static constexpr int TPI = NI / W;              // output tiles per wave
  static constexpr int NTn = N / 16, NTp = P / 16, NT = NTn * NTp;
  static constexpr int TPW = NT / W;              // state tiles per wave
  static constexpr int NNT = TPW >= NTp ? TPW / NTp : 1;  // n-tiles of a wave's state tiles
  static constexpr int NPT = TPW >= NTp ? NTp : TPW;      // p-tiles of a wave's state tiles
  static constexpr int NK = (N + 31) / 32;        // 32-wide n-blocks
  static constexpr int NKS = Q / 32;              // 32-token steps
  static constexpr int NFR = (NI / 2 + 1) * (NI / 2);  // C B^T fragments per chunk
  static constexpr int RX = P / 8;                // 16-byte chunks per x row
  static constexpr int NXL = Q * RX / NTHR;       // 16-byte x chunks per thread
  static constexpr int LDS_S = N + 8;             // pitch of the p-major state (elements)
  static constexpr int LDY = P + 8;               // pitch of the y staging tile
  static_assert(NI % W == 0 && (TPI % 2 == 0 || TPI == 1), "output tiles split over the waves");
  static_assert(NT % W == 0, "state tiles split over the waves");
  static_assert(NXL >= 1 && (Q * RX) % NTHR == 0, "whole x chunks per thread");
};

// First C B^T fragment of output tile it: tile it holds the fragments of
// j-block pairs 0 .. it / 2.
__host__ __device__ constexpr int gfrag_base(int it) {
  return ((it >> 1) + 1) * ((it >> 1) + (it & 1));
}

// Range mode hands out its ranges from eight ticket queues, one per XCD, each
// over a contiguous block of whole streams: queue q holds streams [q S / 8,
// (q + 1) S / 8) split into ranges of R (stream, chunk) units.  Queue words
// live in the workspace header from word kStreamQueueWord on.
constexpr int kStreamQueues = 8;
constexpr int kStreamQueueWord = 16;

struct StreamQueue {
  int64_t u0, u1, nranges;  // the queue's units [u0, u1) and its range count
};
__host__ __device__ inline StreamQueue stream_queue(int64_t streams, int64_t nc, int64_t R, int q) {
  StreamQueue z;
  z.u0 = q * streams / kStreamQueues * nc;
  z.u1 = (q + 1) * streams / kStreamQueues * nc;
  z.nranges = R > 0 ? (z.u1 - z.u0 + R - 1) / R : 0;
  return z;
}

struct StreamArgs {
  Shape sh;
  int nseg;          // segments per stream (segment mode)
  int K;             // chunks per segment (the last one may have fewer)
  int64_t R;         // range mode when > 0: (stream, chunk) units per workgroup
  int64_t streams;   // batch * H
  const bf16* x;
  const float* D;
  const float* init;
  bf16* y;
  float* final_states;
  const float* cs;   // (batch, H, nc, Q) inclusive prefix sums of dt' A log2(e) per chunk
  const float* dtp;  // (batch, H, nc, Q) dt', read when it scales the input
  const int4* escl;  // (batch, nc, G, Q): per token (row) scale exponents of C B^T, C, B
  const f16* gfr;    // (batch, nc, G, NFR, 64 lanes x 8) masked C B^T fragments
  const f16* bfr;    // (batch, nc, G, N/16, Q/32, 64 x 8) B^T fragments
  const f16* cfr;    // (batch, nc, G, Q/16, NK, 64 x 8) C fragments
  unsigned* counter; // ticket counter (zeroed by the preparation kernel)
  unsigned* flags;   // (streams, nseg) segment-entry state published (zeroed likewise)
  float* slots;      // (streams, nseg, N P) segment-entry states, register-tile order
  unsigned* error;   // set when a wait for a segment-entry state gives up
  unsigned spin_limit;
};

template <int N, int Q, int W>
__global__ __launch_bounds__(64 * W, (W == 4 ? 2 : 1)) void k_stream(StreamArgs a) {
  using F = StreamCfg<N, Q, W>;
  constexpr int P = 64, NI = F::NI, TPI = F::TPI, NTp = F::NTp, TPW = F::TPW, NK = F::NK;
  constexpr int NNT = F::NNT, NPT = F::NPT, NKS = F::NKS, RX = F::RX, NXL = F::NXL;
  constexpr int NTHR = F::NTHR, LDS_S = F::LDS_S, LDY = F::LDY;
  constexpr int NP = N * P;

  __shared__ __attribute__((aligned(16))) f16 sX[Q * P];         // x / 2^ex (swizzled)
  __shared__ __attribute__((aligned(16))) f16 sS[P * LDS_S];     // incoming state / 2^eS, p-major
  // per-wave y staging (in the C B^T fragments' space when a wave owns two
  // tiles per pass)
  __shared__ __attribute__((aligned(16))) bf16 sY[TPI >= 2 ? 1 : W][16 * LDY];
  __shared__ __attribute__((aligned(16))) f16 sG[F::NFR * 512];  // the chunk's masked C B^T fragments
  __shared__ __attribute__((aligned(16))) float sCs[Q];          // prefix sums of dt' A (log2 units)
  __shared__ __attribute__((aligned(16))) float sCe[NI];         // the same at each 16-token block end
  __shared__ __attribute__((aligned(16))) f16 sBt[Q];            // exp(r_blk - cs_j) (x dt'_j)
  __shared__ __attribute__((aligned(16))) f16 sW[Q];             // exp(cs_last - cs_j) (x dt'_j) 2^(eb_j - eBm)
  __shared__ __attribute__((aligned(16))) float sSc[Q];          // dt'_j when it scales the input, else 1
  __shared__ __attribute__((aligned(8))) int2 sEi[Q];           // row scales (C B^T row, C row)
  __shared__ float sRed[3][W];
  __shared__ unsigned sTicket, sQueue, sGaveUp;

  const Shape& sh = a.sh;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: everything derived from it (tiles,
  // fragment counts, loop bounds) is uniform and branches on it are scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = (lane >> 4) * 4, g8 = 2 * g4, l16 = lane & 15;
  const bool scales = sh.flags & kFlagScalesInput;

  if (tid == 0) {
    if (a.R > 0) {
      // Range mode: this XCD's queue first (its workgroups then walk
      // neighbouring streams, which share their batch row's fragments in that
      // XCD's L2), the others when it is empty.  Every workgroup gets a range:
      // one that finds every queue empty would leave more ranges than
      // workgroups taken.
      const int xcd = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7;  // XCC_ID
      unsigned t = ~0u, qt = 0;
      for (int k = 0; k < kStreamQueues; ++k) {
        const int qx = (xcd + k) % kStreamQueues;
        const StreamQueue z = stream_queue(a.streams, sh.nc, a.R, qx);
        if (z.nranges == 0) continue;
        const unsigned v = atomicAdd(a.counter + kStreamQueueWord + qx, 1u);
        if ((int64_t)v < z.nranges) {
          t = v;
          qt = (unsigned)qx;
          break;
        }
      }
      sTicket = t;
      sQueue = qt;
    } else {
      sTicket = atomicAdd(a.counter, 1u);
    }
  }
  __syncthreads();
  const unsigned ticket = sTicket;
  // The (batch row, head) stream being walked and its chunk range; set per
  // job below, read by every helper.
  int64_t s = 0;
  int b = 0, h = 0, grp = 0;
  const int nt0 = (wave * TPW) / NTp, pt0 = (wave * TPW) % NTp;
  auto set_stream = [&](int64_t st) {
    s = st;
    b = (int)(s / sh.H);
    h = (int)(s % sh.H);
    grp = h / sh.hpg;
  };

  // Lane-derived values are re-derived from an opaque copy of the thread index
  // in every chunk: derived once outside the loops, the compiler keeps dozens
  // of lane offsets alive across them and spills.
  struct Ln {
    int tid, lane, g4, g8, l16;
  };
  auto fresh_lane = [&]() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    Ln L;
    L.tid = t;
    L.lane = t & 63;
    L.g4 = (L.lane >> 4) * 4;
    L.g8 = 2 * L.g4;
    L.l16 = L.lane & 15;
    return L;
  };
#define SSD_LANE_VARS(L)                                                                  \
  const int tid = (L).tid, lane = (L).lane, g4 = (L).g4, g8 = (L).g8, l16 = (L).l16;       \
  (void)tid;                                                                              \
  (void)lane;                                                                             \
  (void)g4;                                                                               \
  (void)g8;                                                                               \
  (void)l16

  // ---------------------------------------------------------------- per-chunk loads
  struct Tok {
    float cs, cs_last, sc;
    int4 e;  // the token's row scales (C B^T row, C row, B row)
  };
  auto chunk_len = [&](int c) { return (int)min<int64_t>(Q, sh.L - (int64_t)c * Q); };
  auto load_tok = [&](int c, const Ln& L) {
    SSD_LANE_VARS(L);
    const int len = chunk_len(c);
    const int64_t base = (((int64_t)b * sh.H + h) * sh.nc + c) * Q;
    const int t = min(tid, len - 1);
    Tok k;
    k.cs = a.cs[base + t];
    k.cs_last = a.cs[base + len - 1];
    k.sc = scales ? a.dtp[base + t] : 1.f;
    k.e = a.escl[(((int64_t)b * sh.nc + c) * sh.G + grp) * Q + t];
    return k;
  };
  // thread tid holds 16-byte chunks tid + k NTHR of the chunk's x (row r, chunk
  // cc); rows past the chunk end repeat its last row
  auto load_x = [&](int c, const Ln& L, bf16x8 (&xr)[NXL]) {
    SSD_LANE_VARS(L);
    const int len = chunk_len(c);
    const bf16* xb = a.x + (((int64_t)b * sh.L + (int64_t)c * Q) * sh.H + h) * P;
#pragma unroll
    for (int k = 0; k < NXL; ++k) {
      const unsigned qx = (unsigned)tid + k * NTHR;
      const int r = min((int)(qx / RX), len - 1), cc = (int)(qx % RX);
      xr[k] = *reinterpret_cast<const bf16x8*>(xb + (int64_t)r * sh.H * P + 8 * cc);
    }
  };

  // state tile k of this wave: (n-tile, p-tile)
  auto tile_nt = [&](int k) { return nt0 + (TPW >= NTp ? k / NTp : 0); };
  auto tile_pt = [&](int k) { return pt0 + (TPW >= NTp ? k % NTp : k); };
  // state tile k of a row-major N x P state (the caller's initial / final states)
  auto rowmajor = [&](int k, const Ln& L) {
    SSD_LANE_VARS(L);
    return (int64_t)(16 * tile_nt(k) + g4) * P + 16 * tile_pt(k) + l16;
  };

  // ---------------------------------------------------------------- chunk set-up
  // Tables of the chunk, x / 2^ex into sX and (with_s) the incoming state /
  // 2^es into sS.  Returns ex and es, whether the state is zero, and eBm, the
  // largest B row scale of the chunk (the chunk-state operand is B_j w_j
  // 2^(eb_j - eBm), one scale for the whole contraction over tokens).
  // The chunk's maxima (|x|, |S| when with_s, the B row scales of its tokens)
  // per wave into sRed; read by every wave after the next barrier.
  auto maxima = [&](int c, const Ln& L, const Tok& tk, const bf16x8 (&xr)[NXL],
                    const f32x4 (&S)[TPW], bool with_s) {
    SSD_LANE_VARS(L);
    const int len = chunk_len(c);
    float mx = 0.f, ms = 0.f, mb = -1000.f;
#pragma unroll
    for (int k = 0; k < NXL; ++k) {
      // rows past the chunk end repeat its last row: they cannot raise the max
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf((float)xr[k][e]));
    }
    if (with_s) {
#pragma unroll
      for (int k = 0; k < TPW; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) ms = fmaxf(ms, fabsf(S[k][r]));
    }
    if (tid < len) mb = (float)tk.e.z;
    mx = wave_max(mx);
    ms = wave_max(ms);
    mb = wave_max(mb);
    if (lane == 0) {
      sRed[0][wave] = mx;
      sRed[1][wave] = ms;
      sRed[2][wave] = mb;
    }
  };
  // have_max: maxima() already ran for this chunk before a barrier (at the end
  // of the chunk in front, which saves a barrier per chunk)
  auto setup = [&](int c, const Ln& L, const Tok& tk, const bf16x8 (&xr)[NXL],
                   const f32x4 (&S)[TPW], bool with_s, bool have_max, bool& s_zero, int& eBm) {
    SSD_LANE_VARS(L);
    const int len = chunk_len(c);
    // every load in flight has landed (x, the per-token values and the
    // fragments copied into LDS for this chunk)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (!have_max) maxima(c, L, tk, xr, S, with_s);
    const float cs_blk = lane_value(tk.cs, lane | 15);  // end of the token's 16-block
    if (tid < Q) {
      sCs[tid] = tk.cs;
      if ((tid & 15) == 15) sCe[tid >> 4] = tk.cs;
      sBt[tid] = (f16)(exp2_(cs_blk - tk.cs) * tk.sc);
      sSc[tid] = tk.sc;
      sEi[tid] = make_int2(tk.e.x, tk.e.y);
    }
    if (!have_max) lds_barrier();
    float gx = sRed[0][0], gs = sRed[1][0], gb = sRed[2][0];
#pragma unroll
    for (int w = 1; w < W; ++w) {
      gx = fmaxf(gx, sRed[0][w]);
      gs = fmaxf(gs, sRed[1][w]);
      gb = fmaxf(gb, sRed[2][w]);
    }
    const int ex = scale_exp(gx), es = scale_exp(gs);
    s_zero = !(gs > 0.f);
    eBm = (int)gb;
    if (tid < Q) sW[tid] = (f16)ldx(exp2_(tk.cs_last - tk.cs) * tk.sc, tk.e.z - eBm);
    // rows past the chunk end keep the copies of its last row: their B rows
    // and C B^T entries are zero, so they add nothing
    if (ex == 0) {  // wave-uniform
#pragma unroll
      for (int k = 0; k < NXL; ++k) {
        const unsigned qx = (unsigned)tid + k * NTHR;
        const int r = (int)(qx / RX), cc = (int)(qx % RX);
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (f16)(float)xr[k][e];
        *reinterpret_cast<f16x8*>(sX + swz_off<RX>(r, 8 * cc)) = v;
      }
    } else {
#pragma unroll
      for (int k = 0; k < NXL; ++k) {
        const unsigned qx = (unsigned)tid + k * NTHR;
        const int r = (int)(qx / RX), cc = (int)(qx % RX);
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (f16)ldx((float)xr[k][e], -ex);
        *reinterpret_cast<f16x8*>(sX + swz_off<RX>(r, 8 * cc)) = v;
      }
    }
    if (with_s) {
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        f16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (f16)ldx(S[k][r], -es);
        *reinterpret_cast<f16x4*>(sS + (16 * tile_pt(k) + l16) * LDS_S + 16 * tile_nt(k) + g4) = v;
      }
    }
    lds_barrier();
    return make_int2(ex, es);
  };

  // ---------------------------------------------------------------- chunk state
  // S = exp(cs_last) S + sum_j B_j w_j x_j over the chunk (w_j = exp(cs_last -
  // cs_j), times dt'_j when it scales the input); the B^T fragments were
  // requested earlier (issue_state)
  // steps [k0, k1) of the B^T fragments
  auto issue_state = [&](const Ln& L, int64_t bcg, f16x8 (&bf)[NKS][NNT], int k0, int k1) {
    SSD_LANE_VARS(L);
    const f16* bb = a.bfr + bcg * (F::NTn * NKS * 512);  // uniform base; lane offset below
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int nn = 0; nn < NNT; ++nn)
        if (ks >= k0 && ks < k1)
          bf[ks][nn] = *reinterpret_cast<const f16x8*>(bb + ((nt0 + nn) * NKS + ks) * 512 + lane * 8);
  };
  auto state_phase = [&](const Ln& L, int64_t bcg, const Tok& tk, int ex, int eB,
                         const f16x8 (&bf)[NKS][NNT], f32x4 (&S)[TPW]) {
    SSD_LANE_VARS(L);
    f32x4 T[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) T[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    // step ks's x^T fragments and weights; the next step's are read while
    // this step's products run (two buffers)
    struct StepRd {
      f16x8 xf[NPT];
      f16x4 w[2];
    };
    auto read_step = [&](int ks, StepRd& r) {
#pragma unroll
      for (int pp = 0; pp < NPT; ++pp)
        r.xf[pp] = cat_h(tr_h<RX>(sX, 16 * (pt0 + pp), 32 * ks, lane),
                         tr_h<RX>(sX, 16 * (pt0 + pp), 32 * ks + 16, lane));
      r.w[0] = *reinterpret_cast<const f16x4*>(&sW[32 * ks + g4]);
      r.w[1] = *reinterpret_cast<const f16x4*>(&sW[32 * ks + 16 + g4]);
    };
    StepRd r0, r1;
    read_step(0, r0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      StepRd& cur = (ks & 1) ? r1 : r0;
      StepRd& nxt = (ks & 1) ? r0 : r1;
      if (ks + 1 < NKS) read_step(ks + 1, nxt);
      asm volatile("" ::: "memory");
      const f16x8 wv = cat_h(cur.w[0], cur.w[1]);
#pragma unroll
      for (int nn = 0; nn < NNT; ++nn) {
        const f16x8 bw = bf[ks][nn] * wv;  // packed fp16 products
#pragma unroll
        for (int pp = 0; pp < NPT; ++pp) T[nn * NPT + pp] = mma_h(T[nn * NPT + pp], bw, cur.xf[pp]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const float decay = exp2_(tk.cs_last);
#pragma unroll
    for (int k = 0; k < TPW; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[k][r] = decay * S[k][r] + ldx(T[k][r], eB + ex);
  };

  // ---------------------------------------------------------------- outputs
  // y_i = exp(cs_i) C_i S_in + sum_{j <= i} exp(cs_i - cs_j) (C_i . B_j) x_j + D x_i
  //
  // A wave forms its output tiles in passes of two, tiles 2 W k + w and
  // 2 W k + 2 W - 1 - w of pass k (equal causal work per wave; one tile, w,
  // when a wave owns a single tile).  The two tiles of a pass share their x^T
  // operands (the same j-blocks) and their incoming-state operands.  The
  // chunk's masked C B^T fragments sit in LDS (copied there by the DMA path
  // while the previous chunk's state was formed); a tile's C fragments were
  // requested one pass ahead.
  //
  // The accumulator is in units of 2^E_i per token i with E_i = max(eg_i +
  // ex, ec_i + es) (eg_i + ex alone when the incoming state is zero): the left
  // factor C_i S_in is accumulated first and scaled by exp(cs_i) 2^(ec_i + es -
  // E_i) (at most 1), the diagonal blocks then accumulate with 2^(eg_i + ex -
  // E_i) (at most 1) folded into their decay factors, so nothing can overflow
  // and only a term that is negligible next to the other can lose precision.
  constexpr int NU = TPI >= 2 ? 2 : 1;     // tiles per pass
  constexpr int NPASS = TPI >= 2 ? TPI / 2 : 1;
  struct CFr {
    f16x8 v[NU][NK];
  };
  // tile u of pass k
  auto pass_tile = [&](int k, int u) {
    if constexpr (NU == 1) return wave;
    return 2 * W * k + (u ? 2 * W - 1 - wave : wave);
  };
  // the C fragments of pass k (skipped when the incoming state is zero)
  auto issue_cf = [&](int k, const Ln& L, int64_t bcg, CFr& cf) {
    SSD_LANE_VARS(L);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const f16* cb = a.cfr + (bcg * NI + pass_tile(k, u)) * NK * 512 + lane * 8;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) cf.v[u][kk] = *reinterpret_cast<const f16x8*>(cb + kk * 512);
    }
  };
  // LDS reads of j-block pair pr: x^T fragments, the block-end prefix sums,
  // the per-token factors exp(cs_blk_j - cs_j) (x dt'_j) and each tile's C B^T
  // fragment (tiles that reach pair pr)
  struct PairRd {
    f16x8 xa[NTp];
    f16x4 bt[2];
    float ce[2];
    f16x8 g[NU];
  };
  // staging tile of the wave's y rows: the first C B^T fragments of its last
  // tile of the pass once its diagonal blocks are done (each fragment is read
  // by its tile's wave only), else a tile of its own
  constexpr bool kStageInG = NU == 2;

  auto output_pass = [&](auto KC, int c, const Ln& L, const CFr& cf, int ex, int es, bool s_zero) {
    constexpr int k = decltype(KC)::value;
    constexpr int PRM = NU == 2 ? W * (k + 1) : (W + 1) / 2;  // pairs of the pass's last tile, at most
    SSD_LANE_VARS(L);
    const int len = chunk_len(c);
    const float Dx = ldx(a.D ? a.D[h] : 0.f, ex);  // D 2^ex: y gets D x_i = Dx x'_i
    bf16* const ybase = a.y + (((int64_t)b * sh.L + (int64_t)c * Q) * sh.H + h) * P;
    int it[NU], lim[NU], ii[NU], E[NU];
    float csi[NU], fd[NU];
    f32x4 acc[NU][NTp];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      it[u] = pass_tile(k, u);
      lim[u] = it[u] >> 1;
      ii[u] = 16 * it[u] + l16;
      csi[u] = sCs[ii[u]];
      const int2 ei = sEi[ii[u]];
      const int eD = ei.x + ex, eL = ei.y + es;
      E[u] = s_zero ? eD : max(eD, eL);
      fd[u] = ldx(1.f, eD - E[u]);
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) acc[u][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!s_zero) (void)eL;
    }
    // left factors first: acc = exp(cs_i) 2^(eL - E) C_i S_in
    if (!s_zero) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
        for (int pt = 0; pt < NTp; ++pt) {
          const f16x8 v = *reinterpret_cast<const f16x8*>(sS + (16 * pt + l16) * LDS_S + 32 * kk + (g8 % N));
          const f16x8 sv = (N >= 32 || g8 < N) ? v : f16x8{};
#pragma unroll
          for (int u = 0; u < NU; ++u) acc[u][pt] = mma_h(acc[u][pt], sv, cf.v[u][kk]);
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int2 ei = sEi[ii[u]];
        const float f = exp2_(csi[u]) * ldx(1.f, ei.y + es - E[u]);
#pragma unroll
        for (int pt = 0; pt < NTp; ++pt) acc[u][pt] *= f;
      }
    }

    auto read_pair = [&](int pr, PairRd& r) {
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt)
        r.xa[pt] = cat_h(tr_h<RX>(sX, 16 * pt, 32 * pr, lane), tr_h<RX>(sX, 16 * pt, 32 * pr + 16, lane));
      r.bt[0] = *reinterpret_cast<const f16x4*>(&sBt[32 * pr + g4]);
      r.bt[1] = *reinterpret_cast<const f16x4*>(&sBt[32 * pr + 16 + g4]);
      const float2 ce = *reinterpret_cast<const float2*>(&sCe[2 * pr]);
      r.ce[0] = ce.x;
      r.ce[1] = ce.y;
      // unconditional (a tile past its last pair reads that pair again): a read
      // on one path only would make the wait before this pair's products
      // cover the next pair's reads as well
#pragma unroll
      for (int u = 0; u < NU; ++u)
        r.g[u] = *reinterpret_cast<const f16x8*>(sG + (gfrag_base(it[u]) + min(pr, lim[u])) * 512 + lane * 8);
    };
    // decay factors of j-block kb of tile u: below the diagonal block through
    // the block end (both factors at most 1), direct on it, zero above it
    auto below = [&](int u, const PairRd& r, int hf) {
      const f16 e = (f16)(exp2_(csi[u] - r.ce[hf]) * fd[u]);
      return r.bt[hf] * f16x4{e, e, e, e};
    };
    f16x4 fdg[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int j0 = 16 * it[u] + g4;
      const f32x4 dcs = *reinterpret_cast<const f32x4*>(&sCs[j0]);  // the block's prefix sums
      const f32x4 dsc = *reinterpret_cast<const f32x4*>(&sSc[j0]);  // and input scales
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        fdg[u][q4] = (f16)(j0 + q4 <= ii[u] ? exp2_(csi[u] - dcs[q4]) * (dsc[q4] * fd[u]) : 0.f);
    }
    auto on_diag = [&](int u) { return fdg[u]; };
    auto compute_pair = [&](int pr, const PairRd& r) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if (pr <= lim[u]) {  // wave-uniform
          f16x8 f;
          if (pr < lim[u]) {
            f = cat_h(below(u, r, 0), below(u, r, 1));
          } else if (it[u] & 1) {
            f = cat_h(below(u, r, 0), on_diag(u));
          } else {
            f = cat_h(on_diag(u), f16x4{});
          }
          const f16x8 m = r.g[u] * f;  // packed fp16 products
#pragma unroll
          for (int pt = 0; pt < NTp; ++pt) acc[u][pt] = mma_h(acc[u][pt], r.xa[pt], m);
        }
      }
    };
    // diagonal blocks, the next pair's LDS reads in flight during this pair's
    // products (two buffers)
    PairRd r0, r1;
    read_pair(0, r0);
    const int limH = lim[NU - 1];
#pragma unroll
    for (int pr = 0; pr < PRM; ++pr) {
      if (pr <= limH) {  // wave-uniform
        PairRd& cur = (pr & 1) ? r1 : r0;
        PairRd& nxt = (pr & 1) ? r0 : r1;
        read_pair(min(pr + 1, limH), nxt);  // unconditional, as above
        asm volatile("" ::: "memory");
        compute_pair(pr, cur);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // y = acc 2^E + D x_i, through a staging tile so that each store writes
    // whole 128-byte rows
    bf16* const stg = kStageInG ? reinterpret_cast<bf16*>(sG + gfrag_base(it[NU - 1]) * 512) : sY[wave];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) {
        const f16x4 xv = *reinterpret_cast<const f16x4*>(sX + swz_off<RX>(ii[u], 16 * pt + g4));
        f32x4 yv;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) yv[q4] = ldx(acc[u][pt][q4], E[u]) + Dx * (float)xv[q4];
        store_frag(stg + l16 * LDY + 16 * pt + g4, Elem<bf16>::from_f32(yv));
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's own staging writes
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int rr = 8 * mm + (lane >> 3), ch = lane & 7;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + rr * LDY + 8 * ch);
        const int i = 16 * it[u] + rr;
        if (i < len) *reinterpret_cast<bf16x8*>(ybase + (int64_t)i * sh.H * P + 8 * ch) = v;
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the staging tile is rewritten only after these reads
    }
  };

  // the chunk's C B^T fragments into LDS through the DMA path (each lane's 16
  // bytes land at the fragment's base + 16 lane), tracked by vmcnt
  auto issue_g = [&](int c, const Ln& L) {
    SSD_LANE_VARS(L);
    const int64_t bcg = ((int64_t)b * sh.nc + c) * sh.G + grp;
    const f16* src = a.gfr + bcg * (F::NFR * 512) + lane * 8;
    for (int f = wave; f < F::NFR; f += W)  // wave-uniform
      __builtin_amdgcn_global_load_lds(src + f * 512, (__attribute__((address_space(3))) void*)(sG + f * 512),
                                       16, 0, 0);
  };

  // ---------------------------------------------------------------- the walk
  f32x4 S[TPW];
  bf16x8 xr[NXL];
  Tok tk;
  // the caller's initial state of stream s, or zero
  auto initial_state = [&]() {
    const Ln L = fresh_lane();
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      if (a.init) {
        const float* ip = a.init + s * NP + rowmajor(k, L);
        S[k] = f32x4{ip[0], ip[P], ip[2 * P], ip[3 * P]};
      } else {
        S[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  // wait until slot `slot` is published (acquire), then read it into T.  A
  // wait that gives up sets the error word and makes T infinite, so that every
  // output that depends on the missing state is not finite rather than
  // silently wrong (infinite rather than NaN: the block maxima, formed with
  // fmaxf, would drop a NaN and take the state for zero).
  auto wait_slot = [&](int64_t slot, f32x4 (&T)[TPW]) {
    const Ln L = fresh_lane();
    SSD_LANE_VARS(L);
    if (tid == 0) {
      const unsigned* fl = a.flags + slot;
      unsigned spins = 0, gave = 0;
      while (__hip_atomic_load(fl, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > a.spin_limit) {
          atomicOr(a.error, 1u);
          gave = 1;
          break;
        }
      }
      sGaveUp = gave;
    }
    __syncthreads();
    const float* src = a.slots + slot * NP + wave * TPW * 256 + lane * 4;
#pragma unroll
    for (int k = 0; k < TPW; ++k) T[k] = *reinterpret_cast<const f32x4*>(src + k * 256);
    if (sGaveUp) {
      const float inf = __builtin_inff();
#pragma unroll
      for (int k = 0; k < TPW; ++k) T[k] = f32x4{inf, inf, inf, inf};
    }
  };
  // publish the state S in slot `slot`: every wave's stores complete before
  // the flag is set (release)
  auto publish_slot = [&](int64_t slot) {
    const Ln L = fresh_lane();
    SSD_LANE_VARS(L);
    float* dst = a.slots + slot * NP + wave * TPW * 256 + lane * 4;
#pragma unroll
    for (int k = 0; k < TPW; ++k) *reinterpret_cast<f32x4*>(dst + k * 256) = S[k];
    __syncthreads();
    if (tid == 0) __hip_atomic_store(a.flags + slot, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  };

  // chunks [c0, c1) of stream s from the state in S
  auto run_chunks = [&](int c0, int c1) {
    int c = c0;
    CFr cfn;
    {
      // the first chunk's x, per-token values, C B^T fragments (into LDS) and
      // first-pass C fragments; later chunks' are requested during the chunk
      // in front of them
      const Ln L = fresh_lane();
      load_x(c0, L, xr);
      tk = load_tok(c0, L);
      issue_g(c0, L);
      issue_cf(0, L, ((int64_t)b * sh.nc + c0) * sh.G + grp, cfn);
    }
    for (; c < c1; ++c) {
      const Ln L = fresh_lane();
      const int64_t bcg = ((int64_t)b * sh.nc + c) * sh.G + grp;
      bool sz;
      int eB;
      // every load above has landed; the maxima of every chunk after the first
      // were formed at the end of the chunk in front
      const int2 e = setup(c, L, tk, xr, S, true, c > c0, sz, eB);
      const Tok cur = tk;
      static_assert(NPASS == 1 || NPASS == 2, "passes per chunk");
      if constexpr (NPASS == 2) {
        CFr cf1;
        issue_cf(1, L, bcg, cf1);
        asm volatile("" ::: "memory");
        output_pass(std::integral_constant<int, 0>{}, c, L, cfn, e.x, e.y, sz);
        output_pass(std::integral_constant<int, 1>{}, c, L, cf1, e.x, e.y, sz);
      } else {
        output_pass(std::integral_constant<int, 0>{}, c, L, cfn, e.x, e.y, sz);
      }
      // the chunk state's B^T fragments, then the next chunk's C fragments, x
      // and per-token values, in flight while the chunk state is formed
      f16x8 bf[NKS][NNT];
      issue_state(L, bcg, bf, 0, NKS);
      asm volatile("" ::: "memory");
      if (c + 1 < c1) {
        issue_cf(0, L, bcg + sh.G, cfn);
        load_x(c + 1, L, xr);
        tk = load_tok(c + 1, L);
      }
      asm volatile("" ::: "memory");
      state_phase(L, bcg, cur, e.x, eB, bf, S);
      // the next chunk's maxima (its x and per-token values arrived during the
      // chunk state; S is the state entering it)
      if (c + 1 < c1) maxima(c + 1, L, tk, xr, S, true);
      // every wave is done with the C B^T fragments (and the staging tiles in
      // them), sX, sS and the tables; the next chunk's fragments are copied in
      // after the chunk state's last LDS read (LDS reads behind an LDS copy in
      // flight wait for it)
      lds_barrier();
      if (c + 1 < c1) issue_g(c + 1, L);
    }
  };
  auto write_final = [&]() {
    if (!a.final_states) return;
    const Ln L = fresh_lane();
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      float* o = a.final_states + s * NP + rowmajor(k, L);
      o[0] = S[k][0];
      o[P] = S[k][1];
      o[2 * P] = S[k][2];
      o[3 * P] = S[k][3];
    }
  };

  // Range mode (a.R > 0): this workgroup owns units [u0, u1) of the
  // stream-major order of (stream, chunk) units, at most R long and at least
  // one whole stream long unless it ends its queue, so it touches the tail of
  // one stream, whole streams and the head of one more.  The head goes first
  // and publishes the state at its end for the workgroup of the next range
  // (the only hand-off: no chunk is walked twice); the tail goes last, entered
  // with the state the previous range's workgroup published.  A queue starts
  // at a stream boundary, so that range is the one in front in the same
  // queue: it was handed out before this one, to a workgroup that is running
  // or done and walks its head first, so every wait ends.
  //
  // Segment mode: one segment of K chunks of one stream, segment-major
  // tickets; the segment in front of this one always holds a lower ticket, so
  // it is running or done and every wait ends.
  const bool ranged = a.R > 0;
  if (ranged && ticket == ~0u) return;  // not reached (see above)
  const StreamQueue zq = stream_queue(a.streams, sh.nc, a.R, (int)sQueue);
  const int64_t u0 = zq.u0 + (int64_t)ticket * a.R, u1 = min(u0 + a.R, zq.u1);
  const int64_t sa = ranged ? u0 / sh.nc : 0, sz = ranged ? (u1 - 1) / sh.nc : 0;
  const int ca = ranged ? (int)(u0 % sh.nc) : 0, cz = ranged ? (int)((u1 - 1) % sh.nc) + 1 : 0;
  const int q = ranged ? 0 : (int)(ticket / (unsigned)a.streams);
  const int njobs = ranged ? (int)(sz - sa) + 1 : 1;
  for (int jb = 0; jb < njobs; ++jb) {
    int64_t js;
    int jc0, jc1;
    if (!ranged) {
      js = ticket % (unsigned)a.streams, jc0 = q * a.K, jc1 = min(jc0 + a.K, sh.nc);
    } else if (njobs == 1) {
      js = sa, jc0 = ca, jc1 = cz;
    } else if (jb == 0) {
      js = sz, jc0 = 0, jc1 = cz;  // the head of the last stream
    } else if (jb + 1 < njobs) {
      js = sa + jb, jc0 = 0, jc1 = sh.nc;
    } else {
      js = sa, jc0 = ca, jc1 = sh.nc;  // the tail of the first stream
    }
    set_stream(js);
    if (ranged) {
      if (jc0 > 0)
        wait_slot(s, S);
      else
        initial_state();
    } else if (q > 0) {
      // aggregate of the segment in front, from zero: (decay product, state)
#pragma unroll
      for (int k = 0; k < TPW; ++k) S[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      float dec = 1.f;
      int c = jc0 - a.K;
      {
        const Ln L = fresh_lane();
        load_x(c, L, xr);
        tk = load_tok(c, L);
      }
      for (; c < jc0; ++c) {
        const Ln L = fresh_lane();
        const int64_t bcg = ((int64_t)b * sh.nc + c) * sh.G + grp;
        f16x8 bf[NKS][NNT];
        issue_state(L, bcg, bf, 0, NKS);
        asm volatile("" ::: "memory");
        bool szero;
        int eB;
        const int2 e = setup(c, L, tk, xr, S, false, false, szero, eB);
        const Tok cur = tk;
        if (c + 1 < jc0) {
          load_x(c + 1, L, xr);
          tk = load_tok(c + 1, L);
        }
        asm volatile("" ::: "memory");
        state_phase(L, bcg, cur, e.x, eB, bf, S);
        dec *= exp2_(cur.cs_last);
        lds_barrier();
      }
      // the state entering the segment in front: the caller's initial state
      // for the first segment, else what that segment's workgroup published
      f32x4 I[TPW];
      if (q == 1) {
        const Ln L = fresh_lane();
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
          if (a.init) {
            const float* ip = a.init + s * NP + rowmajor(k, L);
            I[k] = f32x4{ip[0], ip[P], ip[2 * P], ip[3 * P]};
          } else {
            I[k] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      } else {
        wait_slot(s * a.nseg + (q - 1), I);
      }
#pragma unroll
      for (int k = 0; k < TPW; ++k) S[k] = dec * I[k] + S[k];
      if (q + 1 < a.nseg) publish_slot(s * a.nseg + q);
    } else {
      initial_state();
    }
    run_chunks(jc0, jc1);
    if (jc1 == sh.nc)
      write_final();
    else if (ranged)
      publish_slot(s);
  }
}
#undef SSD_LANE_VARS

// ---------------------------------------------------------------- preparation
// grid (nc, batch, 4 G + ceil(H / 8)), 256 threads; the heavier C B^T blocks
// come first in dispatch order.
//  z < 4 G: quarter q of group g of the chunk.  The B rows its tiles reach go
//    to LDS; the quarter's slab of B rows gets a power-of-two scale per row
//    (eb_j) and the B^T operand fragments of its 32-token steps (B_j 2^-eb_j in
//    fp16, transposed through LDS).  Output tiles {q, 7 - q, 8 + q, 15 - q}
//    (Q = 256; else q, q + 4, ..., one per wave): the C operand fragments
//    (C_i 2^-ec_i) and the causally masked C B^T fragments (bf16 products,
//    fp32 accumulation, then 2^-eg_i and fp16), each row scaled by its own
//    power of two so that no reduction over the chunk is needed.  Rows past
//    the chunk end are zero with scale 0.
//  z >= 4 G: dt' = clamp(softplus(dt + bias)) and the inclusive prefix sums of
//    dt' A log2(e) over the chunk for 8 heads (loads along the head axis, a transpose
//    through LDS, one wave per head for the scan).
// The grid also resets the ticket counter, the error word and the flags.
constexpr int kStreamPrepHeads = 8;

template <int N, int Q>
__global__ __launch_bounds__(256) void k_stream_prep(const bf16* __restrict__ dt,
                                                     const float* __restrict__ A,
                                                     const float* __restrict__ dt_bias,
                                                     const bf16* __restrict__ Bm,
                                                     const bf16* __restrict__ Cm, Shape sh,
                                                     float* __restrict__ cs_out,
                                                     float* __restrict__ dt_out, int4* escl,
                                                     f16* gfr, f16* bfr, f16* cfr,
                                                     unsigned* counter, unsigned* error,
                                                     unsigned* flags, int64_t nflags) {
  constexpr int NI = Q / 16, NK = (N + 31) / 32, NKS = Q / 32, NTn = N / 16;
  constexpr int NFR = (NI / 2 + 1) * (NI / 2);
  constexpr int LDB = N + 8;  // pitch of the staged B rows (elements)
  const int c = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = (lane >> 4) * 4, g8 = 2 * g4, l16 = lane & 15;
  const int64_t t0 = (int64_t)c * Q;
  const int len = (int)min<int64_t>(Q, sh.L - t0);
  const int64_t row0 = (int64_t)b * sh.L + t0;
  const int zg = 4 * sh.G;  // C B^T blocks first
  if ((int)blockIdx.z >= zg) {
    __shared__ float sD[kStreamPrepHeads][Q + 1];
    __shared__ float sA[kStreamPrepHeads];
    constexpr int TPL = Q / 64;
    const int h0 = ((int)blockIdx.z - zg) * kStreamPrepHeads;
    {
      constexpr int RPT = Q / (256 / kStreamPrepHeads);  // tokens per thread
      const int hl = tid % kStreamPrepHeads, hh = min(h0 + hl, sh.H - 1), i0 = tid / kStreamPrepHeads;
      const float bias = dt_bias ? dt_bias[hh] : 0.f;
      if (tid < kStreamPrepHeads) sA[hl] = A[hh];
      bf16 raw[RPT];
#pragma unroll
      for (int k = 0; k < RPT; ++k)
        raw[k] = dt[(row0 + min(i0 + k * (256 / kStreamPrepHeads), len - 1)) * sh.H + hh];
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int i = i0 + k * (256 / kStreamPrepHeads);
        float dv = (float)raw[k] + bias;
        if (sh.flags & kFlagSoftplus) dv = softplus_f32(dv);
        sD[hl][i] = i < len ? fminf(fmaxf(dv, sh.dt_min), sh.dt_max) : 0.f;
      }
    }
    __syncthreads();
    for (int hl = wave; hl < kStreamPrepHeads && h0 + hl < sh.H; hl += 4) {
      const int hh = h0 + hl;
      const float Ah = sA[hl] * 1.44269504088896341f;  // log2(e): sums in log2 units
      float d[TPL], v[TPL];
      float run = 0.f;
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        d[k] = sD[hl][lane * TPL + k];
        run += d[k] * Ah;
        v[k] = run;
      }
      float incl = run;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      const float excl = incl - run;
      const int64_t base = (((int64_t)b * sh.H + hh) * sh.nc + c) * Q + lane * TPL;
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        cs_out[base + k] = v[k] + excl;
        if (dt_out) dt_out[base + k] = d[k];
      }
    }
  } else {
    // B rows [0, jend) of the chunk, the most any of this block's tiles
    // reaches; the block's own slab of SR rows among them
    __shared__ __attribute__((aligned(16))) bf16 sBs[Q * LDB];
    __shared__ int sEb[Q];
    const int zz = blockIdx.z, grp = zz >> 2, q = zz & 3;
    const int64_t bcg = ((int64_t)b * sh.nc + c) * sh.G + grp;
    const bf16* Bg = Bm + (row0 * sh.G + grp) * N;
    const bf16* Cg = Cm + (row0 * sh.G + grp) * N;
    const int64_t ld = (int64_t)sh.G * N;
    int* es = reinterpret_cast<int*>(escl + bcg * Q);  // (eg, ec, eb, 0) per token

    // output tiles of this block, one per wave: {q, 7 - q, 8 + q, 15 - q} for
    // 16 tiles (equal causal work per block), else q + 4 w
    auto tile_of = [&](int w) {
      if constexpr (NI == 16) return (w & 1) ? 8 * (w >> 1) + 7 - q : 8 * (w >> 1) + q;
      return q + 4 * w;
    };
    int jend = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (tile_of(w) < NI) jend = max(jend, 16 * tile_of(w) + 16);
    constexpr int SR = Q / 4 >= 32 ? Q / 4 : 32, NS = Q / SR;  // the slab: whole 32-token steps
    jend = max(jend, q < NS ? SR * (q + 1) : 0);
    // rows into LDS, 16 bytes a thread at a time (rows past the chunk end
    // zero): every load of a thread is issued before its first LDS store
    constexpr int CPR = N / 8, NLD = (Q * CPR + 255) / 256;  // 16-byte chunks per row, per thread
    {
      bf16x8 v[NLD];
#pragma unroll
      for (int k = 0; k < NLD; ++k) {
        const int idx = tid + 256 * k, j = idx / CPR, cc = idx % CPR;
        v[k] = bf16x8{};
        if (idx < Q * CPR && j < jend && j < len) v[k] = *reinterpret_cast<const bf16x8*>(Bg + j * ld + 8 * cc);
      }
#pragma unroll
      for (int k = 0; k < NLD; ++k) {
        const int idx = tid + 256 * k, j = idx / CPR, cc = idx % CPR;
        if (idx < Q * CPR && j < jend) *reinterpret_cast<bf16x8*>(sBs + j * LDB + 8 * cc) = v[k];
      }
    }
    __syncthreads();
    // the slab's row scales (four threads per row)
    if (q < NS) {
      constexpr int VPT = N / 4;
      const int jl = tid >> 2, part = tid & 3, j = SR * q + jl;
      float m = 0.f;
      if (jl < SR) {
#pragma unroll
        for (int k = 0; k < VPT / 4; ++k) {
          const bf16x4 v = *reinterpret_cast<const bf16x4*>(sBs + j * LDB + part * VPT + 4 * k);
#pragma unroll
          for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf((float)v[e]));
        }
      }
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      m = fmaxf(m, __shfl_xor(m, 2, 64));
      if (jl < SR && part == 0) {
        const int e = scale_exp(m);
        sEb[j] = e;
        es[4 * j + 2] = e;
      }
    }
    __syncthreads();
    // B^T operand fragments of the slab's 32-token steps: (n-tile nt, step ks),
    // lane (g, l): B[32 ks + 16 hf + 4 g + r][16 nt + l] 2^-eb_j
    if (q < NS) {
      constexpr int KQ = SR / 32;  // steps per slab
      f16* bfp = bfr + bcg * (NTn * NKS * 512) + lane * 8;
      for (int f = wave; f < NTn * KQ; f += 4) {
        const int nt = f / KQ, kl = f % KQ, ks = KQ * q + kl;
        f16x8 o;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int j0 = 32 * ks + 16 * hf;
          const bf16x4 v = tr_frag<LDB>(sBs, 16 * nt, j0, lane);
#pragma unroll
          for (int r = 0; r < 4; ++r) o[4 * hf + r] = (f16)ldx((float)v[r], -sEb[j0 + g4 + r]);
        }
        *reinterpret_cast<f16x8*>(bfp + (nt * NKS + ks) * 512) = o;
      }
    }
    // this wave's output tile
    const int it = tile_of(wave);
    if (it < NI) {
      const int i = 16 * it + l16, ic = min(i, len - 1);
      bf16x8 cr[NK];
      float mc = 0.f;
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(Cg + ic * ld + 32 * k + (g8 % N));
        cr[k] = (i < len && (N >= 32 || g8 < N)) ? v : bf16x8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) mc = fmaxf(mc, fabsf((float)cr[k][e]));
      }
      mc = fmaxf(mc, __shfl_xor(mc, 16, 64));
      mc = fmaxf(mc, __shfl_xor(mc, 32, 64));
      const int ec = scale_exp(mc);
      // C operand fragments (tile it, n-block k), lane (g, l): C_i[32 k + 8 g ..] 2^-ec_i
      f16* cf = cfr + bcg * (NI * NK * 512) + lane * 8;
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        f16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (f16)ldx((float)cr[k][e], -ec);
        *reinterpret_cast<f16x8*>(cf + (it * NK + k) * 512) = o;
      }
      // C B^T of the tile's j-block pairs, lane (g, l): G[i][16 kb + 4 g + r],
      // zero above the diagonal and past the chunk end (B rows from LDS)
      constexpr int NPAIR = NI / 2;
      f32x4 gv[NPAIR][2];
      float mg = 0.f;
#pragma unroll
      for (int pr = 0; pr < NPAIR; ++pr) {
        if (pr <= (it >> 1)) {  // wave-uniform
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int kb = 2 * pr + hf;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (kb <= it) {  // wave-uniform
              const bf16* br = sBs + (16 * kb + l16) * LDB + (g8 % N);
#pragma unroll
              for (int k = 0; k < NK; ++k) {
                const bf16x8 v = *reinterpret_cast<const bf16x8*>(br + 32 * k);
                acc = mma8(acc, (N >= 32 || g8 < N) ? v : bf16x8{}, cr[k]);  // rows j (B), columns i (C)
              }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 16 * kb + g4 + r;
              acc[r] = (kb <= it && j <= i && j < len && i < len) ? acc[r] : 0.f;
              mg = fmaxf(mg, fabsf(acc[r]));
            }
            gv[pr][hf] = acc;
          }
        }
      }
      mg = fmaxf(mg, __shfl_xor(mg, 16, 64));
      mg = fmaxf(mg, __shfl_xor(mg, 32, 64));
      const int eg = scale_exp(mg);
      f16* gf = gfr + bcg * (NFR * 512) + lane * 8;
      const int gbase = gfrag_base(it);
#pragma unroll
      for (int pr = 0; pr < NPAIR; ++pr) {
        if (pr <= (it >> 1)) {
          f16x8 o;
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[4 * hf + r] = (f16)ldx(gv[pr][hf][r], -eg);
          *reinterpret_cast<f16x8*>(gf + (gbase + pr) * 512) = o;
        }
      }
      if (lane < 16) {
        es[4 * i + 0] = eg;
        es[4 * i + 1] = ec;
      }
    }
  }

  // bookkeeping, grid-strided over every thread of the launch
  const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * gridDim.z * blockDim.x;
  const int64_t gid =
      (((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x + tid;
  if (gid == 0) {
    *counter = 0u;
    *error = 0u;
  }
  if (gid < kStreamQueues) counter[kStreamQueueWord + gid] = 0u;
  for (int64_t i = gid; i < nflags; i += nthreads) flags[i] = 0u;
}

// ---------------------------------------------------------------- host side
struct StreamLayout {
  size_t flags, slots, cs, dtp, escl, gfr, bfr, cfr, total;
  int64_t nflags;
  int nseg, K;
};

static void stream_segments(int64_t streams, int64_t nc, int target, int* nseg, int* K) {
  int S = 1;
  if (streams > 0 && streams < target)
    S = (int)std::min<int64_t>(nc, (target + streams - 1) / streams);
  if (const char* e = std::getenv("SSD_STREAM_SEGMENTS")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1) S = (int)std::min<int64_t>(nc, v);
  }
  S = std::max(S, 1);
  int k = (int)((nc + S - 1) / S);
  k = std::max(k, 1);
  *K = k;
  *nseg = (int)((nc + k - 1) / k);
}

static StreamLayout stream_layout(const Shape& sh, int Q, int N) {
  constexpr int P = 64;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  StreamLayout l;
  const int64_t streams = (int64_t)sh.batch * sh.H;
  stream_segments(streams, sh.nc, 512, &l.nseg, &l.K);
  const int NI = Q / 16, NK = (N + 31) / 32;
  const int64_t bcg = (int64_t)sh.batch * sh.nc * sh.G;
  l.nflags = streams * l.nseg;
  l.flags = 256;
  l.slots = l.flags + al((size_t)l.nflags * 4);
  l.cs = l.slots + al((size_t)streams * l.nseg * N * P * 4);
  const size_t per = (size_t)sh.batch * sh.H * sh.nc * Q * 4;
  l.dtp = l.cs + al(per);
  l.escl = l.dtp + al((sh.flags & kFlagScalesInput) ? per : 0);
  l.gfr = l.escl + al((size_t)bcg * Q * 16);
  l.bfr = l.gfr + al((size_t)bcg * ((NI / 2 + 1) * (NI / 2)) * 1024);
  l.cfr = l.bfr + al((size_t)bcg * (N / 16) * (Q / 32) * 1024);
  l.total = l.cfr + al((size_t)bcg * NI * NK * 1024);
  return l;
}

bool stream_supported(int N, int P, int Q, bool bf16_storage, bool varlen, int G, int Gc) {
  return bf16_storage && !varlen && P == 64 && G == Gc &&
         (N == 16 || N == 32 || N == 64 || N == 128 || N == 256) && (Q == 64 || Q == 128 || Q == 256);
}

size_t stream_workspace_bytes(const Shape& sh, int N, int Q) { return stream_layout(sh, Q, N).total; }

// Units ((stream, chunk) pairs) per workgroup in range mode, or 0 for segment
// mode.  Range mode spreads the streams' chunks evenly over one wave of
// resident workgroups when that gives every workgroup at least one whole
// stream's worth (no chunk is then walked twice); SSD_STREAM_RANGE forces a
// range length (at least the chunk count), SSD_STREAM_SEGMENTS forces segment
// mode.
template <int N, int Q, int W>
static int64_t stream_range(int64_t streams, int64_t nc) {
  const int64_t U = streams * nc;
  if (U == 0) return 0;
  if (std::getenv("SSD_STREAM_SEGMENTS")) return 0;
  if (const char* e = std::getenv("SSD_STREAM_RANGE")) {
    const long long v = std::strtoll(e, nullptr, 10);
    return v >= nc ? (int64_t)v : 0;
  }
  static int resident[64];  // workgroups resident at once, per device (0: not yet known)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (resident[dev] == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(&k_stream<N, Q, W>),
                                                     64 * W, 0) != hipSuccess)
      return 0;
    resident[dev] = std::max(cus * per, 1);
  }
  // every queue's ranges fit in its share of the resident workgroups
  const int64_t per = std::max(resident[dev] / kStreamQueues, 1);
  int64_t R = 1;
  for (int q = 0; q < kStreamQueues; ++q) {
    const StreamQueue z = stream_queue(streams, nc, 1, q);
    R = std::max(R, (z.u1 - z.u0 + per - 1) / per);
  }
  return R >= nc ? R : 0;
}

template <int N, int Q>
static hipError_t launch_stream_t(const ChunkedArgs& ca, char* base, const StreamLayout& l,
                                  hipStream_t st) {
  const Shape& sh = ca.sh;
  constexpr int W = stream_waves(N, Q);
  StreamArgs a;
  a.sh = sh;
  a.nseg = l.nseg;
  a.K = l.K;
  a.streams = (int64_t)sh.batch * sh.H;
  a.x = static_cast<const bf16*>(ca.x);
  a.D = ca.D;
  a.init = ca.init;
  a.y = static_cast<bf16*>(ca.y);
  a.final_states = ca.final_states;
  a.cs = reinterpret_cast<const float*>(base + l.cs);
  a.dtp = (sh.flags & kFlagScalesInput) ? reinterpret_cast<const float*>(base + l.dtp) : nullptr;
  a.escl = reinterpret_cast<const int4*>(base + l.escl);
  a.gfr = reinterpret_cast<const f16*>(base + l.gfr);
  a.bfr = reinterpret_cast<const f16*>(base + l.bfr);
  a.cfr = reinterpret_cast<const f16*>(base + l.cfr);
  a.counter = reinterpret_cast<unsigned*>(base);
  a.error = reinterpret_cast<unsigned*>(base) + 1;
  a.flags = reinterpret_cast<unsigned*>(base + l.flags);
  a.slots = reinterpret_cast<float*>(base + l.slots);
  a.spin_limit = 1u << 24;
  if (const char* e = std::getenv("SSD_SPIN_LIMIT")) a.spin_limit = (unsigned)std::strtoul(e, nullptr, 10);
  a.R = stream_range<N, Q, W>(a.streams, sh.nc);

  const int zh = (sh.H + kStreamPrepHeads - 1) / kStreamPrepHeads;
  const dim3 pgrid((unsigned)sh.nc, (unsigned)sh.batch, (unsigned)(zh + 4 * sh.G));
  if (mark(ca, "stream_prep", st) != hipSuccess) return hipErrorUnknown;
  hipLaunchKernelGGL((k_stream_prep<N, Q>), pgrid, dim3(256), 0, st,
                     static_cast<const bf16*>(ca.dt), ca.A, ca.dt_bias,
                     static_cast<const bf16*>(ca.B), static_cast<const bf16*>(ca.C), sh,
                     reinterpret_cast<float*>(base + l.cs),
                     (sh.flags & kFlagScalesInput) ? reinterpret_cast<float*>(base + l.dtp) : nullptr,
                     reinterpret_cast<int4*>(base + l.escl), reinterpret_cast<f16*>(base + l.gfr),
                     reinterpret_cast<f16*>(base + l.bfr), reinterpret_cast<f16*>(base + l.cfr),
                     a.counter, a.error, a.flags, l.nflags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mark(ca, "stream", st) != hipSuccess) return hipErrorUnknown;
  int64_t grid = a.streams * l.nseg;
  if (a.R > 0) {
    grid = 0;
    for (int q = 0; q < kStreamQueues; ++q) grid += stream_queue(a.streams, sh.nc, a.R, q).nranges;
  }
  hipLaunchKernelGGL((k_stream<N, Q, W>), dim3((unsigned)grid), dim3(64 * W), 0, st, a);
  return hipGetLastError();
}

template <int N>
static hipError_t stream_q(const ChunkedArgs& ca, char* base, const StreamLayout& l, int Q,
                           hipStream_t st) {
  switch (Q) {
    case 64: return launch_stream_t<N, 64>(ca, base, l, st);
    case 128: return launch_stream_t<N, 128>(ca, base, l, st);
    case 256: return launch_stream_t<N, 256>(ca, base, l, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_stream(const ChunkedArgs& ca, void* ws, int N, int P, int Q, hipStream_t st) {
  const Shape& sh = ca.sh;
  if (sh.nc == 0 || sh.batch == 0 || P != 64) return sh.nc == 0 || sh.batch == 0 ? hipSuccess : hipErrorInvalidValue;
  const StreamLayout l = stream_layout(sh, Q, N);
  char* base = static_cast<char*>(ws);
  switch (N) {
    case 16: return stream_q<16>(ca, base, l, Q, st);
    case 32: return stream_q<32>(ca, base, l, Q, st);
    case 64: return stream_q<64>(ca, base, l, Q, st);
    case 128: return stream_q<128>(ca, base, l, Q, st);
    case 256: return stream_q<256>(ca, base, l, Q, st);
  }
  return hipErrorInvalidValue;
}

template <int N>
static bool range_mode_q(int64_t streams, int64_t nc, int Q) {
  switch (Q) {
    case 64: return stream_range<N, 64, stream_waves(N, 64)>(streams, nc) > 0;
    case 128: return stream_range<N, 128, stream_waves(N, 128)>(streams, nc) > 0;
    case 256: return stream_range<N, 256, stream_waves(N, 256)>(streams, nc) > 0;
  }
  return false;
}

bool stream_range_mode(int64_t streams, int64_t nc, int N, int Q) {
  switch (N) {
    case 16: return range_mode_q<16>(streams, nc, Q);
    case 32: return range_mode_q<32>(streams, nc, Q);
    case 64: return range_mode_q<64>(streams, nc, Q);
    case 128: return range_mode_q<128>(streams, nc, Q);
    case 256: return range_mode_q<256>(streams, nc, Q);
  }
  return false;
}

hipError_t stream_handoff_failed(const void* ws, hipStream_t st, bool* failed) {
  unsigned word = 0;
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess)
    e = hipMemcpy(&word, static_cast<const unsigned*>(ws) + 1, sizeof(word), hipMemcpyDeviceToHost);
  *failed = word != 0;
  return e;
}

}  // namespace ssd
