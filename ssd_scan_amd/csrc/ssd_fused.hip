// Fused single-pass schedule of the SSD forward pass for gfx950 (bf16 storage).
//
// Same block decomposition as the chunked schedule ("Transformers are SSMs"
// section 6: diagonal blocks in the quadratic dual form, section 6.1; chunk
// states, a scan across chunks and left factors, section 6.2), but one kernel
// reads x once and writes y once.  The scan across chunks is a chain: the
// work unit of chunk c for a head waits for the state the unit of chunk c - 1
// published, adds its own chunk state, and publishes the result for chunk
// c + 1 (the sequence-parallel hand-off of section 8.2 done between work units
// of one kernel).  Section 6.3 notes the scan is a small part of the work, so
// the chain only orders a short critical section per chunk.
//
// Work unit = (chunk, batch row, head).  Units are taken from an atomic ticket
// in chunk-major order by persistent workgroups, so a unit only ever waits on a
// lower ticket that a running workgroup holds: the chain always makes
// progress.  Hand-off slots are a 2-deep ring per (row, head), small enough to
// stay in the 256 MB MALL; they are written and read with relaxed agent-scope
// atomics (coherent across XCDs without cache flushes).  A state is published
// with one flag per producing wave holding chunk index + 1; with very few
// streams (the chain bounds the run) every 32-bit value travels instead with
// its chunk tag in one 64-bit atomic word, so the consumer polls the data
// itself and a hand-off costs one store and one load (at twice the bytes).
//
// Inside a unit (8 waves for Q = 256), wave w owns the 16-token output tiles
// {w, Q/16 - 1 - w} (equal causal work per wave).  B and x chunks go from
// global memory straight into LDS (gfx950 global_load_lds_dwordx4, no
// registers involved) while the previous unit still computes, into unpadded
// XOR-swizzled row-major tiles; operands that contract over tokens are read
// with the transposing LDS load (ds_read_b64_tr_b16).  The decay mask
// L[j,i] = exp(cs_i - cs_j) is applied as exp(cs_i - r) * exp(r - cs_j) with r
// the prefix sum at the end of j's 16-token block: one exp per lane per tile
// plus a per-token table, all factors bounded by 1 off the diagonal block.
#include <cstdlib>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"
#include "ssd_lds.hpp"

namespace ssd {

// Hand-off ring entries: a 16 x 16 state tile as two 512-byte halves, lane l's
// values (r = 0, 1) in the first half and (r = 2, 3) in the second, each at
// float offset 2 l.  One wave instruction then moves whole cache lines (a lane's
// 16 bytes in one place would make each 8-byte atomic access half a line).
// The accesses are relaxed 64-bit atomics at agent scope, ordered by the
// hand-off flags without release / acquire fences (which on this part write
// back or invalidate a whole L2 per hand-off): agent-scope stores and loads
// bypass the non-coherent L2 to the device-coherent level, a store counts in
// vmcnt until that level has taken it, the producer waits for its ring stores'
// vmcnt before the flag store, and the consumer issues its ring loads only
// after a poll returned the flag (compiler fences keep that order in the
// code).  The tagged form needs no flag: each 64-bit word carries its own tag.
__device__ inline f32x4 ring_load(const float* tile, int lane) {
  const unsigned long long* q = reinterpret_cast<const unsigned long long*>(tile) + lane;
  const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long b = __hip_atomic_load(q + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float2 fa = __builtin_bit_cast(float2, a), fb = __builtin_bit_cast(float2, b);
  return f32x4{fa.x, fa.y, fb.x, fb.y};
}

__device__ inline void ring_store(float* tile, int lane, f32x4 v) {
  unsigned long long* q = reinterpret_cast<unsigned long long*>(tile) + lane;
  __hip_atomic_store(q, __builtin_bit_cast(unsigned long long, float2{v[0], v[1]}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 64, __builtin_bit_cast(unsigned long long, float2{v[2], v[3]}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tagged ring entries (few-stream launches): a 16 x 16 state tile as four
// 512-byte quarters, quarter r holding lane l's value r as the 64-bit word
// (tag << 32) | bits(value) at word l.  A single-copy-atomic 64-bit access moves
// a value together with the chunk tag that says which state it belongs to.
__device__ inline void ring_store_tagged(float* tile, int lane, f32x4 v, unsigned tag) {
  unsigned long long* q = reinterpret_cast<unsigned long long*>(tile) + lane;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    __hip_atomic_store(q + 64 * r,
                       ((unsigned long long)tag << 32) | __float_as_uint(v[r]),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Loads a tagged tile; false unless all four of this lane's values carry `tag`.
__device__ inline bool ring_load_tagged(const float* tile, int lane, unsigned tag, f32x4& v) {
  const unsigned long long* q = reinterpret_cast<const unsigned long long*>(tile) + lane;
  bool ok = true;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const unsigned long long w = __hip_atomic_load(q + 64 * r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v[r] = __uint_as_float((unsigned)w);
    ok = ok && (unsigned)(w >> 32) == tag;
  }
  return ok;
}

template <int N, int P, int Q>
struct FusedCfg {
  static constexpr int NI = Q / 16;           // 16-token tiles of the chunk
  static constexpr int W = NI / 2;            // waves; wave w owns output tiles w, NI-1-w
  static constexpr int NTHR = 64 * W;
  static constexpr int RB = N / 8, RX = P / 8;  // 16-byte chunks per B / x row
  static constexpr int NKn = N / 16, NKn2 = (NKn + 1) / 2;  // 16- and 32-wide n-blocks
  // Padded pitches (elements): the w-scaled x copy, rows 40 banks apart (a
  // transposed read of 16 rows tiles all banks twice), and the transposed
  // incoming state (P x N), rows 68 = 4 (mod 64) banks apart.
  static constexpr int LDX = P + 16, LDS_T = N + 8, LDY = P + 8;
  static constexpr int NTn = N / 16, NTp = P / 16, NT = NTn * NTp;
  static constexpr int SXW_ELEMS = Q * LDX;
  static constexpr int SS_ELEMS = 2 * P * LDS_T;  // incoming state as hi/lo bf16 terms
  static constexpr int REGION2 = SXW_ELEMS > SS_ELEMS ? SXW_ELEMS : SS_ELEMS;
  // chunk-state tiles: a block of SN n-tiles x SP p-tiles per wave when the
  // tile grid splits evenly over the waves, else tiles w, w + W, ...
  static constexpr bool kBlock = (NTp % 2 == 0) && (W % 2 == 0) && (NTn % (W / 2) == 0);
  static constexpr int SN = kBlock ? NTn / (W / 2) : 1;
  static constexpr int SP = kBlock ? NTp / 2 : 1;
  static constexpr int TPW = kBlock ? SN * SP : (NT + W - 1) / W;
  // memory instructions every wave issues after its last direct-to-LDS load of
  // a unit: the y stores and the next unit's C fragments
  static constexpr int VM_AFTER_DMA = 2 * NKn2 + 4;
};

struct FusedArgs {
  Shape sh;
  const bf16* x;
  const float* A;
  const bf16* B;
  const bf16* C;
  const float* D;
  const float* cs;   // (batch, H, nc, Q) inclusive prefix sums of dt' A per chunk
  const float* dtp;  // (batch, H, nc, Q) dt' (read only when it scales the input)
  const float* init;
  bf16* y;
  bf16* sink;        // 128 bytes that take the stores of rows past a chunk's end
  float* final_states;
  unsigned* counter;  // ticket counter (zeroed before the launch)
  unsigned* flags;    // (batch, H, 2, kFlagWaves) hand-off flags (zeroed before the launch)
  float* slots;       // (batch, H, 2, 2*N*P) hand-off states, ring tile layout
  unsigned* error;    // set when a hand-off wait gives up
  unsigned spin_limit;  // sleeps before a hand-off wait gives up
  // packed sequences (batch 1): cu_seqlens, per token the position in its chunk
  // where its sequence starts (0 if before the chunk), per chunk the first and
  // last sequence and their first tokens
  const int32_t* cu;
  const int32_t* ls;
  const int4* cinfo;
  int nunits;
  // Hand-off placement.  0: wait for chunk c - 1 before the chunk states (the
  // incoming state then loads behind them) and raise the flag after the
  // state-to-output product.  1 (few streams, the chain bounds the run): wait
  // after the chunk states and raise the flag as soon as the ring stores have
  // landed, so that only the update S_out = decay S_in + S_c and two memory
  // round trips separate consecutive chunks of a stream.  2 (fewer streams
  // still): as 1, but through the tagged ring, polled by every wave for the
  // tiles it needs: one store and one load per hand-off.
  int late;
};

// Default bound on the sleeps of one hand-off wait (about half a second):
// every wait ends even if a chunk it depends on never publishes.
constexpr unsigned kSpinLimit = 1u << 24;
// One flag per wave of the producing workgroup (at most 8 waves) and ring slot.
constexpr int kFlagWaves = 8;

// Unit coordinates of ticket t (chunk-major: every unit of chunk c precedes chunk c + 1).
struct Unit {
  int c, b, h, grp, len;
  int64_t row0;
};

__device__ inline Unit unit_of(unsigned t, const Shape& sh, int Q) {
  const int per_chunk = sh.batch * sh.H;
  Unit u;
  u.c = (int)(t / per_chunk);
  const int rem = (int)(t % per_chunk);
  u.b = rem / sh.H;
  u.h = rem % sh.H;
  u.grp = u.h / sh.hpg;
  const int64_t tb = (int64_t)u.c * Q;
  u.len = (int)min<int64_t>(Q, sh.L - tb);
  u.row0 = (int64_t)u.b * sh.L + tb;
  return u;
}

// Per-token values of a unit kept in registers: token tid's prefix sum and dt'
// (threads past the chunk read its last token), and the chunk's last prefix sum;
// with packed sequences also where token tid's sequence starts in the chunk.
struct TokenLoads {
  float cs, cs_last, dtp, D;
  int ls;
};

template <bool VL>
__device__ inline TokenLoads load_tokens(const FusedArgs& a, const Unit& u, int Q) {
  const Shape& sh = a.sh;
  const int tid = threadIdx.x;
  const int64_t cbase = (((int64_t)u.b * sh.H + u.h) * sh.nc + u.c) * Q;
  TokenLoads r;
  r.cs = a.cs[cbase + min(tid, u.len - 1)];
  r.cs_last = a.cs[cbase + u.len - 1];
  // dt' only when it scales the input (else the prefix sum is read again and ignored)
  r.dtp = ((sh.flags & kFlagScalesInput) ? a.dtp : a.cs)[cbase + min(tid, u.len - 1)];
  // the head's D (A is read in its place when D is absent, and dropped at use)
  r.D = (a.D ? a.D : a.A)[u.h];
  r.ls = VL ? a.ls[(int64_t)u.c * Q + min(tid, u.len - 1)] : 0;
  return r;
}

// C fragments of output tiles it0 and it1 of unit u: row it * 16 + l % 16 and
// n = 32 k2 + 8 (l / 16) .. + 7 (rows past the chunk end read the last row; for
// N = 16 the upper half of the only n-block is zero).
template <int N, int P, int Q>
__device__ inline void load_c_tiles(const FusedArgs& a, const Unit& u, int it0, int it1,
                                    bf16x8 (&cf)[2][FusedCfg<N, P, Q>::NKn2]) {
  using F = FusedCfg<N, P, Q>;
  const int lane = threadIdx.x & 63, g8 = (lane >> 4) * 8, l16 = lane & 15;
  const int its[2] = {it0, it1};
  const char* base = reinterpret_cast<const char*>(a.C + (u.row0 * a.sh.Gc + u.h / a.sh.hpgc) * N);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = min(its[t] * 16 + l16, u.len - 1);
    const bf16* cr =
        reinterpret_cast<const bf16*>(base + (unsigned)(i * a.sh.Gc * N + (g8 % N)) * 2u);
#pragma unroll
    for (int k2 = 0; k2 < F::NKn2; ++k2) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(cr + 32 * k2);
      cf[t][k2] = (N >= 32 || g8 < N) ? v : bf16x8{};
    }
  }
}

template <int N, int P, int Q, bool VL, int MODE>
__global__ __launch_bounds__((FusedCfg<N, P, Q>::NTHR), 2) void k_fused(FusedArgs a) {
  using F = FusedCfg<N, P, Q>;
  using E = Elem<bf16>;
  using frag = bf16x4;
  constexpr int NI = F::NI, W = F::W, RB = F::RB, RX = F::RX, LDX = F::LDX;
  constexpr int NKn2 = F::NKn2, NTp = F::NTp, NT = F::NT, TPW = F::TPW;
  constexpr int SN = F::SN, SP = F::SP;
  constexpr int NP = N * P;

  __shared__ __attribute__((aligned(16))) bf16 sB[Q * N];   // B chunk (swizzled)
  __shared__ __attribute__((aligned(16))) bf16 sX[Q * P];   // x chunk (swizzled)
  // x scaled by w_j (padded), later the incoming state as hi/lo terms
  __shared__ __attribute__((aligned(16))) bf16 sXw[F::REGION2];
  __shared__ __attribute__((aligned(16))) float sCs[Q];  // inclusive prefix sums of dt' A
  __shared__ __attribute__((aligned(16))) float sBt[Q];  // exp(r_block - cs_j) (x dt'_j if scaled)
  __shared__ __attribute__((aligned(16))) float sWt[Q];  // exp(cs_last - cs_j) (x dt'_j if scaled)
  // per-wave staging of one 16-row output tile, rows 72 elements (36 banks) apart
  __shared__ __attribute__((aligned(16))) bf16 sY[W][16 * F::LDY];
  // packed sequences: where each token's sequence starts in the chunk
  __shared__ int sLs[VL ? Q : 1];
  __shared__ unsigned sTicket, sGaveUp;
  bf16* const sS = sXw;

  const Shape& sh = a.sh;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: branches on it are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = (lane >> 4) * 4, g8 = 2 * g4, l16 = lane & 15;
  const bool scales = sh.flags & kFlagScalesInput;
  // output tiles of this wave; the pair (w, NI - 1 - w) has equal causal work
  const int it0 = wave, it1 = NI - 1 - wave;
  // chunk-state tiles of this wave
  const int nt0 = F::kBlock ? (wave % (W / 2)) * SN : 0;
  const int pt0 = F::kBlock ? (wave / (W / 2)) * SP : 0;

  // B and x of a unit go straight into LDS, in NB and NTp instructions per wave
  constexpr int NB = (Q * RB / 64) / W;
  static_assert((Q * RX / 64) / W == NTp, "one x instruction per p-tile");
  auto dma_b = [&](const Unit& u, int m) {
    dma_tile_part<RB, Q, W>(sB, a.B + (u.row0 * sh.G + u.grp) * N, sh.G * N, u.len, wave, lane, m);
  };
  auto dma_x = [&](const Unit& u, int m) {
    dma_tile_part<RX, Q, W>(sX, a.x + (u.row0 * sh.H + u.h) * P, sh.H * P, u.len, wave, lane, m);
  };

  if (tid == 0) sTicket = atomicAdd(a.counter, 1u);
  __syncthreads();
  unsigned t = sTicket;
  __syncthreads();

  TokenLoads tk;
  int4 ci = {0, 0, 0, 0};  // packed sequences: the chunk's sequence info
  // C fragments of the wave's two output tiles; rows past the chunk end repeat
  // the last row (they only reach output rows that are never stored)
  bf16x8 cf[2][NKn2];
  if (t < (unsigned)a.nunits) {
    const Unit u0 = unit_of(t, sh, Q);
#pragma unroll
    for (int m = 0; m < NB; ++m) dma_b(u0, m);
#pragma unroll
    for (int m = 0; m < NTp; ++m) dma_x(u0, m);
    tk = load_tokens<VL>(a, u0, Q);
    if constexpr (VL) ci = a.cinfo[u0.c];
    load_c_tiles<N, P, Q>(a, u0, it0, it1, cf);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // chunk-state tile (n-tile, p-tile) of slot k of this wave; slots past the
  // tile count (uneven split) repeat the last tile and store nothing
  auto state_tile = [&](int k, int& nt, int& pt) {
    if constexpr (F::kBlock) {
      nt = nt0 + k / SP;
      pt = pt0 + k % SP;
    } else {
      const int tt = min(wave + W * k, NT - 1);
      nt = tt / NTp;
      pt = tt % NTp;
    }
  };
  auto state_slot_valid = [&](int k) { return F::kBlock || wave + W * k < NT; };

  while (t < (unsigned)a.nunits) {
    // Lane-derived addresses are recomputed in every iteration: hoisted out
    // of the loop they would be kept in registers across it (and spilled).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, g4 = (lane >> 4) * 4, g8 = 2 * g4, l16 = lane & 15;
    const Unit un = unit_of(t, sh, Q);
    const int c = un.c, len = un.len;
    const int64_t row0 = un.row0;
    const int64_t stream = (int64_t)un.b * sh.H + un.h;
    const int64_t t0 = (int64_t)c * Q;
    // packed sequences: the chunk's last sequence starts at ls_last in it (0
    // when it started earlier); fresh: a sequence starts at the first token
    const int ls_last = VL ? (int)max<int64_t>((int64_t)ci.w - t0, 0) : 0;
    const bool fresh = VL && (int64_t)ci.z == t0;

    // ---------------------------------------------------------------- stage
    // this wave's loads into LDS have landed (everything issued after them is
    // the previous unit's y stores and this unit's C fragments); the barrier
    // extends that to every wave's
    {
      constexpr int K = F::VM_AFTER_DMA;
      static_assert(K < 64, "vmcnt field");
      __builtin_amdgcn_s_waitcnt((K & 15) | ((K >> 4) << 14) | (7 << 4) | (15 << 8));
    }
    // the per-token values (loaded before the LDS loads) are first used here,
    // after the wait above
    asm volatile("" : "+v"(tk.cs), "+v"(tk.cs_last), "+v"(tk.dtp), "+v"(tk.D));
    if constexpr (VL) asm volatile("" : "+v"(tk.ls));
    lds_barrier();
    // prefix sums and the decay tables (one token per thread of the first Q);
    // with packed sequences only the last sequence's tokens reach the chunk
    // state
    {
      const float csv = tk.cs;
      const float cs_blk = __shfl(csv, lane | 15, 64);  // end of the token's 16-block
      const float sc = scales ? tk.dtp : 1.f;
      if (tid < Q) {
        sCs[tid] = csv;
        sBt[tid] = fast_exp(cs_blk - csv) * sc;
        sWt[tid] = (VL && tid < ls_last) ? 0.f : fast_exp(tk.cs_last - csv) * sc;
        if constexpr (VL) sLs[tid] = tk.ls;
      }
    }
    lds_barrier();
    // x_j scaled by the weights in sWt (w_j = exp(cs_last - cs_j) (x dt'_j)),
    // rows past the chunk end zero, for the chunk-state product; read only
    // after the wait barrier below
    auto scale_x = [&]() {
      constexpr int KX = (Q * RX) / F::NTHR;  // 16-byte chunks per thread
      static_assert(F::NTHR % RX == 0, "whole rows per pass");
      const int cc = (int)((unsigned)tid % RX), r0 = (int)((unsigned)tid / RX);
      bf16x8 v[KX];
      float w[KX];
#pragma unroll
      for (int k = 0; k < KX; ++k) {  // every read in flight before any use
        const int r = r0 + k * (F::NTHR / RX);
        v[k] = *reinterpret_cast<const bf16x8*>(sX + swz_off<RX>(r, 8 * cc));
        w[k] = sWt[r];
      }
#pragma unroll
      for (int k = 0; k < KX; ++k) {
        const int r = r0 + k * (F::NTHR / RX);
        const f32x4 lo = E::to_f32(bf16x4{v[k][0], v[k][1], v[k][2], v[k][3]}) * w[k];
        const f32x4 hi = E::to_f32(bf16x4{v[k][4], v[k][5], v[k][6], v[k][7]}) * w[k];
        const bf16x4 l4 = E::from_f32(lo), h4 = E::from_f32(hi);
        const bf16x8 o = {l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
        *reinterpret_cast<bf16x8*>(sXw + r * LDX + 8 * cc) = r < len ? o : bf16x8{};
      }
    };
    scale_x();

    // ---------------------------------------------------------------- diagonal blocks
    const float csi0 = sCs[it0 * 16 + l16], csi1 = sCs[it1 * 16 + l16];
    // packed sequences: output row i only sees tokens j of its own sequence,
    // j >= where that sequence starts in the chunk
    const int lsi0 = VL ? sLs[it0 * 16 + l16] : 0, lsi1 = VL ? sLs[it1 * 16 + l16] : 0;
    // B rows of j-block kb for this lane (8 consecutive n per 32-wide n-block)
    auto load_b_rows = [&](int kb, bf16x8 (&ba)[NKn2]) {
      const int j = 16 * kb + l16;
#pragma unroll
      for (int k2 = 0; k2 < NKn2; ++k2) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(sB + swz_off<RB>(j, 32 * k2 + (g8 % N)));
        ba[k2] = (N >= 32 || g8 < N) ? v : bf16x8{};
      }
    };
    // C_i . B_j over n
    auto gram = [&](const bf16x8 (&ba)[NKn2], const bf16x8 (&cc)[NKn2]) {
      f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k2 = 0; k2 < NKn2; ++k2) g = mma8(g, ba[k2], cc[k2]);
      return g;
    };
    // masked tile M[j][i] of j-block kb for output tile it (zero above the
    // diagonal, and across sequence starts), as a bf16 pair hi + lo: hi alone
    // would round every element to 8 bits, lo carries the next 8
    auto mask = [&](f32x4 g, int kb, int it, float csi, int lsi, frag& lo) {
      const float e = fast_exp(csi - sCs[16 * kb + 15]);
      const f32x4 bj = *reinterpret_cast<const f32x4*>(&sBt[16 * kb + g4]);
      f32x4 mv;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mv[r] = ((kb < it || (kb == it && g4 + r <= l16)) && (!VL || 16 * kb + g4 + r >= lsi))
                    ? e * bj[r] * g[r]
                    : 0.f;
      const frag hi = E::from_f32(mv);
      lo = E::from_f32(mv - E::to_f32(hi));
      return hi;
    };
    // D2 operand: x^T of j-blocks 2 pr and 2 pr + 1
    auto load_x_pair = [&](int pr, frag (&xa)[NTp][2]) {
      const int j0 = 32 * min(pr, W - 1);
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) {
        xa[pt][0] = tr_frag_swz<RX>(sX, 16 * pt, j0, lane);
        xa[pt][1] = tr_frag_swz<RX>(sX, 16 * pt, j0 + 16, lane);
      }
    };
    // y starts as the skip term D x
    const float Dh = a.D ? tk.D : 0.f;
    f32x4 acc[2][NTp];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = (u == 0 ? it0 : it1) * 16 + l16;
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt)
        acc[u][pt] = Dh * E::to_f32(load_frag(sX + swz_off<RX>(i, 16 * pt + g4)));
    }
    // One pass over j-block pairs: the C B^T tiles of the pair for both output
    // tiles, masked, then at once Y^T[p][i] += sum_j x^T[p][j] M[j][i].
    static_assert(W % 2 == 0, "an even wave count is assumed");
#pragma unroll
    for (int pr = 0; pr < W; ++pr) {
      if (2 * pr <= it1) {  // wave-uniform
        const int ka = 2 * pr, kc = 2 * pr + 1;
        bf16x8 bc0[NKn2], bc1[NKn2];
        load_b_rows(ka, bc0);
        load_b_rows(kc, bc1);
        frag xcur[NTp][2];
        load_x_pair(pr, xcur);
        frag l1a, l1b;
        const frag m1a = mask(gram(bc0, cf[1]), ka, it1, csi1, lsi1, l1a);
        const frag m1b = mask(gram(bc1, cf[1]), kc, it1, csi1, lsi1, l1b);
#pragma unroll
        for (int pt = 0; pt < NTp; ++pt) {
          acc[1][pt] = E::mma2(acc[1][pt], xcur[pt][0], xcur[pt][1], m1a, m1b);
          acc[1][pt] = E::mma2(acc[1][pt], xcur[pt][0], xcur[pt][1], l1a, l1b);
        }
        if (ka <= it0) {  // wave-uniform
          frag l0a, l0b;
          const frag m0a = mask(gram(bc0, cf[0]), ka, it0, csi0, lsi0, l0a);
          const frag m0b = mask(gram(bc1, cf[0]), kc, it0, csi0, lsi0, l0b);
#pragma unroll
          for (int pt = 0; pt < NTp; ++pt) {
            acc[0][pt] = E::mma2(acc[0][pt], xcur[pt][0], xcur[pt][1], m0a, m0b);
            acc[0][pt] = E::mma2(acc[0][pt], xcur[pt][0], xcur[pt][1], l0a, l0b);
          }
        }
      }
    }

    // ---------------------------------------------------------------- wait
    // take the next ticket; wait until every wave of chunk c - 1 of this
    // (row, head) has published the state entering chunk c
    // the hand-off placement (a.late) of this instance
    // A wait that gives up sets the error word and makes the incoming state NaN
    // (gave_up below), so that every output that depends on it is NaN rather
    // than silently wrong.
    constexpr bool late = MODE != 0, tagged = MODE == 2;
    bool gave_up = false;  // wave-uniform
    if (wave == 0) {
      if (lane == 0) sTicket = atomicAdd(a.counter, 1u);
      unsigned gave = 0;
      if (c > 0 && !late) {
        const unsigned* fl = a.flags + (stream * 2 + ((c - 1) & 1)) * kFlagWaves + (lane % W);
        unsigned spins = 0;
        while (!__all(__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)c)) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > a.spin_limit) {
            if (lane == 0) atomicOr(a.error, 1u);
            gave = 1;
            break;
          }
        }
      }
      if (lane == 0) sGaveUp = gave;
    }
    lds_barrier();  // also: every wave is done reading sX
    const unsigned t_next = sTicket;
    if (!late) gave_up = sGaveUp != 0u;

    // ---------------------------------------------------------------- chunk states
    // the incoming state (ring slot of chunk c - 1; for c = 0 the slot holds
    // the initial state when one is given) is in flight while
    // S_c[n][p] = sum_j B[j][n] w_j x[j][p] is formed
    const float* src = a.slots + (stream * 2 + ((c - 1) & 1)) * (2 * NP);
    f32x4 sin[TPW];
    auto load_incoming = [&]() {
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        int nt, pt;
        state_tile(k, nt, pt);
        sin[k] = ring_load(src + 256 * (nt * NTp + pt), lane);
      }
    };
    if (!late) load_incoming();
    const Unit nx = unit_of(min(t_next, (unsigned)a.nunits - 1u), sh, Q);
    int4 ci_nx = ci;
    if constexpr (VL) ci_nx = a.cinfo[nx.c];
    // sX is free: the next unit's x goes in while the chunk states are formed
    // (with packed sequences only after the final-state passes below, which
    // read this unit's x)
    if constexpr (!VL) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int m = 0; m < NTp; ++m) dma_x(nx, m);
      asm volatile("" ::: "memory");
    }
    // sum_j B[j][n] w_j x[j][p] for this wave's state tiles, w_j from the
    // scaled copy of x in sXw
    auto state_product = [&](f32x4 (&o)[TPW]) {
#pragma unroll
      for (int k = 0; k < TPW; ++k) o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int kb = 0; kb < NI; kb += 2) {
        if constexpr (F::kBlock) {
          frag xw[SP][2], bb[SN][2];
#pragma unroll
          for (int sp = 0; sp < SP; ++sp) {
            xw[sp][0] = tr_frag<LDX>(sXw, 16 * (pt0 + sp), 16 * kb, lane);
            xw[sp][1] = tr_frag<LDX>(sXw, 16 * (pt0 + sp), 16 * kb + 16, lane);
          }
#pragma unroll
          for (int sn = 0; sn < SN; ++sn) {
            bb[sn][0] = tr_frag_swz<RB>(sB, 16 * (nt0 + sn), 16 * kb, lane);
            bb[sn][1] = tr_frag_swz<RB>(sB, 16 * (nt0 + sn), 16 * kb + 16, lane);
          }
#pragma unroll
          for (int sn = 0; sn < SN; ++sn)
#pragma unroll
            for (int sp = 0; sp < SP; ++sp)
              o[sn * SP + sp] = E::mma2(o[sn * SP + sp], bb[sn][0], bb[sn][1], xw[sp][0], xw[sp][1]);
        } else {
#pragma unroll
          for (int k = 0; k < TPW; ++k) {
            int nt, pt;
            state_tile(k, nt, pt);
            const frag x0 = tr_frag<LDX>(sXw, 16 * pt, 16 * kb, lane);
            const frag x1 = tr_frag<LDX>(sXw, 16 * pt, 16 * kb + 16, lane);
            o[k] = E::mma2(o[k], tr_frag_swz<RB>(sB, 16 * nt, 16 * kb, lane),
                           tr_frag_swz<RB>(sB, 16 * nt, 16 * kb + 16, lane), x0, x1);
          }
        }
      }
    };
    f32x4 sc[TPW];
    state_product(sc);
    if (tagged) {
      // This wave's tiles of the incoming state, tagged c by its counterpart
      // wave of chunk c - 1 (for c = 0: the initial state, tagged 0 by the
      // preparation kernel), polled until every tag matches.  Every chunk
      // after the first of a stream waits, also one that starts a sequence and
      // ignores the values (it polls only the last word its counterpart
      // stores): that keeps a chunk from rewriting a ring slot before the
      // chunk in between has read it.
      const bool need = VL ? c > 0 : (c > 0 || a.init != nullptr);
      const bool use = !VL || !fresh;
      if (need) {
        constexpr int NTW = F::kBlock ? 0 : NT;  // last slot holding one of this wave's own tiles
        const int k_last = F::kBlock ? TPW - 1 : (wave < NTW ? (NTW - 1 - wave) / W : 0);
        int ntl, ptl;
        state_tile(k_last, ntl, ptl);
        const unsigned long long* last =
            reinterpret_cast<const unsigned long long*>(src + 512 * (ntl * NTp + ptl)) + 192;
        unsigned spins = 0;
        for (;;) {
          bool ok = true;
          if (use) {
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
              int nt, pt;
              state_tile(k, nt, pt);
              ok = ring_load_tagged(src + 512 * (nt * NTp + pt), lane, (unsigned)c, sin[k]) && ok;
            }
          } else {
            const unsigned long long w = __hip_atomic_load(last, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = (unsigned)(w >> 32) == (unsigned)c;
          }
          if (__all(ok)) break;
          __builtin_amdgcn_s_sleep(1);
          if (++spins > a.spin_limit) {
            if (lane == 0) atomicOr(a.error, 1u);
            if (use) {
              const float nan = __builtin_nanf("");
#pragma unroll
              for (int k = 0; k < TPW; ++k) sin[k] = f32x4{nan, nan, nan, nan};
            }
            break;
          }
        }
      }
    } else if (late) {
      // this wave's tiles of the incoming state come from its counterpart
      // wave of chunk c - 1
      if (c > 0) {
        const unsigned* fl = a.flags + (stream * 2 + ((c - 1) & 1)) * kFlagWaves + wave;
        unsigned spins = 0;
        while (__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (unsigned)c) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > a.spin_limit) {
            if (lane == 0) atomicOr(a.error, 1u);
            gave_up = true;
            break;
          }
        }
      }
      asm volatile("" ::: "memory");  // the ring loads stay behind the poll
      load_incoming();
    }
    if (gave_up) {
      const float nan = __builtin_nanf("");
#pragma unroll
      for (int k = 0; k < TPW; ++k) sin[k] = f32x4{nan, nan, nan, nan};
    }
    // The incoming state: the ring's, or for the first chunk the initial state
    // (held in the ring slot it reads) or zero.  With packed sequences a
    // sequence that starts at the chunk's first token starts from its own
    // initial state (or zero) instead.
    auto init_tile = [&](int64_t seq, int k) {  // state tile k of sequence seq's initial state
      int nt, pt;
      state_tile(k, nt, pt);
      const float* ip = a.init + (seq * sh.H + un.h) * NP + (int64_t)(16 * nt + g4) * P + 16 * pt + l16;
      return f32x4{ip[0], ip[P], ip[2 * P], ip[3 * P]};
    };
    if constexpr (VL) {
      if (fresh) {
#pragma unroll
        for (int k = 0; k < TPW; ++k)
          sin[k] = a.init ? init_tile(ci.x, k) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    } else {
      const bool have_in = c > 0 || a.init != nullptr;
#pragma unroll
      for (int k = 0; k < TPW; ++k) sin[k] = have_in ? sin[k] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // this wave's tile k of a final state goes to the caller (row-major N x P)
    auto store_final = [&](int64_t row, int k, f32x4 v) {
      int nt, pt;
      state_tile(k, nt, pt);
      float* o = a.final_states + row * NP + (int64_t)(16 * nt + g4) * P + 16 * pt + l16;
      o[0] = v[0];
      o[P] = v[1];
      o[2 * P] = v[2];
      o[3 * P] = v[3];
    };
    if constexpr (VL) {
      // Final states of the sequences that end inside this chunk (all but its
      // last): the chunk-state product once more with weights exp(cs_e - cs_j)
      // over the sequence's tokens j <= e, plus what the sequence brought into
      // the chunk decayed to e (the incoming state if it began before the
      // chunk, else its initial state).
      if (a.final_states) {
        for (int sq = ci.x; sq < ci.y; ++sq) {
          const int64_t s0 = a.cu[sq], s1 = a.cu[sq + 1];
          if (s0 == s1) continue;  // empty sequence: set by the preparation kernel
          const int e = (int)(s1 - 1 - t0), lo = (int)max<int64_t>(s0 - t0, 0);
          lds_barrier();  // every wave is done with sWt and sXw
          if (tid < Q)
            sWt[tid] = (tid >= lo && tid <= e) ? fast_exp(sCs[e] - tk.cs) * (scales ? tk.dtp : 1.f) : 0.f;
          lds_barrier();
          scale_x();
          lds_barrier();
          f32x4 fs[TPW];
          state_product(fs);
          const float cse = sCs[e];
#pragma unroll
          for (int k = 0; k < TPW; ++k) {
            if (!state_slot_valid(k)) continue;  // wave-uniform
            f32x4 v = fs[k];
            if (s0 <= t0)
              v += fast_exp(cse) * sin[k];
            else if (a.init)
              v += fast_exp(cse - sCs[lo - 1]) * init_tile(sq, k);
            store_final((int64_t)sq * sh.H + un.h, k, v);
          }
        }
      }
    }
    const float decay = fast_exp(sCs[len - 1]);
    lds_barrier();  // sB and sXw are free: the next unit's B comes in, sXw takes the state

    // ---------------------------------------------------------------- publish
    // S_out = exp(cs_last) S_in + S_c to the ring (and the caller's final state
    // after the last chunk), and the incoming state as two bf16 terms for the
    // state-to-output product
    // (packed sequences: when the chunk's last sequence starts inside it, the
    // incoming state does not pass; that sequence's initial state does, from
    // its start)
    {
      f32x4 sout[TPW];
      const bool starts_inside = VL && ls_last > 0;
      const float di = starts_inside ? 0.f : decay;
#pragma unroll
      for (int k = 0; k < TPW; ++k) sout[k] = di * sin[k] + sc[k];
      if (starts_inside && a.init) {
        const float dl = fast_exp(sCs[len - 1] - sCs[ls_last - 1]);
#pragma unroll
        for (int k = 0; k < TPW; ++k) sout[k] += dl * init_tile(ci.y, k);
      }
      // the caller's final state when the stream (sequence) ends with the chunk
      const bool ends_here = VL ? (int64_t)a.cu[ci.y + 1] == t0 + len : c + 1 == sh.nc;
      if (ends_here && a.final_states) {
        const int64_t row = VL ? (int64_t)ci.y * sh.H + un.h : stream;
#pragma unroll
        for (int k = 0; k < TPW; ++k)
          if (state_slot_valid(k)) store_final(row, k, sout[k]);  // wave-uniform
      }
      // the ring slot is written after the last chunk too (nobody reads it), so
      // that every wave issues the same stores before its loads into LDS
      float* dst = a.slots + (stream * 2 + (c & 1)) * (2 * NP);
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        if (!state_slot_valid(k)) continue;  // wave-uniform
        int nt, pt;
        state_tile(k, nt, pt);
        if (tagged)
          ring_store_tagged(dst + 512 * (nt * NTp + pt), lane, sout[k], (unsigned)(c + 1));
        else
          ring_store(dst + 256 * (nt * NTp + pt), lane, sout[k]);
        // transposed (p-major) so that the state-to-output product reads 8
        // consecutive n per lane
        const frag hi = E::from_f32(sin[k]);
        bf16* st = sS + (16 * pt + l16) * F::LDS_T + 16 * nt + g4;
        store_frag(st, hi);
        store_frag(st + P * F::LDS_T, E::from_f32(sin[k] - E::to_f32(hi)));
      }
    }
    if (late && !tagged && c + 1 < sh.nc) {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): the ring stores have landed
      if (lane == 0)
        __hip_atomic_store(a.flags + (stream * 2 + (c & 1)) * kFlagWaves + wave, (unsigned)(c + 1),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the next unit's per-token values (the incoming state has arrived: a
    // wait for it does not wait for these)
    tk = load_tokens<VL>(a, nx, Q);
    lds_barrier();

    // ---------------------------------------------------------------- left factors
    // y += exp(cs_i) C_i S_in, one p-tile at a time, while the next unit's B
    // (and with packed sequences its x) go into LDS (sX and sB are free).
    // With packed sequences only the chunk's first sequence sees S_in.
    const float ci0 = (VL && lsi0 > 0) ? 0.f : fast_exp(csi0);
    const float ci1 = (VL && lsi1 > 0) ? 0.f : fast_exp(csi1);
#pragma unroll
    for (int pt = 0; pt < NTp; ++pt) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int m = 0; m < NB; ++m)
        if ((m * NTp) / NB == pt) dma_b(nx, m);
      if constexpr (VL) dma_x(nx, pt);
      asm volatile("" ::: "memory");
      // the hi and lo state terms accumulate in separate chains
      f32x4 tso[2][2] = {};
#pragma unroll
      for (int term = 0; term < 2; ++term)
#pragma unroll
        for (int k2 = 0; k2 < NKn2; ++k2) {
          const bf16* sp = sS + term * P * F::LDS_T + (16 * pt + l16) * F::LDS_T + 32 * k2 + (g8 % N);
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(sp);
          const bf16x8 sv = (N >= 32 || g8 < N) ? v : bf16x8{};
#pragma unroll
          for (int u = 0; u < 2; ++u) tso[u][term] = mma8(tso[u][term], sv, cf[u][k2]);
        }
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[u][pt] += (u == 0 ? ci0 : ci1) * (tso[u][0] + tso[u][1]);
    }
    // Publish: this wave's ring stores were issued before the barrier above
    // and only its loads into LDS after it, so once at most that many memory
    // instructions are in flight the stores have landed; the wave's flag then
    // tells chunk c + 1.  (The state-to-output product above gave them time.)
    if (!late && c + 1 < sh.nc) {
      constexpr int K = NB + (VL ? NTp : 0);
      static_assert(K < 64, "vmcnt field");
      __builtin_amdgcn_s_waitcnt((K & 15) | ((K >> 4) << 14) | (7 << 4) | (15 << 8));
      if (lane == 0)
        __hip_atomic_store(a.flags + (stream * 2 + (c & 1)) * kFlagWaves + wave, (unsigned)(c + 1),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if constexpr (VL) {
      // Sequences that start inside the chunk begin from their own initial
      // state: y_i += exp(cs_i - cs_{start-1}) C_i S_init for their tokens, the
      // state put into sS (as hi/lo terms) one sequence at a time.
      if (a.init) {
        for (int sq = ci.x + 1; sq <= ci.y; ++sq) {
          const int64_t s0 = a.cu[sq], s1 = a.cu[sq + 1];
          if (s0 == s1 || s0 <= t0) continue;
          const int lo = (int)(s0 - t0), hi = (int)min<int64_t>(s1 - t0, len);
          lds_barrier();  // every wave is done reading sS
          const float* ip = a.init + ((int64_t)sq * sh.H + un.h) * NP;
          for (int q = tid; q < NP; q += F::NTHR) {
            const int n = q / P, p = q % P;
            const float v = ip[q];
            const bf16 vh = E::from_float(v);
            sS[p * F::LDS_T + n] = vh;
            sS[(P + p) * F::LDS_T + n] = E::from_float(v - E::to_float(vh));
          }
          lds_barrier();
          const float csp = sCs[lo - 1];
          const int i0 = it0 * 16 + l16, i1 = it1 * 16 + l16;
          const float k0 = (i0 >= lo && i0 < hi) ? fast_exp(csi0 - csp) : 0.f;
          const float k1 = (i1 >= lo && i1 < hi) ? fast_exp(csi1 - csp) : 0.f;
#pragma unroll
          for (int pt = 0; pt < NTp; ++pt) {
            f32x4 tso[2][2] = {};
#pragma unroll
            for (int term = 0; term < 2; ++term)
#pragma unroll
              for (int k2 = 0; k2 < NKn2; ++k2) {
                const bf16* sp = sS + term * P * F::LDS_T + (16 * pt + l16) * F::LDS_T + 32 * k2 + (g8 % N);
                const bf16x8 v = *reinterpret_cast<const bf16x8*>(sp);
                const bf16x8 sv = (N >= 32 || g8 < N) ? v : bf16x8{};
#pragma unroll
                for (int u = 0; u < 2; ++u) tso[u][term] = mma8(tso[u][term], sv, cf[u][k2]);
              }
#pragma unroll
            for (int u = 0; u < 2; ++u) acc[u][pt] += (u == 0 ? k0 : k1) * (tso[u][0] + tso[u][1]);
          }
        }
      }
    }
    // y, then the next unit's C fragments (cf is free now): the y stores
    // leave while the memory pipeline is not yet busy with the C loads, and
    // the C loads still have the next stage to land in.
    // Each 16-row output tile goes through the wave's LDS staging area so
    // that every store instruction writes 8 whole rows (8 lanes x 16 bytes
    // per row); rows past the chunk end go to the sink.
    bf16* const ybase = a.y + (row0 * sh.H + un.h) * P;
    bf16* const stg = sY[wave];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt)
        store_frag(stg + l16 * F::LDY + 16 * pt + g4, E::from_f32(acc[u][pt]));
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's own staging writes
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int r = 8 * m + (lane >> 3), ch = lane & 7;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + r * F::LDY + 8 * ch);
        const int i = (u == 0 ? it0 : it1) * 16 + r;
        bf16* dst = i < len ? reinterpret_cast<bf16*>(reinterpret_cast<char*>(ybase) +
                                                      (unsigned)(i * sh.H * P + 8 * ch) * 2u)
                            : a.sink + 8 * (lane & 7);
        *reinterpret_cast<bf16x8*>(dst) = v;
      }
      // the staging area is rewritten for the next tile only after these reads
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    load_c_tiles<N, P, Q>(a, nx, it0, it1, cf);
    lds_barrier();  // sXw (the state) is rewritten by the next unit
    t = t_next;
    ci = ci_nx;
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// Per-chunk preprocessing of dt, and the launch's bookkeeping.
//
// grid (nc, batch, ceil(H / 8)), 256 threads.  Each block takes one chunk of
// one batch row for 8 heads: dt' = clamp(softplus(dt + bias)) with loads that
// run along the head axis (contiguous in memory), a transpose through LDS, then
// one wave per head forms the inclusive prefix sums of dt' A over the chunk
// and writes cs and dt' with contiguous stores along the token axis.  Tokens
// past the end of a short chunk get dt' = 0.
//
// The grid also clears the ticket counter, the error word and the hand-off
// flags, and writes each stream's initial state (row-major N x P) into ring
// slot 1 in the ring tile layout, where chunk 0 reads its incoming state.
// For a launch with tagged hand-offs it rewrites every ring word instead:
// slot 1 with the initial state (or zero) tagged 0, slot 0 with a tag that no
// chunk waits for, so that nothing left by an earlier call can pass for a
// state of this one.
constexpr int kPrepHeads = 8;

template <int Q, bool VL>
__global__ __launch_bounds__(256) void k_fused_prep(const bf16* __restrict__ dt,
                                                    const float* __restrict__ A,
                                                    const float* __restrict__ dt_bias, Shape sh,
                                                    float* __restrict__ cs_out,
                                                    float* __restrict__ dt_out,
                                                    int32_t* __restrict__ ls_out,
                                                    int4* __restrict__ cinfo_out, FusedArgs fa,
                                                    int64_t nflags, int N, int P) {
  constexpr int TPL = Q / 64;
  __shared__ float sD[kPrepHeads][Q + 1];
  __shared__ float sA[kPrepHeads];
  const int c = blockIdx.x, b = blockIdx.y, h0 = blockIdx.z * kPrepHeads;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: branches on it are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)c * Q;
  const int len = (int)min<int64_t>(Q, sh.L - t0);
  const int64_t row0 = (int64_t)b * sh.L + t0;
  // blocks past the last chunk only help with the bookkeeping below
  if (c < sh.nc) {
    if (VL && blockIdx.z == 0 && tid < Q) {
      // packed sequences: where each token's sequence starts in the chunk, and
      // the chunk's first and last sequence with their first tokens
      auto seq_of = [&](int64_t t) {  // the non-empty sequence holding token t
        int lo = 0, hi = sh.nseqs;    // cu[lo] <= t < cu[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (fa.cu[mid] <= t) lo = mid; else hi = mid;
        }
        return lo;
      };
      const int sq = seq_of(t0 + min(tid, len - 1));
      ls_out[t0 + tid] = (int)max<int64_t>(fa.cu[sq] - t0, 0);
      if (tid == 0) {
        const int sl = seq_of(t0 + len - 1);
        cinfo_out[c] = int4{sq, sl, fa.cu[sq], fa.cu[sl]};
      }
    }
    {
      constexpr int RPT = Q / (256 / kPrepHeads);  // tokens per thread
      const int hl = tid % kPrepHeads, h = min(h0 + hl, sh.H - 1), i0 = tid / kPrepHeads;
      const float bias = dt_bias ? dt_bias[h] : 0.f;
      if (tid < kPrepHeads) sA[hl] = A[h];
      bf16 raw[RPT];
#pragma unroll
      for (int k = 0; k < RPT; ++k)  // every load in flight before any use
        raw[k] = dt[(row0 + min(i0 + k * (256 / kPrepHeads), len - 1)) * sh.H + h];
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int i = i0 + k * (256 / kPrepHeads);
        float dv = (float)raw[k] + bias;
        if (sh.flags & kFlagSoftplus) dv = softplus_f32(dv);
        sD[hl][i] = i < len ? fminf(fmaxf(dv, sh.dt_min), sh.dt_max) : 0.f;
      }
    }
    __syncthreads();
    for (int hl = wave; hl < kPrepHeads && h0 + hl < sh.H; hl += 4) {
      const int h = h0 + hl;
      const float Ah = sA[hl];
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
      const int64_t base = (((int64_t)b * sh.H + h) * sh.nc + c) * Q + lane * TPL;
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        cs_out[base + k] = v[k] + excl;
        dt_out[base + k] = d[k];
      }
    }
  }

  // bookkeeping, grid-strided over every thread of the launch
  const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * gridDim.z * blockDim.x;
  const int64_t gid =
      (((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x + tid;
  if (gid == 0) {
    *fa.counter = 0u;
    *fa.error = 0u;
  }
  for (int64_t i = gid; i < nflags; i += nthreads) fa.flags[i] = 0u;
  if (VL && fa.final_states) {
    // empty packed sequences: the final state is the initial state (or zero)
    const int64_t NP = (int64_t)N * P, per = sh.H * NP / 4;
    for (int64_t i = gid; i < (int64_t)sh.nseqs * per; i += nthreads) {
      const int64_t sq = i / per;
      if (fa.cu[sq] != fa.cu[sq + 1]) continue;
      const float4 v = fa.init ? reinterpret_cast<const float4*>(fa.init)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      reinterpret_cast<float4*>(fa.final_states)[i] = v;
    }
  }
  if (fa.late == 2) {
    const int64_t NP = (int64_t)N * P;
    const int64_t total = (int64_t)sh.batch * sh.H * 2 * NP;  // 64-bit words
    const int NTp = P / 16;
    unsigned long long* ring = reinterpret_cast<unsigned long long*>(fa.slots);
    for (int64_t i = gid; i < total; i += nthreads) {
      const int64_t s = i / (2 * NP);
      const int slot = (int)((i / NP) & 1);
      const int w = (int)(i % NP), tile = w >> 8, r = (w >> 6) & 3, l = w & 63;
      unsigned long long word = 0xFFFFFFFFull << 32;
      if (slot == 1 && !VL) {
        const int n = 16 * (tile / NTp) + 4 * (l >> 4) + r, p = 16 * (tile % NTp) + (l & 15);
        const float v = fa.init ? fa.init[s * NP + (int64_t)n * P + p] : 0.f;
        word = __builtin_bit_cast(unsigned, v);
      }
      ring[i] = word;
    }
  } else if (fa.init && !VL) {
    const int64_t NP = (int64_t)N * P, nq = NP / 4;
    const int64_t total = (int64_t)sh.batch * sh.H * nq;
    const int NTp = P / 16;
    for (int64_t i = gid; i < total; i += nthreads) {
      const int64_t s = i / nq;
      const int q = (int)(i % nq), tile = q >> 6, ql = q & 63;
      const int n = 16 * (tile / NTp) + 4 * (ql >> 4), p = 16 * (tile % NTp) + (ql & 15);
      const float* src = fa.init + s * NP + (int64_t)n * P + p;
      float* tile_dst = fa.slots + (s * 2 + 1) * (2 * NP) + 256 * (int64_t)tile;
      *reinterpret_cast<float2*>(tile_dst + 2 * ql) = make_float2(src[0], src[P]);
      *reinterpret_cast<float2*>(tile_dst + 128 + 2 * ql) = make_float2(src[2 * P], src[3 * P]);
    }
  }
}

// Workspace: counter, error word and a 128-byte store sink (256 B), the
// hand-off flags, the hand-off ring, the per-chunk prefix sums and dt', and
// for packed sequences the per-token sequence starts and per-chunk sequence
// info.
struct FusedLayout {
  size_t flags, slots, cs, dtp, ls, cinfo, total;
  int64_t nflags;
};

static FusedLayout fused_layout(int64_t batch, int64_t H, int64_t nc, int Q, int N, int P) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  FusedLayout l;
  l.nflags = batch * H * 2 * kFlagWaves;
  l.flags = 256;
  l.slots = l.flags + al((size_t)l.nflags * sizeof(unsigned));
  l.cs = l.slots + al((size_t)batch * H * 2 * 2 * N * P * sizeof(float));
  const size_t per = (size_t)batch * H * nc * Q * sizeof(float);
  l.dtp = l.cs + al(per);
  l.ls = l.dtp + al(per);
  l.cinfo = l.ls + al((size_t)nc * Q * sizeof(int32_t));
  l.total = l.cinfo + al((size_t)nc * sizeof(int4));
  return l;
}

template <bool VL>
static hipError_t launch_prep(const ChunkedArgs& ca, const FusedArgs& fa, const FusedLayout& l,
                              char* base, int N, int P, int Q, hipStream_t st);

template <int N, int P, int Q, bool VL>
static hipError_t launch_fused_t(const FusedArgs& fa, int ncu, const ChunkedArgs& ca,
                                 const FusedLayout& l, char* base, hipStream_t st) {
  using F = FusedCfg<N, P, Q>;
  // persistent workgroups: as many as fit on the chip at once
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_fused<N, P, Q, VL, 0>, F::NTHR, 0) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int grid = min(fa.nunits, ncu * per_cu);
  // With fewer streams than half the workgroups, consecutive chunks of a
  // stream are in flight together and the hand-off chain bounds the run.
  // With at most a quarter, long streams (16 chunks or more) and a small state
  // (N <= 64), the tagged ring's shorter hand-off pays for its doubled bytes
  // and for rewriting the ring before the launch; at N = 128 the polls of the
  // waiting consumers' whole tiles cost more than the shorter hand-off gains.
  FusedArgs f = fa;
  const int64_t streams = (int64_t)ca.sh.batch * ca.sh.H;
  const bool tagged = streams * 4 <= grid && ca.sh.nc >= 16 && N <= 64;
  f.late = tagged ? 2 : streams * 2 < grid ? 1 : 0;
  // SSD_FUSED_HANDOFF=0|1|2 forces a placement (every one is correct for any
  // shape; tests use it to cover all three at small sizes)
  if (const char* e = std::getenv("SSD_FUSED_HANDOFF"))
    if (e[0] >= '0' && e[0] <= '2' && e[1] == '\0') f.late = e[0] - '0';
  if (mark(ca, "fused_prep", st) != hipSuccess) return hipErrorUnknown;
  const hipError_t e = launch_prep<VL>(ca, f, l, base, N, P, Q, st);
  if (e != hipSuccess) return e;
  if (mark(ca, "fused", st) != hipSuccess) return hipErrorUnknown;
  if (f.late == 2)
    hipLaunchKernelGGL((k_fused<N, P, Q, VL, 2>), dim3(grid), dim3(F::NTHR), 0, st, f);
  else if (f.late == 1)
    hipLaunchKernelGGL((k_fused<N, P, Q, VL, 1>), dim3(grid), dim3(F::NTHR), 0, st, f);
  else
    hipLaunchKernelGGL((k_fused<N, P, Q, VL, 0>), dim3(grid), dim3(F::NTHR), 0, st, f);
  return hipGetLastError();
}


bool fused_supported(int N, int P, int Q, bool bf16_storage, bool /*varlen*/) {
  return bf16_storage && P == 64 && (N == 16 || N == 32 || N == 64 || N == 128) &&
         (Q == 64 || Q == 128 || Q == 256);
}

hipError_t fused_handoff_failed(const void* ws, hipStream_t st, bool* failed) {
  unsigned word = 0;
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess)
    e = hipMemcpy(&word, static_cast<const unsigned*>(ws) + 1, sizeof(word), hipMemcpyDeviceToHost);
  *failed = word != 0;
  return e;
}

size_t fused_workspace_bytes(int64_t batch, int64_t H, int64_t nc, int Q, int N, int P) {
  return fused_layout(batch, H, nc, Q, N, P).total;
}

template <bool VL>
static hipError_t launch_prep(const ChunkedArgs& ca, const FusedArgs& fa, const FusedLayout& l,
                              char* base, int N, int P, int Q, hipStream_t st) {
  const Shape& sh = ca.sh;
  if (sh.nc == 0) return hipSuccess;
  const int64_t gz = (sh.H + kPrepHeads - 1) / kPrepHeads;
  int64_t gx = sh.nc;
  if (fa.late == 2) {  // enough blocks that each thread rewrites at most 16 ring words
    const int64_t words = (int64_t)sh.batch * sh.H * 2 * N * P;
    const int64_t blocks = (words + 256 * 16 - 1) / (256 * 16);
    const int64_t need = (blocks + sh.batch * gz - 1) / (sh.batch * gz);
    if (need > gx) gx = need;
  }
  const dim3 pgrid((unsigned)gx, (unsigned)sh.batch, (unsigned)gz);
  float* cs = reinterpret_cast<float*>(base + l.cs);
  float* dtp = reinterpret_cast<float*>(base + l.dtp);
  int32_t* ls = reinterpret_cast<int32_t*>(base + l.ls);
  int4* cinfo = reinterpret_cast<int4*>(base + l.cinfo);
  const bf16* dt = static_cast<const bf16*>(ca.dt);
  switch (Q) {
    case 64:
      hipLaunchKernelGGL((k_fused_prep<64, VL>), pgrid, dim3(256), 0, st, dt, ca.A, ca.dt_bias, sh, cs, dtp, ls, cinfo, fa, l.nflags, N, P);
      break;
    case 128:
      hipLaunchKernelGGL((k_fused_prep<128, VL>), pgrid, dim3(256), 0, st, dt, ca.A, ca.dt_bias, sh, cs, dtp, ls, cinfo, fa, l.nflags, N, P);
      break;
    case 256:
      hipLaunchKernelGGL((k_fused_prep<256, VL>), pgrid, dim3(256), 0, st, dt, ca.A, ca.dt_bias, sh, cs, dtp, ls, cinfo, fa, l.nflags, N, P);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int N, bool VL>
static hipError_t fused_q(const FusedArgs& fa, int Q, int ncu, const ChunkedArgs& ca,
                          const FusedLayout& l, char* base, hipStream_t st) {
  switch (Q) {
    case 64: return launch_fused_t<N, 64, 64, VL>(fa, ncu, ca, l, base, st);
    case 128: return launch_fused_t<N, 64, 128, VL>(fa, ncu, ca, l, base, st);
    case 256: return launch_fused_t<N, 64, 256, VL>(fa, ncu, ca, l, base, st);
  }
  return hipErrorInvalidValue;
}

template <bool VL>
static hipError_t fused_n(const FusedArgs& fa, int N, int Q, int ncu, const ChunkedArgs& ca,
                          const FusedLayout& l, char* base, hipStream_t st) {
  switch (N) {
    case 16: return fused_q<16, VL>(fa, Q, ncu, ca, l, base, st);
    case 32: return fused_q<32, VL>(fa, Q, ncu, ca, l, base, st);
    case 64: return fused_q<64, VL>(fa, Q, ncu, ca, l, base, st);
    case 128: return fused_q<128, VL>(fa, Q, ncu, ca, l, base, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fused(const ChunkedArgs& ca, void* ws, int N, int P, int Q, hipStream_t st) {
  const Shape& sh = ca.sh;
  if (sh.nc == 0 || sh.batch == 0) return hipSuccess;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorUnknown;
  const FusedLayout l = fused_layout(sh.batch, sh.H, sh.nc, Q, N, P);
  char* base = static_cast<char*>(ws);
  const bool vl = sh.varlen != 0;
  FusedArgs fa;
  fa.sh = sh;
  fa.x = static_cast<const bf16*>(ca.x);
  fa.A = ca.A;
  fa.B = static_cast<const bf16*>(ca.B);
  fa.C = static_cast<const bf16*>(ca.C);
  fa.D = ca.D;
  fa.cs = reinterpret_cast<const float*>(base + l.cs);
  fa.dtp = reinterpret_cast<const float*>(base + l.dtp);
  fa.init = ca.init;
  fa.y = static_cast<bf16*>(ca.y);
  fa.final_states = ca.final_states;
  fa.counter = reinterpret_cast<unsigned*>(base);
  fa.error = reinterpret_cast<unsigned*>(base) + 1;
  fa.sink = reinterpret_cast<bf16*>(base + 128);
  fa.flags = reinterpret_cast<unsigned*>(base + l.flags);
  fa.slots = reinterpret_cast<float*>(base + l.slots);
  fa.cu = vl ? ca.cu : nullptr;
  fa.ls = reinterpret_cast<const int32_t*>(base + l.ls);
  fa.cinfo = reinterpret_cast<const int4*>(base + l.cinfo);
  fa.nunits = sh.nc * sh.batch * sh.H;
  fa.late = 0;
  // SSD_SPIN_LIMIT lowers the bound of the hand-off waits (tests use it to
  // make waits give up and check that the failure is reported)
  fa.spin_limit = kSpinLimit;
  if (const char* e = std::getenv("SSD_SPIN_LIMIT")) fa.spin_limit = (unsigned)std::strtoul(e, nullptr, 10);
  return vl ? fused_n<true>(fa, N, Q, ncu, ca, l, base, st)
            : fused_n<false>(fa, N, Q, ncu, ca, l, base, st);
}

}  // namespace ssd
