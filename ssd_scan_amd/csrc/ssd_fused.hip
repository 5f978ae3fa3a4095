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
// Work unit = (batch row, chunk, NH heads of one B/C group).  Units are taken
// from an atomic ticket in chunk-major order by persistent workgroups (one per
// CU), so a unit only ever waits on a lower ticket that a running workgroup
// holds: the chain always makes progress.  Hand-off slots are a 2-deep ring per
// (row, head), small enough to live in L2 / the 256 MB MALL; they are written
// and read with relaxed agent-scope atomics (coherent across XCDs without
// cache flushes) and published with a per-slot flag holding chunk index + 1.
//
// Inside a unit (8 waves for Q = 256), wave w owns the 16-token output tiles
// {w, Q/16 - 1 - w} (equal causal work per wave).  B and x chunks are staged
// row-major in LDS; operands that contract over tokens are read with the
// gfx950 transposing LDS load (ds_read_b64_tr_b16).  C B^T tiles are computed
// once and used for all NH heads.  The decay mask L[j,i] = exp(cs_i - cs_j) is
// applied as exp(cs_i - r) * exp(r - cs_j) with r the prefix sum at the end of
// j's 16-token block: one exp per lane per tile plus a per-token table, all
// factors bounded by 1 off the diagonal block.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Operand fragment of M[r][k] = T[k][r], T row-major in LDS with leading
// dimension ld: lane (g = lane / 16, i = lane % 16) receives
// M[r0 + i][k0 + 4g .. 4g + 3].  Within each 16-lane group the transposing load
// hands lane i element (i % 4) of source lanes {i/4, 4 + i/4, 8 + i/4, 12 + i/4};
// source lane 4s + q therefore points at row k0 + 4g + s, columns r0 + 4q.
__device__ inline bf16x4 tr_frag(const bf16* T, int ld, int r0, int k0, int lane) {
  const int g = lane >> 4, s = (lane >> 2) & 3, q = lane & 3;
  const bf16* p = T + (k0 + 4 * g + s) * ld + r0 + 4 * q;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ inline f32x4 atomic_load_f32x4(const float* p) {
  const unsigned long long* q = reinterpret_cast<const unsigned long long*>(p);
  const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float2 fa = __builtin_bit_cast(float2, a), fb = __builtin_bit_cast(float2, b);
  return f32x4{fa.x, fa.y, fb.x, fb.y};
}

__device__ inline void atomic_store_f32x4(float* p, f32x4 v) {
  unsigned long long* q = reinterpret_cast<unsigned long long*>(p);
  __hip_atomic_store(q, __builtin_bit_cast(unsigned long long, float2{v[0], v[1]}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, __builtin_bit_cast(unsigned long long, float2{v[2], v[3]}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int N, int P, int Q, int NH>
struct FusedCfg {
  static constexpr int NI = Q / 16;                       // 16-token tiles
  static constexpr int W = NI / 4;                        // waves; each owns 4 tiles
  static constexpr int NTHR = 64 * W;
  static constexpr int LDB = N + 8, LDX = P + 8;          // LDS row pitches (elements)
  static constexpr int NKn = N / 16, NKn2 = (NKn + 1) / 2;
  static constexpr int NTp = P / 16, NT = (N / 16) * NTp;
  static constexpr int TPW = (NT + W - 1) / W;            // state tiles per wave
  static constexpr int SB_ELEMS = Q * LDB;
  static constexpr int SS_ELEMS = NH * 2 * N * P;         // hi/lo state terms of NH heads
  static constexpr int REGION = SB_ELEMS > SS_ELEMS ? SB_ELEMS : SS_ELEMS;
  static constexpr int SX_ELEMS = Q * LDX;
  static constexpr int BQ = Q * N / 8;                    // 16-byte pieces of a B chunk
  static constexpr int XQ = Q * P / 8;                    // 16-byte pieces of an x chunk
  static constexpr int TPL = Q / 64;                      // tokens per lane in the scans
};

struct FusedArgs {
  Shape sh;
  const bf16* x;
  const bf16* dt;
  const float* A;
  const bf16* B;
  const bf16* C;
  const float* D;
  const float* dt_bias;
  const float* init;
  bf16* y;
  float* final_states;
  unsigned* counter;  // ticket counter (zeroed before the launch)
  unsigned* flags;    // (batch, H, 2) hand-off flags (zeroed before the launch)
  float* slots;       // (batch, H, 2, N*P) fragment-layout hand-off states
  unsigned* error;    // set when a hand-off wait gives up
  int nunits;
  int hgroups;        // H / NH
};

constexpr unsigned kSpinLimit = 1u << 24;

// Unit coordinates of ticket t (chunk-major: every unit of chunk c precedes chunk c + 1).
struct Unit {
  int c, b, h0, grp, len;
  int64_t row0;
};

__device__ inline Unit unit_of(unsigned t, const FusedArgs& a, int Q, int NH) {
  const Shape& sh = a.sh;
  const int per_chunk = sh.batch * a.hgroups;
  Unit u;
  u.c = (int)(t / per_chunk);
  const int rem = (int)(t % per_chunk);
  u.b = rem / a.hgroups;
  u.h0 = (rem % a.hgroups) * NH;
  u.grp = u.h0 / sh.hpg;
  const int64_t tb = (int64_t)u.c * Q;
  u.len = (int)min<int64_t>(Q, sh.L - tb);
  u.row0 = (int64_t)u.b * sh.L + tb;
  return u;
}

// C fragments of the wave's four output tiles (B-operand of C B^T and of C S).
// The base pointer goes through an empty asm statement so that the second load
// of the same fragments (before the state-to-output product) is a real reload
// from L2 rather than registers held live across the chunk-state phase.
template <int N>
__device__ inline void load_c_frags(bf16x4 (&cf)[4][2 * ((N / 16 + 1) / 2)], const bf16* Cbase,
                                    int64_t row0, int G, int grp, const int (&itile)[4], int len,
                                    int lane) {
  constexpr int NKn = N / 16, NKn2 = (NKn + 1) / 2;
  const bf16* base = Cbase;
  asm volatile("" : "+s"(base));
  const int g4 = (lane >> 4) * 4, l16 = lane & 15;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = itile[u] * 16 + l16;
    const bf16* cr = base + ((row0 + i) * G + grp) * N + g4;
#pragma unroll
    for (int kb = 0; kb < 2 * NKn2; ++kb)
      cf[u][kb] = (kb < NKn && i < len) ? load_frag(cr + 16 * kb) : zero_frag<bf16>();
  }
}

template <int N, int P, int Q, int NH>
__global__ __launch_bounds__((FusedCfg<N, P, Q, NH>::NTHR), 1) void k_fused(FusedArgs a) {
  using F = FusedCfg<N, P, Q, NH>;
  using E = Elem<bf16>;
  using frag = bf16x4;
  constexpr int NI = F::NI, W = F::W, NTHR = F::NTHR, LDB = F::LDB, LDX = F::LDX;
  constexpr int NKn = F::NKn, NKn2 = F::NKn2, NTp = F::NTp, NT = F::NT, TPW = F::TPW;
  constexpr int NP = N * P;

  __shared__ __attribute__((aligned(16))) bf16 sR[F::REGION];        // B chunk, then states
  __shared__ __attribute__((aligned(16))) bf16 sX[NH][F::SX_ELEMS];  // x chunks (row-major)
  __shared__ __attribute__((aligned(16))) float sCs[NH][Q];  // inclusive prefix sums of dt' A
  __shared__ __attribute__((aligned(16))) float sBt[NH][Q];  // exp(r_block - cs_j) (x dt'_j if scaled)
  __shared__ __attribute__((aligned(16))) float sWt[NH][Q];  // exp(cs_last - cs_j) (x dt'_j if scaled)
  __shared__ unsigned sTicket;

  const Shape& sh = a.sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = (lane >> 4) * 4, l16 = lane & 15;
  const bool scales = sh.flags & kFlagScalesInput;
  const int itile[4] = {wave, 2 * W - 1 - wave, 2 * W + wave, 4 * W - 1 - wave};  // output tiles
  const int it_max = 4 * W - 1 - wave;

  if (tid == 0) sTicket = atomicAdd(a.counter, 1u);
  __syncthreads();
  unsigned t = sTicket;
  __syncthreads();

  while (t < (unsigned)a.nunits) {
    const Unit un = unit_of(t, a, Q, NH);
    const int c = un.c, b = un.b, h0 = un.h0, grp = un.grp, len = un.len;
    const int64_t row0 = un.row0;

    // ---------------------------------------------------------------- stage
    // B chunk and the NH x chunks, row-major, rows past the end zero
    for (int qd = tid; qd < F::BQ; qd += NTHR) {
      const int r = qd / (N / 8), c8 = qd % (N / 8);
      uint4 v = {0u, 0u, 0u, 0u};
      if (r < len) v = *reinterpret_cast<const uint4*>(a.B + ((row0 + r) * sh.G + grp) * N + 8 * c8);
      *reinterpret_cast<uint4*>(sR + r * LDB + 8 * c8) = v;
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
      for (int qd = tid; qd < F::XQ; qd += NTHR) {
        const int r = qd / (P / 8), c8 = qd % (P / 8);
        uint4 v = {0u, 0u, 0u, 0u};
        if (r < len)
          v = *reinterpret_cast<const uint4*>(a.x + ((row0 + r) * sh.H + h0 + hh) * P + 8 * c8);
        *reinterpret_cast<uint4*>(&sX[hh][r * LDX + 8 * c8]) = v;
      }
    // prefix sums of dt' A for each head (wave hh handles head h0 + hh)
    for (int hh = wave; hh < NH; hh += W) {
      const int h = h0 + hh;
      const float Ah = a.A[h];
      const float bias = a.dt_bias ? a.dt_bias[h] : 0.f;
      float d[F::TPL], v[F::TPL];
      float run = 0.f;
#pragma unroll
      for (int k = 0; k < F::TPL; ++k) {
        const int i = lane * F::TPL + k;
        float dv = 0.f;
        if (i < len) {
          dv = (float)a.dt[(row0 + i) * sh.H + h] + bias;
          if (sh.flags & kFlagSoftplus) dv = softplus_f32(dv);
          dv = fminf(fmaxf(dv, sh.dt_min), sh.dt_max);
        }
        d[k] = dv;
        run += dv * Ah;
        v[k] = run;
      }
      float incl = run;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      const float excl = incl - run;
#pragma unroll
      for (int k = 0; k < F::TPL; ++k) sCs[hh][lane * F::TPL + k] = v[k] + excl;
      // the tables read other lanes' prefix sums: wave-local LDS round trip
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      const float cs_last = sCs[hh][len - 1];
#pragma unroll
      for (int k = 0; k < F::TPL; ++k) {
        const int i = lane * F::TPL + k;
        const float csi = sCs[hh][i];
        const float sc = scales ? d[k] : 1.f;
        sBt[hh][i] = fast_exp(sCs[hh][i | 15] - csi) * sc;
        sWt[hh][i] = fast_exp(cs_last - csi) * sc;
      }
    }
    frag cf[4][2 * NKn2];
    load_c_frags<N>(cf, a.C, row0, sh.G, grp, itile, len, lane);
    __syncthreads();

    // ---------------------------------------------------------------- diagonal blocks
    f32x4 acc[NH][4][NTp];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int pt = 0; pt < NTp; ++pt) acc[hh][u][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kb0 = 0; kb0 <= it_max; kb0 += 2) {
      // A-operand (B rows) of the two j-blocks, shared by the wave's output tiles
      frag ba[2][2 * NKn2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bf16* br = sR + (16 * (kb0 + e) + l16) * LDB + g4;
#pragma unroll
        for (int kk = 0; kk < 2 * NKn2; ++kk)
          ba[e][kk] = (kk < NKn) ? load_frag(br + 16 * kk) : zero_frag<bf16>();
      }
      // x^T fragments of the two j-blocks for every head and p-tile
      frag xa[NH][NTp][2];
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int pt = 0; pt < NTp; ++pt) {
          xa[hh][pt][0] = tr_frag(sX[hh], LDX, 16 * pt, 16 * kb0, lane);
          xa[hh][pt][1] = tr_frag(sX[hh], LDX, 16 * pt, 16 * kb0 + 16, lane);
        }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int it = itile[u];
        if (kb0 > it) continue;
        const int i = it * 16 + l16;
        f32x4 gt[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          gt[e] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (kb0 + e <= it) {
#pragma unroll
            for (int k2 = 0; k2 < NKn2; ++k2)
              gt[e] = E::mma2(gt[e], ba[e][2 * k2], ba[e][2 * k2 + 1], cf[u][2 * k2],
                              cf[u][2 * k2 + 1]);
          }
        }
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          frag m[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int kb = kb0 + e;
            if (kb > it) {
              m[e] = zero_frag<bf16>();
              continue;
            }
            const float ei = fast_exp(sCs[hh][i] - sCs[hh][16 * kb + 15]);
            const f32x4 bj = *reinterpret_cast<const f32x4*>(&sBt[hh][16 * kb + g4]);
            f32x4 mv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 16 * kb + g4 + r;
              mv[r] = (kb < it || j <= i) ? ei * bj[r] * gt[e][r] : 0.f;
            }
            m[e] = E::from_f32(mv);
          }
#pragma unroll
          for (int pt = 0; pt < NTp; ++pt)
            acc[hh][u][pt] = E::mma2(acc[hh][u][pt], xa[hh][pt][0], xa[hh][pt][1], m[0], m[1]);
        }
      }
    }

    // ---------------------------------------------------------------- chunk states
    // S_c[n][p] = sum_j B[j][n] w_j x[j][p]; the wave owns tiles wave + W k
    f32x4 sc[NH][TPW];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int k = 0; k < TPW; ++k) sc[hh][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < NI; kb += 2) {
      f32x4 w[NH][2];
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        w[hh][0] = *reinterpret_cast<const f32x4*>(&sWt[hh][16 * kb + g4]);
        w[hh][1] = *reinterpret_cast<const f32x4*>(&sWt[hh][16 * kb + 16 + g4]);
      }
      // tile wave + W k has p-tile (wave + W k) % NTp: the same for every k exactly
      // when W is a multiple of NTp, otherwise it changes from one tile to the next
      constexpr bool kOnePt = (W % NTp) == 0;
      frag xw[NH][2];
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int tt = wave + W * k;
        if (tt < NT) {
          const int nt = tt / NTp, pt = tt % NTp;
          if (!kOnePt || k == 0) {
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
              xw[hh][0] =
                  E::from_f32(E::to_f32(tr_frag(sX[hh], LDX, 16 * pt, 16 * kb, lane)) * w[hh][0]);
              xw[hh][1] = E::from_f32(
                  E::to_f32(tr_frag(sX[hh], LDX, 16 * pt, 16 * kb + 16, lane)) * w[hh][1]);
            }
          }
          const frag b0 = tr_frag(sR, LDB, 16 * nt, 16 * kb, lane);
          const frag b1 = tr_frag(sR, LDB, 16 * nt, 16 * kb + 16, lane);
#pragma unroll
          for (int hh = 0; hh < NH; ++hh)
            sc[hh][k] = E::mma2(sc[hh][k], b0, b1, xw[hh][0], xw[hh][1]);
        }
      }
    }
    __syncthreads();  // B no longer needed: the region now holds the incoming states

    // ---------------------------------------------------------------- hand-off
    // One critical section for all NH heads: wait for chunk c - 1 of every head,
    // publish chunk c of every head, then set the flags.
    if (tid == 0) {
      sTicket = atomicAdd(a.counter, 1u);
      if (c > 0) {
        unsigned spins = 0;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          unsigned* fl = a.flags + ((int64_t)b * sh.H + h0 + hh) * 2 + ((c - 1) & 1);
          while (__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (unsigned)c) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
              atomicOr(a.error, 1u);
              break;
            }
          }
        }
      }
    }
    __syncthreads();
    {
      f32x4 sin[NH][TPW];
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const int64_t stream = (int64_t)b * sh.H + h0 + hh;
        const float* src = a.slots + (stream * 2 + ((c - 1) & 1)) * NP;
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
          const int tt = wave + W * k;
          sin[hh][k] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (tt >= NT) continue;
          if (c > 0) {
            sin[hh][k] = atomic_load_f32x4(src + 4 * (tt * 64 + lane));
          } else if (a.init) {
            const int nt = tt / NTp, pt = tt % NTp;
            const float* ip = a.init + stream * NP + (int64_t)(16 * nt + g4) * P + 16 * pt + l16;
            sin[hh][k] = f32x4{ip[0], ip[P], ip[2 * P], ip[3 * P]};
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const int64_t stream = (int64_t)b * sh.H + h0 + hh;
        const float decay = fast_exp(sCs[hh][len - 1]);
        float* dst = a.slots + (stream * 2 + (c & 1)) * NP;
        bf16* sS = sR + hh * 2 * NP;
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
          const int tt = wave + W * k;
          if (tt >= NT) continue;
          const int q = tt * 64 + lane;  // fragment quad
          const f32x4 sout = decay * sin[hh][k] + sc[hh][k];
          if (c + 1 < sh.nc) {
            atomic_store_f32x4(dst + 4 * q, sout);
          } else if (a.final_states) {
            const int nt = tt / NTp, pt = tt % NTp;
            float* o = a.final_states + stream * NP + (int64_t)(16 * nt + g4) * P + 16 * pt + l16;
            o[0] = sout[0];
            o[P] = sout[1];
            o[2 * P] = sout[2];
            o[3 * P] = sout[3];
          }
          // incoming state as two bf16 terms for the state-to-output product
          const frag hi = E::from_f32(sin[hh][k]);
          store_frag(sS + 4 * q, hi);
          store_frag(sS + NP + 4 * q, E::from_f32(sin[hh][k] - E::to_f32(hi)));
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0 && c + 1 < sh.nc) {
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
        __hip_atomic_store(a.flags + ((int64_t)b * sh.H + h0 + hh) * 2 + (c & 1), (unsigned)(c + 1),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const unsigned t_next = sTicket;

    // ---------------------------------------------------------------- left factors, D, store
    load_c_frags<N>(cf, a.C, row0, sh.G, grp, itile, len, lane);
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const int h = h0 + hh;
      const float Dh = a.D ? a.D[h] : 0.f;
      const bf16* sS = sR + hh * 2 * NP;
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) {
        f32x4 tso[4] = {};
#pragma unroll
        for (int term = 0; term < 2; ++term) {
#pragma unroll
          for (int k2 = 0; k2 < NKn2; ++k2) {
            const frag s0 = load_frag(sS + term * NP + ((2 * k2) * NTp + pt) * 256 + lane * 4);
            const frag s1 = (2 * k2 + 1 < NKn)
                                ? load_frag(sS + term * NP + ((2 * k2 + 1) * NTp + pt) * 256 + lane * 4)
                                : zero_frag<bf16>();
#pragma unroll
            for (int u = 0; u < 4; ++u)
              tso[u] = E::mma2(tso[u], s0, s1, cf[u][2 * k2], cf[u][2 * k2 + 1]);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = itile[u] * 16 + l16;
          if (i < len) {
            const float ci = fast_exp(sCs[hh][i]);
            const f32x4 xv = E::to_f32(load_frag(&sX[hh][i * LDX + 16 * pt + g4]));
            const f32x4 yv = acc[hh][u][pt] + ci * tso[u] + Dh * xv;
            store_frag(a.y + ((row0 + i) * sh.H + h) * P + 16 * pt + g4, E::from_f32(yv));
          }
        }
      }
    }
    __syncthreads();  // LDS is restaged by the next unit
    t = t_next;
  }
}

__global__ void k_fused_reset(unsigned* counter, unsigned* flags, int64_t nflags, unsigned* error) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nflags) flags[i] = 0u;
  if (i == 0) {
    *counter = 0u;
    *error = 0u;
  }
}

template <int N, int P, int Q, int NH>
static hipError_t launch_fused_t(const FusedArgs& fa, int ncu, const ChunkedArgs& ca,
                                 hipStream_t st) {
  using F = FusedCfg<N, P, Q, NH>;
  const int grid = min(fa.nunits, ncu);
  if (mark(ca, "fused", st) != hipSuccess) return hipErrorUnknown;
  hipLaunchKernelGGL((k_fused<N, P, Q, NH>), dim3(grid), dim3(F::NTHR), 0, st, fa);
  return hipGetLastError();
}

template <int N, int Q, int NH>
static hipError_t fused_p(const FusedArgs& fa, int ncu, const ChunkedArgs& ca, hipStream_t st) {
  return launch_fused_t<N, 64, Q, NH>(fa, ncu, ca, st);
}

template <int N, int NH>
static hipError_t fused_q(const FusedArgs& fa, int Q, int ncu, const ChunkedArgs& ca,
                          hipStream_t st) {
  switch (Q) {
    case 64: return fused_p<N, 64, NH>(fa, ncu, ca, st);
    case 128: return fused_p<N, 128, NH>(fa, ncu, ca, st);
    case 256: return fused_p<N, 256, NH>(fa, ncu, ca, st);
  }
  return hipErrorInvalidValue;
}

template <int NH>
static hipError_t fused_n(const FusedArgs& fa, int N, int Q, int ncu, const ChunkedArgs& ca,
                          hipStream_t st) {
  switch (N) {
    case 16: return fused_q<16, NH>(fa, Q, ncu, ca, st);
    case 32: return fused_q<32, NH>(fa, Q, ncu, ca, st);
    case 64: return fused_q<64, NH>(fa, Q, ncu, ca, st);
    case 128: return fused_q<128, NH>(fa, Q, ncu, ca, st);
  }
  return hipErrorInvalidValue;
}

// Heads per work unit: two heads share each C B^T tile where two heads'
// accumulators fit in the register file without spilling (checked from the
// compiler's resource usage of every instance), one head otherwise.
int fused_heads_per_unit(int N, int Q, int heads_per_group) {
  const bool two_fit = Q == 256 || (Q == 128 && N <= 64) || N == 16;
  return (two_fit && heads_per_group % 2 == 0) ? 2 : 1;
}

bool fused_supported(int N, int P, int Q, bool bf16_storage, bool varlen) {
  return bf16_storage && !varlen && P == 64 && (N == 16 || N == 32 || N == 64 || N == 128) &&
         (Q == 64 || Q == 128 || Q == 256);
}

size_t fused_workspace_bytes(int64_t batch, int64_t H, int N, int P) {
  // counter + error word (256 B), flags, then the hand-off ring
  const size_t flags = (size_t)batch * H * 2 * sizeof(unsigned);
  const size_t flags_al = (flags + 255) / 256 * 256;
  return 256 + flags_al + (size_t)batch * H * 2 * N * P * sizeof(float);
}

hipError_t launch_fused(const ChunkedArgs& ca, void* ws, int N, int P, int Q, int heads_per_unit,
                        hipStream_t st) {
  const Shape& sh = ca.sh;
  if (sh.nc == 0 || sh.batch == 0) return hipSuccess;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorUnknown;
  char* base = static_cast<char*>(ws);
  FusedArgs fa;
  fa.sh = sh;
  fa.x = static_cast<const bf16*>(ca.x);
  fa.dt = static_cast<const bf16*>(ca.dt);
  fa.A = ca.A;
  fa.B = static_cast<const bf16*>(ca.B);
  fa.C = static_cast<const bf16*>(ca.C);
  fa.D = ca.D;
  fa.dt_bias = ca.dt_bias;
  fa.init = ca.init;
  fa.y = static_cast<bf16*>(ca.y);
  fa.final_states = ca.final_states;
  fa.counter = reinterpret_cast<unsigned*>(base);
  fa.error = reinterpret_cast<unsigned*>(base) + 1;
  fa.flags = reinterpret_cast<unsigned*>(base + 256);
  const int64_t nflags = (int64_t)sh.batch * sh.H * 2;
  const size_t flags_al = ((size_t)nflags * sizeof(unsigned) + 255) / 256 * 256;
  fa.slots = reinterpret_cast<float*>(base + 256 + flags_al);
  fa.hgroups = sh.H / heads_per_unit;
  fa.nunits = sh.nc * sh.batch * fa.hgroups;
  if (mark(ca, "fused_reset", st) != hipSuccess) return hipErrorUnknown;
  hipLaunchKernelGGL(k_fused_reset, dim3((unsigned)((nflags + 255) / 256)), dim3(256), 0, st,
                     fa.counter, fa.flags, nflags, fa.error);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return heads_per_unit == 2 ? fused_n<2>(fa, N, Q, ncu, ca, st)
                             : fused_n<1>(fa, N, Q, ncu, ca, st);
}

}  // namespace ssd
