// Backward pass (gradients) of the chunked SSD layer for gfx950.
//
// "Transformers are SSMs" section 6 gives the forward pass as a block
// decomposition of the semiseparable matrix; its gradients follow the same
// blocks read in the opposite direction.  With g_t the gradient of the loss
// with respect to the state after token t, the forward's state scan across
// chunks (section 6.3) becomes a reverse scan of adjoints:
//
//   R_c      = sum_{t in c} exp(cs_t) C_t dy_t^T        chunk-local adjoint
//   G_end[c] = exp(cs_end[c+1]) G_end[c+1] + R_{c+1}    adjoint after chunk c
//              (G_end[last] = gradient of the final state)
//
// and inside a chunk (cs the inclusive log-decay prefix sums from its start,
// L[i,j] = exp(cs_i - cs_j) for j <= i, s_j = dt'_j or 1):
//
//   dx_j  = D dy_j + s_j ( sum_{i>=j} L[i,j] (C_i . B_j) dy_i
//                          + exp(cs_end - cs_j) G_end^T B_j )
//   dB_j  = s_j ( sum_{i>=j} L[i,j] (dy_i . x_j) C_i + exp(cs_end - cs_j) G_end x_j )
//   dC_i  = sum_{j<=i} L[i,j] s_j (dy_i . x_j) B_j + exp(cs_i) S_in dy_i
//
// The gradient of the log-decay l_k = dt'_k A of token k collects every
// (output i, input j) pair with j < k <= i, the incoming state counting as an
// input before the chunk and G_end as an output after it:
//
//   dl_k = sum_{i >= k > j} W[i,j]                 W[i,j] = L[i,j] s_j (C_i.B_j)(dy_i.x_j)
//        + sum_{i >= k} dy_i . y_state_i          (incoming state -> outputs)
//        + sum_{j < k} x_j . dxG_j                (inputs -> G_end)
//        + exp(cs_end) <G_end, S_in>              (incoming state -> G_end)
//
// with y_state_i = exp(cs_i) S_in^T C_i and dxG_j = s_j exp(cs_end - cs_j)
// G_end^T B_j.  Every term is formed in fp32 (the pair weights from the C B^T
// and dy x^T tiles the other products need anyway), so no large sums cancel.
// Then ddt'_k = dl_k A + [scaled] x_k . (B_k^T g_k), and the gradient goes
// back through the clamp and the softplus to dt and dt_bias.
//
// Kernels (after the forward's dt prefix sums, chunk states and state scan,
// run on 64-token chunks whatever chunk the forward uses; results do not
// depend on the chunk length):
//
//   k_chunk_state<..., REV>  R_c (in ssd_chunked.hip)
//   k_adjoint_passing        reverse scan of R into G_end, and the
//                            initial-state gradient
//   k_bwd_chunk              one block of heads of a (chunk, row) per
//                            workgroup: dx, dt gradient, dB / dC summed over
//                            the head block, per-chunk dA / dD /
//                            dt_bias partial sums (MFMA on LDS-resident tiles)
//   k_group_sum              dB / dC summed over the head blocks of a group
//   k_head_sums              dA, dD, dt_bias summed over rows and chunks
#include <cstdlib>
#include <type_traits>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"
#include "ssd_lds.hpp"

namespace ssd {

// ------------------------------------------------------------------ reverse scan
// grid (nblk, H, batch), 256 threads; thread q owns fragment quad q of the
// N x P adjoint (4 values: rows n0 .. n0 + 3 of column p).  Walks the chunks
// backwards: stores G_end[c] over R_c, then G <- exp(cs_end[c]) G + R_c.
// G_end[c] is the gradient of the state after chunk c of the chunk's last
// sequence; with packed sequences exp(cs_end[c]) is zero unless one sequence
// spans the whole chunk (the carry decay), and G restarts at zero below a
// chunk that begins a sequence.  No communication between threads: the R_c of
// a batch of chunks are loaded before the previous batch is processed.
__global__ __launch_bounds__(256) void k_adjoint_passing(
    float* __restrict__ adj, const float2* __restrict__ coef, const ChunkInfo* __restrict__ cinfo,
    const float* __restrict__ dfinal, Shape sh, int N, int P, float* __restrict__ dinit) {
  const int NP = N * P, NTp = P / 16;
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q * 4 >= NP) return;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tile = q >> 6, ln = q & 63;
  const int n0 = 16 * (tile / NTp) + 4 * (ln >> 4), p = 16 * (tile % NTp) + (ln & 15);
  const int64_t hb = (int64_t)b * sh.H + h;
  f32x4* aq = reinterpret_cast<f32x4*>(adj + ((int64_t)b * sh.nc * sh.H + h) * NP) + q;
  const int64_t cstride = (int64_t)sh.H * NP / 4;
  const float2* cf = coef + hb * sh.nc;

  f32x4 G = {0.f, 0.f, 0.f, 0.f};
  if (dfinal) {
    const float* e = dfinal + hb * NP + (int64_t)n0 * P + p;
    G = f32x4{e[0], e[P], e[2 * P], e[3 * P]};
  }
  constexpr int BATCH = 8;
  struct Batch {
    f32x4 r[BATCH];
    float k[BATCH];
    int fresh[BATCH];
  };
  // chunks c0, c0 - 1, ..., c0 - BATCH + 1 (clamped at 0)
  auto load = [&](Batch& t, int c0) {
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int c = max(c0 - k, 0);
      t.r[k] = aq[(int64_t)c * cstride];
      t.k[k] = cf[c].x;
      // packed input: nothing flows back across a sequence start at the chunk
      // boundary; a sequence that starts inside chunk c has a zero carry decay
      t.fresh[k] = sh.varlen && cinfo[c].start_first == (int64_t)c * kBwdChunk;
    }
  };
  Batch cur, nxt;
  load(cur, sh.nc - 1);
  for (int c0 = sh.nc - 1; c0 >= 0; c0 -= BATCH) {
    if (c0 - BATCH >= 0) load(nxt, c0 - BATCH);
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int c = c0 - k;
      if (c < 0) break;
      aq[(int64_t)c * cstride] = G;
      G = cur.fresh[k] ? f32x4{0.f, 0.f, 0.f, 0.f} : cur.k[k] * G + cur.r[k];
    }
    cur = nxt;
  }
  if (dinit) {
    float* o = dinit + hb * NP + (int64_t)n0 * P + p;
    o[0] = G[0];
    o[P] = G[1];
    o[2 * P] = G[2];
    o[3 * P] = G[3];
  }
}

// ------------------------------------------------------------------ chunk gradients
// Fragment reads from row-major LDS tiles (see the convention in
// ssd_device.hpp): `row` gives lane l the 4 consecutive k of row r (one vector
// read), `col` gives it 4 consecutive rows k of column c (four reads).
template <typename T>
__device__ inline typename Elem<T>::frag rd_row(const T* a, int ld, int r, int k0) {
  return load_frag(a + r * ld + k0);
}

// rd_col<LD>(a, K, R, lane): lane (g, i) gets a[K + 4g + e][R + i], e = 0..3,
// for tile bases K, R (multiples of 16) of a row-major tile with leading
// dimension LD: the transposing LDS load for bf16 tiles (its preconditions in
// ssd_lds.hpp: LD a multiple of 4, R a multiple of 4, all lanes active), four
// plain LDS reads for fp32 tiles.
template <int LD, typename T>
__device__ inline typename Elem<T>::frag rd_col(const T* a, int K, int R, int lane) {
  if constexpr (std::is_same<T, bf16>::value) {
    return tr_frag<LD>(a, R, K, lane);
  } else {
    const int k0 = K + 4 * (lane >> 4), c = R + (lane & 15);
    typename Elem<T>::frag v;
    v[0] = a[(k0 + 0) * LD + c];
    v[1] = a[(k0 + 1) * LD + c];
    v[2] = a[(k0 + 2) * LD + c];
    v[3] = a[(k0 + 3) * LD + c];
    return v;
  }
}

template <typename T>
__device__ inline float dot4(typename Elem<T>::frag a, f32x4 b) {
  const f32x4 v = Elem<T>::to_f32(a);
  return v[0] * b[0] + v[1] * b[1] + v[2] * b[2] + v[3] * b[3];
}

// sum over the 4 lane groups holding one column of an output tile
__device__ inline float sum_groups(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// A state in LDS is held in the storage type; for bf16 as two terms, S = hi +
// lo with lo = bf16(S - hi), and every state product is done for both terms
// (a single bf16 rounding of G_end or S_in would cost 2^-9 of the state in
// every gradient it reaches, and those are the long-memory terms).
template <typename T>
constexpr int bwd_state_terms() { return sizeof(T) == 2 ? 2 : 1; }

// The state is staged in parts of N / NH rows, one after the other, so that
// the LDS footprint leaves room for two workgroups per CU at N = 128.
template <int N>
constexpr int bwd_state_parts() { return N >= 64 ? 2 : 1; }

// floats of the LDS region of a state part (G_end parts, then S_in parts)
template <typename T, int N, int P>
constexpr int bwd_state_floats() {
  return (bwd_state_terms<T>() * (N / bwd_state_parts<N>()) * (P + 4) * (int)sizeof(T) + 3) / 4;
}

// LDS bytes of one k_bwd_chunk workgroup
template <typename T, int N, int P>
constexpr int bwd_lds_bytes() {
  return (2 * kBwdChunk * (N + 4) + 2 * kBwdChunk * (P + 4)) * (int)sizeof(T) +
         bwd_state_floats<T, N, P>() * 4 + kBwdChunk * (kBwdChunk + 1) / 2 * 4 + 7 * kBwdChunk * 4;
}

// grid (H / hblk, nc, batch), 256 threads = 4 waves, the hblk heads of a
// workgroup one after the other; wave w owns the 16-token tile w
// of the 64-token chunk, as the output rows i of the row-side products (dC:
// sums over j <= i) and as the input columns j of the column-side ones (dx and
// dB: sums over i >= j), which balances the causal work (w + 1 and 4 - w
// tiles, both in one interval between barriers).  B, C, x, dy and a state part
// (G_end's, then S_in's) sit in LDS in the storage type; every product runs on
// the matrix cores with fp32 accumulation; the masked decay is applied to the
// C B^T and dy x^T tiles in registers before they feed the next product.
//
// The decay gradient of token k takes every pair (i, j) with j < k <= i:
//   dl_k = sum_{i >= k, j < k} W[i,j]          W[i,j] = L[i,j] s_j (C_i.B_j)(dy_i.x_j)
//        + sum_{i >= k} dy_i . y_state_i        (incoming state -> outputs)
//        + sum_{j < k} x_j . dxG_j              (inputs -> later chunks)
//        + exp(cs_end) <G_end, S_in>            (incoming state -> later chunks)
// W is formed in fp32 from the C B^T and dy x^T tiles the other products
// already need, kept in a triangular LDS region of its own, and the corner
// sums are two scans over it.
// States and adjoints between the walks and k_bwd_chunk (dense bf16 rows): fp16
// quads in the fragment layout with one power-of-two scale per 16 x 16 tile,
// half the bytes of fp32 (the chunk kernel turns them into two bf16 terms,
// which hold an fp16 value exactly).  Elsewhere fp32 quads.
typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Scale of a tile whose largest magnitude is m: its values times 2^-e are fp16
// with the largest in [2^14, 2^15) (e = 0 for m = 0 or a non-finite m).
__device__ inline int tile_exp(float m) {
  if (!(m > 0.f) || !(m <= 3.0e38f)) return 0;
  return (int)((__float_as_uint(m) >> 23) & 0xFFu) - 127 - 14;
}

template <bool H16, int KS>
struct StateQuads;
template <int KS>
struct StateQuads<false, KS> {
  f32x4 f[KS];
  __device__ f32x4 get(int k) const { return f[k]; }
};
template <int KS>
struct StateQuads<true, KS> {
  f16x4 h[KS];
  int e[KS];
  __device__ f32x4 get(int k) const {
    const f32x4 v = __builtin_convertvector(h[k], f32x4);
    return f32x4{__builtin_amdgcn_ldexpf(v[0], e[k]), __builtin_amdgcn_ldexpf(v[1], e[k]),
                 __builtin_amdgcn_ldexpf(v[2], e[k]), __builtin_amdgcn_ldexpf(v[3], e[k])};
  }
};

// A load of data that is read once (x, dy, the states): marked non-temporal so
// that it leaves the L2 lines of the head block's dB / dC partials alone.
template <typename V>
__device__ inline V load_once(const V* p) { return __builtin_nontemporal_load(p); }

template <typename T, int N, int P, bool H16>
__global__ __launch_bounds__(256, 2) void k_bwd_chunk(
    const T* __restrict__ x, const T* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ dt_bias, const T* __restrict__ dy, const float* __restrict__ cs,
    const float* __restrict__ dtp, const float* __restrict__ states,
    const float* __restrict__ adj, const float2* __restrict__ coef,
    const int32_t* __restrict__ seq_idx, const ChunkInfo* __restrict__ cinfo, Shape sh,
    T* __restrict__ dx, T* __restrict__ ddt, float* __restrict__ dBh, float* __restrict__ dCh,
    float* __restrict__ part, const int* __restrict__ scS, const int* __restrict__ scG, int hblk) {
  using E = Elem<T>;
  // bf16 storage: the fp32 pair weights of the diagonal blocks (the masked
  // (dy_i . x_j), (C_i . B_j) factors) go to the matrix cores as two bf16
  // terms, hi + lo, so that they add no bf16 rounding of their own (a single
  // bf16 weight left dB and dC near 2e-2 where dt' = 0 over many tokens and
  // long causal spans keep large weights undecayed)
  constexpr bool kSplitW = sizeof(T) == 2;
  using frag = typename E::frag;
  constexpr int Q = kBwdChunk, LDN = N + 4, LDP = P + 4;
  constexpr int NTn = N / 16, NTn2 = (NTn + 1) / 2, NTp = P / 16;
  constexpr int NS = bwd_state_terms<T>();                 // bf16 state as hi + lo terms
  constexpr int NH = bwd_state_parts<N>(), NR = N / NH;    // state parts, rows per part
  constexpr int NTr = NR / 16, NTr2 = (NTr + 1) / 2, SL = NR * LDP;  // n-tiles, elements per term
  __shared__ __attribute__((aligned(16))) T sB[Q * LDN];
  __shared__ __attribute__((aligned(16))) T sC[Q * LDN];
  __shared__ __attribute__((aligned(16))) T sX[Q * LDP];
  __shared__ __attribute__((aligned(16))) T sDY[Q * LDP];
  __shared__ __attribute__((aligned(16))) float sU[bwd_state_floats<T, N, P>()];
  T* const sS = reinterpret_cast<T*>(sU);  // NS terms of a state part, row-major, stride LDP
  // pair weights W[i][j] (j < i), then the row prefix sums R[i][k] (k <= i):
  // row i at i (i + 1) / 2
  __shared__ float sW[Q * (Q + 1) / 2];
  auto wrow = [](int i) { return i * (i + 1) / 2; };
  __shared__ float sCs[Q], sDt[Q], sOut[Q], sIn[Q], sDs[Q], sXdy[Q], sT[Q];
  __shared__ int32_t sSeq[Q];  // sequence of each token (packed input)
  __shared__ float sK[4];      // per-wave parts of <G_end, S_in>

  const int64_t NP = (int64_t)N * P;
  const bool scales = sh.flags & kFlagScalesInput;
  const frag fz = zero_frag<T>();
  constexpr int KN = Q * (N / 4) / 256, KP = Q * (P / 4) / 256, KS = NR * P / 4 / 256;
  static_assert(KN * 256 == Q * (N / 4) && KP * 256 == Q * (P / 4) && KS * 256 == NR * P / 4,
                "whole staging rounds");

  // heads hblk blockIdx.x .. + hblk - 1, one after the other: they share their
  // group of B and of C (staged once, here), and their dB and dC rows are
  // summed in place (one partial per head block).  Rows past the chunk end are
  // zero.
  {
    const int tid = threadIdx.x;
    const int64_t tb = (int64_t)blockIdx.y * Q;
    const int len = (int)min<int64_t>(Q, sh.L - tb);
    const int64_t rowbase = (int64_t)blockIdx.z * sh.L + tb;
    const int gB = blockIdx.x * hblk / sh.hpg, gC = blockIdx.x * hblk / sh.hpgc;
    frag vb[KN], vc[KN];
#pragma unroll
    for (int k = 0; k < KN; ++k) {
      const int q = tid + 256 * k, jj = q / (N / 4), c4 = 4 * (q % (N / 4));
      const bool ok = jj < len;
      vb[k] = ok ? load_frag(Bm + ((rowbase + jj) * sh.G + gB) * N + c4) : fz;
      vc[k] = ok ? load_frag(Cm + ((rowbase + jj) * sh.Gc + gC) * N + c4) : fz;
    }
#pragma unroll
    for (int k = 0; k < KN; ++k) {
      const int q = tid + 256 * k, jj = q / (N / 4), c4 = 4 * (q % (N / 4));
      store_frag(sB + jj * LDN + c4, vb[k]);
      store_frag(sC + jj * LDN + c4, vc[k]);
    }
  }
  for (int hi = 0; hi < hblk; ++hi) {
    // indices re-derived per head from opaque copies: derived once outside the
    // loop, the compiler keeps dozens of offsets alive across it and spills
    int ids[4] = {(int)threadIdx.x, (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
    asm volatile("" : "+v"(ids[0]), "+s"(ids[1]), "+s"(ids[2]), "+s"(ids[3]));
    const int c = ids[2], b = ids[3];
    const int tid = ids[0], lane = tid & 63;
    // the wave index in a scalar register: branches on it are scalar branches
    // (a guard the compiler cannot prove uniform becomes an EXEC mask, and the
    // transposing LDS load must not run under one)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = (lane >> 4) * 4, l16 = lane & 15;
    const int64_t tb = (int64_t)c * Q;
    const int len = (int)min<int64_t>(Q, sh.L - tb);
    const int64_t rowbase = (int64_t)b * sh.L + tb;
    const ChunkInfo ci = cinfo[(int64_t)b * sh.nc + c];
    const int nhb = sh.H / hblk, blk = ids[1];
    const int h = blk * hblk + hi;
    const int64_t hb = (int64_t)b * sh.H + h;
    const int64_t cso = (hb * sh.nc + c) * Q;
    if (hi > 0) __syncthreads();  // the previous head's last LDS reads are done

    // ---- stage the head's rows of the chunk (rows past the end are zero); each
    // thread issues all of its loads before the first LDS store
    if (tid < Q) {
      sCs[tid] = cs[cso + tid];
      sDt[tid] = dtp[cso + tid];
      sSeq[tid] = (sh.varlen && tid < len) ? seq_idx[tb + tid] : ci.seq_last;
    }
    {
      frag vx[KP], vd[KP];
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int q = tid + 256 * k, jj = q / (P / 4), c4 = 4 * (q % (P / 4));
        const bool ok = jj < len;
        const int64_t o = ((rowbase + jj) * sh.H + h) * P + c4;
        vx[k] = ok ? load_once(reinterpret_cast<const frag*>(x + o)) : fz;
        vd[k] = ok ? load_once(reinterpret_cast<const frag*>(dy + o)) : fz;
      }
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int q = tid + 256 * k, jj = q / (P / 4), c4 = 4 * (q % (P / 4));
        store_frag(sX + jj * LDP + c4, vx[k]);
        store_frag(sDY + jj * LDP + c4, vd[k]);
      }
    }
    // rows [part NR, part NR + NR) of a state, from the fragment layout (n-tile
    // major, so a part is a contiguous run of quads) into row-major (n, p)
    // (loaded into registers ahead of need, stored to LDS when the region is free)
    using SQ = StateQuads<H16, KS>;
    auto load_state = [&](const float* src, const int* sc, int part, SQ& v) {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int q = part * (NR * P / 4) + tid + 256 * k;
        if constexpr (H16) {
          v.h[k] = load_once(reinterpret_cast<const f16x4*>(src) + q);
          v.e[k] = sc[q >> 6];
        } else {
          v.f[k] = load_once(reinterpret_cast<const f32x4*>(src) + q);
        }
      }
    };
    auto store_state = [&](const SQ& v) {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int q = tid + 256 * k;
        const int tile = q >> 6, ln = q & 63;
        const int n0 = 16 * (tile / NTp) + 4 * (ln >> 4), p = 16 * (tile % NTp) + (ln & 15);
        const f32x4 x4 = v.get(k);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const T hi = E::from_float(x4[e]);
          sS[(n0 + e) * LDP + p] = hi;
          if constexpr (NS == 2)
            sS[SL + (n0 + e) * LDP + p] = E::from_float(x4[e] - E::to_float(hi));
        }
      }
    };
    const int64_t sidx = ((int64_t)b * sh.nc + c) * sh.H + h;
    const float* Sin = H16 ? reinterpret_cast<const float*>(reinterpret_cast<const f16*>(states) + sidx * NP)
                           : states + sidx * NP;
    const float* Gend = H16 ? reinterpret_cast<const float*>(reinterpret_cast<const f16*>(adj) + sidx * NP)
                            : adj + sidx * NP;
    const int* SinE = H16 ? scS + sidx * (NP / 256) : nullptr;
    const int* GendE = H16 ? scG + sidx * (NP / 256) : nullptr;
    // the S_in and G_end quads stay in registers for <G_end, S_in>
    SQ si[NH], sg[NH];
    load_state(Gend, GendE, 0, sg[0]);
    load_state(Sin, SinE, 0, si[0]);
    if constexpr (NH > 1) {
      load_state(Gend, GendE, 1, sg[1]);
      load_state(Sin, SinE, 1, si[1]);
    }
    store_state(sg[0]);
    float kdot = 0.f;  // this thread's part of <G_end, S_in>
#pragma unroll
    for (int part = 0; part < NH; ++part)
#pragma unroll
      for (int k = 0; k < KS; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) kdot += sg[part].get(k)[e] * si[part].get(k)[e];
    __syncthreads();

    const int iw = 16 * w;          // this wave's tile
    const int me = iw + l16;        // this lane's token (output column of every tile)
    const float cs_me = sCs[me];
    const float s_me = scales ? sDt[me] : 1.f;
    const int seq_me = sSeq[me];

    // ---- column side, j = me, from G_end: dx_j += exp(cs_end - cs_j) G^T B_j,
    // dB_j += exp(cs_end - cs_j) G x_j (G_end belongs to the chunk's last sequence)
    f32x4 adx[NTp], adb[NTn];
    float xg_state;  // x_j . (exp(cs_end - cs_j) G_end^T B_j)
    {
      frag bJ[2 * NTn2], xJ[NTp];
#pragma unroll
      for (int kb = 0; kb < 2 * NTn2; ++kb) bJ[kb] = kb < NTn ? rd_row(sB, LDN, me, 16 * kb + g4) : fz;
#pragma unroll
      for (int kb = 0; kb < NTp; ++kb) xJ[kb] = rd_row(sX, LDP, me, 16 * kb + g4);
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) adx[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int part = 0; part < NH; ++part) {
        if (part > 0) {
          __syncthreads();
          store_state(sg[part]);
          __syncthreads();
        }
#pragma unroll
        for (int pt = 0; pt < NTp; ++pt)
#pragma unroll
          for (int term = 0; term < NS; ++term)
#pragma unroll
            for (int k2 = 0; k2 < NTr2; ++k2) {
              const T* st = sS + term * SL;
              const frag a0 = rd_col<LDP>(st, 32 * k2, 16 * pt, lane);
              const frag a1 = (2 * k2 + 1 < NTr) ? rd_col<LDP>(st, 32 * k2 + 16, 16 * pt, lane) : fz;
              adx[pt] = E::mma2(adx[pt], a0, a1, bJ[part * NTr + 2 * k2],
                                2 * k2 + 1 < NTr ? bJ[part * NTr + 2 * k2 + 1] : fz);
            }
#pragma unroll
        for (int nt = 0; nt < NTr; ++nt) {
          f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int term = 0; term < NS; ++term)
#pragma unroll
            for (int k2 = 0; k2 < NTp / 2; ++k2)
              t = E::mma2(t, rd_row(sS + term * SL, LDP, 16 * nt + l16, 32 * k2 + g4),
                          rd_row(sS + term * SL, LDP, 16 * nt + l16, 32 * k2 + 16 + g4),
                          xJ[2 * k2], xJ[2 * k2 + 1]);
          adb[part * NTr + nt] = t;
        }
      }
      const float ej = seq_me == ci.seq_last ? fast_exp(sCs[len - 1] - cs_me) : 0.f;
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) adx[pt] *= ej;
#pragma unroll
      for (int nt = 0; nt < NTn; ++nt) adb[nt] *= ej;
      xg_state = 0.f;
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) xg_state += dot4<T>(xJ[pt], adx[pt]);
      xg_state = sum_groups(xg_state);
    }
    __syncthreads();  // G_end is dead: its region takes S_in
    store_state(si[0]);
    __syncthreads();

    // ---- row side, i = me, from S_in: y_state_i = exp(cs_i) S^T C_i and
    // dC_i = exp(cs_i) S dy_i (S_in belongs to the chunk's first sequence)
    f32x4 adc[NTn];
    {
      frag cI[2 * NTn2], dyI[NTp];
#pragma unroll
      for (int kb = 0; kb < 2 * NTn2; ++kb) cI[kb] = kb < NTn ? rd_row(sC, LDN, me, 16 * kb + g4) : fz;
#pragma unroll
      for (int kb = 0; kb < NTp; ++kb) dyI[kb] = rd_row(sDY, LDP, me, 16 * kb + g4);
      f32x4 ys[NTp];
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) ys[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int part = 0; part < NH; ++part) {
        if (part > 0) {
          __syncthreads();
          store_state(si[part]);
          __syncthreads();
        }
#pragma unroll
        for (int pt = 0; pt < NTp; ++pt)
#pragma unroll
          for (int term = 0; term < NS; ++term)
#pragma unroll
            for (int k2 = 0; k2 < NTr2; ++k2) {
              const T* st = sS + term * SL;
              const frag a0 = rd_col<LDP>(st, 32 * k2, 16 * pt, lane);
              const frag a1 = (2 * k2 + 1 < NTr) ? rd_col<LDP>(st, 32 * k2 + 16, 16 * pt, lane) : fz;
              ys[pt] = E::mma2(ys[pt], a0, a1, cI[part * NTr + 2 * k2],
                               2 * k2 + 1 < NTr ? cI[part * NTr + 2 * k2 + 1] : fz);
            }
#pragma unroll
        for (int nt = 0; nt < NTr; ++nt) {
          f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int term = 0; term < NS; ++term)
#pragma unroll
            for (int k2 = 0; k2 < NTp / 2; ++k2)
              t = E::mma2(t, rd_row(sS + term * SL, LDP, 16 * nt + l16, 32 * k2 + g4),
                          rd_row(sS + term * SL, LDP, 16 * nt + l16, 32 * k2 + 16 + g4),
                          dyI[2 * k2], dyI[2 * k2 + 1]);
          adc[part * NTr + nt] = t;
        }
      }
      // dy_i . y_state_i and dy_i . x_i
      const float ei = seq_me == ci.seq_first ? fast_exp(cs_me) : 0.f;
      float vo = 0.f, vxd = 0.f;
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) {
        vo += dot4<T>(dyI[pt], ys[pt]);
        vxd += dot4<T>(dyI[pt], E::to_f32(rd_row(sX, LDP, me, 16 * pt + g4)));
      }
      vo = sum_groups(vo) * ei;
      vxd = sum_groups(vxd);
      if (g4 == 0) {
        sOut[me] = vo;
        sXdy[me] = vxd;
      }
#pragma unroll
      for (int nt = 0; nt < NTn; ++nt) adc[nt] *= ei;

      // ---- diagonal blocks, both sides in one interval (wave w: w + 1 tiles
      // on the row side, 4 - w on the column side)
      // row side: dC_i += sum_{j <= i} L[i,j] s_j (dy_i . x_j) B_j, and the pair
      // weights W[i][j] (j < i) into their own region
      for (int J0 = 0; J0 <= w; J0 += 2) {
        frag wv[2], wl[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int J = J0 + e2;
          if (J > w) {
            wv[e2] = wl[e2] = fz;
            continue;
          }
          f32x4 cb = {0.f, 0.f, 0.f, 0.f}, xd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k2 = 0; k2 < NTn2; ++k2) {
            const frag a0 = rd_row(sB, LDN, 16 * J + l16, 32 * k2 + g4);
            const frag a1 = (2 * k2 + 1 < NTn) ? rd_row(sB, LDN, 16 * J + l16, 32 * k2 + 16 + g4) : fz;
            cb = E::mma2(cb, a0, a1, cI[2 * k2], cI[2 * k2 + 1]);
          }
#pragma unroll
          for (int k2 = 0; k2 < NTp / 2; ++k2)
            xd = E::mma2(xd, rd_row(sX, LDP, 16 * J + l16, 32 * k2 + g4),
                         rd_row(sX, LDP, 16 * J + l16, 32 * k2 + 16 + g4), dyI[2 * k2],
                         dyI[2 * k2 + 1]);
          f32x4 wvv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 16 * J + g4 + e;
            const float dec = (j <= me && sSeq[j] == seq_me)
                                  ? fast_exp(cs_me - sCs[j]) * (scales ? sDt[j] : 1.f)
                                  : 0.f;
            wvv[e] = dec * xd[e];
            if (j < me) sW[wrow(me) + j] = wvv[e] * cb[e];
          }
          wv[e2] = E::from_f32(wvv);
          if constexpr (kSplitW) wl[e2] = E::from_f32(wvv - E::to_f32(wv[e2]));
        }
#pragma unroll
        for (int nt = 0; nt < NTn; ++nt) {
          const frag b0 = rd_col<LDN>(sB, 16 * J0, 16 * nt, lane);
          const frag b1 = rd_col<LDN>(sB, 16 * (J0 + 1), 16 * nt, lane);
          adc[nt] = E::mma2(adc[nt], b0, b1, wv[0], wv[1]);
          if constexpr (kSplitW) adc[nt] = E::mma2(adc[nt], b0, b1, wl[0], wl[1]);
        }
      }
    }
    if (me < len) {
      // the block's partial: this thread wrote these elements for the heads in
      // front of h (same addresses, same thread)
      float* o = dCh + ((rowbase + me) * nhb + blk) * N + g4;
      if (hi > 0) {
#pragma unroll
        for (int nt = 0; nt < NTn; ++nt) adc[nt] += *reinterpret_cast<const f32x4*>(o + 16 * nt);
      }
#pragma unroll
      for (int nt = 0; nt < NTn; ++nt) *reinterpret_cast<f32x4*>(o + 16 * nt) = adc[nt];
    }
    // column side: tiles i = I0, I0 + 1 with w <= i < 4
    {
      frag bJ[2 * NTn2], xJ[NTp];
#pragma unroll
      for (int kb = 0; kb < 2 * NTn2; ++kb) bJ[kb] = kb < NTn ? rd_row(sB, LDN, me, 16 * kb + g4) : fz;
#pragma unroll
      for (int kb = 0; kb < NTp; ++kb) xJ[kb] = rd_row(sX, LDP, me, 16 * kb + g4);
      for (int I0 = w; I0 < Q / 16; I0 += 2) {
        const bool two = I0 + 1 < Q / 16;
        frag m[2], wv[2], ml[2], wl[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int I = I0 + e2;
          if (e2 == 1 && !two) {
            m[1] = wv[1] = ml[1] = wl[1] = fz;
            continue;
          }
          f32x4 cb = {0.f, 0.f, 0.f, 0.f}, xd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k2 = 0; k2 < NTn2; ++k2) {
            const frag a0 = rd_row(sC, LDN, 16 * I + l16, 32 * k2 + g4);
            const frag a1 = (2 * k2 + 1 < NTn) ? rd_row(sC, LDN, 16 * I + l16, 32 * k2 + 16 + g4) : fz;
            cb = E::mma2(cb, a0, a1, bJ[2 * k2], bJ[2 * k2 + 1]);
          }
#pragma unroll
          for (int k2 = 0; k2 < NTp / 2; ++k2)
            xd = E::mma2(xd, rd_row(sDY, LDP, 16 * I + l16, 32 * k2 + g4),
                         rd_row(sDY, LDP, 16 * I + l16, 32 * k2 + 16 + g4), xJ[2 * k2],
                         xJ[2 * k2 + 1]);
          f32x4 mv, wvv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + g4 + e;
            const float dec = (i >= me && sSeq[i] == seq_me) ? fast_exp(sCs[i] - cs_me) : 0.f;
            mv[e] = dec * cb[e];
            wvv[e] = dec * xd[e];
          }
          m[e2] = E::from_f32(mv);
          wv[e2] = E::from_f32(wvv);
          if constexpr (kSplitW) {
            ml[e2] = E::from_f32(mv - E::to_f32(m[e2]));
            wl[e2] = E::from_f32(wvv - E::to_f32(wv[e2]));
          }
        }
        // dx_j += sum_i L[i,j] (C_i . B_j) dy_i ; dB_j += sum_i L[i,j] (dy_i . x_j) C_i
        // the second tile's column reads always run, inside the tile (its rows
        // for a missing second tile are the first tile's), and the value is
        // dropped afterwards: the transposing load takes no guard
        const int I1 = two ? I0 + 1 : I0;
#pragma unroll
        for (int pt = 0; pt < NTp; ++pt) {
          const frag a0 = rd_col<LDP>(sDY, 16 * I0, 16 * pt, lane);
          const frag r1 = rd_col<LDP>(sDY, 16 * I1, 16 * pt, lane);
          const frag a1 = two ? r1 : fz;
          adx[pt] = E::mma2(adx[pt], a0, a1, m[0], m[1]);
          if constexpr (kSplitW) adx[pt] = E::mma2(adx[pt], a0, a1, ml[0], ml[1]);
        }
#pragma unroll
        for (int nt = 0; nt < NTn; ++nt) {
          const frag a0 = rd_col<LDN>(sC, 16 * I0, 16 * nt, lane);
          const frag r1 = rd_col<LDN>(sC, 16 * I1, 16 * nt, lane);
          const frag a1 = two ? r1 : fz;
          adb[nt] = E::mma2(adb[nt], a0, a1, wv[0], wv[1]);
          if constexpr (kSplitW) adb[nt] = E::mma2(adb[nt], a0, a1, wl[0], wl[1]);
        }
      }
      // x_j . (B_j^T g_j): the dt' gradient of the input scaling
      float xg = 0.f;
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) xg += dot4<T>(xJ[pt], adx[pt]);
      xg = sum_groups(xg);
      if (g4 == 0) {
        sIn[me] = s_me * xg_state;
        sDs[me] = xg;
      }
    }
    if (me < len) {
      const float Dh = D ? D[h] : 0.f;
      const int64_t o = ((rowbase + me) * sh.H + h) * P + g4;
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) {
        const f32x4 dyv = E::to_f32(rd_row(sDY, LDP, me, 16 * pt + g4));
        store_frag(dx + o + 16 * pt, E::from_f32(s_me * adx[pt] + Dh * dyv));
      }
      float* ob = dBh + ((rowbase + me) * nhb + blk) * N + g4;
#pragma unroll
      for (int nt = 0; nt < NTn; ++nt) adb[nt] *= s_me;
      if (hi > 0) {
#pragma unroll
        for (int nt = 0; nt < NTn; ++nt) adb[nt] += *reinterpret_cast<const f32x4*>(ob + 16 * nt);
      }
#pragma unroll
      for (int nt = 0; nt < NTn; ++nt) *reinterpret_cast<f32x4*>(ob + 16 * nt) = adb[nt];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) kdot += __shfl_xor(kdot, off, 64);
    if (lane == 0) sK[w] = kdot;
    __syncthreads();
    // row prefix sums of W: thread (row i, quarter qq) over j in [16 qq, 16 qq + 16)
    // (R[i][k] = sum_{j < k} W[i][j], kept for k <= i)
    {
      const int i = tid >> 2, qq = tid & 3;
      float v[16], run = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int j = 16 * qq + k;
        v[k] = run;  // exclusive prefix inside the quarter
        run += (j < i) ? sW[wrow(i) + j] : 0.f;
      }
      // quarters of one row sit in 4 consecutive lanes
      float off = run;
      const float o1 = __shfl_up(off, 1, 64);
      const float o2 = __shfl_up(off, 2, 64);
      const float o3 = __shfl_up(off, 3, 64);
      off = (qq >= 1 ? o1 : 0.f) + (qq >= 2 ? o2 : 0.f) + (qq >= 3 ? o3 : 0.f);
      __syncthreads();  // every read of W done before the prefix sums overwrite it
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (16 * qq + k <= i) sW[wrow(i) + 16 * qq + k] = off + v[k];  // sum_{j < 16 qq + k}
    }
    __syncthreads();
    // corner sums: sum_{i >= k > j} W[i][j] = sum_{i >= k} R[i][k]; thread
    // (k, quarter qq) over i in [16 qq, 16 qq + 16)
    {
      const int k = tid >> 2, qq = tid & 3;
      float t = 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = 16 * qq + u;
        t += (i >= k) ? sW[wrow(i) + k] : 0.f;
      }
      t += __shfl_xor(t, 1, 64);
      t += __shfl_xor(t, 2, 64);
      if (qq == 0) sT[k] = t;
    }
    __syncthreads();

    // ---- dl, then dt, dA, dD, dt_bias
    if (w == 0) {
      // exp(cs_end) <G_end, S_in>: the carry decay is zero unless one sequence
      // spans the chunk
      const float K = coef[hb * sh.nc + c].x * (sK[0] + sK[1] + sK[2] + sK[3]);
      float suf = lane < len ? sOut[lane] : 0.f;
      const float in = lane < len ? sIn[lane] : 0.f;
      float pre_in = in;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += o;
        const float u = __shfl_up(pre_in, off, 64);
        if (lane >= off) pre_in += u;
      }
      const float dl = sT[lane] + suf + (pre_in - in) + K;
      float gdt = 0.f, gA = 0.f, gD = 0.f;
      if (lane < len) {
        const float Ah = A[h];
        float ddtp = dl * Ah + (scales ? sDs[lane] : 0.f);
        const float pre = E::to_float(dt[(rowbase + lane) * sh.H + h]) + (dt_bias ? dt_bias[h] : 0.f);
        const bool sp = sh.flags & kFlagSoftplus;
        const float act = sp ? softplus_f32(pre) : pre;
        float gate = (act >= sh.dt_min && act <= sh.dt_max) ? 1.f : 0.f;
        if (sp) gate *= 1.f / (1.f + __expf(-pre));
        gdt = ddtp * gate;
        ddt[(rowbase + lane) * sh.H + h] = E::from_float(gdt);
        gA = dl * sDt[lane];
        gD = sXdy[lane];
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        gA += __shfl_xor(gA, off, 64);
        gD += __shfl_xor(gD, off, 64);
        gdt += __shfl_xor(gdt, off, 64);
      }
      if (lane == 0) {
        float* o = part + (hb * sh.nc + c) * 3;
        o[0] = gA;
        o[1] = gD;
        o[2] = gdt;
      }
    }
  }  // heads of the block
}

// ------------------------------------------------------------------ reductions
// out[r, g, n] = sum_{k < hpg} src[r, g hpg + k, n], four n per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_group_sum(const float* __restrict__ src, int64_t rows,
                                                   int H, int ng, int hpg, int N,
                                                   T* __restrict__ out) {
  const int64_t total = rows * ng * (N / 4);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int n4 = (int)(i % (N / 4));
    const int64_t rg = i / (N / 4);
    const int g = (int)(rg % ng);
    const int64_t r = rg / ng;
    const f32x4* s = reinterpret_cast<const f32x4*>(src + (r * H + (int64_t)g * hpg) * N) + n4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < hpg; ++k) acc += s[(int64_t)k * (N / 4)];
    store_frag(out + (r * ng + g) * N + 4 * n4, Elem<T>::from_f32(acc));
  }
}

// grid H, 256 threads: per-head sums of the per-chunk partials over rows and chunks.
__global__ __launch_bounds__(256) void k_head_sums(const float* __restrict__ part, int batch,
                                                   int H, int nc, float* __restrict__ dA,
                                                   float* __restrict__ dD,
                                                   float* __restrict__ dbias) {
  const int h = blockIdx.x;
  float s[3] = {0.f, 0.f, 0.f};
  for (int i = threadIdx.x; i < batch * nc; i += 256) {
    const int b = i / nc, c = i % nc;
    const float* p = part + (((int64_t)b * H + h) * nc + c) * 3;
    s[0] += p[0];
    s[1] += p[1];
    s[2] += p[2];
  }
  __shared__ float red[3][4];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    float v = s[k];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) red[k][threadIdx.x >> 6] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float t[3];
    for (int k = 0; k < 3; ++k) t[k] = red[k][0] + red[k][1] + red[k][2] + red[k][3];
    dA[h] = t[0];
    if (dD) dD[h] = t[1];
    if (dbias) dbias[h] = t[2];
  }
}

// ------------------------------------------------------------------ state walks (dense rows, bf16)
// The chunk states S_in and the adjoints G_end of every chunk, formed by
// walking each (row, head) stream over its chunks with the running state in
// registers (no per-chunk partial states through memory, no separate scans):
//   forward: S_in[c] = S;  S <- exp(cs_end) S + sum_t exp(cs_end - cs_t) s_t B_t x_t^T
//   reverse: G_end[c] = G; G <- exp(cs_end) G + sum_t exp(cs_t) C_t dy_t^T
// the reverse walk going from the last chunk to the first, from the final-state
// gradient to the initial-state gradient.  grid (H, batch, NSPL), 256 threads:
// a workgroup owns N / NSPL state rows (n-tiles from blockIdx.z N / (16 NSPL)
// on, every column), its waves the 16 x 16 tiles wave, wave + 4, ... of them;
// per chunk its columns of the operand rows go to LDS (C or B as read) with
// the weighted x or dy as two bf16 terms, hi + lo (so the weights add no bf16
// rounding), both read back with the transposing load, while the next chunks'
// rows are in flight.  Outputs in the fragment layout of the state buffers.
template <int N, int P, bool REV, int NSPL>
__global__ __launch_bounds__(256, (NSPL > 1 ? 3 : 2)) void k_bwd_walk(const bf16* __restrict__ opA,
                                                     const bf16* __restrict__ opX,
                                                     const float* __restrict__ cs,
                                                     const float* __restrict__ dtp, Shape sh,
                                                     const float* __restrict__ start,
                                                     f16* __restrict__ out, int* __restrict__ osc,
                                                     float* __restrict__ fin) {
  constexpr int NL = N / NSPL;               // state rows of the workgroup
  constexpr int Q = kBwdChunk, RA = NL / 8, RX = P / 8, NTn = NL / 16, NTp = P / 16;
  constexpr int NT = NTn * NTp, TPW = NT / 4, NPW = NTp / 4;  // tiles, per wave; p-tiles per wave
  constexpr int LA = (Q * RA + 255) / 256;  // 16-byte loads of operand rows per thread
  constexpr int LX = Q * RX / 256;          // 16-byte loads of x / dy rows per thread
  constexpr int D = 4;                      // chunks in flight
  static_assert(NT % 4 == 0 && NTp % 4 == 0 && LX * 256 == Q * RX && NL % 16 == 0, "tile split");
  __shared__ __attribute__((aligned(16))) bf16 sA[Q * NL];
  __shared__ __attribute__((aligned(16))) bf16 sXh[Q * P];
  __shared__ __attribute__((aligned(16))) bf16 sXl[Q * P];

  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = (lane >> 4) * 4, l16 = lane & 15;
  const int64_t hb = (int64_t)b * sh.H + h;
  const int64_t NP = (int64_t)N * P;
  const int ng = REV ? sh.Gc : sh.G, grp = REV ? h / sh.hpgc : h / sh.hpg;
  const bool scales = !REV && (sh.flags & kFlagScalesInput);
  const int nt0 = blockIdx.z * NTn;  // the workgroup's first n-tile

  // tile k of this wave: t = wave + 4 k, n-tile nt0 + t / NTp, p-tile t % NTp
  // (the wave's p-tiles are wave + 4 j, j < NPW); tile nt0 NTp + t of the state
  f32x4 S[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = wave + 4 * k;
    S[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (start) {
      const float* sp =
          start + hb * NP + (int64_t)(16 * (nt0 + t / NTp) + g4) * P + 16 * (t % NTp) + l16;
      S[k] = f32x4{sp[0], sp[P], sp[2 * P], sp[3 * P]};
    }
  }
  // fragment-layout offset of local tile t
  auto qoff = [&](int t) { return ((int64_t)(nt0 * NTp + t) * 64 + lane) * 4; };

  // one chunk's operand rows, per-token values and decay, in registers; D
  // chunks are in flight (the walk is otherwise bound by the load latency).
  // Rows past the chunk end are loaded clamped and zeroed when staged: a
  // select right after the load would wait for it.
  struct Buf {
    bf16x8 ra[LA], rx[LX];
    float rcs[LX], rdt[LX], rce;
    int len;
  };
  auto xrow = [&](int j) { return (tid + 256 * j) / RX; };
  auto xcol = [&](int j) { return (tid + 256 * j) % RX; };
  auto fetch = [&](Buf& f, int c) {
    const int64_t tb = (int64_t)c * Q;
    const int len = (int)min<int64_t>(Q, sh.L - tb);
    const int64_t rowbase = (int64_t)b * sh.L + tb;
#pragma unroll
    for (int k = 0; k < LA; ++k) {
      const int q = min(tid + 256 * k, Q * RA - 1), t = q / RA, cc = q % RA;
      f.ra[k] = *reinterpret_cast<const bf16x8*>(opA + ((rowbase + min(t, len - 1)) * ng + grp) * N +
                                                  16 * nt0 + 8 * cc);
    }
    const float* csc = cs + (hb * sh.nc + c) * Q;
#pragma unroll
    for (int j = 0; j < LX; ++j) {
      const int t = min(xrow(j), len - 1);
      f.rx[j] = *reinterpret_cast<const bf16x8*>(opX + ((rowbase + t) * sh.H + h) * P + 8 * xcol(j));
      f.rcs[j] = csc[t];
      f.rdt[j] = scales ? dtp[(hb * sh.nc + c) * Q + t] : 1.f;
    }
    f.rce = csc[len - 1];
    f.len = len;
  };
  auto stage = [&](const Buf& f) {
#pragma unroll
    for (int k = 0; k < LA; ++k) {
      const int q = tid + 256 * k;
      if (q < Q * RA)
        *reinterpret_cast<bf16x8*>(sA + swz_off<RA>(q / RA, 8 * (q % RA))) = q / RA < f.len ? f.ra[k] : bf16x8{};
    }
#pragma unroll
    for (int j = 0; j < LX; ++j) {
      const int t = xrow(j);
      const float w = t < f.len ? (REV ? __expf(f.rcs[j]) : __expf(f.rce - f.rcs[j]) * f.rdt[j]) : 0.f;
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = (float)f.rx[j][e] * w;
        hi[e] = (bf16)v;
        lo[e] = (bf16)(v - (float)hi[e]);
      }
      *reinterpret_cast<bf16x8*>(sXh + swz_off<RX>(t, 8 * xcol(j))) = hi;
      *reinterpret_cast<bf16x8*>(sXl + swz_off<RX>(t, 8 * xcol(j))) = lo;
    }
  };
  auto cat8 = [](bf16x4 a, bf16x4 c) { return __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7); };
  // per 32-token step: the wave's x / dy fragments (one per p-tile it owns),
  // then every tile's operand fragments, then the products
  auto compute = [&]() {
#pragma unroll
    for (int s = 0; s < Q / 32; ++s) {
      bf16x8 xh[NPW], xl[NPW], a[TPW];
#pragma unroll
      for (int j = 0; j < NPW; ++j) {
        const int pl = 16 * (wave + 4 * j);
        xh[j] = cat8(tr_frag_swz<RX>(sXh, pl, 32 * s, lane), tr_frag_swz<RX>(sXh, pl, 32 * s + 16, lane));
        xl[j] = cat8(tr_frag_swz<RX>(sXl, pl, 32 * s, lane), tr_frag_swz<RX>(sXl, pl, 32 * s + 16, lane));
      }
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int t = wave + 4 * k;
        a[k] = cat8(tr_frag_swz<RA>(sA, 16 * (t / NTp), 32 * s, lane),
                    tr_frag_swz<RA>(sA, 16 * (t / NTp), 32 * s + 16, lane));
      }
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int j = k % NPW;  // (wave + 4 k) % NTp = wave + 4 (k % NPW)
        S[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k], xh[j], S[k], 0, 0, 0);
        S[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k], xl[j], S[k], 0, 0, 0);
      }
    }
  };

  const int nc = sh.nc;
  auto chunk_of = [&](int i) { return REV ? nc - 1 - i : i; };  // the i-th chunk walked
  // step i: chunk i's rows (in f) to LDS, the state out and decayed, chunk i + D
  // requested into f, then chunk i's products
  // (barriers wait for LDS traffic only: __syncthreads would also drain the
  // loads in flight and the state stores)
  auto step = [&](Buf& f, int i) {
    lds_barrier();  // the previous chunk's LDS reads are done
    stage(f);
    const int c = chunk_of(i);
    const int64_t sidx = ((int64_t)b * nc + c) * sh.H + h;
    f16* o = out + sidx * NP;
    const float d = __expf(f.rce);
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int t = wave + 4 * k;
      // the tile as fp16 quads with one power-of-two scale
      const float m = wave_max(
          fmaxf(fmaxf(fabsf(S[k][0]), fabsf(S[k][1])), fmaxf(fabsf(S[k][2]), fabsf(S[k][3]))));
      const int e = tile_exp(m);
      const f32x4 v = S[k];
      *reinterpret_cast<f16x4*>(o + qoff(t)) =
          f16x4{(f16)__builtin_amdgcn_ldexpf(v[0], -e), (f16)__builtin_amdgcn_ldexpf(v[1], -e),
                (f16)__builtin_amdgcn_ldexpf(v[2], -e), (f16)__builtin_amdgcn_ldexpf(v[3], -e)};
      if (lane == 0) osc[sidx * (NP / 256) + nt0 * NTp + t] = e;
      S[k] *= d;
    }
    lds_barrier();
    // unconditional (the last steps read the last chunk again): with loads on
    // one path only the wait in the next stage would drain every load
    fetch(f, chunk_of(min(i + D, nc - 1)));
    compute();
  };
  static_assert(D == 4, "four buffers below");
  Buf f0, f1, f2, f3;
  fetch(f0, chunk_of(0));
  fetch(f1, chunk_of(min(1, nc - 1)));
  fetch(f2, chunk_of(min(2, nc - 1)));
  fetch(f3, chunk_of(min(3, nc - 1)));
  int i = 0;
  for (; i + 3 < nc; i += 4) {
    step(f0, i);
    step(f1, i + 1);
    step(f2, i + 2);
    step(f3, i + 3);
  }
  if (i < nc) step(f0, i);
  if (i + 1 < nc) step(f1, i + 1);
  if (i + 2 < nc) step(f2, i + 2);
  if (fin) {
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int t = wave + 4 * k;
      float* fp = fin + hb * NP + (int64_t)(16 * (nt0 + t / NTp) + g4) * P + 16 * (t % NTp) + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) fp[(int64_t)e * P] = S[k][e];
    }
  }
}

// The same walks for larger states (N P > 8192 or P = 128): a workgroup owns
// 32 state columns (grid (H, batch, P / 32)), two chunks in flight, so that
// the state, the operand fragments and the buffers fit the registers.
template <int N, int P, bool REV>
__global__ __launch_bounds__(256, (N <= 128 ? 3 : 1)) void k_bwd_walk_cols(const bf16* __restrict__ opA,
                                                  const bf16* __restrict__ opX,
                                                  const float* __restrict__ cs,
                                                  const float* __restrict__ dtp, Shape sh,
                                                  const float* __restrict__ start,
                                                  f16* __restrict__ out, int* __restrict__ osc,
                                                  float* __restrict__ fin) {
  constexpr int Q = kBwdChunk, RA = N / 8, NTn = N / 16, NTp = P / 16;
  constexpr int NT = 2 * NTn, TPW = (NT + 3) / 4;
  constexpr int LA = (Q * RA + 255) / 256;  // 16-byte loads of operand rows per thread
  static_assert(Q * 4 == 256, "one 16-byte load of x / dy columns per thread");
  __shared__ __attribute__((aligned(16))) bf16 sA[Q * N];
  __shared__ __attribute__((aligned(16))) bf16 sXh[Q * 32];
  __shared__ __attribute__((aligned(16))) bf16 sXl[Q * 32];

  const int h = blockIdx.x, b = blockIdx.y, z = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = (lane >> 4) * 4, l16 = lane & 15;
  const int64_t hb = (int64_t)b * sh.H + h;
  const int64_t NP = (int64_t)N * P;
  const int ng = REV ? sh.Gc : sh.G, grp = REV ? h / sh.hpgc : h / sh.hpg;
  const bool scales = !REV && (sh.flags & kFlagScalesInput);

  // tile k of this wave: n-tile t / 2, p-tile 2 z + t % 2 (t = wave + 4 k)
  f32x4 S[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = wave + 4 * k;
    S[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (start && t < NT) {
      const float* sp = start + hb * NP + (int64_t)(16 * (t >> 1) + g4) * P + 32 * z + 16 * (t & 1) + l16;
      S[k] = f32x4{sp[0], sp[P], sp[2 * P], sp[3 * P]};
    }
  }
  auto qoff = [&](int t) {  // the tile's fragment-layout offset in a state
    return ((int64_t)((t >> 1) * NTp + 2 * z + (t & 1)) * 64 + lane) * 4;
  };

  // one chunk's operand rows, per-token values and decay, in registers; two
  // chunks are in flight
  // (rows past the chunk end are loaded clamped and zeroed when staged: a
  // select right after the load would wait for it)
  struct Buf {
    bf16x8 ra[LA], rx;
    float rcs, rce, rdt;
    int len;
  };
  const int xt = tid >> 2, xc = tid & 3;  // the x / dy row and 8-column group of this thread
  auto fetch = [&](Buf& f, int c) {
    const int64_t tb = (int64_t)c * Q;
    const int len = (int)min<int64_t>(Q, sh.L - tb);
    const int64_t rowbase = (int64_t)b * sh.L + tb;
#pragma unroll
    for (int k = 0; k < LA; ++k) {
      const int q = min(tid + 256 * k, Q * RA - 1), t = q / RA, cc = q % RA;
      f.ra[k] = *reinterpret_cast<const bf16x8*>(opA + ((rowbase + min(t, len - 1)) * ng + grp) * N + 8 * cc);
    }
    f.rx = *reinterpret_cast<const bf16x8*>(opX + ((rowbase + min(xt, len - 1)) * sh.H + h) * P +
                                            32 * z + 8 * xc);
    f.len = len;
    const float* csc = cs + (hb * sh.nc + c) * Q;
    f.rcs = csc[min(xt, len - 1)];
    f.rce = csc[len - 1];
    f.rdt = scales ? dtp[(hb * sh.nc + c) * Q + min(xt, len - 1)] : 1.f;
  };
  auto stage = [&](const Buf& f) {
#pragma unroll
    for (int k = 0; k < LA; ++k) {
      const int q = tid + 256 * k;
      if (q < Q * RA)
        *reinterpret_cast<bf16x8*>(sA + swz_off<RA>(q / RA, 8 * (q % RA))) = q / RA < f.len ? f.ra[k] : bf16x8{};
    }
    const float w = xt < f.len ? (REV ? __expf(f.rcs) : __expf(f.rce - f.rcs) * f.rdt) : 0.f;
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (float)f.rx[e] * w;
      hi[e] = (bf16)v;
      lo[e] = (bf16)(v - (float)hi[e]);
    }
    *reinterpret_cast<bf16x8*>(sXh + swz_off<4>(xt, 8 * xc)) = hi;
    *reinterpret_cast<bf16x8*>(sXl + swz_off<4>(xt, 8 * xc)) = lo;
  };
  auto cat8 = [](bf16x4 a, bf16x4 c) { return __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7); };
  // the wave's tiles share their p-tile (wave % 2): its x / dy fragments are
  // read once per 32-token step; every fragment of the chunk is read before the
  // first product (one LDS round trip per chunk, not one per tile)
  auto compute = [&]() {
    bf16x8 xh[Q / 32], xl[Q / 32], a[Q / 32][TPW];
    const int pl = 16 * (wave & 1);
#pragma unroll
    for (int s = 0; s < Q / 32; ++s) {
      xh[s] = cat8(tr_frag_swz<4>(sXh, pl, 32 * s, lane), tr_frag_swz<4>(sXh, pl, 32 * s + 16, lane));
      xl[s] = cat8(tr_frag_swz<4>(sXl, pl, 32 * s, lane), tr_frag_swz<4>(sXl, pl, 32 * s + 16, lane));
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int t = min(wave + 4 * k, NT - 1);  // a wave past the last tile reads it again
        a[s][k] = cat8(tr_frag_swz<RA>(sA, 16 * (t >> 1), 32 * s, lane),
                       tr_frag_swz<RA>(sA, 16 * (t >> 1), 32 * s + 16, lane));
      }
    }
#pragma unroll
    for (int s = 0; s < Q / 32; ++s)
#pragma unroll
      for (int k = 0; k < TPW; ++k)
        if (wave + 4 * k < NT) {  // wave-uniform
          S[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s][k], xh[s], S[k], 0, 0, 0);
          S[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s][k], xl[s], S[k], 0, 0, 0);
        }
  };

  const int nc = sh.nc;
  auto chunk_of = [&](int i) { return REV ? nc - 1 - i : i; };  // the i-th chunk walked
  // step i: chunk i's rows (in f) to LDS, the state out and decayed, chunk i + 2
  // requested into f, then chunk i's products
  // (barriers wait for LDS traffic only: __syncthreads would also drain the
  // loads in flight and the state stores)
  auto step = [&](Buf& f, int i) {
    lds_barrier();  // the previous chunk's LDS reads are done
    stage(f);
    const int c = chunk_of(i);
    const int64_t sidx = ((int64_t)b * nc + c) * sh.H + h;
    f16* o = out + sidx * NP;
    const float d = __expf(f.rce);
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int t = wave + 4 * k;
      if (t < NT) {  // wave-uniform
        // the tile as fp16 quads with one power-of-two scale
        const float m = wave_max(
            fmaxf(fmaxf(fabsf(S[k][0]), fabsf(S[k][1])), fmaxf(fabsf(S[k][2]), fabsf(S[k][3]))));
        const int e = tile_exp(m);
        const f32x4 v = S[k];
        *reinterpret_cast<f16x4*>(o + qoff(t)) =
            f16x4{(f16)__builtin_amdgcn_ldexpf(v[0], -e), (f16)__builtin_amdgcn_ldexpf(v[1], -e),
                  (f16)__builtin_amdgcn_ldexpf(v[2], -e), (f16)__builtin_amdgcn_ldexpf(v[3], -e)};
        if (lane == 0) osc[sidx * (NP / 256) + (qoff(t) >> 8)] = e;
        S[k] *= d;
      }
    }
    lds_barrier();
    // unconditional (the last steps read the last chunk again): with loads on
    // one path only the wait in the next stage would drain every load
    fetch(f, chunk_of(min(i + 2, nc - 1)));
    compute();
  };
  Buf f0, f1;
  fetch(f0, chunk_of(0));
  fetch(f1, chunk_of(min(1, nc - 1)));
  int i = 0;
  for (; i + 1 < nc; i += 2) {
    step(f0, i);
    step(f1, i + 1);
  }
  if (i < nc) step(f0, i);
  if (fin) {
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int t = wave + 4 * k;
      if (t < NT) {
        float* fp = fin + hb * NP + (int64_t)(16 * (t >> 1) + g4) * P + 32 * z + 16 * (t & 1) + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) fp[(int64_t)e * P] = S[k][e];
      }
    }
  }
}

// ------------------------------------------------------------------ packed-sequence states
// Packed sequences with their own initial states I_s and final-state gradients
// M_s (section 8.3: each sequence is its own scan; its first state decays I_s).
// The layer is linear in I, and the loss term <M, final> separates, so
//   loss = <dy, y0> + <dy, y_init> + <M, final0> + <M, final_init>
// with y0, final0 the outputs from zero initial states (the packed backward
// above computes the gradients of the first term) and, for token t of
// sequence s (f_t = exp(a_first + ... + a_t), e_t = exp(a_{t+1} + ... +
// a_last), E_s = exp(a_first + ... + a_last), s_t = dt'_t or 1):
//   y_init_t   = f_t I_s^T C_t            final_init = E_s I_s
//   final0     = sum_t e_t s_t B_t x_t^T
// whose gradients this kernel adds:
//   dC_t += f_t I_s dy_t                  dI_s  = sum_t f_t C_t dy_t^T + E_s M_s
//   dB_t += e_t s_t M_s x_t               dx_t += e_t s_t M_s^T B_t
//   ds_t += e_t B_t . M_s x_t
//   da_k += sum_{t >= k} pi_t + sum_{t < k} rho_t + E_s <M_s, I_s>    (k in s)
// with pi_t = f_t C_t . I_s dy_t and rho_t = e_t s_t B_t . M_s x_t; da_k goes
// to dt' (times A) and to dA (times dt'), dt' to dt and dt_bias through the
// clamp and the softplus as in the chunk kernel.
//
// grid (sequences, H), 256 threads; one workgroup walks its sequence's tokens
// in blocks of kSeqTB with I_s (then M_s) in LDS: a walk for the I terms and
// dI, a walk for the M terms, then a walk for da.  Every (token, head) belongs
// to one workgroup, so the read-modify-writes of dx, dt, dBh and dCh do not
// race.
constexpr int kSeqTB = 16;

__device__ inline float block_sum256(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// exclusive prefix sum over the 256 threads (in thread order) and the total
__device__ inline float block_exclusive256(float v, float* red, float& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  float before = 0.f;
  for (int k = 0; k < w; ++k) before += red[k];
  total = red[0] + red[1] + red[2] + red[3];
  return before + inc - v;
}

template <typename T, int N, int P>
__global__ __launch_bounds__(256) void k_bwd_seq_terms(
    const T* __restrict__ x, const T* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ dt_bias,
    const T* __restrict__ dy, const float* __restrict__ dtp, const int32_t* __restrict__ cu,
    const float* __restrict__ init, const float* __restrict__ dfinal, Shape sh,
    T* __restrict__ dx, T* __restrict__ ddt, float* __restrict__ dBh, float* __restrict__ dCh,
    float* __restrict__ dinit, float* __restrict__ tmp, float* __restrict__ spart) {
  using E = Elem<T>;
  constexpr int NP = N * P, LDM = P + 1, TB = kSeqTB, ACC = (NP + 255) / 256;
  __shared__ float sM[N * LDM];  // I_s, then M_s (row n, column p)
  __shared__ float sU[TB * N];   // the block's C rows, then B rows
  __shared__ float sV[TB * P];   // the block's dy rows, then x rows
  __shared__ float sA[TB], sDt[TB], sF[TB], sAcc[TB];
  __shared__ float sRed[4];
  const int sq = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  // per-token sums over n in a fixed order (no atomics, so the result does not
  // depend on the order the threads arrive in): item e = (i, n) of a block's
  // nb N items lies in lane e % 64 of iteration e / 256; the SEG lanes of each
  // aligned segment are summed by a butterfly, the segment sums of token i go
  // to sPart[i N / SEG ..] and thread i adds them in order
  constexpr int SEG = N < 64 ? N : 64;
  __shared__ float sPart[TB * N / SEG];
  auto seg_store = [&](float v, int e, int nitems) {
#pragma unroll
    for (int off = SEG / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (e < nitems && e % SEG == 0) sPart[e / SEG] = v;
  };
  auto seg_finish = [&](int nb) {  // after a barrier: token sums into sAcc
    if (tid < nb) {
      float v = 0.f;
      for (int c = 0; c < N / SEG; ++c) v += sPart[tid * (N / SEG) + c];
      sAcc[tid] = v;
    }
  };
  const int64_t a0 = cu[sq], a1 = cu[sq + 1];
  const int64_t hs = (int64_t)sq * sh.H + h;
  const float Ah = A[h];
  const bool scales = sh.flags & kFlagScalesInput;
  const float* dth = dtp + (int64_t)h * sh.nc * kBwdChunk;  // dt' of token t at dth[t]
  const int gB = h / sh.hpg, gC = h / sh.hpgc;

  // a_t = dt'_t A of the block [t0, t0 + nb) into sA (and dt'_t into sDt)
  auto load_decay = [&](int64_t t0, int nb) {
    if (tid < TB) {
      const float d = tid < nb ? dth[t0 + tid] : 0.f;
      sDt[tid] = d;
      sA[tid] = d * Ah;
    }
  };
  // log of f_t for the block's tokens into sF (after a barrier); returns the
  // carry past the block
  auto prefix = [&](float carry, int nb) {
    if (tid < TB) {
      float c = carry;
      for (int k = 0; k <= tid; ++k) c += sA[k];
      sF[tid] = c;
    }
    for (int k = 0; k < nb; ++k) carry += sA[k];
    return carry;
  };
  // The sequence's total log-decay, summed block by block and token by token in
  // the order the walks below form their prefix sums (every thread alike), so
  // that tot - prefix_t is the rounded sum of the terms after t alone: e_t near
  // the end of the sequence, where it is largest, then carries no cancellation
  // error (a tree sum in another order left dB near 2.6e-4 of its scale in
  // fp32 storage on a 400-token sequence).
  float tot = 0.f;
  for (int64_t t0 = a0; t0 < a1; t0 += TB) {
    const int nb = (int)min<int64_t>(TB, a1 - t0);
    __syncthreads();
    load_decay(t0, nb);
    __syncthreads();
    for (int k = 0; k < nb; ++k) tot += sA[k];
  }
  const float Es = __expf(tot);

  // ---- walk 1: I terms (dC, pi) and dI
  float pi_tot = 0.f;
  if (init || dinit) {
    float acc[ACC];
#pragma unroll
    for (int k = 0; k < ACC; ++k) acc[k] = 0.f;
    if (init)
      for (int e = tid; e < NP; e += 256) sM[(e / P) * LDM + e % P] = init[hs * NP + e];
    float carry = 0.f;
    for (int64_t t0 = a0; t0 < a1; t0 += TB) {
      const int nb = (int)min<int64_t>(TB, a1 - t0);
      __syncthreads();
      load_decay(t0, nb);
      for (int e = tid; e < TB * N; e += 256) {
        const int i = e / N, n = e % N;
        sU[e] = i < nb ? E::to_float(Cm[((t0 + i) * sh.Gc + gC) * N + n]) : 0.f;
      }
      for (int e = tid; e < TB * P; e += 256) {
        const int i = e / P, q = e % P;
        sV[e] = i < nb ? E::to_float(dy[((t0 + i) * sh.H + h) * P + q]) : 0.f;
      }
      if (tid < TB) sAcc[tid] = 0.f;
      __syncthreads();
      carry = prefix(carry, nb);
      __syncthreads();
      if (tid < TB) sF[tid] = __expf(sF[tid]);  // f_t
      __syncthreads();
      if (init) {
        for (int e0 = 0; e0 < nb * N; e0 += 256) {  // every lane takes part in the sums
          const int e = e0 + tid;
          float w = 0.f;
          if (e < nb * N) {
            const int i = e / N, n = e % N;
            float v = 0.f;
            for (int q = 0; q < P; ++q) v += sM[n * LDM + q] * sV[i * P + q];  // (I dy_t)_n
            const float f = sF[i];
            dCh[((t0 + i) * sh.H + h) * N + n] += f * v;
            w = f * sU[i * N + n] * v;
          }
          seg_store(w, e, nb * N);
        }
        __syncthreads();
        seg_finish(nb);
      }
      if (dinit) {
#pragma unroll
        for (int k = 0; k < ACC; ++k) {
          const int e = tid + 256 * k;
          if (e < NP) {
            const int n = e / P, q = e % P;
            for (int i = 0; i < nb; ++i) acc[k] += sF[i] * sU[i * N + n] * sV[i * P + q];
          }
        }
      }
      __syncthreads();
      if (init && tid < nb) tmp[((t0 + tid) * sh.H + h) * 3 + 0] = sAcc[tid];
      if (init)
        for (int i = 0; i < nb; ++i) pi_tot += sAcc[i];
    }
    if (dinit) {
#pragma unroll
      for (int k = 0; k < ACC; ++k) {
        const int e = tid + 256 * k;
        if (e < NP) dinit[hs * NP + e] = acc[k] + (dfinal ? Es * dfinal[hs * NP + e] : 0.f);
      }
    }
  }

  // ---- walk 2: M terms (dB, dx, rho, ds)
  if (dfinal) {
    __syncthreads();
    for (int e = tid; e < NP; e += 256) sM[(e / P) * LDM + e % P] = dfinal[hs * NP + e];
    float carry = 0.f;
    for (int64_t t0 = a0; t0 < a1; t0 += TB) {
      const int nb = (int)min<int64_t>(TB, a1 - t0);
      __syncthreads();
      load_decay(t0, nb);
      for (int e = tid; e < TB * N; e += 256) {
        const int i = e / N, n = e % N;
        sU[e] = i < nb ? E::to_float(Bm[((t0 + i) * sh.G + gB) * N + n]) : 0.f;
      }
      for (int e = tid; e < TB * P; e += 256) {
        const int i = e / P, q = e % P;
        sV[e] = i < nb ? E::to_float(x[((t0 + i) * sh.H + h) * P + q]) : 0.f;
      }
      if (tid < TB) sAcc[tid] = 0.f;
      __syncthreads();
      carry = prefix(carry, nb);
      __syncthreads();
      if (tid < TB) sF[tid] = __expf(tot - sF[tid]);  // e_t
      __syncthreads();
      for (int e0 = 0; e0 < nb * N; e0 += 256) {  // every lane takes part in the sums
        const int e = e0 + tid;
        float w = 0.f;
        if (e < nb * N) {
          const int i = e / N, n = e % N;
          float z = 0.f;
          for (int q = 0; q < P; ++q) z += sM[n * LDM + q] * sV[i * P + q];  // (M x_t)_n
          const float es = sF[i] * (scales ? sDt[i] : 1.f);
          dBh[((t0 + i) * sh.H + h) * N + n] += es * z;
          w = sU[i * N + n] * z;
        }
        seg_store(w, e, nb * N);
      }
      __syncthreads();
      seg_finish(nb);
      for (int e = tid; e < nb * P; e += 256) {
        const int i = e / P, q = e % P;
        float w = 0.f;
        for (int n = 0; n < N; ++n) w += sM[n * LDM + q] * sU[i * N + n];  // (M^T B_t)_p
        const float es = sF[i] * (scales ? sDt[i] : 1.f);
        T* o = dx + ((t0 + i) * sh.H + h) * P + q;
        *o = E::from_float(E::to_float(*o) + es * w);
      }
      __syncthreads();
      if (tid < nb) {
        const float zb = sAcc[tid], et = sF[tid];
        tmp[((t0 + tid) * sh.H + h) * 3 + 1] = et * (scales ? sDt[tid] : 1.f) * zb;  // rho_t
        tmp[((t0 + tid) * sh.H + h) * 3 + 2] = et * zb;                              // ds_t
      }
    }
  }

  // ---- walk 3: da_k = (pi_tot - sum_{t<k} pi_t) + sum_{t<k} rho_t + E_s <M, I>
  float gA = 0.f, gb = 0.f;
  if (init || dfinal) {
    float K = 0.f;
    if (init && dfinal) {
      float d = 0.f;
      for (int e = tid; e < NP; e += 256) d += init[hs * NP + e] * dfinal[hs * NP + e];
      K = Es * block_sum256(d, sRed);
    }
    // tmp written above by other threads of this workgroup
    __syncthreads();
    float cpi = 0.f, crho = 0.f;
    for (int64_t t0 = a0; t0 < a1; t0 += 256) {
      const int64_t t = t0 + tid;
      const bool ok = t < a1;
      const float* tp = tmp + (t * sh.H + h) * 3;
      const float pi = ok && init ? tp[0] : 0.f;
      const float rho = ok && dfinal ? tp[1] : 0.f;
      const float ds = ok && dfinal ? tp[2] : 0.f;
      float tpi, trho;
      const float epi = block_exclusive256(pi, sRed, tpi);
      const float erho = block_exclusive256(rho, sRed, trho);
      if (ok) {
        const float da = (pi_tot - (cpi + epi)) + (crho + erho) + K;
        const float dtv = dth[t];
        const float ddtp = da * Ah + (scales ? ds : 0.f);
        const float pre = E::to_float(dt[t * sh.H + h]) + (dt_bias ? dt_bias[h] : 0.f);
        const bool sp = sh.flags & kFlagSoftplus;
        const float act = sp ? softplus_f32(pre) : pre;
        float gate = (act >= sh.dt_min && act <= sh.dt_max) ? 1.f : 0.f;
        if (sp) gate *= 1.f / (1.f + __expf(-pre));
        const float g = ddtp * gate;
        T* o = ddt + t * sh.H + h;
        *o = E::from_float(E::to_float(*o) + g);
        gA += da * dtv;
        gb += g;
      }
      cpi += tpi;
      crho += trho;
    }
  }
  gA = block_sum256(gA, sRed);
  gb = block_sum256(gb, sRed);
  if (tid == 0) {
    spart[hs * 2 + 0] = gA;
    spart[hs * 2 + 1] = gb;
  }
}

// grid H: dA[h] and dt_bias[h] plus the per-sequence partials, in sequence order.
__global__ __launch_bounds__(256) void k_seq_head_sums(const float* __restrict__ spart, int nseqs,
                                                       int H, float* __restrict__ dA,
                                                       float* __restrict__ dbias) {
  const int h = blockIdx.x;
  float s0 = 0.f, s1 = 0.f;
  for (int q = threadIdx.x; q < nseqs; q += 256) {
    s0 += spart[((int64_t)q * H + h) * 2 + 0];
    s1 += spart[((int64_t)q * H + h) * 2 + 1];
  }
  __shared__ float red[4];
  s0 = block_sum256(s0, red);
  s1 = block_sum256(s1, red);
  if (threadIdx.x == 0) {
    dA[h] += s0;
    if (dbias) dbias[h] += s1;
  }
}

// ------------------------------------------------------------------ launch
bool bwd_supported(int N, int P, bool bf16_storage) {
  if (P != 64 && P != 128) return false;
  if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256) return false;
  // LDS: B, C, x, dy of 64 tokens and one state in the storage type
  return N * P <= (bf16_storage ? 16384 : 8192);
}

template <typename T, int N, int P, bool H16>
static hipError_t bwd_chunk_h(const BwdArgs& a, int hblk, hipStream_t st) {
  static_assert(bwd_lds_bytes<T, N, P>() <= 160 * 1024, "k_bwd_chunk LDS");
  const Shape& sh = a.f.sh;
  hipLaunchKernelGGL((k_bwd_chunk<T, N, P, H16>), dim3(sh.H / hblk, sh.nc, sh.batch), dim3(256), 0, st,
                     (const T*)a.f.x, (const T*)a.f.dt, a.f.A, (const T*)a.f.B, (const T*)a.f.C,
                     a.f.D, a.f.dt_bias, (const T*)a.dy, a.f.cs, a.f.dt_out, a.f.states, a.adj,
                     a.f.coef, a.f.seq_idx, a.f.cinfo, sh, (T*)a.dx, (T*)a.ddt,
                     a.dBh, a.dCh, a.part, a.sc_states, a.sc_adj, hblk);
  return hipGetLastError();
}

// the walks (dense bf16 rows) leave fp16 states with tile scales
template <typename T, int N, int P>
static hipError_t bwd_chunk_t(const BwdArgs& a, int hblk, hipStream_t st) {
  if constexpr (sizeof(T) == 2)
    if (a.walked) return bwd_chunk_h<T, N, P, true>(a, hblk, st);
  return bwd_chunk_h<T, N, P, false>(a, hblk, st);
}

template <typename T, int N>
static hipError_t bwd_chunk_p(const BwdArgs& a, int hblk, hipStream_t st) {
  if (a.P == 64) return bwd_chunk_t<T, N, 64>(a, hblk, st);
  if constexpr (N * 128 <= (sizeof(T) == 2 ? 16384 : 8192))
    if (a.P == 128) return bwd_chunk_t<T, N, 128>(a, hblk, st);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t bwd_chunk_n(const BwdArgs& a, int hblk, hipStream_t st) {
  switch (a.N) {
    case 16: return bwd_chunk_p<T, 16>(a, hblk, st);
    case 32: return bwd_chunk_p<T, 32>(a, hblk, st);
    case 64: return bwd_chunk_p<T, 64>(a, hblk, st);
    case 128: return bwd_chunk_p<T, 128>(a, hblk, st);
    case 256:
      if constexpr (sizeof(T) == 2) return bwd_chunk_p<T, 256>(a, hblk, st);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

// Heads per k_bwd_chunk workgroup: the largest of 8, 4, 2 that divides the
// heads of every B group and every C group while the grid keeps at least four
// workgroups per resident slot (two per CU), else 1; always 1 when
// k_bwd_seq_terms adds per-head terms to the dB / dC rows afterwards.
// SSD_BWD_HEAD_BLOCK=k (1 .. 8) caps the block at k and drops the grid-size
// condition (small problems then take the head-block path too).
int bwd_head_block(const BwdArgs& a) {
  const Shape& sh = a.f.sh;
  if (a.seq_terms || sh.H <= 0) return 1;
  const char* force = std::getenv("SSD_BWD_HEAD_BLOCK");
  const int cap = force ? std::atoi(force) : 0;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int64_t units = (int64_t)sh.H * sh.nc * sh.batch, want = cap > 0 ? 0 : 8 * (int64_t)cus;
  for (int k = 8; k >= 2; k /= 2)
    if ((cap <= 0 || k <= cap) && sh.hpg % k == 0 && sh.hpgc % k == 0 && units / k >= want) return k;
  return 1;
}

template <typename T>
static hipError_t group_sums(const BwdArgs& a, int hblk, hipStream_t st) {
  const Shape& sh = a.f.sh;
  const int64_t rows = (int64_t)sh.batch * sh.L;
  hipError_t e;
  const struct {
    const float* src;
    int ng, hpg;
    void* out;
    const char* name;
  } jobs[2] = {{a.dBh, sh.G, sh.hpg, a.dB, "group_sum_B"}, {a.dCh, sh.Gc, sh.hpgc, a.dC, "group_sum_C"}};
  for (const auto& j : jobs) {
    if (mark(a.f, j.name, st) != hipSuccess) return hipErrorUnknown;
    const int64_t total = rows * j.ng * (a.N / 4);
    const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 16384);
    hipLaunchKernelGGL((k_group_sum<T>), dim3(grid), dim3(256), 0, st, j.src, rows, sh.H / hblk,
                       j.ng, j.hpg / hblk, a.N, (T*)j.out);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bwd_sums(const BwdArgs& a, hipStream_t st) {
  const Shape& sh = a.f.sh;
  if (mark(a.f, "head_sums", st) != hipSuccess) return hipErrorUnknown;
  hipLaunchKernelGGL(k_head_sums, dim3(sh.H), dim3(256), 0, st, a.part, sh.batch, sh.H, sh.nc,
                     a.dA, a.dD, a.ddt_bias);
  return hipGetLastError();
}

template <typename T, int N, int P>
static hipError_t seq_terms_t(const BwdArgs& a, hipStream_t st) {
  const Shape& sh = a.f.sh;
  hipLaunchKernelGGL((k_bwd_seq_terms<T, N, P>), dim3(sh.nseqs, sh.H), dim3(256), 0, st,
                     (const T*)a.f.x, (const T*)a.f.dt, a.f.A, (const T*)a.f.B, (const T*)a.f.C,
                     a.f.dt_bias, (const T*)a.dy, a.f.dt_out, a.f.cu, a.seq_init, a.seq_dfinal, sh,
                     (T*)a.dx, (T*)a.ddt, a.dBh, a.dCh, a.seq_dinit, a.seq_tmp, a.seq_part);
  return hipGetLastError();
}

template <typename T, int N>
static hipError_t seq_terms_p(const BwdArgs& a, hipStream_t st) {
  if (a.P == 64) return seq_terms_t<T, N, 64>(a, st);
  if constexpr (N * 128 <= (sizeof(T) == 2 ? 16384 : 8192))
    if (a.P == 128) return seq_terms_t<T, N, 128>(a, st);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t seq_terms_n(const BwdArgs& a, hipStream_t st) {
  switch (a.N) {
    case 16: return seq_terms_p<T, 16>(a, st);
    case 32: return seq_terms_p<T, 32>(a, st);
    case 64: return seq_terms_p<T, 64>(a, st);
    case 128: return seq_terms_p<T, 128>(a, st);
    case 256:
      if constexpr (sizeof(T) == 2) return seq_terms_p<T, 256>(a, st);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

// Workgroups per (row, head) stream of the walks: the whole state (P = 64,
// N <= 128; its rows split in two from N = 64 on: twice the workgroups, half
// the state each), else 32 state columns each.
constexpr int walk_parts(int N, int P) { return (P == 64 && N <= 128) ? (N >= 64 ? 2 : 1) : P / 32; }

template <int N, int P>
static hipError_t walks_t(const BwdArgs& a, hipStream_t st) {
  const Shape& sh = a.f.sh;
  constexpr bool whole = P == 64 && N <= 128;
  constexpr int NSPL = walk_parts(N, P);
  const dim3 grid(sh.H, sh.batch, NSPL);
  void (*fwd)(const bf16*, const bf16*, const float*, const float*, Shape, const float*, f16*, int*,
              float*);
  decltype(fwd) rev;
  if constexpr (whole) {
    fwd = k_bwd_walk<N, P, false, NSPL>;
    rev = k_bwd_walk<N, P, true, NSPL>;
  } else {
    fwd = k_bwd_walk_cols<N, P, false>;
    rev = k_bwd_walk_cols<N, P, true>;
  }
  if (mark(a.f, "state_walk", st) != hipSuccess) return hipErrorUnknown;
  hipLaunchKernelGGL(fwd, grid, dim3(256), 0, st, (const bf16*)a.f.B, (const bf16*)a.f.x, a.f.cs,
                     a.f.dt_out, sh, a.f.init, reinterpret_cast<f16*>(a.f.states), a.sc_states,
                     nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mark(a.f, "adjoint_walk", st) != hipSuccess) return hipErrorUnknown;
  hipLaunchKernelGGL(rev, grid, dim3(256), 0, st, (const bf16*)a.f.C, (const bf16*)a.dy, a.f.cs,
                     a.f.dt_out, sh, a.dfinal, reinterpret_cast<f16*>(a.adj), a.sc_adj, a.dinit);
  return hipGetLastError();
}

template <int N>
static hipError_t walks_p(const BwdArgs& a, hipStream_t st) {
  if (a.P == 64) return walks_t<N, 64>(a, st);
  if constexpr (N <= 128)
    if (a.P == 128) return walks_t<N, 128>(a, st);
  return hipErrorInvalidValue;
}

bool bwd_walks_supported(const Shape& sh, bool is_bf16) { return is_bf16 && !sh.varlen; }

// Each walk is a chain over a stream's chunks: with fewer workgroups than CUs
// the per-chunk state kernels and the two scans, parallel over chunks, are
// faster (b1 H32 L16384 N128: 0.93 against 1.15 ms per pass), with a full
// grid the walks are (b4 H80 L4096 N128: 1.49 against 2.21 ms).
bool bwd_walks_fill(const Shape& sh, int N, int P) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  return (int64_t)sh.H * sh.batch * walk_parts(N, P) >= cus;
}

hipError_t launch_bwd_walks(const BwdArgs& a, hipStream_t st) {
  if (a.f.sh.nc == 0 || a.f.sh.batch == 0) return hipSuccess;
  switch (a.N) {
    case 16: return walks_p<16>(a, st);
    case 32: return walks_p<32>(a, st);
    case 64: return walks_p<64>(a, st);
    case 128: return walks_p<128>(a, st);
    case 256: return walks_p<256>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_tail(const BwdArgs& a, bool is_bf16, hipStream_t st) {
  const Shape& sh = a.f.sh;
  hipError_t e;
  if (!a.walked) {
    if (mark(a.f, "adjoint_passing", st) != hipSuccess) return hipErrorUnknown;
    hipLaunchKernelGGL(k_adjoint_passing, dim3(bwd_nblk(a.N, a.P), sh.H, sh.batch), dim3(256), 0,
                       st, a.adj, a.f.coef, a.f.cinfo, a.dfinal, sh, a.N, a.P, a.dinit);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int hblk = bwd_head_block(a);
  if (mark(a.f, "bwd_chunk", st) != hipSuccess) return hipErrorUnknown;
  if ((e = is_bf16 ? bwd_chunk_n<bf16>(a, hblk, st) : bwd_chunk_n<float>(a, hblk, st)) != hipSuccess)
    return e;
  if (a.seq_terms) {
    if (mark(a.f, "bwd_seq_terms", st) != hipSuccess) return hipErrorUnknown;
    if ((e = is_bf16 ? seq_terms_n<bf16>(a, st) : seq_terms_n<float>(a, st)) != hipSuccess) return e;
  }
  if ((e = is_bf16 ? group_sums<bf16>(a, hblk, st) : group_sums<float>(a, hblk, st)) != hipSuccess)
    return e;
  if ((e = launch_bwd_sums(a, st)) != hipSuccess) return e;
  if (a.seq_terms) {
    if (mark(a.f, "seq_head_sums", st) != hipSuccess) return hipErrorUnknown;
    hipLaunchKernelGGL(k_seq_head_sums, dim3(sh.H), dim3(256), 0, st, a.seq_part, sh.nseqs, sh.H,
                       a.dA, a.ddt_bias);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ssd
