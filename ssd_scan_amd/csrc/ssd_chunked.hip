// Chunked (four-kernel) schedule of the SSD forward pass for gfx950.
//
// "Transformers are SSMs" section 6 splits the sequence into chunks of Q
// tokens.  The semiseparable matrix then has diagonal blocks (section 6.1:
// within-chunk outputs from a zero initial state, in the quadratic dual form
// (L o C B^T) X) and low-rank off-diagonal blocks (section 6.2: right factors
// give each chunk's state assuming no earlier input, a scalar scan passes
// states across chunks, left factors turn the incoming state into outputs).
// Section 6.3 notes the scan is Q times cheaper than a token scan.  Kernels:
//
//   k_seq_index      token -> packed sequence (variable length, section 8.3)
//   k_dt_cumsum      dt' = clamp(softplus(dt + bias)), log-decay dt' A and its
//                    inclusive prefix sum inside each chunk (the a = 1 case of
//                    the scalar scan, appendix B.1), wave-level scans
//   k_chunk_state    right factors: S_c = sum_j exp(cs_end - cs_j) B_j x_j^T
//                    (MFMA, B and x staged transposed through LDS); the same
//                    kernel gives the final state of each packed sequence
//   k_state_passing  S_in[c+1] = exp(cs_end[c]) S_in[c] + S_c, sequential over
//                    chunks, fp32, float4-coalesced, in place
//   k_chunk_scan     Y = (L o C B^T) X + diag(exp(cs)) C S_in + D x per chunk
//                    (MFMA; L built on chip from prefix-sum differences)
//   k_chunk_state_pipe, k_chunk_scan_pipe
//                    the same two steps for bf16 storage with N P <= 16384,
//                    B and x streamed straight into a ring of LDS stages
//
// Chunk states live in the workspace in "fragment layout": 16 x 16 tiles of
// the N x P state in (n-tile, p-tile) order, each tile as 64 lanes x 4 floats
// where lane l holds column p = l % 16 and rows n = 4 (l / 16) .. +3.  That is
// the MFMA output layout of the chunk-state kernels, so every access is a
// 16-byte-per-lane contiguous move.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"
#include "ssd_lds.hpp"

namespace ssd {

// ------------------------------------------------------------------ helpers
template <int TPL>
__device__ inline float pick(const float (&v)[TPL], int k) {
  float r = v[0];
#pragma unroll
  for (int i = 1; i < TPL; ++i) r = (k == i) ? v[i] : r;
  return r;
}

// dst[col * LDT + jj] = src[jj * stride + col] * (w ? w[jj] : 1) for col < W and
// jj in [lo, hi); zero for other jj < KB.  Global reads are 4 consecutive
// elements per thread along col (coalesced); LDS writes land token-contiguous.
template <typename T, int KB, int W, int LDT, int NTHR>
__device__ inline void stage_transposed(T* __restrict__ dst, const T* __restrict__ src,
                                        int64_t stride, int lo, int hi,
                                        const float* __restrict__ w) {
  using E = Elem<T>;
  // every load of a thread is issued before its first LDS store
  if constexpr (sizeof(T) == 2) {
    constexpr int ITEMS = (KB / 2) * (W / 4), IT = (ITEMS + NTHR - 1) / NTHR;
    f32x4 va[IT], vb[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int it = threadIdx.x + NTHR * k;
      const int c4 = it % (W / 4), j0 = 2 * (it / (W / 4));
      va[k] = vb[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (it < ITEMS && j0 >= lo && j0 < hi) va[k] = E::to_f32(load_frag(src + j0 * stride + 4 * c4));
      if (it < ITEMS && j0 + 1 >= lo && j0 + 1 < hi)
        vb[k] = E::to_f32(load_frag(src + (j0 + 1) * stride + 4 * c4));
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int it = threadIdx.x + NTHR * k;
      if (it >= ITEMS) break;
      const int c4 = it % (W / 4), j0 = 2 * (it / (W / 4));
      f32x4 a = va[k], b = vb[k];
      if (w) {
        a *= w[j0];
        b *= w[j0 + 1];
      }
      const bf16x4 ca = E::from_f32(a), cb = E::from_f32(b);
      // tokens j0 and j0 + 1 of column 4 c4 + e are adjacent in dst: one 4-byte store
      *reinterpret_cast<bf16x2*>(dst + (4 * c4 + 0) * LDT + j0) = bf16x2{ca.x, cb.x};
      *reinterpret_cast<bf16x2*>(dst + (4 * c4 + 1) * LDT + j0) = bf16x2{ca.y, cb.y};
      *reinterpret_cast<bf16x2*>(dst + (4 * c4 + 2) * LDT + j0) = bf16x2{ca.z, cb.z};
      *reinterpret_cast<bf16x2*>(dst + (4 * c4 + 3) * LDT + j0) = bf16x2{ca.w, cb.w};
    }
  } else {
    constexpr int ITEMS = KB * (W / 4), IT = (ITEMS + NTHR - 1) / NTHR;
    f32x4 va[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int it = threadIdx.x + NTHR * k;
      const int c4 = it % (W / 4), j = it / (W / 4);
      va[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (it < ITEMS && j >= lo && j < hi) va[k] = E::to_f32(load_frag(src + j * stride + 4 * c4));
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int it = threadIdx.x + NTHR * k;
      if (it >= ITEMS) break;
      const int c4 = it % (W / 4), j = it / (W / 4);
      f32x4 a = va[k];
      if (w) a *= w[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(4 * c4 + e) * LDT + j] = a[e];
    }
  }
}

// The same staging for bf16 with the weighted values split in two bf16 terms,
// v = hi + lo with lo = bf16(v - hi), into dst and dst_lo.
template <int KB, int W, int LDT, int NTHR>
__device__ inline void stage_transposed_split(bf16* __restrict__ dst, bf16* __restrict__ dst_lo,
                                              const bf16* __restrict__ src, int64_t stride,
                                              int lo, int hi, const float* __restrict__ w) {
  using E = Elem<bf16>;
  constexpr int ITEMS = KB * (W / 4), IT = (ITEMS + NTHR - 1) / NTHR;
  bf16x4 va[IT];
#pragma unroll
  for (int k = 0; k < IT; ++k) {  // every load before the first LDS store
    const int it = threadIdx.x + NTHR * k;
    const int c4 = it % (W / 4), j = it / (W / 4);
    va[k] = zero_frag<bf16>();
    if (it < ITEMS && j >= lo && j < hi) va[k] = load_frag(src + j * stride + 4 * c4);
  }
#pragma unroll
  for (int k = 0; k < IT; ++k) {
    const int it = threadIdx.x + NTHR * k;
    if (it >= ITEMS) break;
    const int c4 = it % (W / 4), j = it / (W / 4);
    const f32x4 a = E::to_f32(va[k]) * w[j];
    const bf16x4 h = E::from_f32(a), l = E::from_f32(a - E::to_f32(h));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[(4 * c4 + e) * LDT + j] = h[e];
      dst_lo[(4 * c4 + e) * LDT + j] = l[e];
    }
  }
}

// The incoming state is kept in fp32 by the scan across chunks, but the
// state-to-output product runs on the bf16 matrix cores.  A single bf16
// rounding of the state costs up to 2^-9 of |S| in every output, which does
// not shrink with the chunk (it is the long-memory path), so for bf16 storage
// the state is split into two bf16 terms, S = hi + lo with lo = bf16(S - hi),
// and the product is done twice (relative error ~2^-17).  fp32 storage uses
// fp32 matrix-core products and needs no split.
template <typename T>
struct StateTerms { static constexpr int n = 1; };
template <>
struct StateTerms<bf16> { static constexpr int n = 2; };

// Writes the 4 fp32 state values of fragment quad q as StateTerms<T>::n terms,
// term t at sS[t * NP + 4 q].
template <typename T, int NP>
__device__ inline void put_state_quad(T* sS, int q, f32x4 v) {
  using E = Elem<T>;
  const typename E::frag hi = E::from_f32(v);
  store_frag(sS + 4 * q, hi);
  if constexpr (StateTerms<T>::n == 2) store_frag(sS + NP + 4 * q, E::from_f32(v - E::to_f32(hi)));
}

// (state^T C^T) tile for p-tile pt of a 16-token tile whose C fragments are cfu:
// sum over the state terms and the n k-blocks.
template <typename T, int N, int P>
__device__ inline f32x4 state_to_output(const T* sS, const typename Elem<T>::frag* cfu, int pt,
                                        int lane) {
  using E = Elem<T>;
  constexpr int NKn = N / 16, NKn2 = (NKn + 1) / 2, NTp = P / 16, NP = N * P;
  f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int term = 0; term < StateTerms<T>::n; ++term) {
    const T* base = sS + term * NP + lane * 4;
#pragma unroll
    for (int k2 = 0; k2 < NKn2; ++k2) {
      const typename E::frag a0 = load_frag(base + ((2 * k2) * NTp + pt) * 256);
      const typename E::frag a1 = (2 * k2 + 1 < NKn) ? load_frag(base + ((2 * k2 + 1) * NTp + pt) * 256)
                                                     : zero_frag<T>();
      t = E::mma2(t, a0, a1, cfu[2 * k2], cfu[2 * k2 + 1]);
    }
  }
  return t;
}

// ------------------------------------------------------------------ K0
__global__ void k_seq_index(const int32_t* __restrict__ cu, int nseqs, int64_t T,
                            int32_t* __restrict__ seq_idx) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = nseqs;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  seq_idx[t] = lo;
}

// ------------------------------------------------------------------ K1
// grid (nc, batch, ceil(H / 8)), 256 threads: one chunk of one batch row for 8
// heads.  dt loads run along the head axis (contiguous), dt' goes through LDS,
// and one wave per head forms the prefix sums and writes them token-contiguous.
constexpr int kCumsumHeads = 8;

template <typename T, int Q>
__global__ __launch_bounds__(256) void k_dt_cumsum(
    const T* __restrict__ dt, const float* __restrict__ A, const float* __restrict__ dt_bias,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_idx, Shape sh,
    float* __restrict__ dt_out, float* __restrict__ cs_out, float2* __restrict__ coef,
    ChunkInfo* __restrict__ cinfo) {
  constexpr int TPL = Q / 64;
  constexpr int RPT = Q * kCumsumHeads / 256;  // dt values per thread
  __shared__ float sD[kCumsumHeads][Q + 1];
  __shared__ float sA[kCumsumHeads];
  const int c = blockIdx.x, b = blockIdx.y, h0 = blockIdx.z * kCumsumHeads;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: branches on it are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)c * Q;
  const int len = (int)min<int64_t>(Q, sh.L - t0);
  ChunkInfo ci;
  if (sh.varlen) {
    ci.seq_first = seq_idx[t0];
    ci.seq_last = seq_idx[t0 + len - 1];
    ci.start_first = cu[ci.seq_first];
    ci.start_last = cu[ci.seq_last];
  } else {
    ci.seq_first = ci.seq_last = b;
    ci.start_first = ci.start_last = 0;
  }
  if (tid == 0 && blockIdx.z == 0 && cinfo) cinfo[(int64_t)b * sh.nc + c] = ci;
  const int64_t row0 = (int64_t)b * sh.L + t0;
  {
    const int hl = tid % kCumsumHeads, h = min(h0 + hl, sh.H - 1), i0 = tid / kCumsumHeads;
    const float bias = dt_bias ? dt_bias[h] : 0.f;
    if (tid < kCumsumHeads) sA[hl] = A[h];
    T raw[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k)  // every load in flight before any use
      raw[k] = dt[(row0 + min(i0 + k * (256 / kCumsumHeads), len - 1)) * sh.H + h];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int i = i0 + k * (256 / kCumsumHeads);
      float dv = Elem<T>::to_float(raw[k]) + bias;
      if (sh.flags & kFlagSoftplus) dv = softplus_f32(dv);
      sD[hl][i] = i < len ? fminf(fmaxf(dv, sh.dt_min), sh.dt_max) : 0.f;
    }
  }
  __syncthreads();
  for (int hl = wave; hl < kCumsumHeads && h0 + hl < sh.H; hl += 4) {
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
      v[k] += excl;
      dt_out[base + k] = d[k];
      cs_out[base + k] = v[k];
    }
    if (coef) {
      // decay applied to the incoming state by the end of the chunk: through
      // the whole chunk, or (when the last sequence starts inside it) from
      // that sequence's start, in the second component
      const int il = len - 1;
      const float cs_last = __shfl(pick<TPL>(v, il % TPL), il / TPL, 64);
      float2 cf;
      if (ci.start_last <= t0) {
        cf = make_float2(fast_exp(cs_last), 0.f);
      } else {
        const int ip = ci.start_last - 1 - (int)t0;
        const float csp = __shfl(pick<TPL>(v, ip % TPL), ip / TPL, 64);
        cf = make_float2(0.f, fast_exp(cs_last - csp));
      }
      if (lane == 0) coef[((int64_t)b * sh.H + h) * sh.nc + c] = cf;
    }
  }
}

// ------------------------------------------------------------------ K2 / final states
// FINAL = false: grid (H, nc, batch); S_c of each chunk (for the sequence of the
//   chunk's last token) into the fragment-layout state buffer.
// FINAL = true : grid (H, nseqs), packed sequences only; state after each
//   sequence's last token = in-chunk part + decayed incoming/initial state, in
//   the caller's (S, H, N, P) layout.
// REV = true (with FINAL = false): the backward pass's chunk-local adjoint
//   R_c = sum_t exp(cs_t) C_t dy_t^T over the tokens of the chunk's first
//   sequence, the gradient a chunk's outputs send to the state entering it --
//   the same contraction with C for B (by C group), dy for x and the decay
//   from the chunk start instead of to its end.
// SPLIT = true (bf16 only): the weighted x (or dy) operand goes to the matrix
//   cores as two bf16 terms, so the states carry no bf16 rounding of it (the
//   forward pass's final states and left factors; the backward pass's decay
//   gradient is a sum of state products).
template <typename T, int N, int P, bool FINAL, bool REV = false, bool SPLIT = false>
__global__ __launch_bounds__(256) void k_chunk_state(
    const T* __restrict__ x, const T* __restrict__ Bm, const float* __restrict__ cs,
    const float* __restrict__ dtp, const ChunkInfo* __restrict__ cinfo,
    const int32_t* __restrict__ cu, const float* __restrict__ states,
    const float* __restrict__ init, int Q, Shape sh, float* __restrict__ out) {
  using E = Elem<T>;
  constexpr int KB = E::kStage;
  constexpr int LDT = KB + 4;
  constexpr int NTp = P / 16;
  constexpr int NT = (N / 16) * NTp;
  constexpr int TPW = (NT + 3) / 4;
  static_assert(!SPLIT || sizeof(T) == 2, "the split operand is for bf16 storage");
  __shared__ T sBT[N * LDT];
  __shared__ T sXT[(SPLIT ? 2 : 1) * P * LDT];
  __shared__ float sW[KB];

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: branches on it are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = (lane >> 4) * 4, l16 = lane & 15;
  const int h = blockIdx.x;
  const int64_t NP = (int64_t)N * P;
  int b, c, s = 0;
  int64_t te, js;  // last token and first contributing token (within the row)
  float coef_src = 0.f;
  const float* src = nullptr;
  bool src_frag = false;
  if constexpr (!FINAL) {
    c = blockIdx.y;
    b = blockIdx.z;
    const int64_t tb = (int64_t)c * Q;
    te = min<int64_t>(tb + Q, sh.L) - 1;
    if constexpr (REV) {
      // the adjoint of the state entering the chunk gathers the tokens of the
      // chunk's first sequence only (packed input)
      js = tb;
      if (sh.varlen) te = min<int64_t>(te, (int64_t)cu[cinfo[c].seq_first + 1] - 1);
    } else {
      js = max<int64_t>(tb, cinfo[(int64_t)b * sh.nc + c].start_last);
    }
  } else {
    s = blockIdx.y;
    b = 0;
    const int64_t a0 = cu[s], a1 = cu[s + 1];
    float* o = out + ((int64_t)s * sh.H + h) * NP;
    if (a0 == a1) {  // empty sequence: its final state is its initial state
      const float* ip = init ? init + ((int64_t)s * sh.H + h) * NP : nullptr;
      for (int64_t e = tid; e < NP; e += 256) o[e] = ip ? ip[e] : 0.f;
      return;
    }
    te = a1 - 1;
    c = (int)(te / Q);
    const int64_t tb = (int64_t)c * Q;
    js = max<int64_t>(tb, a0);
    const float* csc = cs + ((int64_t)h * sh.nc + c) * Q;
    const float cs_te = csc[te - tb];
    if (a0 <= tb) {
      coef_src = fast_exp(cs_te);
      src = states + ((int64_t)c * sh.H + h) * NP;
      src_frag = true;
    } else if (init) {
      coef_src = fast_exp(cs_te - csc[a0 - 1 - tb]);
      src = init + ((int64_t)s * sh.H + h) * NP;
    }
  }
  const int grp = REV ? h / sh.hpgc : h / sh.hpg;
  const int ngrp = REV ? sh.Gc : sh.G;
  const int64_t tb = (int64_t)c * Q;
  const float* csc = cs + (((int64_t)b * sh.H + h) * sh.nc + c) * Q;
  const float* dtc = dtp + (((int64_t)b * sh.H + h) * sh.nc + c) * Q;
  const float cs_te = csc[te - tb];
  const bool scales = sh.flags & kFlagScalesInput;
  const int64_t rowbase = (int64_t)b * sh.L + tb;

  f32x4 acc[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ilo = (int)(js - tb), ihi = (int)(te - tb) + 1;  // contributing tokens [ilo, ihi)
  for (int sb = (ilo / KB) * KB; sb < ihi; sb += KB) {
    if (tid < KB) {
      const int i = sb + tid;
      float w = 0.f;
      if (i >= ilo && i < ihi) {
        if constexpr (REV) {
          w = fast_exp(csc[i]);
        } else {
          w = fast_exp(cs_te - csc[i]);
          if (scales) w *= dtc[i];
        }
      }
      sW[tid] = w;
    }
    __syncthreads();
    const int lo = max(ilo - sb, 0), hi = min(ihi - sb, KB);
    stage_transposed<T, KB, N, LDT, 256>(sBT, Bm + ((rowbase + sb) * ngrp + grp) * N,
                                         (int64_t)ngrp * N, lo, hi, nullptr);
    if constexpr (SPLIT) {
      stage_transposed_split<KB, P, LDT, 256>((bf16*)sXT, (bf16*)sXT + P * LDT,
                                              (const bf16*)x + ((rowbase + sb) * sh.H + h) * P,
                                              (int64_t)sh.H * P, lo, hi, sW);
    } else {
      stage_transposed<T, KB, P, LDT, 256>(sXT, x + ((rowbase + sb) * sh.H + h) * P,
                                           (int64_t)sh.H * P, lo, hi, sW);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KB / 32; ++kk) {
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int t = wave + 4 * k;
        if (t < NT) {
          const int nt = t / NTp, pt = t % NTp;
          const T* ar = sBT + (16 * nt + l16) * LDT + 32 * kk + g4;
          const T* br = sXT + (16 * pt + l16) * LDT + 32 * kk + g4;
          acc[k] = E::mma2(acc[k], load_frag(ar), load_frag(ar + 16), load_frag(br),
                           load_frag(br + 16));
          if constexpr (SPLIT)
            acc[k] = E::mma2(acc[k], load_frag(ar), load_frag(ar + 16), load_frag(br + P * LDT),
                             load_frag(br + P * LDT + 16));
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = wave + 4 * k;
    if (t >= NT) continue;
    if constexpr (!FINAL) {
      float* o = out + (((int64_t)b * sh.nc + c) * sh.H + h) * NP + ((int64_t)t * 64 + lane) * 4;
      *reinterpret_cast<f32x4*>(o) = acc[k];
    } else {
      const int nt = t / NTp, pt = t % NTp;
      const int p = 16 * pt + l16;
      float* o = out + ((int64_t)s * sh.H + h) * NP;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = 16 * nt + g4 + r;
        float v = acc[k][r];
        if (src) {
          const float sv = src_frag ? src[((int64_t)t * 64 + lane) * 4 + r] : src[(int64_t)n * P + p];
          v += coef_src * sv;
        }
        o[(int64_t)n * P + p] = v;
      }
    }
  }
}

// ------------------------------------------------------------------ K2, bf16 streaming form
// S_c = sum_j B_j^T w_j x_j for bf16 storage with N P <= 16384: B and x rows go
// straight into a three-deep ring of 32-token LDS stages (as in the streaming
// chunk scan), the contraction over tokens reads both operands with the
// transposing LDS load, and w_j scales the x^T fragments in registers.  The
// 4 waves split the (n-tile, p-tile) grid into equal blocks.
template <int N, int P, int Q>
struct PipeStateCfg {
  static constexpr int W = 4, NTHR = 64 * W;
  static constexpr int RB = N / 8, RX = P / 8;
  static constexpr int NTn = N / 16, NTp = P / 16;
  static constexpr int WN = NTn < W ? NTn : W, WP = W / WN;  // waves along n and p
  static constexpr int SN = NTn / WN, SP = NTp / WP;         // tiles per wave along n and p
  static constexpr int SB = 32 * N, SX = 32 * P, STAGE = SB + SX;
  static constexpr int NSB = SB / 512, NSX = SX / 512;
  static constexpr int KPW = (NSB + NSX + W - 1) / W;
  static_assert(WN * SN == NTn && WP * SP == NTp, "even split of the tile grid");
};

template <int N, int P, int Q>
__global__ __launch_bounds__((PipeStateCfg<N, P, Q>::NTHR)) void k_chunk_state_pipe(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const float* __restrict__ cs,
    const float* __restrict__ dtp, const ChunkInfo* __restrict__ cinfo, Shape sh,
    float* __restrict__ out) {
  using F = PipeStateCfg<N, P, Q>;
  using E = Elem<bf16>;
  constexpr int W = F::W, SN = F::SN, SP = F::SP, NTp = F::NTp;
  __shared__ __attribute__((aligned(16))) bf16 sStage[3][F::STAGE];
  __shared__ __attribute__((aligned(16))) float sW[Q];

  const int h = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: branches on it are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = (lane >> 4) * 4;
  const int grp = h / sh.hpg;
  const int64_t tb = (int64_t)c * Q;
  const int len = (int)min<int64_t>(Q, sh.L - tb);
  const int64_t rowbase = (int64_t)b * sh.L + tb;
  // contributing tokens: those of the chunk's last sequence
  const int ilo = (int)(max<int64_t>(tb, cinfo[(int64_t)b * sh.nc + c].start_last) - tb);
  const int64_t cso = (((int64_t)b * sh.H + h) * sh.nc + c) * Q;
  const bool scales = sh.flags & kFlagScalesInput;
  const int nst = (len + 31) / 32;
  const int nt0 = (wave % F::WN) * SN, pt0 = (wave / F::WN) * SP;

  const bf16* bsrc = Bm + (rowbase * sh.G + grp) * N;
  const bf16* xsrc = x + (rowbase * sh.H + h) * P;
  auto issue = [&](int st) {
    bf16* dst = sStage[st % 3];
#pragma unroll
    for (int m = 0; m < F::KPW; ++m) {
      const int k = (wave + W * m) % (F::NSB + F::NSX);
      if (k < F::NSB)
        dma_rows<F::RB>(dst, bsrc, sh.G * N, 32 * st, len, lane, k);
      else
        dma_rows<F::RX>(dst + F::SB, xsrc, sh.H * P, 32 * st, len, lane, k - F::NSB);
    }
  };
  asm volatile("" ::: "memory");
  issue(0);
  if (nst > 1) issue(1);
  asm volatile("" ::: "memory");
  if (tid < Q) {
    const int i = min(tid, len - 1);
    const float w = fast_exp(cs[cso + len - 1] - cs[cso + i]) * (scales ? dtp[cso + i] : 1.f);
    sW[tid] = (tid >= ilo && tid < len) ? w : 0.f;
  }
  f32x4 acc[SN][SP];
#pragma unroll
  for (int a = 0; a < SN; ++a)
#pragma unroll
    for (int p = 0; p < SP; ++p) acc[a][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) {
      constexpr int K = F::KPW;
      static_assert(K < 64, "vmcnt field");
      __builtin_amdgcn_s_waitcnt((K & 15) | ((K >> 4) << 14) | (7 << 4) | (15 << 8));
    } else {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    }
    lds_barrier();  // (the first one also publishes sW)
    asm volatile("" ::: "memory");
    if (st + 2 < nst) issue(st + 2);
    asm volatile("" ::: "memory");
    const bf16* sB = sStage[st % 3];
    const bf16* sX = sB + F::SB;
    // w_j x_j^T fragments of this wave's p-tiles for the stage's two j-blocks,
    // as two bf16 terms (hi + lo) so that the states carry no bf16 rounding of
    // the weighted x (one term left the final states near 1.5e-2 of their
    // scale with the input-scaling flag)
    bf16x4 xw[SP][2], xl[SP][2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(&sW[32 * st + 16 * e + g4]);
#pragma unroll
      for (int p = 0; p < SP; ++p) {
        const f32x4 v = E::to_f32(tr_frag_swz<F::RX>(sX, 16 * (pt0 + p), 16 * e, lane)) * w;
        xw[p][e] = E::from_f32(v);
        xl[p][e] = E::from_f32(v - E::to_f32(xw[p][e]));
      }
    }
#pragma unroll
    for (int a = 0; a < SN; ++a) {
      const bf16x4 b0 = tr_frag_swz<F::RB>(sB, 16 * (nt0 + a), 0, lane);
      const bf16x4 b1 = tr_frag_swz<F::RB>(sB, 16 * (nt0 + a), 16, lane);
#pragma unroll
      for (int p = 0; p < SP; ++p) {
        acc[a][p] = E::mma2(acc[a][p], b0, b1, xw[p][0], xw[p][1]);
        acc[a][p] = E::mma2(acc[a][p], b0, b1, xl[p][0], xl[p][1]);
      }
    }
  }
  // tile (n-tile, p-tile) in fragment order: lane holds column p, rows 4 (l / 16) .. + 3
  float* o = out + (((int64_t)b * sh.nc + c) * sh.H + h) * (int64_t)(N * P);
#pragma unroll
  for (int a = 0; a < SN; ++a)
#pragma unroll
    for (int p = 0; p < SP; ++p)
      *reinterpret_cast<f32x4*>(o + ((int64_t)((nt0 + a) * NTp + pt0 + p) * 64 + lane) * 4) = acc[a][p];
}

// ------------------------------------------------------------------ K3
// One thread owns 4 consecutive fragment-layout elements of one (row, head)
// state; loops over the row's chunks.  Replaces each chunk state S_c by the
// incoming state S_in[c] (in place) and, without cu_seqlens, writes the state
// after the last chunk as the final state.  The chunks go in batches of 8, and
// the next batch's loads (chunk states, decay coefficients, and with packed
// sequences the next chunks' sequence info) are issued before the current
// batch is processed, so two batches of loads are in flight behind the
// sequential recurrence.
__global__ __launch_bounds__(256) void k_state_passing(
    float* __restrict__ states, const float2* __restrict__ coef,
    const ChunkInfo* __restrict__ cinfo, const float* __restrict__ init, Shape sh, int Q, int N,
    int P, float* __restrict__ final_states) {
  const int NP = N * P;
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q * 4 >= NP) return;
  const int h = blockIdx.y, b = blockIdx.z;
  const int NTp = P / 16;
  const int tile = q >> 6, ln = q & 63;
  const int n0 = 16 * (tile / NTp) + 4 * (ln >> 4), p = 16 * (tile % NTp) + (ln & 15);
  auto load_init = [&](int s) -> f32x4 {
    if (!init) return f32x4{0.f, 0.f, 0.f, 0.f};
    const float* ip = init + ((int64_t)s * sh.H + h) * NP + (int64_t)n0 * P + p;
    return f32x4{ip[0], ip[P], ip[2 * P], ip[3 * P]};
  };
  const ChunkInfo* cib = cinfo + (int64_t)b * sh.nc;
  f32x4* sq = reinterpret_cast<f32x4*>(states + ((int64_t)b * sh.nc * sh.H + h) * NP) + q;
  const int64_t cstride = (int64_t)sh.H * NP / 4;  // f32x4 between consecutive chunks
  const float2* cf = coef + ((int64_t)b * sh.H + h) * sh.nc;
  constexpr int BATCH = 8;
  struct Batch {
    f32x4 s[BATCH];
    float2 k[BATCH];
    int fresh[BATCH];  // chunk c + 1 starts a sequence (packed input)
  };
  auto load = [&](Batch& t, int c0) {
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int c = min(c0 + k, sh.nc - 1);
      t.s[k] = sq[c * cstride];
      t.k[k] = cf[c];
      t.fresh[k] = (sh.varlen && c + 1 < sh.nc) ? (cib[c + 1].start_first == (int64_t)(c + 1) * Q)
                                               : 0;
    }
  };
  f32x4 S = load_init(sh.varlen ? cib[0].seq_first : b);
  f32x4 Send = S;
  Batch cur, nxt;
  load(cur, 0);
  for (int c0 = 0; c0 < sh.nc; c0 += BATCH) {
    if (c0 + BATCH < sh.nc) load(nxt, c0 + BATCH);
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int c = c0 + k;
      if (c >= sh.nc) break;
      sq[c * cstride] = S;
      Send = cur.k[k].x * S + cur.s[k];
      if (init && cur.k[k].y != 0.f) Send += cur.k[k].y * load_init(cib[c].seq_last);
      if (c + 1 < sh.nc) S = cur.fresh[k] ? load_init(cib[c + 1].seq_first) : Send;
    }
    cur = nxt;
  }
  if (final_states) {
    float* o = final_states + ((int64_t)b * sh.H + h) * NP + (int64_t)n0 * P + p;
    o[0] = Send[0];
    o[P] = Send[1];
    o[2 * P] = Send[2];
    o[3 * P] = Send[3];
  }
}

// ------------------------------------------------------------------ K4
template <int Q>
struct ScanShape {
  static constexpr int NI = Q / 16;               // 16-token output tiles
  static constexpr int W = NI >= 16 ? 8 : NI;     // waves per block
  static constexpr int ITW = NI / W;              // tiles per wave (1 or 2)
  static constexpr int NTHR = 64 * W;
};

template <typename T, int N, int P, int Q>
__global__ __launch_bounds__(ScanShape<Q>::NTHR) void k_chunk_scan(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ D, const float* __restrict__ cs, const float* __restrict__ dtp,
    const int32_t* __restrict__ seq_idx, const ChunkInfo* __restrict__ cinfo,
    const int32_t* __restrict__ cu, const float* __restrict__ states,
    const float* __restrict__ init, Shape sh, T* __restrict__ y) {
  using E = Elem<T>;
  using frag = typename E::frag;
  using SS = ScanShape<Q>;
  constexpr int NS = StateTerms<T>::n;
  // the largest bf16 state (N * P = 32768, split in two terms) leaves room for 32-token stages
  constexpr int KB = (NS * N * P * (int)sizeof(T) > 65536) ? 32 : E::kStage;
  constexpr int NI = SS::NI, W = SS::W, ITW = SS::ITW, NTHR = SS::NTHR;
  constexpr int NKn = N / 16, NKn2 = (NKn + 1) / 2, NTp = P / 16;
  constexpr int LDB = N + 4, LDX = KB + 4;
  __shared__ __attribute__((aligned(16))) T sS[NS * N * P];
  __shared__ __attribute__((aligned(16))) T sB[KB * LDB];
  __shared__ __attribute__((aligned(16))) T sX[P * LDX];
  __shared__ float sCs[Q];
  __shared__ float sDt[Q];
  __shared__ int32_t sSeq[Q];

  const int h = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: branches on it are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = (lane >> 4) * 4, l16 = lane & 15;
  const int grp = h / sh.hpg;
  const int64_t tb = (int64_t)c * Q;
  const int len = (int)min<int64_t>(Q, sh.L - tb);
  const int64_t rowbase = (int64_t)b * sh.L + tb;
  const ChunkInfo ci = cinfo[(int64_t)b * sh.nc + c];
  const int64_t cso = (((int64_t)b * sh.H + h) * sh.nc + c) * Q;
  const bool scales = sh.flags & kFlagScalesInput;
  const int64_t NP = (int64_t)N * P;

  for (int i = tid; i < Q; i += NTHR) {
    sCs[i] = cs[cso + i];
    sDt[i] = dtp[cso + i];
    sSeq[i] = (sh.varlen && i < len) ? seq_idx[tb + i] : ci.seq_first;
  }
  int itile[ITW];
  itile[0] = wave;
  if constexpr (ITW == 2) itile[1] = NI - 1 - wave;

  frag cf[ITW][2 * NKn2];
#pragma unroll
  for (int u = 0; u < ITW; ++u) {
    const int i = itile[u] * 16 + l16;
    const T* cr = Cm + ((rowbase + i) * sh.Gc + h / sh.hpgc) * N + g4;
#pragma unroll
    for (int kb = 0; kb < 2 * NKn2; ++kb)
      cf[u][kb] = (kb < NKn && i < len) ? load_frag(cr + 16 * kb) : zero_frag<T>();
  }
  const float* Sin = states + (((int64_t)b * sh.nc + c) * sh.H + h) * NP;
  for (int q = tid; q < N * P / 4; q += NTHR)
    put_state_quad<T, N * P>(sS, q, reinterpret_cast<const f32x4*>(Sin)[q]);
  __syncthreads();

  // left factors: incoming state -> outputs, scaled by the decay from the chunk start
  f32x4 acc[ITW][NTp];
#pragma unroll
  for (int u = 0; u < ITW; ++u) {
    const int i = itile[u] * 16 + l16;
    const float coef = (sSeq[i] == ci.seq_first) ? fast_exp(sCs[i]) : 0.f;
#pragma unroll
    for (int pt = 0; pt < NTp; ++pt)
      acc[u][pt] = state_to_output<T, N, P>(sS, cf[u], pt, lane) * coef;
  }

  // sequences that start strictly inside the chunk begin from their own initial state
  if (sh.varlen && init) {
    for (int s = ci.seq_first + 1; s <= ci.seq_last; ++s) {
      const int a0 = cu[s], a1 = cu[s + 1];
      if (a0 == a1) continue;
      __syncthreads();
      const float* ip = init + ((int64_t)s * sh.H + h) * NP;
      for (int q = tid; q < N * P / 4; q += NTHR) {
        const int tile = q >> 6, ln = q & 63;
        const int n0 = 16 * (tile / NTp) + 4 * (ln >> 4), p = 16 * (tile % NTp) + (ln & 15);
        const float* e = ip + (int64_t)n0 * P + p;
        put_state_quad<T, N * P>(sS, q, f32x4{e[0], e[P], e[2 * P], e[3 * P]});
      }
      __syncthreads();
      const float csp = sCs[a0 - 1 - tb];
#pragma unroll
      for (int u = 0; u < ITW; ++u) {
        const int i0 = itile[u] * 16;
        if (i0 + 15 < a0 - tb || i0 >= a1 - tb) continue;
        const int i = i0 + l16;
        const float coef = (i < len && sSeq[i] == s) ? fast_exp(sCs[i] - csp) : 0.f;
#pragma unroll
        for (int pt = 0; pt < NTp; ++pt)
          acc[u][pt] += state_to_output<T, N, P>(sS, cf[u], pt, lane) * coef;
      }
    }
  }

  // diagonal block: Y^T += X^T (L o C B^T)^T, streamed over KB-token stages of j
  for (int sb = 0; sb < len; sb += KB) {
    __syncthreads();
    for (int q = tid; q < KB * (N / 4); q += NTHR) {
      const int jj = q / (N / 4), c4 = q % (N / 4);
      const int i = sb + jj;
      const frag v = (i < len) ? load_frag(Bm + ((rowbase + i) * sh.G + grp) * N + 4 * c4)
                               : zero_frag<T>();
      store_frag(sB + jj * LDB + 4 * c4, v);
    }
    stage_transposed<T, KB, P, LDX, NTHR>(sX, x + ((rowbase + sb) * sh.H + h) * P,
                                          (int64_t)sh.H * P, 0, min(len - sb, KB),
                                          scales ? sDt + sb : nullptr);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < ITW; ++u) {
      const int it = itile[u];
      const int kb_lo = sb / 16;
      if (kb_lo > it) continue;
      const int i = it * 16 + l16;
      const float csi = sCs[i];
      const int seqi = sSeq[i];
#pragma unroll
      for (int kp = 0; kp < KB / 32; ++kp) {
        const int kb0 = kb_lo + 2 * kp;
        if (kb0 > it) break;
        frag m[2], ml[2];  // hi + lo (lo stays zero in fp32)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int kb = kb0 + e;
          ml[e] = zero_frag<T>();
          if (kb > it) {
            m[e] = zero_frag<T>();
            continue;
          }
          f32x4 gacc = {0.f, 0.f, 0.f, 0.f};
          const T* br = sB + (kb * 16 - sb + l16) * LDB + g4;
#pragma unroll
          for (int k2 = 0; k2 < NKn2; ++k2) {
            const frag a0 = load_frag(br + 32 * k2);
            const frag a1 = (2 * k2 + 1 < NKn) ? load_frag(br + 32 * k2 + 16) : zero_frag<T>();
            gacc = E::mma2(gacc, a0, a1, cf[u][2 * k2], cf[u][2 * k2 + 1]);
          }
          f32x4 mv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = kb * 16 + g4 + r;
            const bool ok = (j <= i) && (i < len) && (sSeq[j] == seqi);
            mv[r] = ok ? fast_exp(csi - sCs[j]) * gacc[r] : 0.f;
          }
          m[e] = E::from_f32(mv);
          if constexpr (!std::is_same<T, float>::value) ml[e] = E::from_f32(mv - E::to_f32(m[e]));
        }
#pragma unroll
        for (int pt = 0; pt < NTp; ++pt) {
          const T* xr = sX + (16 * pt + l16) * LDX + (kb0 * 16 - sb) + g4;
          const frag x0 = load_frag(xr), x1 = load_frag(xr + 16);
          acc[u][pt] = E::mma2(acc[u][pt], x0, x1, m[0], m[1]);
          if constexpr (!std::is_same<T, float>::value) acc[u][pt] = E::mma2(acc[u][pt], x0, x1, ml[0], ml[1]);
        }
      }
    }
  }

  // skip term and store
  const float Dh = D ? D[h] : 0.f;
#pragma unroll
  for (int u = 0; u < ITW; ++u) {
    const int i = itile[u] * 16 + l16;
    if (i >= len) continue;
    const int64_t xo = ((rowbase + i) * sh.H + h) * P;
#pragma unroll
    for (int pt = 0; pt < NTp; ++pt) {
      const int p0 = 16 * pt + g4;
      const f32x4 xv = E::to_f32(load_frag(x + xo + p0));
      store_frag(y + xo + p0, E::from_f32(acc[u][pt] + Dh * xv));
    }
  }
}

// ------------------------------------------------------------------ K4, bf16 streaming form
// The same chunk scan for bf16 storage when the incoming state, as two bf16
// terms, fits next to a three-deep ring of 32-token stages (N P <= 16384).
// Wave w owns the output tiles w and Q/16 - 1 - w (equal causal work).  B and
// x rows go from global memory straight into swizzled LDS tiles
// (global_load_lds_dwordx4, no registers), two stages ahead of the one being
// used, so every stage's loads have the products of the stages before it to
// land behind.  The decay mask exp(cs_i - cs_j) is applied as
// exp(cs_i - r) exp(r - cs_j), r the prefix sum at the end of j's 16-token
// block: one exp per lane and tile plus a per-token table.  The C fragments
// carry 8 consecutive n per lane, the layout both C B^T (over B rows) and the
// state-to-output product (over the transposed state) consume.
template <int N, int P, int Q>
struct PipeScanCfg {
  static constexpr int NI = Q / 16, W = NI / 2, NTHR = 64 * W;
  static constexpr int RB = N / 8, RX = P / 8;  // 16-byte chunks per B / x row
  static constexpr int NKn2 = (N / 16 + 1) / 2, NTp = P / 16, NTn = N / 16;
  static constexpr int LDS_T = N + 8;           // pitch of the transposed state's rows
  static constexpr int SB = 32 * N, SX = 32 * P, STAGE = SB + SX;  // stage tiles (elements)
  static constexpr int NSB = SB / 512, NSX = SX / 512;             // 1 KB loads per stage tile
  // loads each wave issues per stage (the count is the same for every wave,
  // so waits can count them; padding repeats a real load of the same bytes)
  static constexpr int KPW = (NSB + NSX + W - 1) / W;
  static constexpr int NQ = (N * P / 4 + NTHR - 1) / NTHR;  // state quads per thread
  // LDS bytes, and the waves per SIMD to build for: two blocks per CU when
  // their LDS fits and, at 8 waves per block (registers then capped at 128 per
  // lane), the C fragments and accumulators are small enough (P = 64, N <= 64)
  // for the stage loop to stay clear of spills; else one
  static constexpr int LDS = 2 * (2 * P * LDS_T + 3 * STAGE) + 12 * Q;
  static constexpr int BPC = (2 * LDS <= 160 * 1024 && (W < 8 || (P == 64 && N <= 64))) ? 2 : 1;
  static constexpr int WPE = BPC * W / 4 > 1 ? BPC * W / 4 : 1;
};

template <int N, int P, int Q>
__global__ __launch_bounds__((PipeScanCfg<N, P, Q>::NTHR)) __attribute__((amdgpu_waves_per_eu(PipeScanCfg<N, P, Q>::WPE, PipeScanCfg<N, P, Q>::WPE)))
void k_chunk_scan_pipe(const bf16* __restrict__ x, const bf16* __restrict__ Bm,
                       const bf16* __restrict__ Cm, const float* __restrict__ D,
                       const float* __restrict__ cs, const float* __restrict__ dtp,
                       const int32_t* __restrict__ seq_idx, const ChunkInfo* __restrict__ cinfo,
                       const int32_t* __restrict__ cu, const float* __restrict__ states,
                       const float* __restrict__ init, Shape sh, bf16* __restrict__ y) {
  using F = PipeScanCfg<N, P, Q>;
  using E = Elem<bf16>;
  constexpr int NI = F::NI, W = F::W, NTHR = F::NTHR, NKn2 = F::NKn2, NTp = F::NTp;
  constexpr int LDS_T = F::LDS_T, NP = N * P;
  __shared__ __attribute__((aligned(16))) bf16 sS[2 * P * LDS_T];  // S_in as hi/lo terms, p-major
  __shared__ __attribute__((aligned(16))) bf16 sStage[3][F::STAGE];
  __shared__ __attribute__((aligned(16))) float sCs[Q];  // prefix sums of dt' A
  __shared__ __attribute__((aligned(16))) float sBt[Q];  // exp(r_block - cs_j) (x dt'_j if scaled)
  __shared__ int sLs[Q];                                 // where token j's sequence starts in the chunk

  const int h = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: branches on it are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = (lane >> 4) * 4, g8 = 2 * g4, l16 = lane & 15;
  const int grp = h / sh.hpg;
  const int64_t tb = (int64_t)c * Q;
  const int len = (int)min<int64_t>(Q, sh.L - tb);
  const int64_t rowbase = (int64_t)b * sh.L + tb;
  const ChunkInfo ci = cinfo[(int64_t)b * sh.nc + c];
  const int64_t cso = (((int64_t)b * sh.H + h) * sh.nc + c) * Q;
  const bool scales = sh.flags & kFlagScalesInput;
  const int it0 = wave, it1 = NI - 1 - wave;
  const int nst = (len + 31) / 32;

  const bf16* bsrc = Bm + (rowbase * sh.G + grp) * N;
  const bf16* xsrc = x + (rowbase * sh.H + h) * P;
  auto issue = [&](int st) {  // this wave's loads of stage st into ring slot st % 3
    bf16* dst = sStage[st % 3];
#pragma unroll
    for (int m = 0; m < F::KPW; ++m) {
      const int k = (wave + W * m) % (F::NSB + F::NSX);
      if (k < F::NSB)
        dma_rows<F::RB>(dst, bsrc, sh.G * N, 32 * st, len, lane, k);
      else
        dma_rows<F::RX>(dst + F::SB, xsrc, sh.H * P, 32 * st, len, lane, k - F::NSB);
    }
  };
  asm volatile("" ::: "memory");
  issue(0);
  if (nst > 1) issue(1);
  asm volatile("" ::: "memory");

  // per-token tables (threads past the chunk repeat its last token)
  if (tid < Q) {
    const int i = min(tid, len - 1);
    const float csv = cs[cso + i];
    const float csb = cs[cso + min(tid | 15, len - 1)];
    sCs[tid] = csv;
    sBt[tid] = fast_exp(csb - csv) * (scales ? dtp[cso + i] : 1.f);
    sLs[tid] = sh.varlen ? (int)max<int64_t>((int64_t)cu[seq_idx[tb + i]] - tb, 0) : 0;
  }
  // C fragments of the two output tiles: row 16 it + l % 16 (rows past the
  // chunk repeat the last), n = 32 k2 + 8 (l / 16) .. + 7 (zero past N)
  bf16x8 cf[2][NKn2];
  {
    const int its[2] = {it0, it1};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = min(its[t] * 16 + l16, len - 1);
      const char* cr = reinterpret_cast<const char*>(Cm + (rowbase * sh.Gc + h / sh.hpgc) * N) +
                       (unsigned)(i * sh.Gc * N + (g8 % N)) * 2u;
#pragma unroll
      for (int k2 = 0; k2 < NKn2; ++k2) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(cr + 64 * k2);
        cf[t][k2] = (N >= 32 || g8 < N) ? v : bf16x8{};
      }
    }
  }
  // the incoming state (fragment layout) into LDS as two bf16 terms, p-major
  auto put_state = [&](const float* src_frag) {
    f32x4 v[F::NQ];
#pragma unroll
    for (int k = 0; k < F::NQ; ++k) {
      const int q = tid + k * NTHR;
      v[k] = q < NP / 4 ? reinterpret_cast<const f32x4*>(src_frag)[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < F::NQ; ++k) {
      const int q = tid + k * NTHR;
      if (q >= NP / 4) continue;
      const int tile = q >> 6, ql = q & 63;
      bf16* st = sS + (16 * (tile % NTp) + (ql & 15)) * LDS_T + 16 * (tile / NTp) + 4 * (ql >> 4);
      const bf16x4 hi = E::from_f32(v[k]);
      store_frag(st, hi);
      store_frag(st + P * LDS_T, E::from_f32(v[k] - E::to_f32(hi)));
    }
  };
  put_state(states + (((int64_t)b * sh.nc + c) * sh.H + h) * NP);
  lds_barrier();

  const float csi0 = sCs[it0 * 16 + l16], csi1 = sCs[it1 * 16 + l16];
  const int lsi0 = sLs[it0 * 16 + l16], lsi1 = sLs[it1 * 16 + l16];
  // y^T[p][i] += k_i sum_n S[n][p] C[i][n] for both output tiles
  f32x4 acc[2][NTp];
  auto state_out = [&](float k0, float k1, bool first) {
#pragma unroll
    for (int pt = 0; pt < NTp; ++pt) {
      f32x4 tso[2][2] = {};
#pragma unroll
      for (int term = 0; term < 2; ++term)
#pragma unroll
        for (int k2 = 0; k2 < NKn2; ++k2) {
          const bf16* sp = sS + term * P * LDS_T + (16 * pt + l16) * LDS_T + 32 * k2 + (g8 % N);
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(sp);
          const bf16x8 sv = (N >= 32 || g8 < N) ? v : bf16x8{};
#pragma unroll
          for (int u = 0; u < 2; ++u) tso[u][term] = mma8(tso[u][term], sv, cf[u][k2]);
        }
      const f32x4 a0 = k0 * (tso[0][0] + tso[0][1]), a1 = k1 * (tso[1][0] + tso[1][1]);
      acc[0][pt] = first ? a0 : acc[0][pt] + a0;
      acc[1][pt] = first ? a1 : acc[1][pt] + a1;
    }
  };
  // left factors: only the chunk's first sequence sees S_in
  state_out(lsi0 > 0 ? 0.f : fast_exp(csi0), lsi1 > 0 ? 0.f : fast_exp(csi1), true);
  // sequences that start strictly inside the chunk begin from their own initial state
  if (sh.varlen && init) {
    for (int sq = ci.seq_first + 1; sq <= ci.seq_last; ++sq) {
      const int64_t a0 = cu[sq], a1 = cu[sq + 1];
      if (a0 == a1) continue;
      const int lo = (int)(a0 - tb), hi = (int)min<int64_t>(a1 - tb, len);
      lds_barrier();  // every wave is done reading sS
      const float* ip = init + ((int64_t)sq * sh.H + h) * NP;
      for (int q = tid; q < NP; q += NTHR) {
        const int n = q / P, p = q % P;
        const float v = ip[q];
        const bf16 vh = E::from_float(v);
        sS[p * LDS_T + n] = vh;
        sS[(P + p) * LDS_T + n] = E::from_float(v - E::to_float(vh));
      }
      lds_barrier();
      const float csp = sCs[lo - 1];
      const int i0 = it0 * 16 + l16, i1 = it1 * 16 + l16;
      state_out((i0 >= lo && i0 < hi) ? fast_exp(csi0 - csp) : 0.f,
                (i1 >= lo && i1 < hi) ? fast_exp(csi1 - csp) : 0.f, false);
    }
  }

  // diagonal blocks, one 32-token stage (two j-blocks) at a time
  auto load_b_rows = [&](const bf16* sB, int jb, bf16x8 (&ba)[NKn2]) {
    const int j = 16 * jb + l16;
#pragma unroll
    for (int k2 = 0; k2 < NKn2; ++k2) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(sB + swz_off<F::RB>(j, 32 * k2 + (g8 % N)));
      ba[k2] = (N >= 32 || g8 < N) ? v : bf16x8{};
    }
  };
  auto gram = [&](const bf16x8 (&ba)[NKn2], const bf16x8 (&cc)[NKn2]) {
    f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < NKn2; ++k2) g = mma8(g, ba[k2], cc[k2]);
    return g;
  };
  // masked C B^T tile as a bf16 pair hi + lo (hi alone keeps 8 bits)
  auto mask = [&](f32x4 g, int kb, int it, float csi, int lsi, bf16x4& lo) {
    const float e = fast_exp(csi - sCs[16 * kb + 15]);
    const f32x4 bj = *reinterpret_cast<const f32x4*>(&sBt[16 * kb + g4]);
    f32x4 mv;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      mv[r] = ((kb < it || (kb == it && g4 + r <= l16)) && 16 * kb + g4 + r >= lsi) ? e * bj[r] * g[r]
                                                                                     : 0.f;
    const bf16x4 hi = E::from_f32(mv);
    lo = E::from_f32(mv - E::to_f32(hi));
    return hi;
  };
  for (int st = 0; st < nst; ++st) {
    // this wave's loads of stage st have landed once at most those of stage
    // st + 1 are in flight; the barrier extends that to every wave's
    if (st + 1 < nst) {
      constexpr int K = F::KPW;
      static_assert(K < 64, "vmcnt field");
      __builtin_amdgcn_s_waitcnt((K & 15) | ((K >> 4) << 14) | (7 << 4) | (15 << 8));
    } else {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    }
    lds_barrier();
    asm volatile("" ::: "memory");
    if (st + 2 < nst) issue(st + 2);
    asm volatile("" ::: "memory");
    const bf16* sB = sStage[st % 3];
    const bf16* sX = sB + F::SB;
    const int ka = 2 * st, kc = 2 * st + 1;
    if (ka <= it1) {  // wave-uniform
      const bool both = ka <= it0;  // wave-uniform
      // the masked C B^T tiles of the two j-blocks, one j-block's B rows at a time
      bf16x4 m1[2], m0[2], l1[2], l0[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        bf16x8 bc[NKn2];
        load_b_rows(sB, e, bc);
        m1[e] = mask(gram(bc, cf[1]), ka + e, it1, csi1, lsi1, l1[e]);
        l0[e] = bf16x4{};
        m0[e] = both ? mask(gram(bc, cf[0]), ka + e, it0, csi0, lsi0, l0[e]) : bf16x4{};
      }
#pragma unroll
      for (int pt = 0; pt < NTp; ++pt) {
        const bf16x4 xa0 = tr_frag_swz<F::RX>(sX, 16 * pt, 0, lane);
        const bf16x4 xa1 = tr_frag_swz<F::RX>(sX, 16 * pt, 16, lane);
        acc[1][pt] = E::mma2(acc[1][pt], xa0, xa1, m1[0], m1[1]);
        acc[1][pt] = E::mma2(acc[1][pt], xa0, xa1, l1[0], l1[1]);
        if (both) {
          acc[0][pt] = E::mma2(acc[0][pt], xa0, xa1, m0[0], m0[1]);
          acc[0][pt] = E::mma2(acc[0][pt], xa0, xa1, l0[0], l0[1]);
        }
      }
    }
  }

  // skip term and store: lane holds y[16 it + l % 16][16 pt + 4 (l / 16) .. + 3]
  const float Dh = D ? D[h] : 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = (u == 0 ? it0 : it1) * 16 + l16;
    if (i >= len) continue;
    const int64_t xo = ((rowbase + i) * sh.H + h) * P;
#pragma unroll
    for (int pt = 0; pt < NTp; ++pt) {
      const int p0 = 16 * pt + g4;
      const f32x4 xv = E::to_f32(load_frag(x + xo + p0));
      store_frag(y + xo + p0, E::from_f32(acc[u][pt] + Dh * xv));
    }
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_seq_index(const int32_t* cu, int nseqs, int64_t T, int32_t* seq_idx,
                            hipStream_t st) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_seq_index, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, cu, nseqs,
                     T, seq_idx);
  return hipGetLastError();
}

template <typename T, int Q>
static hipError_t dt_cumsum_t(const ChunkedArgs& a, hipStream_t st) {
  if (mark(a, "dt_cumsum", st) != hipSuccess) return hipErrorUnknown;
  hipLaunchKernelGGL((k_dt_cumsum<T, Q>),
                     dim3(a.sh.nc, a.sh.batch, (a.sh.H + kCumsumHeads - 1) / kCumsumHeads),
                     dim3(256), 0, st,
                     (const T*)a.dt, a.A, a.dt_bias, a.cu, a.seq_idx, a.sh, a.dt_out, a.cs,
                     a.coef, a.cinfo);
  return hipGetLastError();
}

template <typename T>
static hipError_t dt_cumsum_q(const ChunkedArgs& a, int Q, hipStream_t st) {
  switch (Q) {
    case 64: return dt_cumsum_t<T, 64>(a, st);
    case 128: return dt_cumsum_t<T, 128>(a, st);
    case 256: return dt_cumsum_t<T, 256>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dt_cumsum(const ChunkedArgs& a, int Q, bool is_bf16, hipStream_t st) {
  if (a.sh.nc == 0 || a.sh.batch == 0) return hipSuccess;
  return is_bf16 ? dt_cumsum_q<bf16>(a, Q, st) : dt_cumsum_q<float>(a, Q, st);
}

template <typename T, int N, int P, int Q>
static hipError_t chunked_tail(const ChunkedArgs& a, bool with_scan, hipStream_t st) {
  const Shape& sh = a.sh;
  if (mark(a, "chunk_state", st) != hipSuccess) return hipErrorUnknown;
  if constexpr (sizeof(T) == 2) {
    if (!with_scan) {  // states for the backward pass: bf16 operand in two terms
      hipLaunchKernelGGL((k_chunk_state<T, N, P, false, false, true>), dim3(sh.H, sh.nc, sh.batch),
                         dim3(256), 0, st, (const T*)a.x, (const T*)a.B, a.cs, a.dt_out, a.cinfo,
                         a.cu, a.states, a.init, Q, sh, a.states);
      goto passing;
    }
  }
  if constexpr (sizeof(T) == 2 && N * P <= 16384) {
    hipLaunchKernelGGL((k_chunk_state_pipe<N, P, Q>), dim3(sh.H, sh.nc, sh.batch),
                       dim3(PipeStateCfg<N, P, Q>::NTHR), 0, st, (const bf16*)a.x,
                       (const bf16*)a.B, a.cs, a.dt_out, a.cinfo, sh, a.states);
  } else {
    hipLaunchKernelGGL((k_chunk_state<T, N, P, false, false, sizeof(T) == 2>),
                       dim3(sh.H, sh.nc, sh.batch), dim3(256), 0, st, (const T*)a.x,
                       (const T*)a.B, a.cs, a.dt_out, a.cinfo, a.cu, a.states, a.init, Q, sh,
                       a.states);
  }
passing:
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int NP = N * P;
  if (mark(a, "state_passing", st) != hipSuccess) return hipErrorUnknown;
  hipLaunchKernelGGL(k_state_passing, dim3((NP / 4 + 255) / 256, sh.H, sh.batch), dim3(256), 0,
                     st, a.states, a.coef, a.cinfo, a.init, sh, Q, N, P,
                     sh.varlen ? nullptr : a.final_states);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!with_scan) return hipSuccess;
  if (mark(a, "chunk_scan", st) != hipSuccess) return hipErrorUnknown;
  if constexpr (sizeof(T) == 2 && N * P <= 16384) {
    hipLaunchKernelGGL((k_chunk_scan_pipe<N, P, Q>), dim3(sh.H, sh.nc, sh.batch),
                       dim3(PipeScanCfg<N, P, Q>::NTHR), 0, st, (const bf16*)a.x, (const bf16*)a.B,
                       (const bf16*)a.C, a.D, a.cs, a.dt_out, a.seq_idx, a.cinfo, a.cu, a.states,
                       a.init, sh, (bf16*)a.y);
  } else {
    hipLaunchKernelGGL((k_chunk_scan<T, N, P, Q>), dim3(sh.H, sh.nc, sh.batch),
                       dim3(ScanShape<Q>::NTHR), 0, st, (const T*)a.x, (const T*)a.B,
                       (const T*)a.C, a.D, a.cs, a.dt_out, a.seq_idx, a.cinfo, a.cu, a.states,
                       a.init, sh, (T*)a.y);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (sh.varlen && a.final_states && sh.nseqs > 0) {
    if (mark(a, "final_states", st) != hipSuccess) return hipErrorUnknown;
    hipLaunchKernelGGL((k_chunk_state<T, N, P, true, false, sizeof(T) == 2>), dim3(sh.H, sh.nseqs),
                       dim3(256), 0, st,
                       (const T*)a.x, (const T*)a.B, a.cs, a.dt_out, a.cinfo, a.cu, a.states,
                       a.init, Q, sh, a.final_states);
    e = hipGetLastError();
  }
  return e;
}

// Final states of a problem with no tokens at all (nothing else to do).
__global__ void k_copy_init(const float* __restrict__ init, int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = init ? init[i] : 0.f;
}

hipError_t launch_empty_final(const float* init, int64_t n, float* out, hipStream_t st) {
  if (n <= 0 || !out) return hipSuccess;
  hipLaunchKernelGGL(k_copy_init, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, init, n,
                     out);
  return hipGetLastError();
}

#define SSD_DISPATCH_Q(T, N, P)                                     \
  switch (Q) {                                                      \
    case 64: return chunked_tail<T, N, P, 64>(a, with_scan, st);               \
    case 128: return chunked_tail<T, N, P, 128>(a, with_scan, st);             \
    case 256: return chunked_tail<T, N, P, 256>(a, with_scan, st);             \
  }                                                                 \
  return hipErrorInvalidValue;

template <typename T, int N>
static hipError_t chunked_p(const ChunkedArgs& a, int P, int Q, bool with_scan, hipStream_t st) {
  if (P == 64) { SSD_DISPATCH_Q(T, N, 64) }
  if (P == 128) { SSD_DISPATCH_Q(T, N, 128) }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t chunked_n(const ChunkedArgs& a, int N, int P, int Q, bool with_scan,
                            hipStream_t st) {
  switch (N) {
    case 16: return chunked_p<T, 16>(a, P, Q, with_scan, st);
    case 32: return chunked_p<T, 32>(a, P, Q, with_scan, st);
    case 64: return chunked_p<T, 64>(a, P, Q, with_scan, st);
    case 128: return chunked_p<T, 128>(a, P, Q, with_scan, st);
    case 256:
      if constexpr (sizeof(T) == 2) return chunked_p<T, 256>(a, P, Q, with_scan, st);
      else if (P == 64) { SSD_DISPATCH_Q(T, 256, 64) }
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunked_tail(const ChunkedArgs& a, int N, int P, int Q, bool is_bf16,
                               hipStream_t st) {
  if (a.sh.nc == 0 || a.sh.batch == 0) return hipSuccess;
  return is_bf16 ? chunked_n<bf16>(a, N, P, Q, true, st) : chunked_n<float>(a, N, P, Q, true, st);
}

hipError_t launch_chunk_states(const ChunkedArgs& a, int N, int P, int Q, bool is_bf16,
                               hipStream_t st) {
  if (a.sh.nc == 0 || a.sh.batch == 0) return hipSuccess;
  return is_bf16 ? chunked_n<bf16>(a, N, P, Q, false, st)
                 : chunked_n<float>(a, N, P, Q, false, st);
}

// Chunk-local adjoints of the backward pass (dense rows): dy plays x and C
// plays B in the chunk-state contraction; out in the fragment layout.
template <typename T, int N>
static hipError_t adjoint_p(const ChunkedArgs& a, const void* dy, float* out, int P, int Q,
                            hipStream_t st) {
  const Shape& sh = a.sh;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(sh.H, sh.nc, sh.batch), dim3(256), 0, st, (const T*)dy,
                       (const T*)a.C, a.cs, a.dt_out, a.cinfo, a.cu, a.states, a.init, Q, sh, out);
    return hipGetLastError();
  };
  constexpr bool split = sizeof(T) == 2;
  if (P == 64) return go(k_chunk_state<T, N, 64, false, true, split>);
  if (P == 128) return go(k_chunk_state<T, N, 128, false, true, split>);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_adjoint(const ChunkedArgs& a, const void* dy, float* out, int N, int P,
                                int Q, bool is_bf16, hipStream_t st) {
  if (a.sh.nc == 0 || a.sh.batch == 0) return hipSuccess;
  if (mark(a, "chunk_adjoint", st) != hipSuccess) return hipErrorUnknown;
  switch (N) {
    case 16: return is_bf16 ? adjoint_p<bf16, 16>(a, dy, out, P, Q, st) : adjoint_p<float, 16>(a, dy, out, P, Q, st);
    case 32: return is_bf16 ? adjoint_p<bf16, 32>(a, dy, out, P, Q, st) : adjoint_p<float, 32>(a, dy, out, P, Q, st);
    case 64: return is_bf16 ? adjoint_p<bf16, 64>(a, dy, out, P, Q, st) : adjoint_p<float, 64>(a, dy, out, P, Q, st);
    case 128: return is_bf16 ? adjoint_p<bf16, 128>(a, dy, out, P, Q, st) : adjoint_p<float, 128>(a, dy, out, P, Q, st);
    case 256: return is_bf16 ? adjoint_p<bf16, 256>(a, dy, out, P, Q, st) : hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
