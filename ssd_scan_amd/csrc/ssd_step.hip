// Single-token step of the SSD layer (recurrent / decode mode).
//
// "Transformers are SSMs" section 3.4.1 (the linear mode, one token at a
// time) with the scalar-times-identity transition of section 2.4: per (row,
// head), from the state S (N x P, fp32, the caller's buffer, updated in place)
//
//     dt' = clamp(act(dt + dt_bias), dt_min, dt_max),  a = exp(dt' A_h)
//     S   = a S + B x^T          (times dt' with the input-scaling flag)
//     y   = S^T C + D_h x
//
// It moves the N x P state through HBM once in each direction and does
// 4 N P flops per (row, head): bound by HBM bandwidth, with no matrix-core
// work.  One workgroup per (head, row); each thread owns one 4-column slice
// p .. p+3 of the state (the same slice in every row it visits), so every
// state access is a coalesced 16-byte load or store, and the column sums of
// y = S^T C reduce through LDS at the end.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kStepThreads = 256;

template <typename T, int P>
__global__ __launch_bounds__(kStepThreads) void k_step(const T* __restrict__ x,
                                                       const T* __restrict__ dt,
                                                       const float* __restrict__ A,
                                                       const T* __restrict__ B,
                                                       const T* __restrict__ C,
                                                       const float* __restrict__ D,
                                                       const float* __restrict__ dt_bias,
                                                       float* __restrict__ state,
                                                       T* __restrict__ y, Shape sh, int N) {
  using E = Elem<T>;
  constexpr int Q4 = P / 4;                   // 16-byte slices per state row
  constexpr int RPP = kStepThreads / Q4;      // state rows per pass of the block
  constexpr int UNROLL = 8;                   // passes whose loads are in flight together
  static_assert(kStepThreads % Q4 == 0, "whole rows per pass");
  __shared__ f32x4 sPart[kStepThreads];

  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int g = h / sh.hpg;
  const int q = tid % Q4, r0 = tid / Q4;  // this thread's column slice and first row

  float dv = E::to_float(dt[(int64_t)b * sh.H + h]) + (dt_bias ? dt_bias[h] : 0.f);
  if (sh.flags & kFlagSoftplus) dv = softplus_f32(dv);
  dv = fminf(fmaxf(dv, sh.dt_min), sh.dt_max);
  const float a = fast_exp(dv * A[h]);
  const float sc = (sh.flags & kFlagScalesInput) ? dv : 1.f;

  const int64_t row = (int64_t)b * sh.H + h;
  const T* xr = x + row * P + 4 * q;
  const f32x4 xv = f32x4{E::to_float(xr[0]), E::to_float(xr[1]), E::to_float(xr[2]),
                         E::to_float(xr[3])};
  const f32x4 sx = sc * xv;
  const T* Br = B + ((int64_t)b * sh.G + g) * N;
  const T* Cr = C + ((int64_t)b * sh.Gc + h / sh.hpgc) * N;
  f32x4* S = reinterpret_cast<f32x4*>(state + row * (int64_t)N * P) + q;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int n0 = r0; n0 < N; n0 += RPP * UNROLL) {
    f32x4 sv[UNROLL];
    float bn[UNROLL], cn[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {  // every load of the group in flight first
      const int n = n0 + k * RPP;
      if (n < N) {
        sv[k] = S[(int64_t)n * Q4];
        bn[k] = E::to_float(Br[n]);
        cn[k] = E::to_float(Cr[n]);
      }
    }
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const int n = n0 + k * RPP;
      if (n < N) {
        const f32x4 s = a * sv[k] + bn[k] * sx;
        S[(int64_t)n * Q4] = s;
        acc += cn[k] * s;
      }
    }
  }
  // y[p] = sum over the rows of C[n] S[n][p]: the RPP partial sums of each
  // column slice meet in LDS
  sPart[tid] = acc;
  __syncthreads();
  if (tid < Q4) {
    f32x4 s = D ? D[h] * xv : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k = 0; k < RPP; ++k) s += sPart[k * Q4 + tid];
    T* yr = y + row * P + 4 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) yr[e] = E::from_float(s[e]);
  }
}

template <typename T>
static hipError_t step_p(const StepArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.sh.H, (unsigned)a.sh.batch);
  const T* x = static_cast<const T*>(a.x);
  const T* dt = static_cast<const T*>(a.dt);
  const T* B = static_cast<const T*>(a.B);
  const T* C = static_cast<const T*>(a.C);
  T* y = static_cast<T*>(a.y);
  switch (a.P) {
    case 64:
      hipLaunchKernelGGL((k_step<T, 64>), grid, dim3(kStepThreads), 0, st, x, dt, a.A, B, C, a.D,
                         a.dt_bias, a.state, y, a.sh, a.N);
      break;
    case 128:
      hipLaunchKernelGGL((k_step<T, 128>), grid, dim3(kStepThreads), 0, st, x, dt, a.A, B, C, a.D,
                         a.dt_bias, a.state, y, a.sh, a.N);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs& a, bool is_bf16, hipStream_t st) {
  if (a.sh.batch == 0 || a.sh.H == 0) return hipSuccess;
  return is_bf16 ? step_p<bf16>(a, st) : step_p<float>(a, st);
}

}  // namespace ssd
