/*
 * Oracle for the SSD (state space duality) forward pass and its gradients
 * (ssd_ref_bwd, at the end of this file).  TEST INFRASTRUCTURE
 * ONLY: nothing on the product path may link, load or call this file.  It is
 * used by tests/, by __graft_entry__.smoke() and by the cpu_baseline leg of
 * bench.py, and nowhere else.
 *
 * What it computes is the plain definition of the layer, run as the
 * token-by-token linear (recurrent) mode ("Transformers are SSMs", paperlayer
 * summary, section 3.4.1 "The Linear (Recurrent) Mode", with the scalar
 * recurrence of section 3.2.2 and the scalar-times-identity transition of
 * section 2.4).  Per head h (B group g = h / (H/G) and C group
 * gc = h / (H/Gc), section 7.1 / 7.2: B heads shared by H/G and C heads by
 * H/Gc consecutive x heads; G = Gc is the multi-value pattern, G = 1 with
 * Gc = H the multi-contract one, G = H with Gc = 1 the multi-expand one),
 * starting from the initial state S (N x P, zero when none is given):
 *
 *     dt'   = clamp(act(dt[t,h] + dt_bias[h]), dt_min, dt_max)
 *     a_t   = exp(dt' * A[h])
 *     S     = a_t * S + B[t,g,:] (x) x[t,h,:]     (times dt' if SCALES_INPUT)
 *     y[t,h,:] = S^T C[t,gc,:] + D[h] * x[t,h,:]
 *
 * act is the identity, or softplus(v) = max(v,0) + log1p(exp(-|v|)) when
 * flag bit 0 is set.  The D skip term is the feed-through of the continuous
 * state space model y = C h + D x (explainer page, "The state-space scan
 * primitive").  Variable-length batches (section 8.3, "Variable Length"):
 * several sequences packed into one stream, given by cu_seqlens; each starts
 * from its own initial state (or zero) so nothing crosses a boundary.  The
 * final state of every sequence is returned, which is what a sequence-parallel
 * worker hands to the next one (section 8.2).
 *
 * Everything is in fp64 on inputs widened exactly from their stored fp32 (or
 * bf16, already widened to fp32) values.  Sequences x heads are independent
 * and are spread over OpenMP threads; the per-token loop is sequential.
 *
 * Flag bits (plain integers, defined here on their own):
 *   1 : dt' = softplus(dt + dt_bias) before the clamp
 *   2 : the input term is multiplied by dt'
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_FLAG_SOFTPLUS 1u
#define REF_FLAG_SCALES_INPUT 2u

static double ref_softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }

/* One (sequence, head) stream: tokens [tok0, tok0 + len) of the packed token
 * axis.  Strides are in elements of the flat row-major arrays. */
static void ref_stream(int64_t tok0, int64_t len, int64_t h, int64_t H, int64_t P,
                       int64_t N, int64_t G, int64_t Gc, const float* x, const float* dt,
                       const float* A, const float* B, const float* C,
                       const float* D, const float* dt_bias, const float* init,
                       unsigned flags, double dt_min, double dt_max, double* y,
                       double* final_state, double* S) {
  const int64_t g = h / (H / G), gc = h / (H / Gc);
  const double Ah = (double)A[h];
  const double Dh = D ? (double)D[h] : 0.0;
  const double bias = dt_bias ? (double)dt_bias[h] : 0.0;

  if (init) {
    for (int64_t i = 0; i < N * P; ++i) S[i] = (double)init[i];
  } else {
    memset(S, 0, sizeof(double) * (size_t)(N * P));
  }

  for (int64_t t = tok0; t < tok0 + len; ++t) {
    double dtv = (double)dt[t * H + h] + bias;
    if (flags & REF_FLAG_SOFTPLUS) dtv = ref_softplus(dtv);
    dtv = fmin(fmax(dtv, dt_min), dt_max);
    const double a = exp(dtv * Ah);
    const double in_scale = (flags & REF_FLAG_SCALES_INPUT) ? dtv : 1.0;

    const float* xt = x + (t * H + h) * P;
    const float* Bt = B + (t * G + g) * N;
    const float* Ct = C + (t * Gc + gc) * N;

    /* state update: S[n,p] = a * S[n,p] + in_scale * B[n] * x[p] */
    for (int64_t n = 0; n < N; ++n) {
      const double bn = in_scale * (double)Bt[n];
      double* Sn = S + n * P;
      for (int64_t p = 0; p < P; ++p) Sn[p] = a * Sn[p] + bn * (double)xt[p];
    }
    /* readout: y[p] = sum_n C[n] * S[n,p] + D * x[p] */
    double* yt = y + (t * H + h) * P;
    for (int64_t p = 0; p < P; ++p) yt[p] = Dh * (double)xt[p];
    for (int64_t n = 0; n < N; ++n) {
      const double cn = (double)Ct[n];
      const double* Sn = S + n * P;
      for (int64_t p = 0; p < P; ++p) yt[p] += cn * Sn[p];
    }
  }
  if (final_state) memcpy(final_state, S, sizeof(double) * (size_t)(N * P));
}

/*
 * Layouts (row-major, host memory):
 *   x, y  (batch, seqlen, H, P)      dt (batch, seqlen, H)
 *   B     (batch, seqlen, G, N)      C (batch, seqlen, Gc, N)
 *   A, D, dt_bias (H)
 *   init, final (nseq, H, N, P)      cu_seqlens (nseqs + 1) int32
 * Without cu_seqlens the sequences are the batch rows (nseq = batch).  With
 * it, batch must be 1, seqlen is the total token count and sequence s covers
 * tokens [cu_seqlens[s], cu_seqlens[s+1]).
 * pairs (optional): n_pairs (sequence, head) pairs; only those streams are
 * computed (y of the other streams is left untouched).  NULL = all.
 * Returns 0, or -1 on an inconsistent argument.
 */
int ssd_ref_fwd(int64_t batch, int64_t seqlen, int64_t H, int64_t P, int64_t N,
                int64_t G, int64_t Gc, int64_t nseqs, const int32_t* cu_seqlens,
                const float* x, const float* dt, const float* A, const float* B,
                const float* C, const float* D, const float* dt_bias,
                const float* init, unsigned flags, double dt_min, double dt_max,
                int64_t n_pairs, const int64_t* pairs, double* y,
                double* final_states) {
  if (batch < 0 || seqlen < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || Gc <= 0) return -1;
  if (H % G != 0 || H % Gc != 0) return -1;
  if (cu_seqlens && batch != 1) return -1;
  const int64_t S_count = cu_seqlens ? nseqs : batch;
  if (cu_seqlens) {
    if (cu_seqlens[0] != 0 || cu_seqlens[nseqs] != seqlen) return -1;
    for (int64_t s = 0; s < nseqs; ++s)
      if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
  }
  const int64_t total = pairs ? n_pairs : S_count * H;
  for (int64_t i = 0; pairs && i < n_pairs; ++i)
    if (pairs[2 * i] < 0 || pairs[2 * i] >= S_count || pairs[2 * i + 1] < 0 ||
        pairs[2 * i + 1] >= H)
      return -1;

  int failed = 0;
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)(N * P));
    if (!S) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < total; ++i) {
      if (!S) continue;
      const int64_t s = pairs ? pairs[2 * i] : i / H;
      const int64_t h = pairs ? pairs[2 * i + 1] : i % H;
      const int64_t tok0 = cu_seqlens ? cu_seqlens[s] : s * seqlen;
      const int64_t len = cu_seqlens ? cu_seqlens[s + 1] - cu_seqlens[s] : seqlen;
      const float* init_sh = init ? init + (s * H + h) * N * P : NULL;
      double* fin_sh = final_states ? final_states + (s * H + h) * N * P : NULL;
      ref_stream(tok0, len, h, H, P, N, G, Gc, x, dt, A, B, C, D, dt_bias, init_sh, flags,
                 dt_min, dt_max, y, fin_sh, S);
    }
    free(S);
  }
  return failed ? -1 : 0;
}

/* Number of OpenMP threads the oracle will use (1 without OpenMP). */
int ssd_ref_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Backward pass (gradients) of the same layer, for a loss whose gradient with
 * respect to y is dy and with respect to the final states is dfinal (zero when
 * NULL).  Section 6 of "Transformers are SSMs" counts the method's training
 * cost; the gradients themselves are those of the recurrence above, taken by
 * reverse-mode differentiation of the token loop (the adjoint of the linear
 * mode, section 3.4.1), with no chunking.  Per stream, with s_t the input
 * scale (dt' or 1) and g the adjoint dLoss/dS of the state after token t:
 *
 *     g      = dfinal
 *     for t = last .. first:
 *       g     += C_t (x) dy_t                        (readout of token t)
 *       dx_t   = D dy_t + s_t * g^T B_t
 *       dB_t  += s_t * g x_t          (summed over the heads of B's group)
 *       dC_t  += S_t dy_t             (summed over the heads of C's group)
 *       dl_t   = a_t <g, S_{t-1}>     (l_t = dt'_t A, the log of a_t)
 *       ddt'_t = dl_t A + [scaled] <g, B_t (x) x_t>
 *       dA    += dl_t dt'_t
 *       dD    += <dy_t, x_t>
 *       ddt_t  = ddt'_t * [dt_min <= act <= dt_max] * act'(dt_t + bias)
 *       dbias += ddt_t
 *       g     *= a_t                                 (back through the decay)
 *     dinit  = g
 *
 * act' is 1, or the logistic sigmoid for softplus.  The clamp passes the
 * gradient where the activated value lies inside [dt_min, dt_max], edges
 * included.  The states S_t of the forward sweep are kept for the whole
 * stream (len * N * P doubles per thread).
 *
 * Layouts as in ssd_ref_fwd; dy (batch, seqlen, H, P) and dfinal (nseq, H, N,
 * P) float32; outputs in double: dx like x, ddt like dt, dB like B, dC like C,
 * dA / dD / ddt_bias (H), dinit like init (optional).  Returns 0, or -1 on an
 * inconsistent argument or when memory runs out.
 */
static double ref_sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

static void ref_stream_bwd(int64_t tok0, int64_t len, int64_t h, int64_t H, int64_t P,
                           int64_t N, int64_t G, int64_t Gc, const float* x, const float* dt,
                           const float* A, const float* B, const float* C, const float* D,
                           const float* dt_bias, const float* init, unsigned flags,
                           double dt_min, double dt_max, const float* dy, const float* dfinal,
                           double* dx, double* ddt, double* dBh, double* dCh, double* sums,
                           double* dinit, double* S, double* g) {
  const int64_t NP = N * P;
  const int64_t gb = h / (H / G), gc = h / (H / Gc);
  const double Ah = (double)A[h];
  const double Dh = D ? (double)D[h] : 0.0;
  const double bias = dt_bias ? (double)dt_bias[h] : 0.0;

  /* forward sweep, keeping every state: S + (t - tok0 + 1) * NP is the state
   * after token t, S itself the initial state */
  for (int64_t i = 0; i < NP; ++i) S[i] = init ? (double)init[i] : 0.0;
  for (int64_t t = tok0; t < tok0 + len; ++t) {
    double dtv = (double)dt[t * H + h] + bias;
    if (flags & REF_FLAG_SOFTPLUS) dtv = ref_softplus(dtv);
    dtv = fmin(fmax(dtv, dt_min), dt_max);
    const double a = exp(dtv * Ah);
    const double sc = (flags & REF_FLAG_SCALES_INPUT) ? dtv : 1.0;
    const float* xt = x + (t * H + h) * P;
    const float* Bt = B + (t * G + gb) * N;
    const double* prev = S + (t - tok0) * NP;
    double* cur = S + (t - tok0 + 1) * NP;
    for (int64_t n = 0; n < N; ++n)
      for (int64_t p = 0; p < P; ++p)
        cur[n * P + p] = a * prev[n * P + p] + sc * (double)Bt[n] * (double)xt[p];
  }

  for (int64_t i = 0; i < NP; ++i) g[i] = dfinal ? (double)dfinal[i] : 0.0;
  double dA_acc = 0.0, dD_acc = 0.0, db_acc = 0.0;
  for (int64_t t = tok0 + len - 1; t >= tok0; --t) {
    const double pre = (double)dt[t * H + h] + bias;
    const double act = (flags & REF_FLAG_SOFTPLUS) ? ref_softplus(pre) : pre;
    const double dtv = fmin(fmax(act, dt_min), dt_max);
    const double a = exp(dtv * Ah);
    const double sc = (flags & REF_FLAG_SCALES_INPUT) ? dtv : 1.0;
    const float* xt = x + (t * H + h) * P;
    const float* dyt = dy + (t * H + h) * P;
    const float* Bt = B + (t * G + gb) * N;
    const float* Ct = C + (t * Gc + gc) * N;
    const double* cur = S + (t - tok0 + 1) * NP;
    const double* prev = S + (t - tok0) * NP;

    for (int64_t n = 0; n < N; ++n)
      for (int64_t p = 0; p < P; ++p) g[n * P + p] += (double)Ct[n] * (double)dyt[p];

    double* dxt = dx + (t * H + h) * P;
    for (int64_t p = 0; p < P; ++p) {
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) acc += (double)Bt[n] * g[n * P + p];
      dxt[p] = Dh * (double)dyt[p] + sc * acc;
    }
    double* dBt = dBh + (t * H + h) * N;
    double* dCt = dCh + (t * H + h) * N;
    double gBx = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double gx = 0.0, sd = 0.0;
      for (int64_t p = 0; p < P; ++p) {
        gx += g[n * P + p] * (double)xt[p];
        sd += cur[n * P + p] * (double)dyt[p];
      }
      dBt[n] = sc * gx;
      dCt[n] = sd;
      gBx += (double)Bt[n] * gx;
    }
    double gS = 0.0;
    for (int64_t i = 0; i < NP; ++i) gS += g[i] * prev[i];
    const double dl = a * gS;
    double ddtp = dl * Ah;
    if (flags & REF_FLAG_SCALES_INPUT) ddtp += gBx;
    dA_acc += dl * dtv;
    for (int64_t p = 0; p < P; ++p) dD_acc += (double)dyt[p] * (double)xt[p];
    double gate = (act >= dt_min && act <= dt_max) ? 1.0 : 0.0;
    if (flags & REF_FLAG_SOFTPLUS) gate *= ref_sigmoid(pre);
    ddt[t * H + h] = ddtp * gate;
    db_acc += ddtp * gate;
    for (int64_t i = 0; i < NP; ++i) g[i] *= a;
  }
  sums[0] = dA_acc;
  sums[1] = dD_acc;
  sums[2] = db_acc;
  if (dinit) memcpy(dinit, g, sizeof(double) * (size_t)NP);
}

int ssd_ref_bwd(int64_t batch, int64_t seqlen, int64_t H, int64_t P, int64_t N, int64_t G,
                int64_t Gc, int64_t nseqs, const int32_t* cu_seqlens, const float* x,
                const float* dt, const float* A, const float* B, const float* C, const float* D,
                const float* dt_bias, const float* init, unsigned flags, double dt_min,
                double dt_max, const float* dy, const float* dfinal, double* dx, double* ddt,
                double* dA, double* dB, double* dC, double* dD, double* ddt_bias,
                double* dinit) {
  if (batch < 0 || seqlen < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || Gc <= 0) return -1;
  if (H % G != 0 || H % Gc != 0) return -1;
  if (cu_seqlens && batch != 1) return -1;
  if (!dx || !ddt || !dA || !dB || !dC || !dD || !ddt_bias) return -1;
  const int64_t S_count = cu_seqlens ? nseqs : batch;
  int64_t max_len = seqlen;
  if (cu_seqlens) {
    if (cu_seqlens[0] != 0 || cu_seqlens[nseqs] != seqlen) return -1;
    max_len = 0;
    for (int64_t s = 0; s < nseqs; ++s) {
      if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
      if (cu_seqlens[s + 1] - cu_seqlens[s] > max_len) max_len = cu_seqlens[s + 1] - cu_seqlens[s];
    }
  }
  const int64_t T = batch * seqlen, NP = N * P;
  double* dBh = (double*)calloc((size_t)(T * H * N) + 1, sizeof(double));
  double* dCh = (double*)calloc((size_t)(T * H * N) + 1, sizeof(double));
  double* sums = (double*)calloc((size_t)(S_count * H * 3) + 1, sizeof(double));
  int failed = (!dBh || !dCh || !sums);
#pragma omp parallel if (!failed)
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)((max_len + 1) * NP));
    double* g = (double*)malloc(sizeof(double) * (size_t)NP);
    if (!S || !g) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < S_count * H; ++i) {
      if (!S || !g) continue;
      const int64_t s = i / H, h = i % H;
      const int64_t tok0 = cu_seqlens ? cu_seqlens[s] : s * seqlen;
      const int64_t len = cu_seqlens ? cu_seqlens[s + 1] - cu_seqlens[s] : seqlen;
      ref_stream_bwd(tok0, len, h, H, P, N, G, Gc, x, dt, A, B, C, D, dt_bias,
                     init ? init + (s * H + h) * NP : NULL, flags, dt_min, dt_max, dy,
                     dfinal ? dfinal + (s * H + h) * NP : NULL, dx, ddt, dBh, dCh,
                     sums + i * 3, dinit ? dinit + (s * H + h) * NP : NULL, S, g);
    }
    free(S);
    free(g);
  }
  if (!failed) {
    /* sum the per-head contributions over the heads that share each group */
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t k = 0; k < G * N; ++k) dB[t * G * N + k] = 0.0;
      for (int64_t k = 0; k < Gc * N; ++k) dC[t * Gc * N + k] = 0.0;
      for (int64_t h = 0; h < H; ++h)
        for (int64_t n = 0; n < N; ++n) {
          dB[(t * G + h / (H / G)) * N + n] += dBh[(t * H + h) * N + n];
          dC[(t * Gc + h / (H / Gc)) * N + n] += dCh[(t * H + h) * N + n];
        }
    }
    for (int64_t h = 0; h < H; ++h) {
      dA[h] = dD[h] = ddt_bias[h] = 0.0;
      for (int64_t s = 0; s < S_count; ++s) {
        dA[h] += sums[(s * H + h) * 3 + 0];
        dD[h] += sums[(s * H + h) * 3 + 1];
        ddt_bias[h] += sums[(s * H + h) * 3 + 2];
      }
    }
  }
  free(dBh);
  free(dCh);
  free(sums);
  return failed ? -1 : 0;
}
