/*
 * ssd.h - C ABI of the chunked SSD (state space duality) forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation ("Transformers are SSMs: Generalized Models and Efficient
 * Algorithms Through Structured State Space Duality", arXiv 2405.21060):
 * per head h, with the groups g = h / (H / G) and gc = h / (H / Gc) whose B and
 * C heads it shares (section 7.1 "Block Design"; section 7.2 head patterns:
 * Gc = G multi-value, G = 1 with Gc = H multi-contract, G = H with Gc = 1
 * multi-expand), the
 * scalar-times-identity selective SSM of section 2.4 / section 5.1:
 *
 *     dt'_t = clamp(act(dt[t,h] + dt_bias[h]), dt_min, dt_max)
 *     S_t   = exp(dt'_t A[h]) S_{t-1} + B[t,g,:] x[t,h,:]^T      (N x P state)
 *     y_t   = S_t^T C[t,gc,:] + D[h] x[t,h,:]
 *
 * with act = softplus when SSD_DT_SOFTPLUS is set, and the input term scaled by
 * dt'_t when SSD_DT_SCALES_INPUT is set.  S_{-1} is the caller's initial state
 * (zero when none is given).  It is evaluated by the block decomposition of
 * section 6 (diagonal blocks in the quadratic, attention-like dual form of
 * section 6.1; chunk states, a scan across chunks and the state-to-output
 * left factors of section 6.2), whose result equals the recurrence up to
 * rounding.  Variable-length batches (section 8.3) pack sequences into one
 * stream given by cu_seqlens; nothing crosses a sequence boundary, and each
 * sequence starts from its own initial state.  Final states are what a
 * sequence-parallel worker passes on (section 8.2).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to row-major, contiguous memory
 *     owned by the caller.  The library allocates no device memory and keeps
 *     no mutable state; concurrent calls on different workspaces are safe.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     null stream).  Host-side validation runs before anything is enqueued;
 *     on any error nothing is launched and no output is touched.
 *   - No C++ exception crosses this boundary.
 */
#ifndef SSD_SCAN_AMD_SSD_H
#define SSD_SCAN_AMD_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1, /* null required pointer, bad shape, H % G != 0, ... */
  SSD_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype, P, N, chunk)     */
  SSD_ERR_WORKSPACE = 3,   /* workspace missing or smaller than ssd_workspace_size */
  SSD_ERR_HIP = 4          /* a HIP launch or runtime call failed                 */
} ssd_status;

/* Storage type of x, dt, B, C and y.  Arithmetic is fp32 (MFMA with fp32
 * accumulation) in both cases; A, D, dt_bias and the states are always fp32. */
typedef enum ssd_dtype { SSD_DTYPE_F32 = 0, SSD_DTYPE_BF16 = 1 } ssd_dtype;

enum {
  SSD_DT_SOFTPLUS = 1u << 0,    /* dt' = softplus(dt + dt_bias) before the clamp      */
  SSD_DT_SCALES_INPUT = 1u << 1 /* input term is dt' B x^T instead of B x^T           */
};

/* Evaluation schedule; every schedule computes the same function.  STREAM
 * supports bf16 storage, P = 64, dense rows with one group count for B and C;
 * FUSED bf16 storage, P = 64, N <= 128, with or without cu_seqlens; CHUNKED
 * every supported shape.  AUTO takes STREAM where it supports the shape and
 * has enough chunks for every resident workgroup of the device to walk whole
 * (row, head) streams; where it supports the shape with fewer, STREAM only for
 * N >= 64 on rows of at least 256 or at most 2 chunks and for N = 256 from 64
 * chunks on (CHUNKED below), FUSED otherwise; outside STREAM, FUSED where it
 * supports the shape unless the problem is small (fewer than 512 (row, head,
 * chunk) units with N >= 64), CHUNKED otherwise.  The choice depends on the
 * current device (its compute units), as does the workspace size. */
typedef enum ssd_algo {
  SSD_ALGO_AUTO = 0,    /* library picks from the shape (see above)                     */
  SSD_ALGO_CHUNKED = 1, /* four kernels: dt/cumsum, chunk states, state passing, scan   */
  SSD_ALGO_FUSED = 2,   /* one pass over x: states handed chunk to chunk on chip/in MALL */
  SSD_ALGO_STREAM = 3   /* one pass over x: a workgroup walks a run of chunks of a
                           (row, head) with the state in registers; C B^T shared by
                           the heads of a group; fp16 matrix-core operands           */
} ssd_algo;

typedef struct ssd_problem {
  int64_t batch;      /* b (must be 1 with cu_seqlens)                              */
  int64_t seqlen;     /* L (with cu_seqlens: total packed tokens)                   */
  int64_t nheads;     /* H                                                          */
  int64_t headdim;    /* P  (supported: 64, 128)                                    */
  int64_t dstate;     /* N  (supported: 16, 32, 64, 128, 256)                       */
  int64_t ngroups;    /* G  (H % G == 0)                                            */
  int64_t chunk_size; /* Q  (supported: 64, 128, 256)                               */
  int64_t nseqs;      /* number of packed sequences (>= 1) with cu_seqlens, else 0 */
  int32_t dtype;      /* ssd_dtype                                                  */
  uint32_t flags;     /* SSD_DT_* bits                                              */
  float dt_min;       /* clamp bounds, dt_min <= dt_max (use 0 and +inf for none)   */
  float dt_max;
  int32_t algo;       /* ssd_algo                                                   */
  int32_t ngroups_c;  /* Gc, groups of C (0: same as ngroups; must divide H)        */
} ssd_problem;

/*
 * Bytes of device workspace ssd_fwd needs for this problem (0 for an invalid
 * problem).  The workspace holds per-chunk log-decay prefix sums, chunk
 * states and hand-off flags; its contents need not be initialised and are
 * garbage after the call.
 */
size_t ssd_workspace_size(const ssd_problem* p);

/*
 * Forward pass.
 *   x      (b, L, H, P)  dtype          dt  (b, L, H)  dtype (raw, see flags)
 *   A      (H) fp32                      B (b, L, G, N), C (b, L, Gc, N) dtype
 *   D      (H) fp32, nullable (no skip)  dt_bias (H) fp32, nullable (zero)
 *   initial_states (S, H, N, P) fp32, nullable (zero); S = b, or nseqs with
 *                  cu_seqlens
 *   cu_seqlens (nseqs + 1) int32, nullable; cu[0] = 0, non-decreasing,
 *                  cu[nseqs] = L.  Empty sequences are allowed (their final
 *                  state is their initial state).  Contents are trusted unless
 *                  the environment variable SSD_VALIDATE=1 is set, in which case
 *                  they are copied to the host and checked (this synchronises
 *                  the stream).
 *   y      (b, L, H, P) dtype, written
 *   final_states (S, H, N, P) fp32, nullable (not computed)
 *   workspace: device memory of at least ssd_workspace_size(p) bytes, 256-byte
 *              aligned; must not be in use by another call in flight.
 * Returns SSD_OK once the work is enqueued.  fp32 exponents can overflow for
 * A * dt' > 0 over long spans; the result is then inf/NaN, as in any fp32
 * evaluation.
 * The fused and stream schedules hand states between workgroups; every such
 * wait is bounded (about half a second of sleeps; the environment variable
 * SSD_SPIN_LIMIT sets the number of sleeps).  A wait that gives up (which the
 * ticket order rules out in a normal run) takes the missing state as NaN (fused)
 * or infinite (stream), so that the outputs that depend on it are not finite
 * rather than silently wrong.  With SSD_VALIDATE=1 the call synchronises the
 * stream after the launch and returns SSD_ERR_HIP when a wait gave up.
 */
ssd_status ssd_fwd(const ssd_problem* p, const void* x, const void* dt, const float* A,
                   const void* B, const void* C, const float* D, const float* dt_bias,
                   const float* initial_states, const int32_t* cu_seqlens, void* y,
                   float* final_states, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Profiling variant of ssd_fwd: same arguments, same work, and additionally
 * records events[k] (hipEvent_t handles created by the caller) on `stream`
 * right before the k-th kernel launch of the call, and one more after the last
 * launch, for as many events as max_events allows.  names (nullable) receives a
 * static string per recorded event (the kernel about to run, "end" for the
 * last).  *n_events (nullable) receives the number of events recorded.
 * Elapsed time between consecutive events is the duration of one kernel.
 */
ssd_status ssd_fwd_events(const ssd_problem* p, const void* x, const void* dt, const float* A,
                          const void* B, const void* C, const float* D, const float* dt_bias,
                          const float* initial_states, const int32_t* cu_seqlens, void* y,
                          float* final_states, void* workspace, size_t workspace_bytes,
                          void* stream, void* const* events, const char** names, int max_events,
                          int* n_events);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ssd_fwd with
 * the library's own device scratch buffer in place of the workspace argument.
 * The buffer is a static device array of SSD_NOALLOC_SCRATCH_BYTES bytes that
 * every GPU the library runs on holds until the process ends; its address is
 * looked up once per device on the first call on that device.  The call
 * allocates nothing and never synchronises (SSD_VALIDATE is ignored).  A
 * problem whose ssd_workspace_size exceeds the buffer returns
 * SSD_ERR_WORKSPACE.  All calls on one GPU share the buffer: calls that can
 * overlap on one GPU (different streams, or host threads) race and must be
 * serialised by the caller.  Other arguments and results as for ssd_fwd.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ssd_status ssd_fwd_noalloc(const ssd_problem* p, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, const float* dt_bias,
                           const float* initial_states, const int32_t* cu_seqlens, void* y,
                           float* final_states, void* stream);

/*
 * The dt preprocessing and per-chunk log-decay prefix sums on their own (the
 * first step of the chunked schedule), for testing: writes
 *   dt_out (b, H, nchunks, Q) fp32 = dt' of every token (0 in the padding of a
 *          short last chunk)
 *   cs_out (b, H, nchunks, Q) fp32 = sum of dt' A[h] from the chunk start to
 *          the token, inclusive (the last valid value repeated in the padding)
 * where nchunks = ceil(L / Q) per batch row (with cu_seqlens, chunks tile the
 * packed stream).  Same validation as ssd_fwd for the arguments it takes.
 */
ssd_status ssd_dt_cumsum(const ssd_problem* p, const void* dt, const float* A,
                         const float* dt_bias, float* dt_out, float* cs_out, void* stream);

/*
 * Single-token step (the recurrent / decode mode, section 3.4.1, one token):
 * for each of the b rows, the recurrence above applied to one token from the
 * caller's state, which it overwrites with the new state.
 *   x      (b, H, P)  dtype          dt (b, H) dtype (raw, see flags)
 *   A      (H) fp32                   B (b, G, N), C (b, Gc, N) dtype
 *   D      (H) fp32, nullable         dt_bias (H) fp32, nullable
 *   state  (b, H, N, P) fp32, read as S_{t-1} and overwritten with S_t
 *   y      (b, H, P) dtype, written (must not overlap state)
 * p->seqlen must be 1; chunk_size, nseqs and algo are not used.  P must be
 * 64 or 128; any N.  No workspace.  One kernel, bound by moving the state
 * through HBM (N P fp32 values read and written per row and head).
 */
ssd_status ssd_step(const ssd_problem* p, const void* x, const void* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* dt_bias,
                    float* state, void* y, void* stream);

/*
 * Bytes of device workspace ssd_bwd needs for this problem (0 when the
 * problem is invalid or the backward pass does not support it).  Besides the
 * forward's per-chunk buffers it holds the adjoint of every chunk (N P fp32
 * values per row, head and 64-token chunk) and per-head dB / dC (b L H N fp32
 * each); with packed sequences also 3 fp32 per token and head and 2 per
 * sequence and head.
 */
size_t ssd_bwd_workspace_size(const ssd_problem* p);

/*
 * Backward pass: the gradients of a loss, given its gradient dy with respect
 * to y and d_final_states with respect to the final states, with respect to
 * every input of ssd_fwd.  "Transformers are SSMs" section 6 counts the
 * method's training cost; the gradients are those of the recurrence above
 * (reverse-mode differentiation), evaluated on the same block decomposition:
 * a reverse scan of per-chunk adjoints across chunks and, inside each chunk,
 * the transposed quadratic products.
 *   x, dt, A, B, C, D, dt_bias, initial_states: as for ssd_fwd (the forward
 *                  pass is recomputed; nothing from a previous ssd_fwd call is
 *                  needed)
 *   cu_seqlens     nullable; packed sequences as for ssd_fwd, each with its
 *                  own initial state, final-state gradient and initial-state
 *                  gradient (section 8.3)
 *   dy             (b, L, H, P) dtype
 *   d_final_states (S, H, N, P) fp32, nullable (zero); S = b, or nseqs with
 *                  cu_seqlens
 *   dx  (b, L, H, P) dtype    ddt (b, L, H) dtype (gradient of the raw dt)
 *   dA  (H) fp32              dB (b, L, G, N), dC (b, L, Gc, N) dtype
 *   dD  (H) fp32, nullable    ddt_bias (H) fp32, nullable
 *   d_initial_states (S, H, N, P) fp32, nullable
 * All outputs are written (not accumulated).  dD and ddt_bias are the
 * gradients with respect to D and dt_bias also when those inputs are NULL
 * (taken as zero); d_initial_states likewise.  The clamp passes the gradient
 * where the activated dt lies inside [dt_min, dt_max], edges included.
 * chunk_size and algo are not used: the pass runs on 64-token chunks (the
 * result does not depend on the chunk).  Supported: P 64 or 128, N 16 .. 256,
 * N P <= 16384 for bf16 storage and N P <= 8192 for fp32; other shapes return
 * SSD_ERR_UNSUPPORTED.  workspace as for ssd_fwd, of ssd_bwd_workspace_size(p)
 * bytes.  Returns SSD_OK once the work is enqueued.
 */
ssd_status ssd_bwd(const ssd_problem* p, const void* x, const void* dt, const float* A,
                   const void* B, const void* C, const float* D, const float* dt_bias,
                   const float* initial_states, const int32_t* cu_seqlens, const void* dy,
                   const float* d_final_states, void* dx, void* ddt, float* dA, void* dB, void* dC,
                   float* dD, float* ddt_bias, float* d_initial_states, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Profiling variant of ssd_bwd, with the event arguments of ssd_fwd_events. */
ssd_status ssd_bwd_events(const ssd_problem* p, const void* x, const void* dt, const float* A,
                          const void* B, const void* C, const float* D, const float* dt_bias,
                          const float* initial_states, const int32_t* cu_seqlens, const void* dy,
                          const float* d_final_states, void* dx, void* ddt, float* dA, void* dB,
                          void* dC, float* dD, float* ddt_bias, float* d_initial_states,
                          void* workspace, size_t workspace_bytes, void* stream,
                          void* const* events, const char** names, int max_events,
                          int* n_events);

/* Human-readable name of a status code (static storage). */
const char* ssd_status_string(ssd_status s);

/* Library version string, including the target architecture. */
const char* ssd_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SSD_SCAN_AMD_SSD_H */
