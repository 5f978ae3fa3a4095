// Internal launch interface between the C ABI (ssd_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_device.hpp"

namespace ssd {

// Optional profiling hook: HIP events recorded on the launch stream right
// before each kernel launch (and once after the last one).
struct LaunchMarks {
  void* const* events;  // hipEvent_t[max_events]
  const char** names;   // nullable; receives the kernel name of each mark
  int max_events;
  int count;            // marks recorded so far
};

// Everything one call needs: caller tensors plus carved workspace pointers.
struct ChunkedArgs {
  Shape sh;
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const float* dt_bias;
  const float* init;
  const int32_t* cu;
  void* y;
  float* final_states;
  // workspace
  float* cs;          // (batch, H, nc, Q) inclusive log-decay prefix sums
  float* dt_out;      // (batch, H, nc, Q) dt'
  float2* coef;       // (batch, H, nc)   (carry decay, initial-state decay) per chunk
  ChunkInfo* cinfo;   // (batch, nc)
  float* states;      // (batch, nc, H, N*P) fragment layout
  int32_t* seq_idx;   // (L) packed streams only
  uint32_t* flags;    // hand-off flags of the fused schedule
  LaunchMarks* marks; // nullable
};

inline hipError_t mark(const ChunkedArgs& a, const char* name, hipStream_t st) {
  if (!a.marks || a.marks->count >= a.marks->max_events) return hipSuccess;
  LaunchMarks& m = *a.marks;
  if (m.names) m.names[m.count] = name;
  const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(m.events[m.count]), st);
  ++m.count;
  return e;
}

hipError_t launch_seq_index(const int32_t* cu, int nseqs, int64_t T, int32_t* seq_idx,
                            hipStream_t st);
hipError_t launch_dt_cumsum(const ChunkedArgs& a, int Q, bool is_bf16, hipStream_t st);
hipError_t launch_chunked_tail(const ChunkedArgs& a, int N, int P, int Q, bool is_bf16,
                               hipStream_t st);
hipError_t launch_empty_final(const float* init, int64_t n, float* out, hipStream_t st);
// chunk states and the scan across chunks only (states in place, final states
// of dense rows into a.final_states), no outputs
hipError_t launch_chunk_states(const ChunkedArgs& a, int N, int P, int Q, bool is_bf16,
                               hipStream_t st);
// backward pass: chunk-local adjoints sum_t exp(cs_t) C_t dy_t^T (fragment layout)
hipError_t launch_chunk_adjoint(const ChunkedArgs& a, const void* dy, float* out, int N, int P,
                                int Q, bool is_bf16, hipStream_t st);

// The rest of the backward pass (dense rows, 64-token chunks): reverse scan of
// the adjoints across chunks, the per-chunk gradient kernel and the reductions
// over shared heads and over chunks.
struct BwdArgs {
  ChunkedArgs f;        // forward inputs and the forward workspace (cs, dt', states)
  int N, P;
  const void* dy;
  const float* dfinal;  // nullable
  void* dx;
  void* ddt;
  float* dA;
  void* dB;
  void* dC;
  float* dD;            // nullable
  float* ddt_bias;      // nullable
  float* dinit;         // nullable
  // workspace
  float* adj;           // (batch, nc, H, N*P) fragment layout: R_c, then G_end[c] in place
  float* dBh;           // (batch, L, H / hb, N) B gradients summed over blocks of hb heads
  float* dCh;           // (batch, L, H / hb, N) the same for C (hb = bwd_head_block)
  float* part;          // (batch, H, nc, 3) per-chunk dA, dD, ddt_bias
  // packed sequences with per-sequence states: the terms of the initial states
  // and the final-state gradients, added by k_bwd_seq_terms (the chunk
  // kernels then run from zero states with no final-state gradient)
  bool walked;  // S_in and G_end formed by the state walks (k_adjoint_passing skipped):
                // then fp16 quads in states / adj with one scale per 16 x 16 tile
  int* sc_states;  // (batch, nc, H, N P / 256) tile scales of S_in (walked)
  int* sc_adj;     // the same for G_end
  bool seq_terms;
  const float* seq_init;    // (nseqs, H, N, P), nullable
  const float* seq_dfinal;  // (nseqs, H, N, P), nullable
  float* seq_dinit;         // (nseqs, H, N, P), nullable
  float* seq_tmp;           // (L, H, 3) per-token pi, rho, ds
  float* seq_part;          // (nseqs, H, 2) per-sequence dA and dt_bias sums
};
constexpr int kBwdChunk = 64;
inline int bwd_nblk(int N, int P) { return (N * P / 4 + 255) / 256; }
bool bwd_supported(int N, int P, bool bf16_storage);
hipError_t launch_bwd_tail(const BwdArgs& a, bool is_bf16, hipStream_t st);
int bwd_head_block(const BwdArgs& a);
bool bwd_walks_supported(const Shape& sh, bool is_bf16);
bool bwd_walks_fill(const Shape& sh, int N, int P);
hipError_t launch_bwd_walks(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_sums(const BwdArgs& a, hipStream_t st);

// single-token step: state (b, H, N, P) fp32 updated in place
struct StepArgs {
  Shape sh;  // batch, H, G, hpg, flags, dt_min, dt_max are used
  int N, P;
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const float* dt_bias;
  float* state;
  void* y;
};
hipError_t launch_step(const StepArgs& a, bool is_bf16, hipStream_t st);

// fused single-pass schedule (bf16 storage, P = 64, N <= 128)
bool fused_supported(int N, int P, int Q, bool bf16_storage, bool varlen);
size_t fused_workspace_bytes(int64_t batch, int64_t H, int64_t nc, int Q, int N, int P);
hipError_t launch_fused(const ChunkedArgs& a, void* ws, int N, int P, int Q, hipStream_t st);
// Waits for the stream, then reports whether a hand-off wait of the last fused
// launch on this workspace gave up (its error word is set).
hipError_t fused_handoff_failed(const void* ws, hipStream_t st, bool* failed);

// stream-resident schedule (bf16 storage, P = 64, dense rows, one group count)
bool stream_supported(int N, int P, int Q, bool bf16_storage, bool varlen, int G, int Gc);
size_t stream_workspace_bytes(const Shape& sh, int N, int Q);
// whether the stream schedule runs in range mode (whole streams per workgroup)
// for this many streams and chunks per stream on the current device
bool stream_range_mode(int64_t streams, int64_t nc, int N, int Q);
hipError_t launch_stream(const ChunkedArgs& a, void* ws, int N, int P, int Q, hipStream_t st);
// Waits for the stream, then reports whether a segment hand-off wait of the
// last stream launch on this workspace gave up (its error word is set).
hipError_t stream_handoff_failed(const void* ws, hipStream_t st, bool* failed);

}  // namespace ssd
