// C ABI of the SSD forward pass: argument validation, workspace plan and the
// launch sequence on the caller's stream.  Declarations and the contract of
// every entry point are in include/ssd.h.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include <mutex>

#include "ssd.h"
#include "ssd_launch.hpp"

namespace {

// The no-allocation entry point's buffer: one copy per GPU, which the device
// code object holds from its load until the process ends.  Host code uses the
// address hipGetSymbolAddress returns for the current device, never the
// array's name (a host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on the first call on the
// device (with that device current).
ssd_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SSD_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SSD_OK;
}

using ssd::ChunkedArgs;
using ssd::ChunkInfo;
using ssd::Shape;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] == '1';
}

bool env_validate() { return env_flag("SSD_VALIDATE"); }

bool supported_shape(const ssd_problem& p) {
  const int64_t P = p.headdim, N = p.dstate, Q = p.chunk_size;
  if (P != 64 && P != 128) return false;
  if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256) return false;
  if (Q != 64 && Q != 128 && Q != 256) return false;
  if (p.dtype == SSD_DTYPE_F32 && N * P > 16384) return false;  // LDS budget of the fp32 scan
  return true;
}

// Shape checks that need no pointers.
ssd_status check_problem(const ssd_problem* p) {
  if (!p) return SSD_ERR_INVALID_ARG;
  if (p->batch < 0 || p->seqlen < 0 || p->nheads <= 0 || p->headdim <= 0 || p->dstate <= 0 ||
      p->ngroups <= 0 || p->chunk_size <= 0 || p->ngroups_c < 0)
    return SSD_ERR_INVALID_ARG;
  if (p->nheads % p->ngroups != 0) return SSD_ERR_INVALID_ARG;
  if (p->ngroups_c > 0 && p->nheads % p->ngroups_c != 0) return SSD_ERR_INVALID_ARG;
  if (p->dtype != SSD_DTYPE_F32 && p->dtype != SSD_DTYPE_BF16) return SSD_ERR_INVALID_ARG;
  if (p->flags & ~(uint32_t)(SSD_DT_SOFTPLUS | SSD_DT_SCALES_INPUT)) return SSD_ERR_INVALID_ARG;
  if (std::isnan(p->dt_min) || std::isnan(p->dt_max) || p->dt_min > p->dt_max)
    return SSD_ERR_INVALID_ARG;
  if (p->algo != SSD_ALGO_AUTO && p->algo != SSD_ALGO_CHUNKED && p->algo != SSD_ALGO_FUSED &&
      p->algo != SSD_ALGO_STREAM)
    return SSD_ERR_INVALID_ARG;
  if (!supported_shape(*p)) return SSD_ERR_UNSUPPORTED;
  // index ranges of the launch grids and of the 32-bit token positions (the
  // size checks come first: the chunk count is formed from bounded values)
  if (p->batch > 65535 || p->nheads > 65535 || p->seqlen > (int64_t)1 << 30)
    return SSD_ERR_UNSUPPORTED;
  const int64_t nc = (p->seqlen + p->chunk_size - 1) / p->chunk_size;
  if (nc > 65535) return SSD_ERR_UNSUPPORTED;
  // no tensor or workspace size can overflow: at most 2^40 elements of x
  // (and of the per-chunk fp32 tables), and of the chunk states (every
  // factor below is positive and bounded, so the divisions are exact tests)
  const int64_t kMaxElems = (int64_t)1 << 40;
  const int64_t rows = p->batch * p->nheads;                           // < 2^32
  const int64_t per_row = std::max(nc * p->chunk_size, p->seqlen);    // < 2^31
  if (rows > 0 && per_row > kMaxElems / (rows * p->headdim)) return SSD_ERR_UNSUPPORTED;
  if (rows > 0 && nc > kMaxElems / (rows * p->headdim * p->dstate)) return SSD_ERR_UNSUPPORTED;
  if (p->nseqs > (int64_t)1 << 31 ||
      (p->nseqs > 0 && p->nseqs > kMaxElems / (p->nheads * p->headdim * p->dstate)))
    return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

// The schedule a problem runs with: AUTO takes the stream-resident schedule
// wherever it supports the shape (dense rows, bf16, P = 64, B and C with one
// group count), else the fused single pass wherever it supports the shape (it
// reads x once and keeps the chunk states on chip), the chunked schedule
// otherwise -- and also for small problems with N >= 64: with fewer (row, head,
// chunk) units than about two per CU (512) the fused kernel's units run nearly
// one per workgroup with nothing to overlap them, and the four short chunked
// kernels finish first (b1 H32 L512: 42 vs 66 us at N = 128, 38 vs 43 us at
// N = 64).
int resolve_algo(const ssd_problem& p, bool varlen) {
  const bool bf16 = p.dtype == SSD_DTYPE_BF16;
  const int G = (int)p.ngroups, Gc = (int)(p.ngroups_c > 0 ? p.ngroups_c : p.ngroups);
  const bool stream_ok = ssd::stream_supported((int)p.dstate, (int)p.headdim, (int)p.chunk_size,
                                               bf16, varlen, G, Gc);
  const bool fused_ok = ssd::fused_supported((int)p.dstate, (int)p.headdim, (int)p.chunk_size,
                                             bf16, varlen);
  if (p.algo == SSD_ALGO_STREAM) return stream_ok ? SSD_ALGO_STREAM : -1;
  if (p.algo == SSD_ALGO_FUSED) return fused_ok ? SSD_ALGO_FUSED : -1;
  if (p.algo == SSD_ALGO_CHUNKED) return SSD_ALGO_CHUNKED;
  const int64_t nc = (p.seqlen + p.chunk_size - 1) / p.chunk_size;
  if (stream_ok) {
    // Range mode (enough chunks for every resident workgroup to walk whole
    // streams) is the stream schedule's own case.  In segment mode (few
    // streams, or few chunks per stream) each segment re-walks the one in
    // front of it for its entering state, and the other schedules win except
    // on very long or very short streams with larger states (crossovers
    // measured on b1 H32 rows of 512 to 65536 tokens, N 16 to 256, and the
    // 130M-shaped layer).
    if (ssd::stream_range_mode(p.batch * p.nheads, nc, (int)p.dstate, (int)p.chunk_size))
      return SSD_ALGO_STREAM;
    if (p.dstate >= 64 && (nc >= 256 || nc <= 2)) return SSD_ALGO_STREAM;
    if (p.dstate == 256) return nc >= 64 ? SSD_ALGO_STREAM : SSD_ALGO_CHUNKED;
    if (fused_ok) return SSD_ALGO_FUSED;
    return SSD_ALGO_STREAM;
  }
  const bool small = p.batch * p.nheads * nc < 512 && p.dstate >= 64;
  return fused_ok && !small ? SSD_ALGO_FUSED : SSD_ALGO_CHUNKED;
}

struct Plan {
  int algo = SSD_ALGO_CHUNKED;
  int64_t nc = 0;
  size_t cs = 0, dt = 0, coef = 0, cinfo = 0, states = 0, seq = 0, flags = 0, total = 0;
};

Shape make_shape(const ssd_problem& p, const Plan& pl, bool varlen, bool has_init);

Plan make_plan(const ssd_problem& p, bool varlen) {
  Plan pl;
  pl.algo = resolve_algo(p, varlen);
  if (pl.algo == SSD_ALGO_STREAM) {
    pl.nc = (p.seqlen + p.chunk_size - 1) / p.chunk_size;
    const Shape sh = make_shape(p, pl, varlen, false);
    pl.total = ssd::stream_workspace_bytes(sh, (int)p.dstate, (int)p.chunk_size);
    return pl;
  }
  if (pl.algo == SSD_ALGO_FUSED) {
    pl.nc = (p.seqlen + p.chunk_size - 1) / p.chunk_size;
    pl.total = ssd::fused_workspace_bytes(p.batch, p.nheads, pl.nc, (int)p.chunk_size,
                                          (int)p.dstate, (int)p.headdim);
    return pl;
  }
  const int64_t rows = p.batch, H = p.nheads, Q = p.chunk_size;
  pl.nc = (p.seqlen + Q - 1) / Q;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t per_chunk = (size_t)(rows * H * pl.nc);
  pl.cs = take(per_chunk * Q * sizeof(float));
  pl.dt = take(per_chunk * Q * sizeof(float));
  pl.coef = take(per_chunk * sizeof(float2));
  pl.cinfo = take((size_t)(rows * pl.nc) * sizeof(ChunkInfo));
  pl.states = take(per_chunk * (size_t)(p.dstate * p.headdim) * sizeof(float));
  pl.seq = take(varlen ? (size_t)p.seqlen * sizeof(int32_t) : 0);
  pl.total = off;
  return pl;
}

Shape make_shape(const ssd_problem& p, const Plan& pl, bool varlen, bool has_init) {
  Shape sh;
  sh.L = p.seqlen;
  sh.batch = (int32_t)p.batch;
  sh.H = (int32_t)p.nheads;
  sh.G = (int32_t)p.ngroups;
  sh.hpg = (int32_t)(p.nheads / p.ngroups);
  sh.Gc = (int32_t)(p.ngroups_c > 0 ? p.ngroups_c : p.ngroups);
  sh.hpgc = (int32_t)(p.nheads / sh.Gc);
  sh.nc = (int32_t)pl.nc;
  sh.nseqs = varlen ? (int32_t)p.nseqs : (int32_t)p.batch;
  sh.flags = p.flags;
  sh.dt_min = p.dt_min;
  sh.dt_max = p.dt_max;
  sh.varlen = varlen ? 1 : 0;
  sh.has_init = has_init ? 1 : 0;
  return sh;
}

ssd_status check_cu_seqlens_on_host(const ssd_problem& p, const int32_t* cu, hipStream_t st) {
  std::vector<int32_t> h((size_t)p.nseqs + 1);
  if (hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return SSD_ERR_HIP;
  if (h[0] != 0 || h.back() != p.seqlen) return SSD_ERR_INVALID_ARG;
  for (size_t i = 1; i < h.size(); ++i)
    if (h[i] < h[i - 1]) return SSD_ERR_INVALID_ARG;
  return SSD_OK;
}

ssd_status fwd_impl(const ssd_problem* p, const void* x, const void* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* dt_bias,
                    const float* initial_states, const int32_t* cu_seqlens, void* y,
                    float* final_states, void* workspace, size_t workspace_bytes, void* stream,
                    ssd::LaunchMarks* marks, bool validate);

}  // namespace

extern "C" {

size_t ssd_workspace_size(const ssd_problem* p) {
  if (check_problem(p) != SSD_OK) return 0;
  if (resolve_algo(*p, p->nseqs > 0) < 0) return 0;
  // packed sequences (cu_seqlens) are announced by nseqs > 0
  return make_plan(*p, p->nseqs > 0).total;
}

ssd_status ssd_fwd(const ssd_problem* p, const void* x, const void* dt, const float* A,
                   const void* B, const void* C, const float* D, const float* dt_bias,
                   const float* initial_states, const int32_t* cu_seqlens, void* y,
                   float* final_states, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(p, x, dt, A, B, C, D, dt_bias, initial_states, cu_seqlens, y, final_states,
                  workspace, workspace_bytes, stream, nullptr, env_validate());
}

ssd_status ssd_fwd_noalloc(const ssd_problem* p, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, const float* dt_bias,
                           const float* initial_states, const int32_t* cu_seqlens, void* y,
                           float* final_states, void* stream) {
  const ssd_status s = check_problem(p);
  if (s != SSD_OK) return s;
  if (resolve_algo(*p, cu_seqlens != nullptr) < 0) return SSD_ERR_UNSUPPORTED;
  const size_t need = make_plan(*p, cu_seqlens != nullptr).total;
  if (need > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_address(&ws) != SSD_OK) return SSD_ERR_HIP;
  return fwd_impl(p, x, dt, A, B, C, D, dt_bias, initial_states, cu_seqlens, y, final_states, ws,
                  SSD_NOALLOC_SCRATCH_BYTES, stream, nullptr, false);
}

ssd_status ssd_fwd_events(const ssd_problem* p, const void* x, const void* dt, const float* A,
                          const void* B, const void* C, const float* D, const float* dt_bias,
                          const float* initial_states, const int32_t* cu_seqlens, void* y,
                          float* final_states, void* workspace, size_t workspace_bytes,
                          void* stream, void* const* events, const char** names, int max_events,
                          int* n_events) {
  if (n_events) *n_events = 0;
  if (max_events < 0 || (max_events > 0 && !events)) return SSD_ERR_INVALID_ARG;
  ssd::LaunchMarks m{events, names, max_events, 0};
  const ssd_status s = fwd_impl(p, x, dt, A, B, C, D, dt_bias, initial_states, cu_seqlens, y,
                                final_states, workspace, workspace_bytes, stream, &m,
                                env_validate());
  if (s == SSD_OK && m.count < m.max_events) {
    if (m.names) m.names[m.count] = "end";
    if (hipEventRecord(static_cast<hipEvent_t>(m.events[m.count]), (hipStream_t)stream) !=
        hipSuccess)
      return SSD_ERR_HIP;
    ++m.count;
  }
  if (n_events) *n_events = m.count;
  return s;
}

}  // extern "C"

namespace {

ssd_status fwd_impl(const ssd_problem* p, const void* x, const void* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* dt_bias,
                    const float* initial_states, const int32_t* cu_seqlens, void* y,
                    float* final_states, void* workspace, size_t workspace_bytes, void* stream,
                    ssd::LaunchMarks* marks, bool validate) {
  ssd_status s = check_problem(p);
  if (s != SSD_OK) return s;
  const bool varlen = cu_seqlens != nullptr;
  if (varlen && (p->batch != 1 || p->nseqs < 1)) return SSD_ERR_INVALID_ARG;
  const int64_t tokens = p->batch * p->seqlen;
  if (tokens > 0 && (!x || !dt || !A || !B || !C || !y)) return SSD_ERR_INVALID_ARG;
  if (resolve_algo(*p, varlen) < 0) return SSD_ERR_UNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t nstates = varlen ? p->nseqs : p->batch;

  if (varlen && validate) {
    s = check_cu_seqlens_on_host(*p, cu_seqlens, st);
    if (s != SSD_OK) return s;
  }
  if (tokens == 0) {
    const int64_t n = nstates * p->nheads * p->dstate * p->headdim;
    return ssd::launch_empty_final(initial_states, n, final_states, st) == hipSuccess
               ? SSD_OK
               : SSD_ERR_HIP;
  }

  const Plan pl = make_plan(*p, varlen);
  if (!workspace || workspace_bytes < pl.total) return SSD_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return SSD_ERR_INVALID_ARG;

  char* ws = static_cast<char*>(workspace);
  ChunkedArgs a;
  a.sh = make_shape(*p, pl, varlen, initial_states != nullptr);
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.dt_bias = dt_bias;
  a.init = initial_states;
  a.cu = cu_seqlens;
  a.y = y;
  a.final_states = final_states;
  a.cs = reinterpret_cast<float*>(ws + pl.cs);
  a.dt_out = reinterpret_cast<float*>(ws + pl.dt);
  a.coef = reinterpret_cast<float2*>(ws + pl.coef);
  a.cinfo = reinterpret_cast<ChunkInfo*>(ws + pl.cinfo);
  a.states = reinterpret_cast<float*>(ws + pl.states);
  a.seq_idx = varlen ? reinterpret_cast<int32_t*>(ws + pl.seq) : nullptr;
  a.flags = nullptr;
  a.marks = marks;

  const bool bf16 = p->dtype == SSD_DTYPE_BF16;
  const int N = (int)p->dstate, P = (int)p->headdim, Q = (int)p->chunk_size;
  if (pl.algo == SSD_ALGO_STREAM) {
    if (ssd::launch_stream(a, workspace, N, P, Q, st) != hipSuccess) return SSD_ERR_HIP;
    if (validate) {
      bool failed = false;
      if (ssd::stream_handoff_failed(workspace, st, &failed) != hipSuccess || failed)
        return SSD_ERR_HIP;
    }
    return SSD_OK;
  }
  if (pl.algo == SSD_ALGO_FUSED) {
    if (ssd::launch_fused(a, workspace, N, P, Q, st) != hipSuccess)
      return SSD_ERR_HIP;
    if (validate) {
      bool failed = false;
      if (ssd::fused_handoff_failed(workspace, st, &failed) != hipSuccess || failed)
        return SSD_ERR_HIP;
    }
    return SSD_OK;
  }
  if (varlen &&
      ssd::launch_seq_index(cu_seqlens, (int)p->nseqs, p->seqlen, a.seq_idx, st) != hipSuccess)
    return SSD_ERR_HIP;
  if (ssd::launch_dt_cumsum(a, Q, bf16, st) != hipSuccess) return SSD_ERR_HIP;
  if (ssd::launch_chunked_tail(a, N, P, Q, bf16, st) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

}  // namespace

extern "C" {

ssd_status ssd_step(const ssd_problem* p, const void* x, const void* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* dt_bias,
                    float* state, void* y, void* stream) {
  if (!p) return SSD_ERR_INVALID_ARG;
  if (p->batch < 0 || p->seqlen != 1 || p->nheads <= 0 || p->headdim <= 0 || p->dstate <= 0 ||
      p->ngroups <= 0 || p->nheads % p->ngroups != 0 || p->ngroups_c < 0 ||
      (p->ngroups_c > 0 && p->nheads % p->ngroups_c != 0))
    return SSD_ERR_INVALID_ARG;
  if (p->dtype != SSD_DTYPE_F32 && p->dtype != SSD_DTYPE_BF16) return SSD_ERR_INVALID_ARG;
  if (p->flags & ~(uint32_t)(SSD_DT_SOFTPLUS | SSD_DT_SCALES_INPUT)) return SSD_ERR_INVALID_ARG;
  if (std::isnan(p->dt_min) || std::isnan(p->dt_max) || p->dt_min > p->dt_max)
    return SSD_ERR_INVALID_ARG;
  if (p->headdim != 64 && p->headdim != 128) return SSD_ERR_UNSUPPORTED;
  if (p->batch > 65535 || p->nheads > 65535 || p->dstate > 65536) return SSD_ERR_UNSUPPORTED;
  if (p->batch > 0 && (!x || !dt || !A || !B || !C || !state || !y)) return SSD_ERR_INVALID_ARG;
  ssd::StepArgs a{};
  a.sh.L = 1;
  a.sh.batch = (int32_t)p->batch;
  a.sh.H = (int32_t)p->nheads;
  a.sh.G = (int32_t)p->ngroups;
  a.sh.hpg = (int32_t)(p->nheads / p->ngroups);
  a.sh.Gc = (int32_t)(p->ngroups_c > 0 ? p->ngroups_c : p->ngroups);
  a.sh.hpgc = (int32_t)(p->nheads / a.sh.Gc);
  a.sh.flags = p->flags;
  a.sh.dt_min = p->dt_min;
  a.sh.dt_max = p->dt_max;
  a.N = (int)p->dstate;
  a.P = (int)p->headdim;
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.dt_bias = dt_bias;
  a.state = state;
  a.y = y;
  return ssd::launch_step(a, p->dtype == SSD_DTYPE_BF16, reinterpret_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? SSD_OK
             : SSD_ERR_HIP;
}

ssd_status ssd_dt_cumsum(const ssd_problem* p, const void* dt, const float* A,
                         const float* dt_bias, float* dt_out, float* cs_out, void* stream) {
  ssd_status s = check_problem(p);
  if (s != SSD_OK) return s;
  if (p->batch * p->seqlen > 0 && (!dt || !A || !dt_out || !cs_out)) return SSD_ERR_INVALID_ARG;
  const Plan pl = make_plan(*p, false);
  ChunkedArgs a{};
  a.sh = make_shape(*p, pl, false, false);
  a.marks = nullptr;
  a.dt = dt;
  a.A = A;
  a.dt_bias = dt_bias;
  a.dt_out = dt_out;
  a.cs = cs_out;
  a.coef = nullptr;
  a.cinfo = nullptr;
  return ssd::launch_dt_cumsum(a, (int)p->chunk_size, p->dtype == SSD_DTYPE_BF16,
                               reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? SSD_OK
             : SSD_ERR_HIP;
}

}  // extern "C"

namespace {

// Backward workspace: the forward's dt / prefix-sum / state buffers on
// 64-token chunks, the adjoints, the per-chunk partial sums and the per-head
// dB / dC; with packed sequences also the per-token and per-sequence sums of
// the sequence-state terms.
struct BwdPlan {
  int64_t nc = 0;
  size_t cs = 0, dt = 0, coef = 0, cinfo = 0, states = 0, adj = 0, dBh = 0, dCh = 0,
         part = 0, seq = 0, seq_tmp = 0, seq_part = 0, sc_states = 0, sc_adj = 0, total = 0;
};

BwdPlan make_bwd_plan(const ssd_problem& p) {
  BwdPlan pl;
  const int64_t rows = p.batch, H = p.nheads, Q = ssd::kBwdChunk;
  const int64_t NP = p.dstate * p.headdim;
  pl.nc = (p.seqlen + Q - 1) / Q;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t per_chunk = (size_t)(rows * H * pl.nc);
  pl.cs = take(per_chunk * Q * sizeof(float));
  pl.dt = take(per_chunk * Q * sizeof(float));
  pl.coef = take(per_chunk * sizeof(float2));
  pl.cinfo = take((size_t)(rows * pl.nc) * sizeof(ChunkInfo));
  pl.states = take(per_chunk * (size_t)NP * sizeof(float));
  pl.adj = take(per_chunk * (size_t)NP * sizeof(float));
  pl.dBh = take((size_t)(rows * p.seqlen * H * p.dstate) * sizeof(float));
  pl.dCh = take((size_t)(rows * p.seqlen * H * p.dstate) * sizeof(float));
  pl.part = take(per_chunk * 3 * sizeof(float));
  pl.seq = take(p.nseqs > 0 ? (size_t)p.seqlen * sizeof(int32_t) : 0);
  pl.seq_tmp = take(p.nseqs > 0 ? (size_t)(p.seqlen * H * 3) * sizeof(float) : 0);
  pl.sc_states = take(per_chunk * (size_t)(NP / 256) * sizeof(int));
  pl.sc_adj = take(per_chunk * (size_t)(NP / 256) * sizeof(int));
  pl.seq_part = take(p.nseqs > 0 ? (size_t)(p.nseqs * H * 2) * sizeof(float) : 0);
  pl.total = off;
  return pl;
}

ssd_status check_bwd_problem(const ssd_problem* p) {
  ssd_status s = check_problem(p);
  if (s != SSD_OK) return s;
  if (!ssd::bwd_supported((int)p->dstate, (int)p->headdim, p->dtype == SSD_DTYPE_BF16))
    return SSD_ERR_UNSUPPORTED;
  if ((p->seqlen + ssd::kBwdChunk - 1) / ssd::kBwdChunk > 65535) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

ssd_status bwd_impl(const ssd_problem* p, const void* x, const void* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* dt_bias,
                    const float* initial_states, const int32_t* cu_seqlens, const void* dy,
                    const float* d_final_states, void* dx, void* ddt, float* dA, void* dB,
                    void* dC, float* dD, float* ddt_bias, float* d_initial_states,
                    void* workspace, size_t workspace_bytes, void* stream,
                    ssd::LaunchMarks* marks) {
  if (!p) return SSD_ERR_INVALID_ARG;
  ssd_status s = check_bwd_problem(p);
  if (s != SSD_OK) return s;
  const bool varlen = cu_seqlens != nullptr;
  if (varlen && (p->batch != 1 || p->nseqs < 1)) return SSD_ERR_INVALID_ARG;
  if (!varlen && p->nseqs > 0) return SSD_ERR_INVALID_ARG;
  // packed sequences with per-sequence states: the chunk kernels run from zero
  // states and k_bwd_seq_terms adds what the states contribute
  const bool seq_terms = varlen && (initial_states || d_final_states || d_initial_states);
  const int64_t tokens = p->batch * p->seqlen;
  if (!A || !dA) return SSD_ERR_INVALID_ARG;
  if (tokens > 0 && (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC))
    return SSD_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const BwdPlan pl = make_bwd_plan(*p);
  if (tokens > 0) {
    if (!workspace || workspace_bytes < pl.total) return SSD_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return SSD_ERR_INVALID_ARG;
  }
  char* ws = static_cast<char*>(workspace);
  Plan fpl;
  fpl.nc = pl.nc;
  ssd::BwdArgs a{};
  a.f.sh = make_shape(*p, fpl, varlen, initial_states != nullptr && !seq_terms);
  a.f.x = x;
  a.f.dt = dt;
  a.f.A = A;
  a.f.B = B;
  a.f.C = C;
  a.f.D = D;
  a.f.dt_bias = dt_bias;
  a.f.init = seq_terms ? nullptr : initial_states;
  a.f.cu = cu_seqlens;
  a.f.y = nullptr;
  a.f.seq_idx = nullptr;
  a.f.flags = nullptr;
  a.f.marks = marks;
  a.N = (int)p->dstate;
  a.P = (int)p->headdim;
  a.dy = dy;
  a.dfinal = seq_terms ? nullptr : d_final_states;
  a.dx = dx;
  a.ddt = ddt;
  a.dA = dA;
  a.dB = dB;
  a.dC = dC;
  a.dD = dD;
  a.ddt_bias = ddt_bias;
  a.dinit = seq_terms ? nullptr : d_initial_states;
  a.seq_terms = seq_terms;
  a.seq_init = initial_states;
  a.seq_dfinal = d_final_states;
  a.seq_dinit = d_initial_states;
  if (tokens == 0) {
    // nothing but the states: dinit = dfinal, and zero head sums
    const int64_t n = (varlen ? p->nseqs : p->batch) * p->nheads * p->dstate * p->headdim;
    if (d_initial_states && ssd::launch_empty_final(d_final_states, n, d_initial_states, st) != hipSuccess)
      return SSD_ERR_HIP;
    a.part = nullptr;
    return ssd::launch_bwd_sums(a, st) == hipSuccess ? SSD_OK : SSD_ERR_HIP;
  }
  a.f.cs = reinterpret_cast<float*>(ws + pl.cs);
  a.f.dt_out = reinterpret_cast<float*>(ws + pl.dt);
  a.f.coef = reinterpret_cast<float2*>(ws + pl.coef);
  a.f.cinfo = reinterpret_cast<ChunkInfo*>(ws + pl.cinfo);
  a.f.states = reinterpret_cast<float*>(ws + pl.states);
  a.f.final_states = nullptr;
  a.adj = reinterpret_cast<float*>(ws + pl.adj);
  a.dBh = reinterpret_cast<float*>(ws + pl.dBh);
  a.dCh = reinterpret_cast<float*>(ws + pl.dCh);
  a.part = reinterpret_cast<float*>(ws + pl.part);
  a.seq_tmp = varlen ? reinterpret_cast<float*>(ws + pl.seq_tmp) : nullptr;
  a.seq_part = varlen ? reinterpret_cast<float*>(ws + pl.seq_part) : nullptr;
  a.sc_states = reinterpret_cast<int*>(ws + pl.sc_states);
  a.sc_adj = reinterpret_cast<int*>(ws + pl.sc_adj);

  const bool bf16 = p->dtype == SSD_DTYPE_BF16;
  const int Q = ssd::kBwdChunk;
  if (varlen) {
    if (env_validate() && (s = check_cu_seqlens_on_host(*p, cu_seqlens, st)) != SSD_OK) return s;
    a.f.seq_idx = reinterpret_cast<int32_t*>(ws + pl.seq);
    if (ssd::launch_seq_index(cu_seqlens, (int)p->nseqs, p->seqlen, a.f.seq_idx, st) != hipSuccess)
      return SSD_ERR_HIP;
  }
  if (ssd::launch_dt_cumsum(a.f, Q, bf16, st) != hipSuccess) return SSD_ERR_HIP;
  // the state walks for dense bf16 rows when their grid fills the device;
  // SSD_BWD_WALK=1 takes them whenever they can run, SSD_BWD_NO_WALK=1 never
  a.walked = ssd::bwd_walks_supported(a.f.sh, bf16) && !env_flag("SSD_BWD_NO_WALK") &&
             (env_flag("SSD_BWD_WALK") || ssd::bwd_walks_fill(a.f.sh, a.N, a.P));
  if (a.walked) {
    if (ssd::launch_bwd_walks(a, st) != hipSuccess) return SSD_ERR_HIP;
  } else {
    if (ssd::launch_chunk_states(a.f, a.N, a.P, Q, bf16, st) != hipSuccess) return SSD_ERR_HIP;
    if (ssd::launch_chunk_adjoint(a.f, dy, a.adj, a.N, a.P, Q, bf16, st) != hipSuccess)
      return SSD_ERR_HIP;
  }
  if (ssd::launch_bwd_tail(a, bf16, st) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

}  // namespace

extern "C" {

size_t ssd_bwd_workspace_size(const ssd_problem* p) {
  if (check_bwd_problem(p) != SSD_OK) return 0;
  return make_bwd_plan(*p).total;
}

ssd_status ssd_bwd(const ssd_problem* p, const void* x, const void* dt, const float* A,
                   const void* B, const void* C, const float* D, const float* dt_bias,
                   const float* initial_states, const int32_t* cu_seqlens, const void* dy,
                   const float* d_final_states, void* dx, void* ddt, float* dA, void* dB, void* dC,
                   float* dD, float* ddt_bias, float* d_initial_states, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return bwd_impl(p, x, dt, A, B, C, D, dt_bias, initial_states, cu_seqlens, dy, d_final_states,
                  dx, ddt, dA, dB, dC, dD, ddt_bias, d_initial_states, workspace, workspace_bytes,
                  stream, nullptr);
}

ssd_status ssd_bwd_events(const ssd_problem* p, const void* x, const void* dt, const float* A,
                          const void* B, const void* C, const float* D, const float* dt_bias,
                          const float* initial_states, const int32_t* cu_seqlens, const void* dy,
                          const float* d_final_states, void* dx, void* ddt, float* dA, void* dB,
                          void* dC, float* dD, float* ddt_bias, float* d_initial_states,
                          void* workspace, size_t workspace_bytes, void* stream,
                          void* const* events, const char** names, int max_events,
                          int* n_events) {
  if (n_events) *n_events = 0;
  if (max_events < 0 || (max_events > 0 && !events)) return SSD_ERR_INVALID_ARG;
  ssd::LaunchMarks m{events, names, max_events, 0};
  const ssd_status s = bwd_impl(p, x, dt, A, B, C, D, dt_bias, initial_states, cu_seqlens, dy,
                                d_final_states, dx, ddt, dA, dB, dC, dD, ddt_bias,
                                d_initial_states, workspace, workspace_bytes, stream, &m);
  if (s == SSD_OK && m.count < m.max_events) {
    if (m.names) m.names[m.count] = "end";
    if (hipEventRecord(static_cast<hipEvent_t>(m.events[m.count]), (hipStream_t)stream) !=
        hipSuccess)
      return SSD_ERR_HIP;
    ++m.count;
  }
  if (n_events) *n_events = m.count;
  return s;
}

const char* ssd_status_string(ssd_status s) {
  // a C caller may pass any int: read it as one (a C++ load of an enum outside
  // its range is undefined)
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARG: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported problem (dtype, head dim, state dim or chunk)";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

const char* ssd_version(void) { return "ssd_scan_amd 0.1.0 (gfx950, HIP)"; }

}  // extern "C"
