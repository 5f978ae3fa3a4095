// Drives the host side of libssd's C ABI (problem validation, schedule choice,
// workspace plans, status strings) with valid, invalid and extreme problems,
// for a build whose host code runs under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Nothing here needs a GPU: every call returns
// before its first launch.  Exit status 0 when every call returned what it
// should.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "ssd.h"

static int failures = 0;
#define CHECK(cond, what)                                  \
  do {                                                     \
    if (!(cond)) {                                         \
      std::fprintf(stderr, "host check failed: %s\n", what); \
      ++failures;                                          \
    }                                                      \
  } while (0)

static ssd_problem base() {
  ssd_problem p{};
  p.batch = 2, p.seqlen = 1000, p.nheads = 8, p.headdim = 64, p.dstate = 128;
  p.ngroups = 2, p.chunk_size = 256, p.nseqs = 0, p.dtype = SSD_DTYPE_BF16;
  p.flags = SSD_DT_SOFTPLUS, p.dt_min = 0.f, p.dt_max = std::numeric_limits<float>::infinity();
  p.algo = SSD_ALGO_AUTO, p.ngroups_c = 0;
  return p;
}

int main() {
  CHECK(ssd_version() != nullptr && ssd_version()[0] != '\0', "version");
  for (int s = -2; s < 8; ++s) CHECK(ssd_status_string((ssd_status)s) != nullptr, "status string");
  CHECK(ssd_workspace_size(nullptr) == 0, "null problem");
  CHECK(ssd_bwd_workspace_size(nullptr) == 0, "null problem (backward)");

  // every supported shape, schedule, storage type and packing has a plan
  const int64_t Ps[] = {64, 128}, Ns[] = {16, 32, 64, 128, 256}, Qs[] = {64, 128, 256};
  const int32_t dtypes[] = {SSD_DTYPE_BF16, SSD_DTYPE_F32};
  const int32_t algos[] = {SSD_ALGO_AUTO, SSD_ALGO_CHUNKED, SSD_ALGO_FUSED, SSD_ALGO_STREAM};
  int planned = 0;
  for (int64_t P : Ps)
    for (int64_t N : Ns)
      for (int64_t Q : Qs)
        for (int32_t dt : dtypes)
          for (int32_t algo : algos)
            for (int packed = 0; packed < 2; ++packed)
              for (int64_t L : {int64_t(1), int64_t(255), int64_t(4097), int64_t(65536)}) {
                ssd_problem p = base();
                p.headdim = P, p.dstate = N, p.chunk_size = Q, p.dtype = dt, p.algo = algo;
                p.seqlen = L;
                if (packed) p.batch = 1, p.nseqs = 7;
                const size_t ws = ssd_workspace_size(&p);
                const bool f32_too_big = dt == SSD_DTYPE_F32 && N * P > 16384;
                if (algo == SSD_ALGO_AUTO || algo == SSD_ALGO_CHUNKED)
                  CHECK((ws > 0) == !f32_too_big, "auto and chunked plans");
                planned += ws > 0;
                (void)ssd_bwd_workspace_size(&p);
              }
  CHECK(planned > 0, "some plans");

  // invalid problems: no workspace, and the entry points refuse them before
  // touching any pointer
  auto refused = [](ssd_problem p, const char* what) {
    CHECK(ssd_workspace_size(&p) == 0, what);
    CHECK(ssd_bwd_workspace_size(&p) == 0, what);
    const ssd_status s = ssd_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr);
    CHECK(s == SSD_ERR_INVALID_ARG || s == SSD_ERR_UNSUPPORTED, what);
  };
  ssd_problem p = base();
  p.batch = -1, refused(p, "negative batch");
  p = base(), p.seqlen = -5, refused(p, "negative seqlen");
  p = base(), p.nheads = 0, refused(p, "no heads");
  p = base(), p.nheads = 6, p.ngroups = 4, refused(p, "H % G");
  p = base(), p.ngroups_c = 3, refused(p, "H % Gc");
  p = base(), p.ngroups_c = -1, refused(p, "negative Gc");
  p = base(), p.headdim = 32, refused(p, "P = 32");
  p = base(), p.dstate = 48, refused(p, "N = 48");
  p = base(), p.chunk_size = 96, refused(p, "Q = 96");
  p = base(), p.chunk_size = 0, refused(p, "Q = 0");
  p = base(), p.dtype = 7, refused(p, "dtype");
  p = base(), p.flags = 1u << 5, refused(p, "flags");
  p = base(), p.dt_min = std::nanf(""), refused(p, "NaN dt_min");
  p = base(), p.dt_min = 2.f, p.dt_max = 1.f, refused(p, "dt_min > dt_max");
  p = base(), p.algo = 9, refused(p, "algo");
  // a forced schedule that does not take the shape (the backward pass has no
  // schedule choice)
  p = base(), p.dtype = SSD_DTYPE_F32, p.algo = SSD_ALGO_STREAM;
  CHECK(ssd_workspace_size(&p) == 0, "stream takes bf16 only");
  p = base(), p.headdim = 128, p.algo = SSD_ALGO_FUSED;
  CHECK(ssd_workspace_size(&p) == 0, "fused takes P = 64 only");
  // every size within its own limit, their product beyond any memory
  p = base(), p.batch = 65535, p.seqlen = int64_t(1) << 24, p.nheads = 65535, p.ngroups = 1;
  refused(p, "layer beyond 2^40 elements");
  p = base(), p.batch = 1, p.nseqs = int64_t(1) << 40, refused(p, "too many sequences");
  p = base(), p.batch = 70000, refused(p, "batch beyond the grid");
  p = base(), p.seqlen = int64_t(1) << 40, refused(p, "seqlen beyond 32-bit positions");
  p = base(), p.nheads = std::numeric_limits<int64_t>::max(), p.ngroups = 1, refused(p, "huge H");
  p = base(), p.batch = std::numeric_limits<int64_t>::max(), refused(p, "huge batch");
  p = base(), p.seqlen = std::numeric_limits<int64_t>::max(), refused(p, "huge seqlen");

  // packed sequences need batch 1 and nseqs >= 1
  int32_t cu[2] = {0, 1000};
  p = base();
  CHECK(ssd_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, cu,
                nullptr, nullptr, nullptr, 0, nullptr) == SSD_ERR_INVALID_ARG,
        "packed sequences with batch 2");
  // tokens but no x
  p = base();
  CHECK(ssd_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                nullptr, nullptr, nullptr, nullptr, 0, nullptr) == SSD_ERR_INVALID_ARG,
        "missing inputs");
  // a negative event count
  int n = -1;
  CHECK(ssd_fwd_events(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                       nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, -1,
                       &n) == SSD_ERR_INVALID_ARG && n == 0,
        "negative event count");
  if (failures == 0) std::printf("host checks passed\n");
  return failures != 0;
}
