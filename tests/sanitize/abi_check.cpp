// Host-side check of the C-ABI's argument handling, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only (no GPU is touched).
//
// Every call below must be refused by the host-side validation before anything is enqueued:
// sizes at and beyond the documented limits (negative, zero, INT32_MAX, INT64_MAX), pointers
// that are fake but well aligned, and an output placed on top of an input so that a call whose
// sizes are valid ends at the aliasing check.  The size and plan queries are swept over the
// same extremes and must agree with one another.  A return code outside the allowed set, a
// sanitizer report or a crash fails the run.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mambamix.h"

static int failures = 0;

#define EXPECT(cond, ...)                                \
  do {                                                   \
    if (!(cond)) {                                       \
      ++failures;                                        \
      if (failures <= 20) {                              \
        std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        std::fprintf(stderr, __VA_ARGS__);               \
        std::fprintf(stderr, "\n");                      \
      }                                                  \
    }                                                    \
  } while (0)

// fake device addresses 2^40 bytes apart: aligned for every element type, never overlapping
static void* fake(int i) { return reinterpret_cast<void*>((uintptr_t(1) << 44) + (uintptr_t(i) << 40)); }

static bool refused(int rc) { return rc == MM_ERR_NULL || rc == MM_ERR_DIM || rc == MM_ERR_UNSUPPORTED ||
                                     rc == MM_ERR_ALIGN || rc == MM_ERR_WORKSPACE || rc == MM_ERR_ALIAS; }

static const int32_t I32[] = {-1, 0, 1, 7, 16, 4096, MM_ROW_MAX_D, MM_ROW_MAX_D + 16, 65536 * 1024, INT32_MAX};
static const int64_t I64[] = {-1, 0, 1, 100, 16384, INT32_MAX, int64_t(INT32_MAX) + 1, int64_t(1) << 40, INT64_MAX};
static const int32_t NS[] = {0, 1, 4, 16, 17, INT32_MAX};
static const int64_t CH[] = {INT64_MIN, -1, 0, 1, 16, 2048, int64_t(1) << 40, INT64_MAX};

static bool valid_sizes(int32_t S, int64_t T, int32_t d, int32_t N) {
  if (S < 0 || T < 0 || d < 0 || T > INT32_MAX || N < 1 || N > MM_MAX_N || (S == 0 && T > 0)) return false;
  return d == 0 || (uint64_t(T) <= MM_MAX_ROWS_X_D / uint64_t(d) && uint64_t(S) <= MM_MAX_ROWS_X_D / uint64_t(d));
}

static void sweep_plans() {
  long calls = 0;
  for (int32_t S : I32)
    for (int64_t T : I64)
      for (int32_t d : I32)
        for (int32_t N : NS)
          for (int64_t ch : CH)
            for (int32_t eng = -1; eng <= 3; ++eng) {
              int64_t cl = -7;
              int32_t en = -7, nk = -7;
              size_t ws = 12345;
              const int rc = mamba_mixer_prefill_plan(S, T, d, N, 4, ch, eng, &cl, &en, &ws, &nk);
              ++calls;
              EXPECT(rc == MM_OK || refused(rc), "plan rc %d", rc);
              if (!valid_sizes(S, T, d, N)) EXPECT(rc != MM_OK, "plan accepted S=%d T=%lld d=%d N=%d", S,
                                                   (long long)T, d, N);
              const bool empty = T == 0 || d == 0 || S == 0;
              if ((eng < 0 || eng > 2) && !empty)
                EXPECT(rc == MM_ERR_UNSUPPORTED || rc == MM_ERR_DIM, "engine %d rc %d", eng, rc);
              if (rc != MM_OK) continue;
              if (empty) {  // nothing to do: no kernels, no workspace, whatever the engine
                EXPECT(nk == 0 && ws == 0, "empty problem: %d kernels, %zu bytes", nk, ws);
                continue;
              }
              EXPECT(cl >= 16 && cl % 16 == 0 && cl <= 4 * T + 512, "chunk length %lld (T %lld)",
                     (long long)cl, (long long)T);
              EXPECT(nk >= 0 && nk <= 8, "kernel count %d", nk);
              EXPECT(en == MM_ENGINE_LANE || en == MM_ENGINE_ROW, "engine out %d", en);
              EXPECT(mamba_mixer_prefill_workspace_bytes_chunked(S, T, d, N, 4, ch) ==
                         (eng == MM_ENGINE_AUTO ? ws : mamba_mixer_prefill_workspace_bytes_chunked(S, T, d, N, 4, ch)),
                     "workspace query disagrees with the plan");
              for (int32_t i = -1; i <= nk; ++i) {
                const char* name = mamba_mixer_prefill_kernel_name(S, T, d, N, 4, ch, eng, i);
                EXPECT(name != nullptr, "kernel name NULL");
                if (name == nullptr) continue;
                const bool in = i >= 0 && i < nk;
                EXPECT(in == (name[0] != '\0'), "kernel name %d of %d: '%s'", i, nk, name);
              }
            }
  // the plain workspace query and the plan with chunk_len 0 / automatic engine agree
  for (int32_t S : I32)
    for (int64_t T : I64)
      for (int32_t d : I32)
        for (int32_t N : NS) {
          size_t ws = 0;
          const int rc = mamba_mixer_prefill_plan(S, T, d, N, 4, 0, MM_ENGINE_AUTO, nullptr, nullptr, &ws, nullptr);
          const size_t q = mamba_mixer_prefill_workspace_bytes(S, T, d, N, 4);
          EXPECT(rc == MM_OK ? q == ws : q == 0, "workspace query %zu vs plan %zu (rc %d)", q, ws, rc);
          for (int has = 0; has <= 1; ++has) {
            size_t bw = 777;
            int32_t bk = -1;
            const int brc = mamba_mixer_prefill_backward_plan(S, T, d, N, 4, has, &bw, &bk);
            EXPECT(brc == MM_OK || refused(brc), "backward plan rc %d", brc);
            const size_t bq = mamba_mixer_prefill_backward_workspace_bytes(S, T, d, N, 4, has);
            EXPECT(brc == MM_OK ? bq == bw : bq == 0, "backward workspace %zu vs plan %zu", bq, bw);
            if (brc == MM_OK && d == 0) EXPECT(bk == 0 && bw == 0, "backward with d == 0: %d kernels", bk);
            if (brc == MM_OK && d > 0) EXPECT(bk >= 1 && bk <= 8, "backward kernels %d", bk);
          }
          (void)mamba_mixer_checkpoint_bytes(S, T, d);
          calls += 4;
        }
  for (int32_t d : I32)
    for (int32_t N : NS)
      for (int32_t R : {-1, 0, 1, 64, 256, 257, INT32_MAX})
        for (int64_t T : I64) (void)mamba_mixer_project_workspace_bytes(T, d, N, R);
  for (int code : {INT_MIN, -8, -7, -1, 0, 1, INT_MAX}) EXPECT(mamba_mixer_status_string(code) != nullptr, "status");
  EXPECT(mamba_mixer_version() != nullptr && std::strlen(mamba_mixer_version()) > 0, "version");
  {  // the host check of cu_seqlens reads exactly S + 1 entries (the vectors are sized to that)
    const std::vector<int32_t> ok{0, 3, 3, 10}, bad{0, 5, 4, 10}, one{0};
    EXPECT(mamba_mixer_check_cu_seqlens(ok.data(), 3, 10) == MM_OK, "cu ok");
    EXPECT(mamba_mixer_check_cu_seqlens(bad.data(), 3, 10) == MM_ERR_DIM, "cu decreasing");
    EXPECT(mamba_mixer_check_cu_seqlens(ok.data(), 3, 9) == MM_ERR_DIM, "cu end");
    EXPECT(mamba_mixer_check_cu_seqlens(one.data(), 0, 0) == MM_OK, "cu empty");
    EXPECT(mamba_mixer_check_cu_seqlens(one.data(), -1, 0) == MM_ERR_DIM, "cu S");
    EXPECT(mamba_mixer_check_cu_seqlens(nullptr, 2, 10) == MM_ERR_NULL, "cu null");
  }
  std::printf("plan queries: %ld calls\n", calls);
}

// Entry points with fake pointers and one output on top of an input: every call is refused.
static void sweep_calls() {
  long calls = 0;
  void* p[32];
  for (int i = 0; i < 32; ++i) p[i] = fake(i);
  const int32_t* cu = static_cast<const int32_t*>(p[10]);
  for (int32_t S : I32)
    for (int64_t T : I64)
      for (int32_t d : I32)
        for (int32_t N : NS)
          for (int32_t io : {0, 1, 2}) {
            const bool empty = valid_sizes(S, T, d, N) && (io == 0 || io == 1) && (T == 0 || d == 0 || S == 0);
            // prefill: y on top of x
            int rc = mamba_mixer_prefill_chunked(p[0], p[1], p[2], p[3], p[4], (float*)p[5], (float*)p[6],
                                                 (float*)p[7], (float*)p[8], (float*)p[9], cu, (float*)p[11],
                                                 (float*)p[12], p[0], S, T, d, N, 4, io, 0, nullptr, 0, nullptr);
            EXPECT(empty ? rc == MM_OK : refused(rc), "prefill rc %d S=%d T=%lld d=%d N=%d io=%d", rc, S,
                   (long long)T, d, N, io);
            rc = mamba_mixer_prefill_noalloc(p[0], p[1], p[2], p[3], p[4], (float*)p[5], (float*)p[6],
                                             (float*)p[7], (float*)p[8], (float*)p[9], cu, (float*)p[11],
                                             (float*)p[12], p[0], S, T, d, N, 4, io, nullptr);
            EXPECT(empty ? rc == MM_OK : refused(rc), "noalloc rc %d", rc);
            // training forward: checkpoints on top of y
            rc = mamba_mixer_prefill_train(p[0], p[1], p[2], p[3], p[4], (float*)p[5], (float*)p[6], (float*)p[7],
                                           (float*)p[8], (float*)p[9], cu, (float*)p[11], (float*)p[12], p[13],
                                           (float*)p[13], S, T, d, N, 4, io, 0, p[20], SIZE_MAX & ~size_t(255),
                                           nullptr, nullptr, 0);
            EXPECT(rc == MM_OK ? empty : refused(rc), "train rc %d", rc);
            // backward: dA_log on top of A_log (a parameter gradient: written even when T == 0)
            rc = mamba_mixer_prefill_backward(p[0], p[1], p[2], p[3], p[4], (float*)p[5], (float*)p[6],
                                              (float*)p[7], (float*)p[8], (float*)p[9], cu, (float*)p[11],
                                              (float*)p[12], p[13], nullptr, p[14], p[15], p[16], p[17], p[18],
                                              (float*)p[5], (float*)p[20], (float*)p[21], (float*)p[22],
                                              (float*)p[23], (float*)p[24], (float*)p[25], S, T, d, N, 4, io,
                                              p[26], SIZE_MAX & ~size_t(255), nullptr, nullptr, 0);
            EXPECT(rc == MM_OK ? d == 0 : refused(rc), "backward rc %d S=%d T=%lld d=%d",
                   rc, S, (long long)T, d);
            // projection: dt on top of x
            for (int32_t R : {0, 16, 257}) {
              rc = mamba_mixer_project(p[0], (float*)p[1], (float*)p[2], cu, (float*)p[4], p[5], p[6], p[0], p[8],
                                       p[9], S, T, d, N, R, 4, io, p[26], SIZE_MAX & ~size_t(255), nullptr, nullptr,
                                       0);
              EXPECT(rc == MM_OK ? T == 0 || d == 0 : refused(rc), "project rc %d", rc);
              ++calls;
            }
            calls += 4;
          }
  // decode-side entry points: rows = T clipped to int32
  for (int32_t Bs : I32)
    for (int32_t d : I32)
      for (int32_t N : NS)
        for (int32_t io : {0, 1, 2}) {
          const bool empty = Bs >= 0 && d >= 0 && N >= 1 && N <= MM_MAX_N && (io == 0 || io == 1) && (Bs == 0 || d == 0);
          int rc = mamba_mixer_decode(p[0], p[1], p[2], p[3], p[4], (float*)p[5], (float*)p[6], (float*)p[7],
                                      (float*)p[8], (float*)p[9], (float*)p[10], (float*)p[11], p[0], Bs, d, N, 4, io,
                                      nullptr);
          EXPECT(empty ? rc == MM_OK : refused(rc), "decode rc %d Bs=%d d=%d N=%d", rc, Bs, d, N);
          for (int32_t W : {-1, 0, 1, 4, 5, INT32_MAX})
            for (int32_t k : {-1, 0, 3, INT32_MAX}) {
              rc = mamba_mixer_decode_replay(p[0], p[1], p[2], p[3], p[4], (float*)p[5], (float*)p[6], (float*)p[7],
                                             (float*)p[8], (float*)p[9], (float*)p[10], (float*)p[11], p[3], Bs, d,
                                             N, 4, io, W, k, 0, nullptr);
              EXPECT(rc == MM_OK ? Bs == 0 || d == 0 : refused(rc), "replay rc %d", rc);
              rc = mamba_mixer_decode_replay_dual(p[0], p[1], p[2], p[3], p[4], (float*)p[5], (float*)p[6],
                                                  (float*)p[7], (float*)p[8], (float*)p[9], (float*)p[10],
                                                  (float*)p[11], p[12], p[11], p[14], Bs, d, N, 4, io, W, k, 0,
                                                  nullptr);
              EXPECT(rc == MM_OK ? Bs == 0 || d == 0 : refused(rc), "replay dual rc %d", rc);
              rc = mamba_mixer_decode_replay_multi(p[0], p[1], p[2], p[3], p[4], (float*)p[5], (float*)p[6],
                                                   (float*)p[7], (float*)p[8], (float*)p[9], (float*)p[10],
                                                   (float*)p[11], p[3], Bs, d, N, 4, io, W, 0, k, -1, nullptr);
              EXPECT(rc == MM_OK ? Bs == 0 || d == 0 : refused(rc), "replay multi rc %d", rc);
              calls += 3;
            }
          rc = mamba_mixer_replay_checkpoint_lo((float*)p[0], (float*)p[1], p[0], p[3], Bs, d, N, 4, nullptr);
          EXPECT(rc == MM_OK ? Bs == 0 || d == 0 : refused(rc), "checkpoint_lo rc %d", rc);
          calls += 2;
        }
  std::printf("entry points: %ld calls\n", calls);
}

int main() {
  sweep_plans();
  sweep_calls();
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
