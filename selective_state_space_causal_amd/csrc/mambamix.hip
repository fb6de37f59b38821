// libmambamix -- HIP kernels for gfx950 (MI355X) and the C ABI declared in include/mambamix.h.
//
// The mixer step (TensorRT Mamba tensor-parallel builder, _add_mamba_tp_layer):
//   u = SiLU(conv_b + sum_k conv_w[k] * window[k]),  delta = softplus(dt + dt_bias),
//   h = exp(delta * A) * h + delta * B * u,  y = (C . h + D * u) * SiLU(z),
// run token after token over packed sequences (PackMamba: no state crosses a
// cu_seqlens boundary), with the final conv/SSM state left in the caller's slots
// (the state cache carried from prefill into decode on the tensor-parallel SSM page).
//
// Cost model (gfx950, wave64): per token and channel the method does 22
// transcendental ops (16 exp for the decays, exp+log for softplus, exp+rcp for each
// SiLU) and ~77 plain fp32 ops, and moves 8 bytes of token io in bf16 -- prefill is
// bound by VALU issue, not HBM.  Decode streams the fp32 state once in and once out
// and is bound by HBM.  The prefill engines and the chunking are described in
// mm_prefill.h, the decode kernels in mm_decode.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <utility>

#include <stdint.h>
#include <string.h>

#include <cmath>

#include "mambamix.h"
#include "mm_backward.h"
#include "mm_decode.h"
#include "mm_device.h"
#include "mm_prefill.h"
#include "mm_project.h"
#include "mm_row.h"

namespace mm {
namespace {

// ---------------------------------------------------------------- prefill plan

// The lane engine needs this many (sequence, 64-channel block) waves to keep the
// GPU busy without splitting sequences and to beat the row engine, which needs fewer
// instructions' worth of parallelism but more instructions per (token, channel):
// measured crossover between 8192 waves (the engines within 4% either way) and 16384
// (the lane engine 10% ahead at 512-token sequences); at 4096 the row engine is 6% ahead.
constexpr int64_t kLaneMinWaves = 8192;
constexpr int64_t kCUs = 256;
// replay decode: N = 16 (4 lanes x 4 state entries per channel), windows of at most 4 steps
constexpr int kReplayN = 16;
constexpr int kReplayMaxW = 4;

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
inline int nmax_for(int N) { return N <= 4 ? 4 : (N <= 8 ? 8 : 16); }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  int engine;  // MM_ENGINE_LANE or MM_ENGINE_ROW
  int nmax;
  int64_t Lc;    // chunk length
  int64_t Pmax;  // chunk grid bound: ceil(T / Lc) + S
  int64_t Mmax;  // non-last-chunk bound: floor(T / Lc) (every non-last chunk holds Lc tokens)
  int ksub;      // row engine: pass 1 scans a non-last chunk as ksub pieces (carry slots: Mmax * ksub)
  bool inl;      // row engine: the kernels compute the chunk plan themselves (S <= kPlanInline)
  int64_t Tpad;  // B/C rows incl. zero padding past T
  size_t off_off, off_moff, off_bc, off_a, off_b, off_stash, total;
  int kernels;   // kernels one call enqueues
  bool whole;    // row engine with one chunk per sequence: no plan, no carries
};

// Pieces per non-last chunk in the row engine's pass 1: the smallest power of two that gives
// the pass about 8 workgroups per CU (it only has the non-last chunks to work on), keeping
// pieces at >= 128 tokens.  Chunk lengths are rounded to multiples of 16 * ksub.
int row_pieces(int64_t Lc, double nonlast_chunks, int64_t nchb) {
  int k = 1;
  while (k < 16 && nonlast_chunks * k * nchb < 8.0 * kCUs && Lc / (2 * k) >= 128) k *= 2;
  return k;
}

// Modelled time (microseconds) of the row engine with P chunks per (average) sequence,
// fitted to measurements on MI355X.  A pass is as slow as its busiest CU: with
// g = workgroups / 256, some CU runs ceil(g) workgroups, each taking (its W / wgs
// (token, channel) pairs) / rate + a fixed cost per workgroup.  Final pass: ~996 pairs per
// us per CU with >= 3 workgroups on the CU, x 0.82 with 2, less with 1, plus 7.8 us per
// workgroup (staging fill and drain, carry fold, final states).  Pass 1: 1.54x the rate,
// 1.5 us per workgroup.  Fitted to: the 130m-shaped call (3 per CU, 0.117 ms), and one
// 8192-token call at d_inner 5120 in whole-sequence mode (0.338 ms), in two chunks (pass 1
// in 8 pieces: 0.070 + 0.221 ms) and in four (pass 1 in 4 pieces: 0.100 + 0.204 ms).
// Chunking adds the plan (inside the kernels for S <= kPlanInline) and a launch (~3 us).
double row_pass_us(double W, double wgs, double speed, double per_wg) {
  if (wgs <= 0) return 0.0;
  const double g = std::ceil(wgs / kCUs);
  const double rate = 996.0 * (g >= 3 ? 1.0 : (g >= 2 ? 0.82 : 0.55)) * speed;  // pairs per us per CU
  return g * ((W / wgs) / rate + per_wg);
}
double row_cost(int64_t S, int64_t T, int d, int64_t P) {
  const double W = static_cast<double>(T) * d;
  const int64_t nchb = cdiv(d, kRowChans);
  const double wgs = static_cast<double>(S) * nchb;
  double t = row_pass_us(W, wgs * P, 1.0, 7.8);
  if (P > 1) {
    const int k = row_pieces(cdiv(cdiv(T, S), P), static_cast<double>(S) * (P - 1), nchb);
    t += row_pass_us(W * (P - 1) / P, wgs * (P - 1) * k, 1.54, 1.5) + (S <= kPlanInline ? 3.0 : 8.0);
  }
  return t;
}

// workgroups of a row-engine launch: (chunk, channel-group) items, 8 per 32 workgroups
int64_t row_grid(int64_t chunks, int d) {
  const int64_t items = chunks * cdiv(cdiv(d, kRowChans), kRowGroup);
  return cdiv(items, kXcds) * kXcds * kRowGroup;
}

int make_plan(Plan& p, int64_t S, int64_t T, int d, int N, int64_t chunk_len, int engine) {
  p = Plan{};
  p.nmax = nmax_for(N);
  const int64_t nblk = cdiv(d, kWave);
  const int64_t avg = cdiv(T, S > 0 ? S : 1);
  if (engine == MM_ENGINE_AUTO) engine = (S * nblk >= kLaneMinWaves || d > kRowMaxD) ? MM_ENGINE_LANE : MM_ENGINE_ROW;
  if (engine != MM_ENGINE_LANE && engine != MM_ENGINE_ROW) return MM_ERR_UNSUPPORTED;
  if (engine == MM_ENGINE_ROW && d > kRowMaxD) return MM_ERR_UNSUPPORTED;
  p.engine = engine;
  if (engine == MM_ENGINE_ROW) p.nmax = kRow;  // one state entry per lane of a 16-lane row
  if (chunk_len > 0) {
    // a chunk longer than the stream is the same as one of T + 1 tokens (whole sequences)
    p.Lc = std::min<int64_t>(chunk_len, T + 1);
  } else if (engine == MM_ENGINE_ROW) {
    // chunks shorter than ~256 tokens are not worth their carries
    const int64_t pmax = avg / 256 < 16 ? avg / 256 : 16;
    int64_t best = 1;
    for (int64_t P = 2; P <= pmax; ++P)
      if (row_cost(S, T, d, P) < row_cost(S, T, d, best)) best = P;
    // one chunk per sequence: a chunk longer than the whole stream leaves no carries
    p.Lc = best == 1 ? T + 1 : cdiv(avg, best);
  } else {
    // lane engine: sequences up to 4x the mean length stay whole; longer ones are split for balance
    p.Lc = 4 * avg;
    if (p.Lc < 512) p.Lc = 512;
  }
  if (p.Lc < 16) p.Lc = 16;  // >= 3 keeps a continuing chunk's conv window inside its sequence
  p.Lc = (p.Lc + 15) / 16 * 16;
  p.ksub = 1;
  if (engine == MM_ENGINE_ROW && p.Lc <= T) {
    // pass 1 in pieces; the chunk length a multiple of 16 pieces' worth of tokens
    const int64_t nchb = cdiv(d, kRowChans);
    // at least T / Lc - S non-last chunks (sequences longer than Lc have all but one)
    p.ksub = row_pieces(p.Lc, static_cast<double>(std::max<int64_t>(T / p.Lc - S, 1)), nchb);
    while (p.ksub > 1 && p.Lc % (16 * p.ksub) != 0) p.ksub /= 2;
    p.inl = S <= kPlanInline;
  }
  p.Pmax = cdiv(T, p.Lc) + S;
  p.Mmax = T / p.Lc;
  p.Tpad = T + 16;
  // packed B/C rows (the row engine stages B/C itself)
  const size_t nbc = engine == MM_ENGINE_ROW ? 0 : static_cast<size_t>(p.Tpad) * 2 * p.nmax;
  p.whole = engine == MM_ENGINE_ROW && p.Lc > T;
  size_t off = 0;
  p.off_off = off; off += align256(static_cast<size_t>(S + 1) * sizeof(int32_t));
  p.off_moff = off; off += align256(static_cast<size_t>(S + 1) * sizeof(int32_t));
  p.off_bc = off; off += align256(nbc * sizeof(float));
  if (p.whole) off = 0;  // nothing in the workspace is used
  if (p.Mmax > 0) {
    const size_t m1 = static_cast<size_t>(p.Mmax) * p.ksub;  // carry slots (pass-1 pieces)
    p.off_a = off; off += align256(m1 * d * sizeof(float));
    p.off_b = off; off += align256(m1 * d * p.nmax * sizeof(float));
    p.off_stash = off; off += align256(static_cast<size_t>(p.Mmax) * d * (p.nmax + kKS) * sizeof(float));
  }
  p.total = off;
  p.kernels = p.Mmax > 0 ? 5 : 3;
  // row engine: [k_chunk_plan unless the kernels compute it], [pass 1], pass 2
  if (engine == MM_ENGINE_ROW) p.kernels = p.whole ? 1 : (p.inl ? 0 : 1) + (p.Mmax > 0 ? 1 : 0) + 1;
  const int64_t wgs = engine == MM_ENGINE_LANE ? p.Pmax * cdiv(d, kBlock)
                                               : row_grid(p.whole ? S : std::max(p.Pmax, p.Mmax * p.ksub), d);
  if (wgs > INT32_MAX || p.Pmax > INT32_MAX) return MM_ERR_DIM;
  return MM_OK;
}

const char* kernel_name(const Plan& p, int i) {
  const char* agg = p.engine == MM_ENGINE_LANE ? "k_lane_agg" : "k_row_agg";
  const char* fin = p.engine == MM_ENGINE_LANE ? "k_lane_final" : "k_row_final";
  if (p.engine == MM_ENGINE_ROW) {  // stages B/C itself: no packing kernel; carries folded in pass 2
    if (p.whole) return i == 0 ? fin : "";
    const char* names[3];
    int n = 0;
    if (!p.inl) names[n++] = "k_chunk_plan";
    if (p.Mmax > 0) names[n++] = agg;
    names[n++] = fin;
    return i >= 0 && i < n ? names[i] : "";
  }
  if (i == 0) return "k_chunk_plan";
  if (i == 1) return "k_pack_bc";
  if (p.Mmax > 0) {
    if (i == 2) return agg;
    if (i == 3) return "k_carry";
    if (i == 4) return fin;
  } else if (i == 2) {
    return fin;
  }
  return "";
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && a0 < b0 + nb && b0 < a0 + na;
}

// Records events[k] (if given) on the stream before the k-th kernel and events[n]
// after the last one.
struct StageEvents {
  void* const* ev;
  int n;
  int k;
  void mark(hipStream_t st) {
    if (ev != nullptr && k < n) (void)hipEventRecord(static_cast<hipEvent_t>(ev[k]), st);
    ++k;
  }
};

struct PrefillArgs {
  const void *x, *z, *dt, *B, *C;
  const float *A_log, *D, *dt_bias, *conv_w, *conv_b;
  const int32_t* cu;
  float *conv_state, *ssm_state;
  void* y;
  int S;
  int64_t T;
  int d, N;
};

// The row kernel stages with 4-element vector loads when N = 16, d % 4 == 0 and every io
// tensor is aligned to 4 elements; otherwise element by element.
template <typename IO>
bool row_vec(int d, int N, std::initializer_list<const void*> io) {
  if (N != kRow || d % 4 != 0) return false;
  for (const void* q : io)
    if (q != nullptr && !aligned(q, 4 * sizeof(IO))) return false;
  return true;
}

template <typename IO, bool FINAL, bool CKPT>
void launch_k_row(bool vec, dim3 grid, hipStream_t st, const PrefillArgs& a, const IO* x, const IO* z, const IO* dt,
                  const IO* B, const IO* C, float* conv_state, float* ssm_state, IO* y, CarryWs cw, int64_t Lc,
                  int whole, float* ckpt) {
  const dim3 block(kRowThreads);
  if (vec)
    hipLaunchKernelGGL((k_row<IO, FINAL, CKPT, true>), grid, block, 0, st, x, z, dt, B, C, a.A_log, a.D, a.dt_bias,
                       a.conv_w, a.conv_b, a.cu, conv_state, ssm_state, y, cw, a.S, a.T, a.d, a.N, Lc, whole, ckpt);
  else
    hipLaunchKernelGGL((k_row<IO, FINAL, CKPT, false>), grid, block, 0, st, x, z, dt, B, C, a.A_log, a.D, a.dt_bias,
                       a.conv_w, a.conv_b, a.cu, conv_state, ssm_state, y, cw, a.S, a.T, a.d, a.N, Lc, whole, ckpt);
}

template <typename IO>
void launch_row(const Plan& p, const PrefillArgs& a, CarryWs cw, hipStream_t st, StageEvents& evs, float* ckpt) {
  const IO* xi = static_cast<const IO*>(a.x);
  const IO* zi = static_cast<const IO*>(a.z);
  const IO* di = static_cast<const IO*>(a.dt);
  const IO* Bi = static_cast<const IO*>(a.B);
  const IO* Ci = static_cast<const IO*>(a.C);
  const dim3 grid(static_cast<unsigned>(row_grid(p.whole ? a.S : p.Pmax, a.d)));
  const int whole = p.whole ? 1 : 0;
  const bool vec = row_vec<IO>(a.d, a.N, {a.x, a.z, a.dt, a.B, a.C, a.y});
  IO* yo = static_cast<IO*>(a.y);
  if (!p.whole && !p.inl) {
    evs.mark(st);
    hipLaunchKernelGGL(k_chunk_plan, dim3(1), dim3(kPlanThreads), 0, st, a.cu, a.S, p.Lc, cw.off, cw.moff);
  }
  if (!p.whole && p.Mmax > 0) {
    evs.mark(st);
    const dim3 grid1(static_cast<unsigned>(row_grid(p.Mmax * p.ksub, a.d)));  // pass-1 pieces
    launch_k_row<IO, false, false>(vec, grid1, st, a, xi, zi, di, Bi, Ci, a.conv_state, a.ssm_state, yo, cw, p.Lc,
                                   whole, nullptr);
  }
  evs.mark(st);
  if (ckpt != nullptr)
    launch_k_row<IO, true, true>(vec, grid, st, a, xi, zi, di, Bi, Ci, a.conv_state, a.ssm_state, yo, cw, p.Lc, whole,
                                 ckpt);
  else
    launch_k_row<IO, true, false>(vec, grid, st, a, xi, zi, di, Bi, Ci, a.conv_state, a.ssm_state, yo, cw, p.Lc,
                                  whole, nullptr);
}

template <typename IO, int NMAX>
int launch_prefill(const Plan& p, const PrefillArgs& a, char* ws, hipStream_t st, StageEvents evs,
                   float* ckpt = nullptr) {
  CarryWs cw{};
  cw.off = reinterpret_cast<int32_t*>(ws + p.off_off);
  cw.moff = reinterpret_cast<int32_t*>(ws + p.off_moff);
  cw.ksub = p.ksub;
  cw.inl = p.inl ? 1 : 0;
  if (p.Mmax > 0) {
    cw.a = reinterpret_cast<float*>(ws + p.off_a);
    cw.b = reinterpret_cast<float*>(ws + p.off_b);
    cw.stash = reinterpret_cast<float*>(ws + p.off_stash);
  }
  if (p.engine == MM_ENGINE_ROW) {
    if constexpr (NMAX == kRow) launch_row<IO>(p, a, cw, st, evs, ckpt);
    evs.mark(st);
    return hipGetLastError() == hipSuccess ? MM_OK : MM_ERR_HIP;
  }
  float* bc = reinterpret_cast<float*>(ws + p.off_bc);
  evs.mark(st);
  hipLaunchKernelGGL(k_chunk_plan, dim3(1), dim3(kPlanThreads), 0, st, a.cu, a.S, p.Lc, cw.off, cw.moff);
  evs.mark(st);
  const int64_t nbc = p.Tpad * 2 * NMAX;
  const dim3 gbc(static_cast<unsigned>(cdiv(nbc, kBlock)));
  const IO* Bi = static_cast<const IO*>(a.B);
  const IO* Ci = static_cast<const IO*>(a.C);
  {
    hipLaunchKernelGGL((k_pack_bc_rows<IO, NMAX>), gbc, dim3(kBlock), 0, st, Bi, Ci, bc, a.T, p.Tpad, a.N);
    const IO* xi = static_cast<const IO*>(a.x);
    const IO* zi = static_cast<const IO*>(a.z);
    const IO* di = static_cast<const IO*>(a.dt);
    const dim3 grid(static_cast<unsigned>(p.Pmax * cdiv(a.d, kBlock)));
    if (p.Mmax > 0) {
      evs.mark(st);
      hipLaunchKernelGGL((k_lane_agg<IO, NMAX>), grid, dim3(kBlock), 0, st, xi, di, bc, a.A_log, a.D, a.dt_bias,
                         a.conv_w, a.conv_b, a.cu, a.conv_state, a.ssm_state, cw, a.S, a.d, a.N, p.Lc);
      evs.mark(st);
      const int64_t q = static_cast<int64_t>(a.d) * NMAX;
      hipLaunchKernelGGL((k_carry<NMAX>), dim3(static_cast<unsigned>(cdiv(q, kBlock))), dim3(kBlock), 0, st, cw,
                         a.A_log, a.S, a.d, a.N);
    }
    evs.mark(st);
    hipLaunchKernelGGL((k_lane_final<IO, NMAX>), grid, dim3(kBlock), 0, st, xi, zi, di, bc, a.A_log, a.D,
                       a.dt_bias, a.conv_w, a.conv_b, a.cu, a.conv_state, a.ssm_state, static_cast<IO*>(a.y), cw,
                       a.S, a.d, a.N, p.Lc);
  }
  evs.mark(st);
  return hipGetLastError() == hipSuccess ? MM_OK : MM_ERR_HIP;
}

// ---------------------------------------------------------------- decode launch

template <typename IO, int NMAX>
int launch_decode(const void* x, const void* z, const void* dt, const void* B, const void* C, const float* A_log,
                  const float* D, const float* dt_bias, const float* conv_w, const float* conv_b,
                  float* conv_state, float* ssm_state, void* y, int Bs, int d, int N, hipStream_t st) {
  const size_t bca = 4 * sizeof(IO);  // B/C rows are read four elements at a time
  const bool vec = N == NMAX && aligned(ssm_state, 16) && aligned(A_log, 16) && aligned(conv_w, 16) &&
                   aligned(B, bca) && aligned(C, bca);
  if (vec) {
    constexpr int CPB = kBlock / (NMAX / 4);
    const dim3 grid(static_cast<unsigned>(cdiv(d, CPB) * cdiv(Bs, NMAX / 4)));
    hipLaunchKernelGGL((k_decode_vec<IO, NMAX>), grid, dim3(kBlock), 0, st, static_cast<const IO*>(x),
                       static_cast<const IO*>(z), static_cast<const IO*>(dt), static_cast<const IO*>(B),
                       static_cast<const IO*>(C), A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state,
                       static_cast<IO*>(y), Bs, d);
  } else {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>((d + kBlock - 1) / kBlock) * Bs));
    hipLaunchKernelGGL((k_decode<IO, NMAX>), grid, dim3(kBlock), 0, st, static_cast<const IO*>(x),
                       static_cast<const IO*>(z), static_cast<const IO*>(dt), static_cast<const IO*>(B),
                       static_cast<const IO*>(C), A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state,
                       static_cast<IO*>(y), d, N);
  }
  return hipGetLastError() == hipSuccess ? MM_OK : MM_ERR_HIP;
}

int check_common(int64_t rows, int32_t d, int32_t N, int32_t K, int32_t io) {
  if (rows < 0 || d < 0 || N < 0 || K < 0) return MM_ERR_DIM;
  // keeps every byte extent (rows x d x 16 x 4 at most) far inside 64 bits
  if (d > 0 && static_cast<uint64_t>(rows) > MM_MAX_ROWS_X_D / static_cast<uint64_t>(d)) return MM_ERR_DIM;
  if (K != kK || N < 1 || N > MM_MAX_N) return MM_ERR_UNSUPPORTED;
  if (io != MM_IO_F32 && io != MM_IO_BF16) return MM_ERR_UNSUPPORTED;
  return MM_OK;
}

// size checks shared by the plan queries and the prefill call
int check_prefill_sizes(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io) {
  const int rc = check_common(T, d, N, K, io);
  if (rc != MM_OK) return rc;
  if (S < 0 || T > INT32_MAX) return MM_ERR_DIM;
  if (S == 0 && T > 0) return MM_ERR_DIM;
  if (d > 0 && static_cast<uint64_t>(S) > MM_MAX_ROWS_X_D / static_cast<uint64_t>(d)) return MM_ERR_DIM;
  return MM_OK;
}

struct Span {
  const void* p;
  size_t n;
};

// Validation and launch shared by the replay entry points.  multi: z, C and y are rings
// [W][Bs][...] indexed by window step; otherwise they are this step's [Bs][...].  dual: the
// checkpoint's bf16 copy (conv_lo [Bs][d][4], ssm_lo [Bs][d][16]) is read by a call that
// commits nothing and rewritten by one that commits (bf16 io only).
int replay_launch(const void* x_ring, const void* dt_ring, const void* B_ring, const void* z, const void* C,
                  const float* A_log, const float* D, const float* dt_bias, const float* conv_w, const float* conv_b,
                  float* conv_state, float* ssm_state, void* y, int32_t Bs, int32_t d, int32_t N, int32_t K,
                  int32_t io_dtype, int32_t W, int32_t k0, int32_t k1, int32_t cstep, bool multi, void* stream,
                  bool dual = false, void* conv_lo = nullptr, void* ssm_lo = nullptr) {
  int rc = check_common(Bs, d, N, K, io_dtype);
  if (rc != MM_OK) return rc;
  if (N != kReplayN) return MM_ERR_UNSUPPORTED;
  if (dual && io_dtype != MM_IO_BF16) return MM_ERR_UNSUPPORTED;
  if (W < 1 || W > kReplayMaxW || k0 < 0 || k0 > k1 || k1 >= W || cstep < -1 || cstep > k1) return MM_ERR_DIM;
  if (Bs == 0 || d == 0) return MM_OK;
  const void* req[] = {x_ring, dt_ring, B_ring, z, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y};
  for (const void* p : req)
    if (p == nullptr) return MM_ERR_NULL;
  const size_t es = io_dtype == MM_IO_BF16 ? 2 : 4;
  const void* iop[] = {x_ring, dt_ring, z, y};
  for (const void* p : iop)
    if (!aligned(p, es)) return MM_ERR_ALIGN;
  const void* vec[] = {B_ring, C};  // rows are read four elements at a time
  for (const void* p : vec)
    if (!aligned(p, 4 * es)) return MM_ERR_ALIGN;
  const void* fp[] = {D, dt_bias, conv_b, conv_state};
  for (const void* p : fp)
    if (!aligned(p, 4)) return MM_ERR_ALIGN;
  const void* f16[] = {A_log, conv_w, ssm_state};
  for (const void* p : f16)
    if (!aligned(p, 16)) return MM_ERR_ALIGN;
  const size_t slot_d = static_cast<size_t>(Bs) * d * es, slot_n = static_cast<size_t>(Bs) * N * es;
  const size_t nring = static_cast<size_t>(W) * slot_d, nbr = static_cast<size_t>(W) * slot_n;
  const size_t ny = multi ? nring : slot_d, nz = multi ? nring : slot_d, nc = multi ? nbr : slot_n;
  if (overlap(y, ny, x_ring, nring) || overlap(y, ny, dt_ring, nring) || overlap(y, ny, B_ring, nbr) ||
      overlap(y, ny, z, nz) || overlap(y, ny, C, nc))
    return MM_ERR_ALIAS;
  if (overlap(conv_state, static_cast<size_t>(Bs) * d * kKS * 4, ssm_state, static_cast<size_t>(Bs) * d * N * 4))
    return MM_ERR_ALIAS;
  if (dual) {
    if (conv_lo == nullptr || ssm_lo == nullptr) return MM_ERR_NULL;
    if (!aligned(ssm_lo, 16) || !aligned(conv_lo, 8)) return MM_ERR_ALIGN;
    const size_t nsl = static_cast<size_t>(Bs) * d * N * 2, ncl = static_cast<size_t>(Bs) * d * 4 * 2;
    const Span other[] = {{x_ring, nring}, {dt_ring, nring}, {B_ring, nbr}, {z, nz}, {C, nc}, {y, ny},
                          {conv_state, static_cast<size_t>(Bs) * d * kKS * 4},
                          {ssm_state, static_cast<size_t>(Bs) * d * N * 4}, {conv_lo, ncl}};
    for (const Span& v : other)
      if (overlap(ssm_lo, nsl, v.p, v.n) || (v.p != conv_lo && overlap(conv_lo, ncl, v.p, v.n))) return MM_ERR_ALIAS;
  }
  // z/C/y of step t sit at slot t - k0 of the pointers passed to the kernel
  const int64_t zs = multi ? static_cast<int64_t>(Bs) * d : 0, cs = multi ? static_cast<int64_t>(Bs) * N : 0;
  const int64_t off_d = multi ? static_cast<int64_t>(k0) * Bs * d : 0;
  const int64_t off_n = multi ? static_cast<int64_t>(k0) * Bs * N : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(cdiv(d, kBlock) * Bs));
  uint16_t* slo = static_cast<uint16_t*>(ssm_lo);
  uint16_t* clo = static_cast<uint16_t*>(conv_lo);
  if (io_dtype == MM_IO_BF16) {
    using T = uint16_t;
    if (dual && cstep < 0)  // outputs from the bf16 copy, nothing committed
      hipLaunchKernelGGL((k_decode_replay<T, true>), grid, dim3(kBlock), 0, st, static_cast<const T*>(x_ring),
                         static_cast<const T*>(dt_ring), static_cast<const T*>(B_ring),
                         static_cast<const T*>(z) + off_d, static_cast<const T*>(C) + off_n, A_log, D, dt_bias,
                         conv_w, conv_b, conv_state, ssm_state, static_cast<T*>(y) + off_d, Bs, d, k0, k1, cstep,
                         zs, cs, zs, slo, clo, nullptr, nullptr);
    else  // from the fp32 checkpoint; a dual commit also rewrites the bf16 copy
      hipLaunchKernelGGL((k_decode_replay<T, false>), grid, dim3(kBlock), 0, st, static_cast<const T*>(x_ring),
                         static_cast<const T*>(dt_ring), static_cast<const T*>(B_ring),
                         static_cast<const T*>(z) + off_d, static_cast<const T*>(C) + off_n, A_log, D, dt_bias,
                         conv_w, conv_b, conv_state, ssm_state, static_cast<T*>(y) + off_d, Bs, d, k0, k1, cstep,
                         zs, cs, zs, nullptr, nullptr, dual ? slo : nullptr, dual ? clo : nullptr);
  } else {
    using T = float;
    hipLaunchKernelGGL((k_decode_replay<T, false>), grid, dim3(kBlock), 0, st, static_cast<const T*>(x_ring),
                       static_cast<const T*>(dt_ring), static_cast<const T*>(B_ring),
                       static_cast<const T*>(z) + off_d, static_cast<const T*>(C) + off_n, A_log, D, dt_bias,
                       conv_w, conv_b, conv_state, ssm_state, static_cast<T*>(y) + off_d, Bs, d, k0, k1, cstep, zs,
                       cs, zs, nullptr, nullptr, nullptr, nullptr);
  }
  return hipGetLastError() == hipSuccess ? MM_OK : MM_ERR_HIP;
}

// ---------------------------------------------------------------- prefill backward

// The reverse pass gives each workgroup row every G-th sequence; G is chosen for
// about this many workgroups (8 per CU).
constexpr int64_t kBwdWgs = 2048;

struct BwdPlan {
  int nchb;      // 16-channel blocks
  int G;         // workgroup rows of the reverse pass (0 when S == 0)
  int64_t rows;  // checkpoint rows: ceil(T / 16) + S
  size_t off_ckpt, off_pbc, off_prm, total;
  int kernels;
};

int make_bwd_plan(BwdPlan& p, int64_t S, int64_t T, int d, int N, bool has_ckpt) {
  p = BwdPlan{};
  if (d > kRowMaxD) return MM_ERR_UNSUPPORTED;
  p.nchb = static_cast<int>(cdiv(d, kRowChans));
  p.rows = cdiv(T, kRow) + S;
  int64_t g = cdiv(kBwdWgs, p.nchb > 0 ? p.nchb : 1);
  if (g > S) g = S;
  p.G = static_cast<int>(g);
  size_t off = 0;
  p.off_ckpt = off;
  if (!has_ckpt) off += align256(static_cast<size_t>(p.rows) * d * kRow * sizeof(float));
  p.off_pbc = off; off += align256(static_cast<size_t>(p.nchb) * 2 * T * N * sizeof(float));
  p.off_prm = off; off += align256(static_cast<size_t>(p.G) * kPrm * d * sizeof(float));
  p.total = off;
  p.kernels = S > 0 ? (has_ckpt ? 3 : 4) : 1;
  if (row_grid(S, d) > INT32_MAX || cdiv(2 * T * N, kBlock) > INT32_MAX) return MM_ERR_DIM;
  return MM_OK;
}

struct BwdArgs {
  const void *x, *z, *dt, *B, *C, *dy;
  const float *A_log, *D, *dt_bias, *conv_w, *conv_b;
  const int32_t* cu;
  const float *conv_state, *ssm_state, *ckpt;  // ckpt: NULL, or the training forward's checkpoints
  void *dx, *dz, *ddt, *dB, *dC;
  float *dA_log, *dD, *ddt_bias, *dconv_w, *dconv_b, *dconv_state, *dssm_state;
  int S;
  int64_t T;
  int d, N;
};

template <typename IO>
int launch_backward(const BwdPlan& p, const BwdArgs& a, char* ws, hipStream_t st, StageEvents evs) {
  float* ckpt = a.ckpt != nullptr ? const_cast<float*>(a.ckpt) : reinterpret_cast<float*>(ws + p.off_ckpt);
  float* pbc = reinterpret_cast<float*>(ws + p.off_pbc);
  float* pprm = reinterpret_cast<float*>(ws + p.off_prm);
  const IO* xi = static_cast<const IO*>(a.x);
  const IO* zi = static_cast<const IO*>(a.z);
  const IO* di = static_cast<const IO*>(a.dt);
  const IO* Bi = static_cast<const IO*>(a.B);
  const IO* Ci = static_cast<const IO*>(a.C);
  const dim3 block(kRowThreads);
  if (a.S > 0) {
    // 1. checkpoints: the forward's states before every 16-token block (unless given)
    if (a.ckpt == nullptr) {
      evs.mark(st);
      const PrefillArgs fa{a.x, a.z, a.dt, a.B, a.C, a.A_log, a.D, a.dt_bias, a.conv_w, a.conv_b, a.cu,
                           nullptr, nullptr, nullptr, a.S, a.T, a.d, a.N};
      launch_k_row<IO, false, true>(row_vec<IO>(a.d, a.N, {a.x, a.dt, a.B}), dim3(static_cast<unsigned>(row_grid(a.S, a.d))),
                                    st, fa, xi, zi, di, Bi, Ci, const_cast<float*>(a.conv_state),
                                    const_cast<float*>(a.ssm_state), static_cast<IO*>(nullptr), CarryWs{}, a.T + 1, 1,
                                    ckpt);
    }
    // 2. the reverse pass
    evs.mark(st);
    hipLaunchKernelGGL((k_row_bwd<IO>), dim3(static_cast<unsigned>(row_grid(p.G, a.d))), block, 0, st, xi, zi, di, Bi,
                       Ci, static_cast<const IO*>(a.dy), a.A_log, a.D, a.dt_bias, a.conv_w, a.conv_b, a.cu,
                       a.conv_state, ckpt, static_cast<IO*>(a.dx), static_cast<IO*>(a.dz), static_cast<IO*>(a.ddt),
                       a.dconv_state, a.dssm_state, pbc, pprm, a.S, a.T, a.d, a.N, p.G);
    // 3. dB, dC
    evs.mark(st);
    const int64_t TN = a.T * a.N;
    const int64_t nbc = cdiv(2 * TN, kBlock);
    hipLaunchKernelGGL((k_bwd_sum_bc<IO>), dim3(static_cast<unsigned>(nbc > 0 ? nbc : 1)), dim3(kBlock), 0, st, pbc,
                       static_cast<IO*>(a.dB), static_cast<IO*>(a.dC), TN, p.nchb);
  }
  // 4. parameter gradients (zeros when there is no sequence)
  evs.mark(st);
  hipLaunchKernelGGL(k_bwd_sum_params, dim3(static_cast<unsigned>(cdiv(static_cast<int64_t>(kPrm) * a.d, kBlock))),
                     dim3(kBlock), 0, st, pprm, a.dA_log, a.dD, a.ddt_bias, a.dconv_b, a.dconv_w, a.d, a.N, p.G);
  evs.mark(st);
  return hipGetLastError() == hipSuccess ? MM_OK : MM_ERR_HIP;
}

// ---------------------------------------------------------------- projections

// the projection kernels for NT output column tiles (1 .. 18) and KR K steps of dt_in (1 .. 8)
using KernIn = void (*)(const uint16_t*, const float*, const float*, const int32_t*, const float*, const uint16_t*,
                        uint16_t*, uint16_t*, uint16_t*, uint16_t*, int, int64_t, int, int, int, int, int, const float*,
                       int);
using KernDt = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int64_t, int, int, int);
template <int... I>
KernIn proj_in_table(int nt, std::integer_sequence<int, I...>) {
  static const KernIn t[] = {k_proj_in<I + 1>...};
  return t[nt - 1];
}
template <int... I>
KernDt proj_dt_table(int kr, std::integer_sequence<int, I...>) {
  static const KernDt t[] = {k_proj_dt<I + 1>...};
  return t[kr - 1];
}
KernIn proj_in_kernel(int nt) { return proj_in_table(nt, std::make_integer_sequence<int, kProjMaxP / 16>{}); }
template <int... I>
size_t proj_in_lds_table(int nt, std::integer_sequence<int, I...>) {
  static const size_t t[] = {pin_lds_bytes_t<I + 1>()...};
  return t[nt - 1];
}
size_t proj_in_lds(int nt) { return proj_in_lds_table(nt, std::make_integer_sequence<int, kProjMaxP / 16>{}); }
template <int... I>
int proj_in_threads_table(int nt, std::integer_sequence<int, I...>) {
  static const int t[] = {PinGeo<I + 1>::THREADS...};
  return t[nt - 1];
}
int proj_in_threads(int nt) { return proj_in_threads_table(nt, std::make_integer_sequence<int, kProjMaxP / 16>{}); }
KernDt proj_dt_kernel(int kr) { return proj_dt_table(kr, std::make_integer_sequence<int, kProjMaxR / kProjK>{}); }

struct ProjPlan {
  int P, Pp, dk, Rp;
  size_t off_wx, off_wdt, off_dth, off_dtl, total;
};

// workspace: the re-laid w_x and w_dt, then dt_in's bf16 high and low parts [T][Rp]
void make_proj_plan(ProjPlan& p, int64_t T, int d, int N, int R) {
  p.P = R + 2 * N;
  p.Pp = static_cast<int>(cdiv(p.P, 16) * 16);
  p.dk = static_cast<int>(cdiv(d, kProjK) * kProjK);
  p.Rp = static_cast<int>(cdiv(R, kProjK) * kProjK);
  size_t off = 0;
  p.off_wx = off; off += align256(static_cast<size_t>(p.Pp) * p.dk * 2);
  p.off_wdt = off; off += align256(static_cast<size_t>(d) * p.Rp * 2);
  p.off_dth = off; off += align256(static_cast<size_t>(T) * p.Rp * 2);
  p.off_dtl = off; off += align256(static_cast<size_t>(T) * p.Rp * 2);
  p.total = off;
}

int check_proj_sizes(int32_t S, int64_t T, int32_t d, int32_t N, int32_t R, int32_t K, int32_t io) {
  const int rc = check_prefill_sizes(S, T, d, N, K, io);
  if (rc != MM_OK) return rc;
  if (R < 0) return MM_ERR_DIM;
  if (io != MM_IO_BF16 || R < 1 || R > kProjMaxR || d % 16 != 0 || d > MM_PROJECT_MAX_D) return MM_ERR_UNSUPPORTED;
  return MM_OK;
}

// ---------------------------------------------------------------- fixed scratch

// The workspace of mamba_mixer_prefill_noalloc: a file-scope device array that every GPU the
// library runs on holds from the loading of the library's code until the process ends.  Host
// code never passes the array's name to a kernel or a copy (on the host it names a stand-in,
// not device memory): it passes the device address hipGetSymbolAddress returns, looked up once
// per device with that device current and kept per device.
static __device__ __align__(256) unsigned char scratch[MM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (MM_OK), or MM_ERR_HIP when the device or the
// symbol cannot be resolved.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MM_OK;
}

}  // namespace
}  // namespace mm

using namespace mm;

extern "C" {

const char* mamba_mixer_status_string(int status) {
  switch (status) {
    case MM_OK: return "ok";
    case MM_ERR_NULL: return "a required pointer is NULL";
    case MM_ERR_DIM: return "invalid size (negative, T > INT32_MAX, S == 0 with T > 0, or too few events)";
    case MM_ERR_UNSUPPORTED: return "unsupported K, N, io dtype or engine (K must be 4, N in 1..16, io F32 or BF16)";
    case MM_ERR_ALIGN: return "pointer not aligned to its element size";
    case MM_ERR_WORKSPACE: return "workspace too small or NULL";
    case MM_ERR_ALIAS: return "output overlaps an input, or conv_state overlaps ssm_state";
    case MM_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

const char* mamba_mixer_version(void) { return "libmambamix 0.4 gfx950"; }

int mamba_mixer_check_cu_seqlens(const int32_t* cu_seqlens_host, int32_t S, int64_t T) {
  if (S < 0 || T < 0) return MM_ERR_DIM;
  if (cu_seqlens_host == nullptr) return MM_ERR_NULL;
  if (cu_seqlens_host[0] != 0 || cu_seqlens_host[S] != T) return MM_ERR_DIM;
  for (int32_t s = 0; s < S; ++s)
    if (cu_seqlens_host[s + 1] < cu_seqlens_host[s]) return MM_ERR_DIM;
  return MM_OK;
}

int mamba_mixer_prefill_plan(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int64_t chunk_len,
                             int32_t engine, int64_t* chunk_len_out, int32_t* engine_out, size_t* workspace_out,
                             int32_t* kernels_out) {
  int rc = check_prefill_sizes(S, T, d, N, K, MM_IO_F32);
  if (rc != MM_OK) return rc;
  Plan p{};
  if (T > 0 && d > 0 && S > 0) {
    rc = make_plan(p, S, T, d, N, chunk_len, engine);
    if (rc != MM_OK) return rc;
  }
  if (chunk_len_out) *chunk_len_out = p.Lc;
  if (engine_out) *engine_out = p.engine;
  if (workspace_out) *workspace_out = p.total;
  if (kernels_out) *kernels_out = p.kernels;
  return MM_OK;
}

const char* mamba_mixer_prefill_kernel_name(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int64_t chunk_len,
                                            int32_t engine, int32_t i) {
  if (check_prefill_sizes(S, T, d, N, K, MM_IO_F32) != MM_OK || T == 0 || d == 0 || S == 0) return "";
  Plan p{};
  if (make_plan(p, S, T, d, N, chunk_len, engine) != MM_OK || i < 0 || i >= p.kernels) return "";
  return kernel_name(p, i);
}

size_t mamba_mixer_prefill_workspace_bytes_chunked(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K,
                                                   int64_t chunk_len) {
  size_t w = 0;
  if (mamba_mixer_prefill_plan(S, T, d, N, K, chunk_len, MM_ENGINE_AUTO, nullptr, nullptr, &w, nullptr) != MM_OK)
    return 0;
  return w;
}

size_t mamba_mixer_prefill_workspace_bytes(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K) {
  return mamba_mixer_prefill_workspace_bytes_chunked(S, T, d, N, K, 0);
}

// The prefill call; with ckpt != NULL (row engine only) the final pass also stores the
// state before every 16-token block.
// use_scratch: the workspace is the library's fixed device scratch (mamba_mixer_prefill_noalloc);
// a plan that needs more than it holds is MM_ERR_WORKSPACE, found before anything is enqueued.
static int prefill_call(const void* x, const void* z, const void* dt, const void* B, const void* C,
                        const float* A_log, const float* D, const float* dt_bias, const float* conv_w,
                        const float* conv_b, const int32_t* cu_seqlens, float* conv_state, float* ssm_state,
                        void* y, float* ckpt, int32_t S, int64_t T, int32_t d, int32_t N, int32_t K,
                        int32_t io_dtype, int64_t chunk_len, int32_t engine, void* workspace,
                        size_t workspace_bytes, void* stream, void* const* events, int32_t n_events,
                        bool use_scratch = false) {
  int rc = check_prefill_sizes(S, T, d, N, K, io_dtype);
  if (rc != MM_OK) return rc;
  if (T == 0 || d == 0 || S == 0) return MM_OK;
  const void* req[] = {x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state, y};
  for (const void* p : req)
    if (p == nullptr) return MM_ERR_NULL;
  const size_t es = io_dtype == MM_IO_BF16 ? 2 : 4;
  const void* iop[] = {x, z, dt, B, C, y};
  for (const void* p : iop)
    if (!aligned(p, es)) return MM_ERR_ALIGN;
  const void* fp[] = {A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state};
  for (const void* p : fp)
    if (!aligned(p, 4)) return MM_ERR_ALIGN;
  const size_t ny = static_cast<size_t>(T) * d * es, nbc = static_cast<size_t>(T) * N * es;
  if (overlap(y, ny, x, ny) || overlap(y, ny, z, ny) || overlap(y, ny, dt, ny) || overlap(y, ny, B, nbc) ||
      overlap(y, ny, C, nbc))
    return MM_ERR_ALIAS;
  if (overlap(conv_state, static_cast<size_t>(S) * d * kKS * 4, ssm_state, static_cast<size_t>(S) * d * N * 4))
    return MM_ERR_ALIAS;
  if (ckpt != nullptr) {
    const size_t nck = static_cast<size_t>(cdiv(T, kRow) + S) * d * kRow * 4;
    const Span other[] = {{x, ny}, {z, ny}, {dt, ny}, {B, nbc}, {C, nbc}, {y, ny},
                          {conv_state, static_cast<size_t>(S) * d * kKS * 4},
                          {ssm_state, static_cast<size_t>(S) * d * N * 4}};
    for (const Span& v : other)
      if (overlap(ckpt, nck, v.p, v.n)) return MM_ERR_ALIAS;
    if (!aligned(ckpt, 4)) return MM_ERR_ALIGN;
  }
  Plan p{};
  rc = make_plan(p, S, T, d, N, chunk_len, engine);
  if (rc != MM_OK) return rc;
  if (use_scratch) {
    if (p.total > MM_NOALLOC_SCRATCH_BYTES) return MM_ERR_WORKSPACE;
    workspace = nullptr;
    workspace_bytes = 0;
    if (p.total > 0) {
      rc = scratch_address(&workspace);
      if (rc != MM_OK) return rc;
      workspace_bytes = MM_NOALLOC_SCRATCH_BYTES;
    }
  }
  if (p.total > 0 && (workspace == nullptr || workspace_bytes < p.total)) return MM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MM_ERR_ALIGN;
  if (events != nullptr && n_events < p.kernels + 1) return MM_ERR_DIM;
  const PrefillArgs a{x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state, y,
                      S, T, d, N};
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const StageEvents evs{events, n_events, 0};
  if (ckpt != nullptr) {
    if (p.engine != MM_ENGINE_ROW) return MM_ERR_UNSUPPORTED;
    if (io_dtype == MM_IO_BF16) return launch_prefill<uint16_t, 16>(p, a, ws, st, evs, ckpt);
    return launch_prefill<float, 16>(p, a, ws, st, evs, ckpt);
  }
  if (io_dtype == MM_IO_BF16) {
    if (p.nmax == 4) return launch_prefill<uint16_t, 4>(p, a, ws, st, evs);
    if (p.nmax == 8) return launch_prefill<uint16_t, 8>(p, a, ws, st, evs);
    return launch_prefill<uint16_t, 16>(p, a, ws, st, evs);
  }
  if (p.nmax == 4) return launch_prefill<float, 4>(p, a, ws, st, evs);
  if (p.nmax == 8) return launch_prefill<float, 8>(p, a, ws, st, evs);
  return launch_prefill<float, 16>(p, a, ws, st, evs);
}

int mamba_mixer_prefill_ex(const void* x, const void* z, const void* dt, const void* B, const void* C,
                           const float* A_log, const float* D, const float* dt_bias,
                           const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                           float* conv_state, float* ssm_state, void* y,
                           int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                           int64_t chunk_len, int32_t engine, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* events, int32_t n_events) {
  return prefill_call(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state, y,
                      nullptr, S, T, d, N, K, io_dtype, chunk_len, engine, workspace, workspace_bytes, stream,
                      events, n_events);
}

size_t mamba_mixer_checkpoint_bytes(int32_t S, int64_t T, int32_t d) {
  if (S < 0 || T < 0 || d < 0 || T > INT32_MAX) return 0;
  const uint64_t rows = static_cast<uint64_t>(cdiv(T, kRow) + S);
  if (d > 0 && rows > MM_MAX_ROWS_X_D / static_cast<uint64_t>(d)) return 0;
  return static_cast<size_t>(rows) * d * kRow * sizeof(float);
}

int mamba_mixer_prefill_train(const void* x, const void* z, const void* dt, const void* B, const void* C,
                              const float* A_log, const float* D, const float* dt_bias, const float* conv_w,
                              const float* conv_b, const int32_t* cu_seqlens, float* conv_state, float* ssm_state,
                              void* y, float* ckpt, int32_t S, int64_t T, int32_t d, int32_t N, int32_t K,
                              int32_t io_dtype, int64_t chunk_len, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* events, int32_t n_events) {
  if (ckpt == nullptr && T > 0 && d > 0 && S > 0) return MM_ERR_NULL;
  return prefill_call(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state, y,
                      ckpt, S, T, d, N, K, io_dtype, chunk_len, MM_ENGINE_ROW, workspace, workspace_bytes, stream,
                      events, n_events);
}

int mamba_mixer_prefill_chunked(const void* x, const void* z, const void* dt, const void* B, const void* C,
                                const float* A_log, const float* D, const float* dt_bias,
                                const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                                float* conv_state, float* ssm_state, void* y,
                                int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                                int64_t chunk_len, void* workspace, size_t workspace_bytes, void* stream) {
  return mamba_mixer_prefill_ex(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state,
                                ssm_state, y, S, T, d, N, K, io_dtype, chunk_len, MM_ENGINE_AUTO, workspace,
                                workspace_bytes, stream, nullptr, 0);
}

int mamba_mixer_prefill(const void* x, const void* z, const void* dt, const void* B, const void* C,
                        const float* A_log, const float* D, const float* dt_bias,
                        const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                        float* conv_state, float* ssm_state, void* y,
                        int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return mamba_mixer_prefill_chunked(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state,
                                     ssm_state, y, S, T, d, N, K, io_dtype, 0, workspace, workspace_bytes, stream);
}

int mamba_mixer_prefill_noalloc(const void* x, const void* z, const void* dt, const void* B, const void* C,
                                const float* A_log, const float* D, const float* dt_bias,
                                const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                                float* conv_state, float* ssm_state, void* y,
                                int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                                void* stream) {
  return prefill_call(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state, y,
                      nullptr, S, T, d, N, K, io_dtype, 0, MM_ENGINE_AUTO, nullptr, 0, stream, nullptr, 0, true);
}

int mamba_mixer_decode(const void* x, const void* z, const void* dt, const void* B, const void* C,
                       const float* A_log, const float* D, const float* dt_bias,
                       const float* conv_w, const float* conv_b,
                       float* conv_state, float* ssm_state, void* y,
                       int32_t Bs, int32_t d, int32_t N, int32_t K, int32_t io_dtype, void* stream) {
  int rc = check_common(Bs, d, N, K, io_dtype);
  if (rc != MM_OK) return rc;
  if (Bs == 0 || d == 0) return MM_OK;
  const void* req[] = {x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y};
  for (const void* p : req)
    if (p == nullptr) return MM_ERR_NULL;
  const size_t es = io_dtype == MM_IO_BF16 ? 2 : 4;
  const void* iop[] = {x, z, dt, B, C, y};
  for (const void* p : iop)
    if (!aligned(p, es)) return MM_ERR_ALIGN;
  const void* fp[] = {A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state};
  for (const void* p : fp)
    if (!aligned(p, 4)) return MM_ERR_ALIGN;
  const size_t ny = static_cast<size_t>(Bs) * d * es, nbc = static_cast<size_t>(Bs) * N * es;
  if (overlap(y, ny, x, ny) || overlap(y, ny, z, ny) || overlap(y, ny, dt, ny) || overlap(y, ny, B, nbc) ||
      overlap(y, ny, C, nbc))
    return MM_ERR_ALIAS;
  if (overlap(conv_state, static_cast<size_t>(Bs) * d * kKS * 4, ssm_state, static_cast<size_t>(Bs) * d * N * 4))
    return MM_ERR_ALIAS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int nm = nmax_for(N);
#define MM_DECODE(IO, NM)                                                                                       \
  launch_decode<IO, NM>(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y, Bs, d, N, st)
  if (io_dtype == MM_IO_BF16) {
    if (nm == 4) return MM_DECODE(uint16_t, 4);
    if (nm == 8) return MM_DECODE(uint16_t, 8);
    return MM_DECODE(uint16_t, 16);
  }
  if (nm == 4) return MM_DECODE(float, 4);
  if (nm == 8) return MM_DECODE(float, 8);
  return MM_DECODE(float, 16);
#undef MM_DECODE
}

int mamba_mixer_decode_replay(const void* x_ring, const void* dt_ring, const void* B_ring, const void* z,
                              const void* C, const float* A_log, const float* D, const float* dt_bias,
                              const float* conv_w, const float* conv_b, float* conv_state, float* ssm_state,
                              void* y, int32_t Bs, int32_t d, int32_t N, int32_t K, int32_t io_dtype, int32_t W,
                              int32_t k, int32_t commit, void* stream) {
  const int cstep = (commit != 0 || k == W - 1) ? k : -1;
  return replay_launch(x_ring, dt_ring, B_ring, z, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y,
                       Bs, d, N, K, io_dtype, W, k, k, cstep, false, stream);
}

int mamba_mixer_decode_replay_dual(const void* x_ring, const void* dt_ring, const void* B_ring, const void* z,
                                   const void* C, const float* A_log, const float* D, const float* dt_bias,
                                   const float* conv_w, const float* conv_b, float* conv_state, float* ssm_state,
                                   void* conv_lo, void* ssm_lo, void* y, int32_t Bs, int32_t d, int32_t N, int32_t K,
                                   int32_t io_dtype, int32_t W, int32_t k, int32_t commit, void* stream) {
  const int cstep = (commit != 0 || k == W - 1) ? k : -1;
  return replay_launch(x_ring, dt_ring, B_ring, z, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y,
                       Bs, d, N, K, io_dtype, W, k, k, cstep, false, stream, true, conv_lo, ssm_lo);
}

int mamba_mixer_replay_checkpoint_lo(const float* conv_state, const float* ssm_state, void* conv_lo, void* ssm_lo,
                                     int32_t Bs, int32_t d, int32_t N, int32_t K, void* stream) {
  int rc = check_common(Bs, d, N, K, MM_IO_BF16);
  if (rc != MM_OK) return rc;
  if (N != kReplayN) return MM_ERR_UNSUPPORTED;
  if (Bs == 0 || d == 0) return MM_OK;
  if (conv_state == nullptr || ssm_state == nullptr || conv_lo == nullptr || ssm_lo == nullptr) return MM_ERR_NULL;
  if (!aligned(conv_state, 4) || !aligned(ssm_state, 16) || !aligned(ssm_lo, 16) || !aligned(conv_lo, 8))
    return MM_ERR_ALIGN;
  const size_t n = static_cast<size_t>(Bs) * d;
  const Span all[] = {{conv_state, n * kKS * 4}, {ssm_state, n * N * 4}, {conv_lo, n * 4 * 2}, {ssm_lo, n * N * 2}};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(all[i].p, all[i].n, all[j].p, all[j].n)) return MM_ERR_ALIAS;
  hipLaunchKernelGGL(k_checkpoint_lo, dim3(static_cast<unsigned>(cdiv(static_cast<int64_t>(n), kBlock))), dim3(kBlock),
                     0, static_cast<hipStream_t>(stream), conv_state, ssm_state, static_cast<uint16_t*>(conv_lo),
                     static_cast<uint16_t*>(ssm_lo), static_cast<int64_t>(n));
  return hipGetLastError() == hipSuccess ? MM_OK : MM_ERR_HIP;
}

int mamba_mixer_decode_replay_multi(const void* x_ring, const void* dt_ring, const void* B_ring, const void* z_ring,
                                    const void* C_ring, const float* A_log, const float* D, const float* dt_bias,
                                    const float* conv_w, const float* conv_b, float* conv_state, float* ssm_state,
                                    void* y_ring, int32_t Bs, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                                    int32_t W, int32_t k0, int32_t k1, int32_t commit_step, void* stream) {
  return replay_launch(x_ring, dt_ring, B_ring, z_ring, C_ring, A_log, D, dt_bias, conv_w, conv_b, conv_state,
                       ssm_state, y_ring, Bs, d, N, K, io_dtype, W, k0, k1, commit_step, true, stream);
}

int mamba_mixer_prefill_backward_plan(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t has_ckpt,
                                      size_t* workspace_out, int32_t* kernels_out) {
  int rc = check_prefill_sizes(S, T, d, N, K, MM_IO_F32);
  if (rc != MM_OK) return rc;
  BwdPlan p{};
  if (d > 0) {
    rc = make_bwd_plan(p, S, T, d, N, has_ckpt != 0);
    if (rc != MM_OK) return rc;
  }
  if (workspace_out) *workspace_out = p.total;
  if (kernels_out) *kernels_out = p.kernels;
  return MM_OK;
}

size_t mamba_mixer_prefill_backward_workspace_bytes(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K,
                                                    int32_t has_ckpt) {
  size_t w = 0;
  if (mamba_mixer_prefill_backward_plan(S, T, d, N, K, has_ckpt, &w, nullptr) != MM_OK) return 0;
  return w;
}

int mamba_mixer_prefill_backward(const void* x, const void* z, const void* dt, const void* B, const void* C,
                                 const float* A_log, const float* D, const float* dt_bias, const float* conv_w,
                                 const float* conv_b, const int32_t* cu_seqlens, const float* conv_state,
                                 const float* ssm_state, const void* dy, const float* ckpt, void* dx, void* dz,
                                 void* ddt, void* dB,
                                 void* dC, float* dA_log, float* dD, float* ddt_bias, float* dconv_w, float* dconv_b,
                                 float* dconv_state, float* dssm_state, int32_t S, int64_t T, int32_t d, int32_t N,
                                 int32_t K, int32_t io_dtype, void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events, int32_t n_events) {
  int rc = check_prefill_sizes(S, T, d, N, K, io_dtype);
  if (rc != MM_OK) return rc;
  if (d == 0) return MM_OK;
  const size_t es = io_dtype == MM_IO_BF16 ? 2 : 4;
  const size_t ntd = static_cast<size_t>(T) * d * es, ntn = static_cast<size_t>(T) * N * es;
  const size_t nsk = static_cast<size_t>(S) * d * kKS * 4, nsn = static_cast<size_t>(S) * d * N * 4;
  const size_t nd = static_cast<size_t>(d) * 4;
  // inputs and outputs; an array of zero bytes may be NULL
  // with checkpoints given, the initial SSM state is not read (their first rows hold it)
  const size_t nck = ckpt != nullptr ? mamba_mixer_checkpoint_bytes(S, T, d) : 0;
  const Span in[] = {{x, ntd}, {z, ntd}, {dt, ntd}, {B, ntn}, {C, ntn}, {dy, ntd},
                     {A_log, nd * N}, {D, nd}, {dt_bias, nd}, {conv_w, nd * K}, {conv_b, nd},
                     {cu_seqlens, (static_cast<size_t>(S) + 1) * 4}, {conv_state, nsk},
                     {ssm_state, ckpt != nullptr ? 0 : nsn}, {ckpt, nck}};
  const Span out[] = {{dx, ntd}, {dz, ntd}, {ddt, ntd}, {dB, ntn}, {dC, ntn},
                      {dA_log, nd * N}, {dD, nd}, {ddt_bias, nd}, {dconv_w, nd * K}, {dconv_b, nd},
                      {dconv_state, nsk}, {dssm_state, nsn}};
  for (const Span& v : in)
    if (v.n > 0 && v.p == nullptr) return MM_ERR_NULL;
  for (const Span& v : out)
    if (v.n > 0 && v.p == nullptr) return MM_ERR_NULL;
  for (int i = 0; i < 6; ++i)
    if (!aligned(in[i].p, es)) return MM_ERR_ALIGN;
  for (int i = 0; i < 5; ++i)
    if (!aligned(out[i].p, es)) return MM_ERR_ALIGN;
  for (size_t i = 6; i < sizeof(in) / sizeof(in[0]); ++i)
    if (!aligned(in[i].p, 4)) return MM_ERR_ALIGN;
  for (size_t i = 5; i < sizeof(out) / sizeof(out[0]); ++i)
    if (!aligned(out[i].p, 4)) return MM_ERR_ALIGN;
  for (size_t i = 0; i < sizeof(out) / sizeof(out[0]); ++i) {
    for (const Span& v : in)
      if (overlap(out[i].p, out[i].n, v.p, v.n)) return MM_ERR_ALIAS;
    for (size_t k = i + 1; k < sizeof(out) / sizeof(out[0]); ++k)
      if (overlap(out[i].p, out[i].n, out[k].p, out[k].n)) return MM_ERR_ALIAS;
  }
  BwdPlan p{};
  rc = make_bwd_plan(p, S, T, d, N, ckpt != nullptr);
  if (rc != MM_OK) return rc;
  if (p.total > 0 && (workspace == nullptr || workspace_bytes < p.total)) return MM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MM_ERR_ALIGN;
  if (events != nullptr && n_events < p.kernels + 1) return MM_ERR_DIM;
  const BwdArgs a{x, z, dt, B, C, dy, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state, ckpt,
                  dx, dz, ddt, dB, dC, dA_log, dD, ddt_bias, dconv_w, dconv_b, dconv_state, dssm_state,
                  S, T, d, N};
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const StageEvents evs{events, n_events, 0};
  if (io_dtype == MM_IO_BF16) return launch_backward<uint16_t>(p, a, ws, st, evs);
  return launch_backward<float>(p, a, ws, st, evs);
}

size_t mamba_mixer_project_workspace_bytes(int64_t T, int32_t d, int32_t N, int32_t R) {
  if (T < 0 || T > INT32_MAX || d < 0 || N < 1 || N > MM_MAX_N || R < 1 || R > kProjMaxR) return 0;
  if (d > 0 && static_cast<uint64_t>(T) > MM_MAX_ROWS_X_D / static_cast<uint64_t>(d)) return 0;
  ProjPlan p{};
  make_proj_plan(p, T, d, N, R);
  return p.total;
}

int mamba_mixer_project(const void* x, const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                        const float* conv_state, const void* w_x, const void* w_dt, void* dt, void* B, void* C,
                        int32_t S, int64_t T, int32_t d, int32_t N, int32_t R, int32_t K, int32_t io_dtype,
                        void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                        int32_t n_events) {
  int rc = check_proj_sizes(S, T, d, N, R, K, io_dtype);
  if (rc != MM_OK) return rc;
  if (T == 0 || d == 0) return MM_OK;
  const size_t P = static_cast<size_t>(R) + 2 * N;
  const size_t ntd = static_cast<size_t>(T) * d * 2, ntn = static_cast<size_t>(T) * N * 2;
  const Span in[] = {{x, ntd}, {conv_w, static_cast<size_t>(d) * kK * 4}, {conv_b, static_cast<size_t>(d) * 4},
                     {cu_seqlens, (static_cast<size_t>(S) + 1) * 4}, {conv_state, static_cast<size_t>(S) * d * kKS * 4},
                     {w_x, static_cast<size_t>(d) * P * 2}, {w_dt, static_cast<size_t>(R) * d * 2}};
  const Span out[] = {{dt, ntd}, {B, ntn}, {C, ntn}};
  for (const Span& v : in)
    if (v.p == nullptr) return MM_ERR_NULL;
  for (const Span& v : out)
    if (v.p == nullptr) return MM_ERR_NULL;
  // x, conv_w and conv_b are read, and dt written, in 16-byte pieces
  if (!aligned(x, 16) || !aligned(conv_w, 16) || !aligned(conv_b, 16) || !aligned(dt, 16)) return MM_ERR_ALIGN;
  if (!aligned(cu_seqlens, 4) || !aligned(conv_state, 4)) return MM_ERR_ALIGN;
  const void* two[] = {w_x, w_dt, B, C};
  for (const void* q : two)
    if (!aligned(q, 2)) return MM_ERR_ALIGN;
  for (size_t i = 0; i < 3; ++i) {
    for (const Span& v : in)
      if (overlap(out[i].p, out[i].n, v.p, v.n)) return MM_ERR_ALIAS;
    for (size_t k = i + 1; k < 3; ++k)
      if (overlap(out[i].p, out[i].n, out[k].p, out[k].n)) return MM_ERR_ALIAS;
  }
  ProjPlan p{};
  make_proj_plan(p, T, d, N, R);
  if (workspace == nullptr || workspace_bytes < p.total) return MM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MM_ERR_ALIGN;
  const int ncb = static_cast<int>(cdiv(d, kPdtCh));
  if (cdiv(T, kPinTok) > INT32_MAX) return MM_ERR_DIM;
  if (events != nullptr && n_events < 4) return MM_ERR_DIM;
  StageEvents evs{events, n_events, 0};
  char* ws = static_cast<char*>(workspace);
  uint16_t* wxP = reinterpret_cast<uint16_t*>(ws + p.off_wx);
  uint16_t* wdtP = reinterpret_cast<uint16_t*>(ws + p.off_wdt);
  uint16_t* dth = reinterpret_cast<uint16_t*>(ws + p.off_dth);
  uint16_t* dtl = reinterpret_cast<uint16_t*>(ws + p.off_dtl);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t npack = static_cast<int64_t>(p.dk / 8) * p.Pp + static_cast<int64_t>(p.Rp / 8) * d;
  evs.mark(st);
  hipLaunchKernelGGL(k_proj_pack, dim3(static_cast<unsigned>(cdiv(npack, kBlock))), dim3(kBlock), 0, st,
                     static_cast<const uint16_t*>(w_x), static_cast<const uint16_t*>(w_dt), wxP, wdtP, d,
                     static_cast<int>(P), p.Pp, p.dk, R, p.Rp);
  const int nt = p.Pp / 16;
  const int nkr = p.Rp / kProjK;
  const KernIn kin = proj_in_kernel(nt);
  const size_t lds = std::max(proj_in_lds(nt), pin_out_bytes(p.Pp, p.Rp));
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(kin), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) != hipSuccess)
    return MM_ERR_HIP;
  evs.mark(st);
  hipLaunchKernelGGL(kin, dim3(static_cast<unsigned>(cdiv(T, kPinTok))), dim3(proj_in_threads(nt)), lds, st,
                     static_cast<const uint16_t*>(x), conv_w, conv_b, cu_seqlens, conv_state, wxP, dth, dtl,
                     static_cast<uint16_t*>(B), static_cast<uint16_t*>(C), S, T, d, N, R, p.Rp, p.dk / kProjK,
                     reinterpret_cast<const float*>(reinterpret_cast<uintptr_t>(conv_state) & ~static_cast<uintptr_t>(15)),
                     aligned(conv_state, 16) ? 1 : 0);
  // dt: about kPdtWGs workgroups, each a 128-channel block and a run of 16-token tiles
  const int64_t ntt = cdiv(T, 16);
  const int64_t G = std::max<int64_t>(1, std::min<int64_t>(cdiv(kPdtWGs, ncb), cdiv(ntt, kPdtWaves)));
  const int64_t per = cdiv(cdiv(ntt, G), kPdtWaves) * kPdtWaves;
  const int64_t groups = cdiv(ntt, per);
  const KernDt kdt = proj_dt_kernel(nkr);
  const size_t ldt = pdt_lds_bytes(nkr);
  if (ldt > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(kdt), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(ldt)) != hipSuccess)
    return MM_ERR_HIP;
  evs.mark(st);
  hipLaunchKernelGGL(kdt, dim3(static_cast<unsigned>(groups * ncb)), dim3(kPdtThreads), ldt, st, dth, dtl, wdtP,
                     static_cast<uint16_t*>(dt), T, d, ncb, static_cast<int>(per));
  evs.mark(st);
  return hipGetLastError() == hipSuccess ? MM_OK : MM_ERR_HIP;
}

}  // extern "C"
