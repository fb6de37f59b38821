// libmambamix -- HIP kernels for gfx950 (MI355X) and the C ABI declared in include/mambamix.h.
//
// The mixer step (TensorRT Mamba tensor-parallel builder, _add_mamba_tp_layer):
//   u = SiLU(conv_b + sum_k conv_w[k] * window[k]),  delta = softplus(dt + dt_bias),
//   h = exp(delta * A) * h + delta * B * u,  y = (C . h + D * u) * SiLU(z),
// run token after token over packed sequences (PackMamba: no state crosses a
// cu_seqlens boundary), with the final conv/SSM state left in the caller's slots
// (the state cache carried from prefill into decode on the tensor-parallel SSM page).
//
// Design (gfx950, wave64):
//  * One lane owns one channel and keeps all N state values of that channel in
//    registers; a wave covers 64 consecutive channels of one token, so every lane
//    of a wave reads the same B_t / C_t row: those come through the scalar unit
//    (SMEM loads of a float32 copy of B/C packed per token), not through VGPR loads.
//  * Per token and channel the work is 22 transcendental ops (16 exp for the
//    decays, exp+log for softplus, exp+rcp for each SiLU) and ~80 plain VALU ops;
//    reading x/z/dt and writing y is 8 bytes in bf16.  Prefill is therefore bound by
//    VALU issue, not by HBM; decode streams the fp32 state once in and once out and
//    is bound by HBM.
//  * Time parallelism: the packed token stream is cut into chunks of Lc tokens.
//    Chunks run in parallel.  A chunk whose first token continues a sequence needs
//    the state at the end of the previous chunk: k_tail_aggregate computes, for each
//    chunk, the pair (a, b) of the associative combine (a, b) o (a', b') =
//    (a a', a' b + b') over the tokens of its last sequence (a = 0 when that sequence
//    starts inside the chunk, i.e. the segmented reset), k_carry folds the pairs in
//    chunk order, and k_prefill_final rescans every chunk from its carry-in and
//    writes y and the final states.  Initial states of sequences that start in one
//    chunk and end in a later one are copied to the workspace by k_tail_aggregate
//    so that no kernel reads a slot that another workgroup of the same launch writes.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "mambamix.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kK = MM_CONV_K;   // conv width
constexpr int kKS = kK - 1;     // stored conv-state columns
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// ---------------------------------------------------------------- element I/O
__device__ __forceinline__ float ld_io(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_io(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ void st_io(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_io(uint16_t* p, int64_t i, float v) {
  // float32 -> bfloat16, round to nearest even; NaN stays a quiet NaN
  uint32_t u = __float_as_uint(v);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  p[i] = static_cast<uint16_t>((v != v) ? 0x7FC0u : r);
}

// ---------------------------------------------------------------- math
// v_exp_f32 / v_log_f32 / v_rcp_f32 are the hardware base-2 exponential, base-2
// logarithm and reciprocal (about 1 ulp).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// x * sigmoid(x)
__device__ __forceinline__ float silu(float x) { return x * rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// softplus(v) = log(1 + e^v).  For v > 20 it is v to within 2.1e-9.  For
// e = e^v < 1/64 the rounding of 1 + e would cost up to ~4e-6 relative, so the
// Taylor series e - e^2/2 + e^3/3 - e^4/4 (error < e^5/5) is used there.
__device__ __forceinline__ float softplus(float v) {
  const float e = exp2_hw(fminf(v, 20.0f) * kLog2e);
  const float series = e * __builtin_fmaf(e, __builtin_fmaf(e, __builtin_fmaf(e, -0.25f, 1.0f / 3.0f), -0.5f), 1.0f);
  const float viaLog = log2_hw(1.0f + e) * kLn2;
  const float r = (e < 0.015625f) ? series : viaLog;
  return (v > 20.0f) ? v : r;
}

// largest s in [0, S-1] with cu[s] <= g (the sequence that holds token g; empty
// sequences have cu[s] == cu[s+1] and are never returned for g < T)
__device__ __forceinline__ int seq_of(const int32_t* __restrict__ cu, int S, int64_t g) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (static_cast<int64_t>(cu[mid]) <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// per-channel constants held in registers for the whole launch
template <int NMAX>
struct Chan {
  float A2[NMAX];   // A * log2(e), so that exp(delta * A) = exp2(delta * A2)
  float w[kK];
  float cb, Dc, dtb;
};

template <int NMAX>
__device__ __forceinline__ void load_chan(Chan<NMAX>& ch, int c, int N, const float* __restrict__ A_log,
                                          const float* __restrict__ D, const float* __restrict__ dt_bias,
                                          const float* __restrict__ conv_w, const float* __restrict__ conv_b) {
#pragma unroll
  for (int n = 0; n < NMAX; ++n)
    ch.A2[n] = (n < N) ? -exp2_hw(A_log[static_cast<int64_t>(c) * N + n] * kLog2e) * kLog2e : 0.0f;
#pragma unroll
  for (int k = 0; k < kK; ++k) ch.w[k] = conv_w[static_cast<int64_t>(c) * kK + k];
  ch.cb = conv_b[c];
  ch.Dc = D[c];
  ch.dtb = dt_bias[c];
}

// One token of one channel.  win[0..2] = the three previous raw inputs (oldest
// first), shifted in place.  bc points at the token's packed float32 row
// [B_0..B_{NMAX-1}, C_0..C_{NMAX-1}] (uniform across the wave).
template <int NMAX, bool READOUT>
__device__ __forceinline__ float mixer_token(const Chan<NMAX>& ch, float xv, float zv, float dtv,
                                             const float* __restrict__ bc, float (&win)[kKS], float (&h)[NMAX],
                                             float& dsum) {
  float xc = ch.cb;
  xc = __builtin_fmaf(ch.w[0], win[0], xc);
  xc = __builtin_fmaf(ch.w[1], win[1], xc);
  xc = __builtin_fmaf(ch.w[2], win[2], xc);
  xc = __builtin_fmaf(ch.w[3], xv, xc);
  win[0] = win[1];
  win[1] = win[2];
  win[2] = xv;
  const float u = silu(xc);
  const float delta = softplus(dtv + ch.dtb);
  const float du = delta * u;
  dsum += delta;
  float yv = ch.Dc * u;
#pragma unroll
  for (int n = 0; n < NMAX; ++n) {
    const float a = exp2_hw(delta * ch.A2[n]);
    h[n] = __builtin_fmaf(a, h[n], du * bc[n]);
    if (READOUT) yv = __builtin_fmaf(h[n], bc[NMAX + n], yv);
  }
  if (READOUT) return yv * silu(zv);
  return 0.0f;
}

// Scan tokens [g, g_end) of one sequence for channel c.  Full groups of U tokens
// run as straight-line code (no per-token branch), so the scheduler can overlap
// the independent per-token work (conv, softplus, decays) of the whole group
// around the serial state updates; the next group's loads are issued before the
// current group's arithmetic (their indices are clamped into the range, so the
// last group's prefetch re-reads valid data instead of branching).  The < U
// leftover tokens run one at a time.
template <typename IO, int NMAX, bool READOUT>
__device__ __forceinline__ void scan_range(const Chan<NMAX>& ch, int64_t g, int64_t g_end, int c, int d,
                                           const IO* __restrict__ x, const IO* __restrict__ z,
                                           const IO* __restrict__ dt, const float* __restrict__ bc,
                                           IO* __restrict__ y, float (&win)[kKS], float (&h)[NMAX], float& dsum) {
  constexpr int U = 8;
  const int64_t last = g_end - 1;
  int64_t nfull = (g_end - g) / U;
  if (nfull > 0) {
    float xb[U], zb[U], db[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int64_t off = (g + i) * d + c;
      xb[i] = ld_io(x, off);
      if (READOUT) zb[i] = ld_io(z, off);
      db[i] = ld_io(dt, off);
    }
    for (; nfull > 0; --nfull, g += U) {
      float xn[U], zn[U], dn[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int64_t gi = g + U + i;
        const int64_t off = (gi < last ? gi : last) * d + c;
        xn[i] = ld_io(x, off);
        if (READOUT) zn[i] = ld_io(z, off);
        dn[i] = ld_io(dt, off);
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int64_t gi = g + i;
        const float out = mixer_token<NMAX, READOUT>(ch, xb[i], READOUT ? zb[i] : 0.0f, db[i],
                                                     bc + gi * (2 * NMAX), win, h, dsum);
        if (READOUT) st_io(y, gi * d + c, out);
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        xb[i] = xn[i];
        if (READOUT) zb[i] = zn[i];
        db[i] = dn[i];
      }
    }
  }
  for (; g < g_end; ++g) {
    const int64_t off = g * d + c;
    const float out = mixer_token<NMAX, READOUT>(ch, ld_io(x, off), READOUT ? ld_io(z, off) : 0.0f, ld_io(dt, off),
                                                 bc + g * (2 * NMAX), win, h, dsum);
    if (READOUT) st_io(y, off, out);
  }
}

// ---------------------------------------------------------------- kernels

// B, C [T, N] io -> float32 rows [T][2][NMAX] (B then C, zero-padded past N)
template <typename IO, int NMAX>
__global__ void __launch_bounds__(kBlock) k_pack_bc(const IO* __restrict__ B, const IO* __restrict__ C,
                                                   float* __restrict__ bc, int64_t T, int N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= T * 2 * NMAX) return;
  const int n = static_cast<int>(i % NMAX);
  const int which = static_cast<int>((i / NMAX) & 1);
  const int64_t g = i / (2 * NMAX);
  float v = 0.0f;
  if (n < N) v = ld_io(which ? C : B, g * N + n);
  bc[i] = v;
}

struct ChunkWs {
  float* a;        // [P][d]        sum of delta over the chunk's last segment, or -1 when that segment
                   //               starts a sequence (its decay product is then 0: the segmented reset)
  float* b;        // [P][d][NMAX]  state at the chunk end from a zero (or slot) state
  float* hin;      // [P][d][NMAX]  carry-in state of chunks whose first token continues a sequence
  float* halo;     // [P][d][3]     raw inputs before the chunk start (same sequence / its conv state)
  float* stash_h;  // [P][d][NMAX]  initial ssm state of the sequence starting in the chunk and ending later
  float* stash_c;  // [P][d][3]     its initial conv state
  int32_t* flags;  // [P]           bit 0: the chunk's first token continues a sequence;
                   //               bit 1: (a, b) of the chunk is needed (the next chunk continues)
};

// Pass 1: per chunk j and channel, (i) the halo of raw inputs before the chunk
// start, (ii) the stash of the initial state of the sequence that starts in the
// chunk and runs past its end, (iii) the combine pair (a, b) of the chunk's last
// segment when the next chunk continues that sequence.
template <typename IO, int NMAX>
__global__ void __launch_bounds__(kBlock) k_tail_aggregate(
    const IO* __restrict__ x, const IO* __restrict__ dt, const float* __restrict__ bc,
    const float* __restrict__ A_log, const float* __restrict__ D, const float* __restrict__ dt_bias,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b, const int32_t* __restrict__ cu,
    const float* __restrict__ conv_state, const float* __restrict__ ssm_state, ChunkWs ws,
    int S, int64_t T, int d, int N, int64_t Lc) {
  const int nb = (d + kBlock - 1) / kBlock;
  const int j = static_cast<int>(blockIdx.x / nb);
  const int c = static_cast<int>(blockIdx.x % nb) * kBlock + threadIdx.x;
  const int64_t g0 = static_cast<int64_t>(j) * Lc;
  const int64_t g1 = (g0 + Lc < T) ? g0 + Lc : T;
  const int s0 = seq_of(cu, S, g0);
  const int64_t st0 = cu[s0];
  // the next chunk continues a sequence of this one: then its carry-in needs (a, b) of this chunk
  const bool next_cont = g1 < T && g1 > static_cast<int64_t>(cu[seq_of(cu, S, g1)]);
  if (c == 0) ws.flags[j] = ((g0 > st0) ? 1 : 0) | (next_cont ? 2 : 0);
  if (c >= d) return;
  const int64_t pc = static_cast<int64_t>(j) * d + c;

  float halo[kKS] = {0.0f, 0.0f, 0.0f};
  if (g0 > st0) {
#pragma unroll
    for (int k = 0; k < kKS; ++k) {
      const int64_t q = g0 - kKS + k;
      halo[k] = (q >= st0) ? ld_io(x, q * d + c)
                           : conv_state[(static_cast<int64_t>(s0) * d + c) * kKS + kKS + (q - st0)];
      ws.halo[pc * kKS + k] = halo[k];
    }
  }
  if (!next_cont) return;

  const int s1 = seq_of(cu, S, g1);
  const int64_t st1 = cu[s1];
  const bool has_start = st1 >= g0;
  float h[NMAX];
  float win[kKS];
  if (has_start) {
    const int64_t sc = static_cast<int64_t>(s1) * d + c;
#pragma unroll
    for (int k = 0; k < kKS; ++k) {
      win[k] = conv_state[sc * kKS + k];
      ws.stash_c[pc * kKS + k] = win[k];
    }
#pragma unroll
    for (int n = 0; n < NMAX; ++n) {
      h[n] = (n < N) ? ssm_state[sc * N + n] : 0.0f;
      ws.stash_h[pc * NMAX + n] = h[n];
    }
  } else {
#pragma unroll
    for (int k = 0; k < kKS; ++k) win[k] = halo[k];
#pragma unroll
    for (int n = 0; n < NMAX; ++n) h[n] = 0.0f;
  }
  Chan<NMAX> ch;
  load_chan(ch, c, N, A_log, D, dt_bias, conv_w, conv_b);
  float dsum = 0.0f;
  scan_range<IO, NMAX, false>(ch, has_start ? st1 : g0, g1, c, d, x, x, dt, bc, nullptr, win, h, dsum);
  ws.a[pc] = has_start ? -1.0f : dsum;
#pragma unroll
  for (int n = 0; n < NMAX; ++n) ws.b[pc * NMAX + n] = h[n];
}

// Pass 2: fold the chunk pairs in order; the carry-in of chunk j is the state at
// the end of chunk j-1.  One thread per (channel, state index).  The per-chunk flags
// are read U at a time (uniform scalar loads), the pair loads are unconditional
// (entries of chunks whose pair is not needed hold stale data and are masked out),
// so the loop has no memory round trip on its critical path.
template <int NMAX>
__global__ void __launch_bounds__(kBlock) k_carry(ChunkWs ws, const float* __restrict__ A_log, int d, int N,
                                                  int P) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (q >= static_cast<int64_t>(d) * NMAX) return;
  const int c = static_cast<int>(q / NMAX);
  const int n = static_cast<int>(q % NMAX);
  const float A2 = (n < N) ? -exp2_hw(A_log[static_cast<int64_t>(c) * N + n] * kLog2e) * kLog2e : 0.0f;
  const int64_t stride = static_cast<int64_t>(d) * NMAX;
  float cur = 0.0f;
  constexpr int U = 32;
  for (int j0 = 0; j0 < P; j0 += U) {
    int fl[U];
    float sv[U], bv[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int j = (j0 + i < P) ? j0 + i : P - 1;
      fl[i] = (j0 + i < P) ? ws.flags[j] : 0;
      sv[i] = ws.a[static_cast<int64_t>(j) * d + c];
      bv[i] = ws.b[j * stride + q];
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (fl[i] & 1) ws.hin[(j0 + i) * stride + q] = cur;
      const bool need = (fl[i] & 2) != 0;
      const float a = (need && sv[i] >= 0.0f) ? exp2_hw(A2 * sv[i]) : 0.0f;
      cur = need ? __builtin_fmaf(a, cur, bv[i]) : 0.0f;
    }
  }
}

// Pass 3 (or the only pass when there is one chunk): scan each chunk from its
// carry-in, write y, and write the final state of every sequence that ends in it.
template <typename IO, int NMAX>
__global__ void __launch_bounds__(kBlock) k_prefill_final(
    const IO* __restrict__ x, const IO* __restrict__ z, const IO* __restrict__ dt, const float* __restrict__ bc,
    const float* __restrict__ A_log, const float* __restrict__ D, const float* __restrict__ dt_bias,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b, const int32_t* __restrict__ cu,
    float* __restrict__ conv_state, float* __restrict__ ssm_state, IO* __restrict__ y, ChunkWs ws,
    int S, int64_t T, int d, int N, int64_t Lc) {
  const int nb = (d + kBlock - 1) / kBlock;
  const int j = static_cast<int>(blockIdx.x / nb);
  const int c = static_cast<int>(blockIdx.x % nb) * kBlock + threadIdx.x;
  if (c >= d) return;
  const int64_t g0 = static_cast<int64_t>(j) * Lc;
  const int64_t g1 = (g0 + Lc < T) ? g0 + Lc : T;
  const int64_t pc = static_cast<int64_t>(j) * d + c;

  Chan<NMAX> ch;
  load_chan(ch, c, N, A_log, D, dt_bias, conv_w, conv_b);

  int s = seq_of(cu, S, g0);
  float win[kKS];
  float h[NMAX];
  int64_t g = g0;
  if (g0 > cu[s]) {  // continues a sequence from the previous chunk
#pragma unroll
    for (int k = 0; k < kKS; ++k) win[k] = ws.halo[pc * kKS + k];
#pragma unroll
    for (int n = 0; n < NMAX; ++n) h[n] = ws.hin[pc * NMAX + n];
  }
  bool need_init = !(g0 > cu[s]);
  float dsum = 0.0f;
  while (true) {
    const int64_t seq_end = cu[s + 1];
    const int64_t sc = static_cast<int64_t>(s) * d + c;
    if (need_init) {
      if (seq_end > g1) {  // runs past this chunk: its slot is written by a later chunk
#pragma unroll
        for (int k = 0; k < kKS; ++k) win[k] = ws.stash_c[pc * kKS + k];
#pragma unroll
        for (int n = 0; n < NMAX; ++n) h[n] = ws.stash_h[pc * NMAX + n];
      } else {
#pragma unroll
        for (int k = 0; k < kKS; ++k) win[k] = conv_state[sc * kKS + k];
#pragma unroll
        for (int n = 0; n < NMAX; ++n) h[n] = (n < N) ? ssm_state[sc * N + n] : 0.0f;
      }
    }
    const int64_t seg_end = seq_end < g1 ? seq_end : g1;
    scan_range<IO, NMAX, true>(ch, g, seg_end, c, d, x, z, dt, bc, y, win, h, dsum);
    if (seg_end == seq_end) {  // sequence s ends here: write its slot
#pragma unroll
      for (int k = 0; k < kKS; ++k) conv_state[sc * kKS + k] = win[k];
#pragma unroll
      for (int n = 0; n < NMAX; ++n)
        if (n < N) ssm_state[sc * N + n] = h[n];
    }
    if (seg_end >= g1) break;
    g = seg_end;
    s = seq_of(cu, S, g);
    need_init = true;
  }
}

// Decode: one token per row; lane = channel, block = 256 channels of one row.
template <typename IO, int NMAX>
__global__ void __launch_bounds__(kBlock) k_decode(
    const IO* __restrict__ x, const IO* __restrict__ z, const IO* __restrict__ dt, const IO* __restrict__ B,
    const IO* __restrict__ C, const float* __restrict__ A_log, const float* __restrict__ D,
    const float* __restrict__ dt_bias, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    float* __restrict__ conv_state, float* __restrict__ ssm_state, IO* __restrict__ y, int d, int N) {
  const int nb = (d + kBlock - 1) / kBlock;
  const int r = static_cast<int>(blockIdx.x / nb);
  const int c = static_cast<int>(blockIdx.x % nb) * kBlock + threadIdx.x;
  if (c >= d) return;
  const int64_t rc = static_cast<int64_t>(r) * d + c;
  float bcr[2 * NMAX];
#pragma unroll
  for (int n = 0; n < NMAX; ++n) {
    bcr[n] = (n < N) ? ld_io(B, static_cast<int64_t>(r) * N + n) : 0.0f;
    bcr[NMAX + n] = (n < N) ? ld_io(C, static_cast<int64_t>(r) * N + n) : 0.0f;
  }
  float h[NMAX];
#pragma unroll
  for (int n = 0; n < NMAX; ++n) h[n] = (n < N) ? ssm_state[rc * N + n] : 0.0f;
  float win[kKS];
#pragma unroll
  for (int k = 0; k < kKS; ++k) win[k] = conv_state[rc * kKS + k];
  const float xv = ld_io(x, rc), zv = ld_io(z, rc), dtv = ld_io(dt, rc);
  Chan<NMAX> ch;
  load_chan(ch, c, N, A_log, D, dt_bias, conv_w, conv_b);
  float dsum = 0.0f;
  const float out = mixer_token<NMAX, true>(ch, xv, zv, dtv, bcr, win, h, dsum);
  st_io(y, rc, out);
#pragma unroll
  for (int k = 0; k < kKS; ++k) conv_state[rc * kKS + k] = win[k];
#pragma unroll
  for (int n = 0; n < NMAX; ++n)
    if (n < N) ssm_state[rc * N + n] = h[n];
}

// Decode, streaming layout: G = NMAX/4 lanes per channel, each lane owning four
// consecutive state entries, so every state load/store instruction of a wave moves
// one contiguous 1 KiB run.  The fp32 state is touched exactly once in each
// direction, with nontemporal loads/stores (it is not reused by this kernel and
// should not displace other data from the caches).  The three conv-state values of
// a channel are loaded by three different lanes of its group (one dword each, one
// contiguous run per wave) and shared within the group by lane shuffles.  The
// per-channel work (conv, SiLU, softplus, gate) is repeated by the G lanes of a
// channel (the kernel is bound by HBM with ALU to spare) and the readout is summed
// across them with lane exchanges.  Requires N == NMAX, 16-byte aligned ssm_state,
// A_log and conv_w, and B/C rows aligned for 4-element vector loads.
template <typename T>
__device__ __forceinline__ T nt_load(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void nt_store(T v, T* p) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ void ld4_io(const float* p, float (&o)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void ld4_io(const uint16_t* p, float (&o)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xFFFF0000u);
  o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xFFFF0000u);
}

template <typename IO, int NMAX>
__global__ void __launch_bounds__(kBlock) k_decode_vec(
    const IO* __restrict__ x, const IO* __restrict__ z, const IO* __restrict__ dt, const IO* __restrict__ B,
    const IO* __restrict__ C, const float* __restrict__ A_log, const float* __restrict__ D,
    const float* __restrict__ dt_bias, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    float* __restrict__ conv_state, float* __restrict__ ssm_state, IO* __restrict__ y, int d) {
  constexpr int G = NMAX / 4;      // lanes per channel
  constexpr int CPB = kBlock / G;  // channels per block
  constexpr int KPL = (kKS + G - 1) / G;  // conv-state entries loaded per lane
  const int nb = (d + CPB - 1) / CPB;
  const int r = static_cast<int>(blockIdx.x / nb);
  const int q = static_cast<int>(threadIdx.x) % G;
  const int c = static_cast<int>(blockIdx.x % nb) * CPB + static_cast<int>(threadIdx.x) / G;
  if (c >= d) return;
  const int64_t rc = static_cast<int64_t>(r) * d + c;
  float* srow = ssm_state + rc * NMAX + 4 * q;
  float h[4] = {nt_load(srow), nt_load(srow + 1), nt_load(srow + 2), nt_load(srow + 3)};
  // conv state entry k is loaded by lane k % G of the channel's group
  float cv[KPL];
#pragma unroll
  for (int m = 0; m < KPL; ++m) {
    const int k = m * G + q;
    cv[m] = (k < kKS) ? nt_load(conv_state + rc * kKS + k) : 0.0f;
  }
  float win[kKS];
  if constexpr (G == 1) {
#pragma unroll
    for (int k = 0; k < kKS; ++k) win[k] = cv[k];
  } else {
    const int base = (static_cast<int>(threadIdx.x) & (kWave - 1)) - q;
#pragma unroll
    for (int k = 0; k < kKS; ++k) win[k] = __shfl(cv[k / G], base + k % G, kWave);
  }
  const float xv = ld_io(x, rc), zv = ld_io(z, rc), dtv = ld_io(dt, rc);
  float bq[4], cq[4];
  ld4_io(B + static_cast<int64_t>(r) * NMAX + 4 * q, bq);
  ld4_io(C + static_cast<int64_t>(r) * NMAX + 4 * q, cq);
  const float4 w = reinterpret_cast<const float4*>(conv_w)[c];
  float xc = conv_b[c];
  xc = __builtin_fmaf(w.x, win[0], xc);
  xc = __builtin_fmaf(w.y, win[1], xc);
  xc = __builtin_fmaf(w.z, win[2], xc);
  xc = __builtin_fmaf(w.w, xv, xc);
  const float u = silu(xc);
  const float delta = softplus(dtv + dt_bias[c]);
  const float du = delta * u;
  const float4 al = reinterpret_cast<const float4*>(A_log + static_cast<int64_t>(c) * NMAX)[q];
  const float alv[4] = {al.x, al.y, al.z, al.w};
  float yp = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float A2 = -exp2_hw(alv[i] * kLog2e) * kLog2e;
    const float a = exp2_hw(delta * A2);
    h[i] = __builtin_fmaf(a, h[i], du * bq[i]);
    yp = __builtin_fmaf(h[i], cq[i], yp);
  }
  if (G >= 2) yp += __shfl_xor(yp, 1);
  if (G >= 4) yp += __shfl_xor(yp, 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) nt_store(h[i], srow + i);
  if (q == 0) st_io(y, rc, (yp + D[c] * u) * silu(zv));
  // new conv state = [win1, win2, x]; entry k is written by lane k % G
  const float nw[kKS] = {win[1], win[2], xv};
#pragma unroll
  for (int m = 0; m < KPL; ++m) {
    const int k = m * G + q;
    if (k < kKS) nt_store(nw[k], conv_state + rc * kKS + k);
  }
}

// ---------------------------------------------------------------- host side

struct Plan {
  int nmax;
  int64_t Lc, P;
  size_t off_bc, off_a, off_b, off_hin, off_halo, off_stash_h, off_stash_c, off_flags, total;
};

// Enough chunks for ~32 waves per CU (short waves balance well), but never below
// 128 tokens: below that the chunk-aggregate recompute and the carry fold cost more
// than the extra parallelism returns.
constexpr int64_t kTargetWaves = 32768;
constexpr int64_t kMinChunk = 128;

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

inline int nmax_for(int N) { return N <= 4 ? 4 : (N <= 8 ? 8 : 16); }

int64_t auto_chunk(int64_t T, int d) {
  const int64_t nblk = (d + kWave - 1) / kWave;
  int64_t Lc = (T * nblk + kTargetWaves - 1) / kTargetWaves;
  if (Lc < kMinChunk) Lc = kMinChunk;
  Lc = (Lc + 63) / 64 * 64;
  if (Lc > T) Lc = T;
  return Lc;
}

Plan make_plan(int64_t T, int d, int N, int64_t chunk_len) {
  Plan p{};
  p.nmax = nmax_for(N);
  p.Lc = chunk_len > 0 ? chunk_len : auto_chunk(T, d);
  if (p.Lc > T) p.Lc = T;
  if (p.Lc < 1) p.Lc = 1;
  p.P = T > 0 ? (T + p.Lc - 1) / p.Lc : 0;
  size_t off = 0;
  p.off_bc = off;
  off += align256(static_cast<size_t>(T) * 2 * p.nmax * sizeof(float));
  if (p.P > 1) {
    const size_t pdn = static_cast<size_t>(p.P) * d * p.nmax * sizeof(float);
    const size_t pd3 = static_cast<size_t>(p.P) * d * kKS * sizeof(float);
    p.off_a = off; off += align256(static_cast<size_t>(p.P) * d * sizeof(float));
    p.off_b = off; off += align256(pdn);
    p.off_hin = off; off += align256(pdn);
    p.off_stash_h = off; off += align256(pdn);
    p.off_halo = off; off += align256(pd3);
    p.off_stash_c = off; off += align256(pd3);
    p.off_flags = off; off += align256(static_cast<size_t>(p.P) * sizeof(int32_t));
  }
  p.total = off;
  return p;
}

int prefill_kernel_count(const Plan& p) { return p.P > 1 ? 4 : 2; }

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

template <typename IO, int NMAX>
int launch_prefill(const Plan& p, const void* x, const void* z, const void* dt, const void* B, const void* C,
                   const float* A_log, const float* D, const float* dt_bias, const float* conv_w,
                   const float* conv_b, const int32_t* cu, float* conv_state, float* ssm_state, void* y, int S,
                   int64_t T, int d, int N, char* ws, hipStream_t st, StageEvents evs) {
  const IO* xi = static_cast<const IO*>(x);
  const IO* zi = static_cast<const IO*>(z);
  const IO* di = static_cast<const IO*>(dt);
  float* bc = reinterpret_cast<float*>(ws + p.off_bc);
  const int64_t nbc = T * 2 * NMAX;
  evs.mark(st);
  hipLaunchKernelGGL((k_pack_bc<IO, NMAX>), dim3(static_cast<unsigned>((nbc + kBlock - 1) / kBlock)), dim3(kBlock),
                     0, st, static_cast<const IO*>(B), static_cast<const IO*>(C), bc, T, N);
  ChunkWs cw{};
  if (p.P > 1) {
    cw.a = reinterpret_cast<float*>(ws + p.off_a);
    cw.b = reinterpret_cast<float*>(ws + p.off_b);
    cw.hin = reinterpret_cast<float*>(ws + p.off_hin);
    cw.halo = reinterpret_cast<float*>(ws + p.off_halo);
    cw.stash_h = reinterpret_cast<float*>(ws + p.off_stash_h);
    cw.stash_c = reinterpret_cast<float*>(ws + p.off_stash_c);
    cw.flags = reinterpret_cast<int32_t*>(ws + p.off_flags);
  }
  const dim3 grid(static_cast<unsigned>(((d + kBlock - 1) / kBlock) * p.P));
  if (p.P > 1) {
    evs.mark(st);
    hipLaunchKernelGGL((k_tail_aggregate<IO, NMAX>), grid, dim3(kBlock), 0, st, xi, di, bc, A_log, D, dt_bias,
                       conv_w, conv_b, cu, conv_state, ssm_state, cw, S, T, d, N, p.Lc);
    const int64_t q = static_cast<int64_t>(d) * NMAX;
    evs.mark(st);
    hipLaunchKernelGGL((k_carry<NMAX>), dim3(static_cast<unsigned>((q + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                       st, cw, A_log, d, N, static_cast<int>(p.P));
  }
  evs.mark(st);
  hipLaunchKernelGGL((k_prefill_final<IO, NMAX>), grid, dim3(kBlock), 0, st, xi, zi, di, bc, A_log, D, dt_bias,
                     conv_w, conv_b, cu, conv_state, ssm_state, static_cast<IO*>(y), cw, S, T, d, N, p.Lc);
  evs.mark(st);
  return hipGetLastError() == hipSuccess ? MM_OK : MM_ERR_HIP;
}

template <typename IO, int NMAX>
int launch_decode(const void* x, const void* z, const void* dt, const void* B, const void* C, const float* A_log,
                  const float* D, const float* dt_bias, const float* conv_w, const float* conv_b,
                  float* conv_state, float* ssm_state, void* y, int Bs, int d, int N, hipStream_t st) {
  const size_t bca = 4 * sizeof(IO);  // B/C rows are read four elements at a time
  const bool vec = N == NMAX && aligned(ssm_state, 16) && aligned(A_log, 16) && aligned(conv_w, 16) &&
                   aligned(B, bca) && aligned(C, bca);
  if (vec) {
    constexpr int CPB = kBlock / (NMAX / 4);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>((d + CPB - 1) / CPB) * Bs));
    hipLaunchKernelGGL((k_decode_vec<IO, NMAX>), grid, dim3(kBlock), 0, st, static_cast<const IO*>(x),
                       static_cast<const IO*>(z), static_cast<const IO*>(dt), static_cast<const IO*>(B),
                       static_cast<const IO*>(C), A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state,
                       static_cast<IO*>(y), d);
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
  if (K != kK || N < 1 || N > MM_MAX_N) return MM_ERR_UNSUPPORTED;
  if (io != MM_IO_F32 && io != MM_IO_BF16) return MM_ERR_UNSUPPORTED;
  return MM_OK;
}

}  // namespace

extern "C" {

const char* mamba_mixer_status_string(int status) {
  switch (status) {
    case MM_OK: return "ok";
    case MM_ERR_NULL: return "a required pointer is NULL";
    case MM_ERR_DIM: return "invalid size (negative, T > INT32_MAX, or S == 0 with T > 0)";
    case MM_ERR_UNSUPPORTED: return "unsupported K, N or io dtype (K must be 4, N in 1..16, io F32 or BF16)";
    case MM_ERR_ALIGN: return "pointer not aligned to its element size";
    case MM_ERR_WORKSPACE: return "workspace too small or NULL";
    case MM_ERR_ALIAS: return "output overlaps an input, or conv_state overlaps ssm_state";
    case MM_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

const char* mamba_mixer_version(void) { return "libmambamix 0.1 gfx950"; }

int64_t mamba_mixer_prefill_chunk_len(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K) {
  (void)S; (void)N; (void)K;
  if (T <= 0 || d <= 0) return 0;
  return auto_chunk(T, d);
}

size_t mamba_mixer_prefill_workspace_bytes_chunked(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K,
                                                   int64_t chunk_len) {
  if (check_common(T, d, N, K, MM_IO_F32) != MM_OK || S < 0) return 0;
  if (T == 0 || d == 0 || S == 0) return 0;
  return make_plan(T, d, N, chunk_len).total;
}

size_t mamba_mixer_prefill_workspace_bytes(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K) {
  return mamba_mixer_prefill_workspace_bytes_chunked(S, T, d, N, K, 0);
}

int mamba_mixer_prefill_timed(const void* x, const void* z, const void* dt, const void* B, const void* C,
                              const float* A_log, const float* D, const float* dt_bias,
                              const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                              float* conv_state, float* ssm_state, void* y,
                              int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                              int64_t chunk_len, void* workspace, size_t workspace_bytes, void* stream,
                              void* const* events, int32_t n_events) {
  int rc = check_common(T, d, N, K, io_dtype);
  if (rc != MM_OK) return rc;
  if (S < 0 || T > INT32_MAX) return MM_ERR_DIM;
  if (S == 0 && T > 0) return MM_ERR_DIM;
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
  const Plan p = make_plan(T, d, N, chunk_len);
  if (p.total > 0 && (workspace == nullptr || workspace_bytes < p.total)) return MM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MM_ERR_ALIGN;
  if (events != nullptr && n_events < prefill_kernel_count(p) + 1) return MM_ERR_DIM;
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const StageEvents evs{events, n_events, 0};
#define MM_PREFILL(IO, NM)                                                                                      \
  launch_prefill<IO, NM>(p, x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state, \
                         y, S, T, d, N, ws, st, evs)
  if (io_dtype == MM_IO_BF16) {
    if (p.nmax == 4) return MM_PREFILL(uint16_t, 4);
    if (p.nmax == 8) return MM_PREFILL(uint16_t, 8);
    return MM_PREFILL(uint16_t, 16);
  }
  if (p.nmax == 4) return MM_PREFILL(float, 4);
  if (p.nmax == 8) return MM_PREFILL(float, 8);
  return MM_PREFILL(float, 16);
#undef MM_PREFILL
}

int mamba_mixer_prefill_chunked(const void* x, const void* z, const void* dt, const void* B, const void* C,
                                const float* A_log, const float* D, const float* dt_bias,
                                const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                                float* conv_state, float* ssm_state, void* y,
                                int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                                int64_t chunk_len, void* workspace, size_t workspace_bytes, void* stream) {
  return mamba_mixer_prefill_timed(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state,
                                   ssm_state, y, S, T, d, N, K, io_dtype, chunk_len, workspace, workspace_bytes,
                                   stream, nullptr, 0);
}

int32_t mamba_mixer_prefill_kernel_count(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int64_t chunk_len) {
  if (check_common(T, d, N, K, MM_IO_F32) != MM_OK || S <= 0 || T == 0 || d == 0) return 0;
  return prefill_kernel_count(make_plan(T, d, N, chunk_len));
}

const char* mamba_mixer_prefill_kernel_name(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int64_t chunk_len,
                                            int32_t i) {
  const int32_t n = mamba_mixer_prefill_kernel_count(S, T, d, N, K, chunk_len);
  if (i < 0 || i >= n) return "";
  static const char* const multi[] = {"k_pack_bc", "k_tail_aggregate", "k_carry", "k_prefill_final"};
  static const char* const single[] = {"k_pack_bc", "k_prefill_final"};
  return n == 4 ? multi[i] : single[i];
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
  if (io_dtype == MM_IO_BF16) {
    if (nm == 4) return launch_decode<uint16_t, 4>(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y, Bs, d, N, st);
    if (nm == 8) return launch_decode<uint16_t, 8>(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y, Bs, d, N, st);
    return launch_decode<uint16_t, 16>(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y, Bs, d, N, st);
  }
  if (nm == 4) return launch_decode<float, 4>(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y, Bs, d, N, st);
  if (nm == 8) return launch_decode<float, 8>(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y, Bs, d, N, st);
  return launch_decode<float, 16>(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y, Bs, d, N, st);
}

}  // extern "C"
