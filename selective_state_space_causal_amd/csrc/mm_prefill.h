// Prefill kernels: the mixer over packed sequences, with time chunks stitched by
// the associative combine of the recurrence.
//
// Chunks.  Every sequence s of length L_s is cut into n_s = ceil(L_s / Lc) chunks
// of Lc tokens (the last one shorter); a chunk never crosses a sequence boundary,
// so a sequence starts afresh from its slot at its first chunk and nothing passes
// between sequences (the PackMamba requirement).  k_chunk_plan turns cu_seqlens
// into chunk offsets off[s] (first chunk of s) and carry offsets moff[s] (first of
// the n_s - 1 non-last chunks of s) on the device.
//
// Carries.  For the recurrence h_t = a_t h_{t-1} + b_t the pairs (a, b) combine
// associatively: (a, b) o (a', b') = (a a', a' b + b').  Over a chunk, the product
// of the decays is exp(A * sum(delta)), so the pass-1 kernels record, for every
// non-last chunk, sum(delta) and the chunk-end state from a zero start (the first
// chunk of a sequence starts from the slot instead and records -1: its decay
// product is not needed, the segmented reset).  k_carry folds them in order into
// true chunk-end states; pass 2 rescans every chunk from its carry-in and writes y
// and, for the last chunk of a sequence, the final states.  The initial states of
// multi-chunk sequences are copied to the workspace in pass 1, so no kernel reads a
// slot that another workgroup of the same launch writes.
//
// Two engines run the same chunks:
//  * lane engine (k_lane_*, this file): one lane per channel with all N state
//    entries in registers; 64 channels of one token per wave, so B_t/C_t are
//    wave-uniform and come through the scalar unit.  Fewest instructions per
//    token; needs many (chunk, channel block) pairs to fill the GPU.
//  * row engine (k_row, mm_row.h): one channel per 16-lane row, one state entry
//    per lane, 16x more waves from the same chunks; for few, long sequences.
#pragma once

#include "mm_device.h"

namespace mm {

// ---------------------------------------------------------------- chunk plan

// off[s] = sum_{s'<s} ceil(L_s' / Lc), moff[s] = sum_{s'<s} max(ceil(L_s' / Lc) - 1, 0),
// for s = 0..S.  One workgroup of 1024 threads scans S in tiles.
constexpr int kPlanThreads = 1024;

__global__ void __launch_bounds__(kPlanThreads) k_chunk_plan(const int32_t* __restrict__ cu, int S, int64_t Lc,
                                                             int32_t* __restrict__ off, int32_t* __restrict__ moff) {
  __shared__ int32_t wsum[2][kPlanThreads / kWave];
  __shared__ int32_t carry[2];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  if (tid == 0) {
    off[0] = 0;
    moff[0] = 0;
    carry[0] = 0;
    carry[1] = 0;
  }
  __syncthreads();
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int n = 0;
    if (s < S) {
      const int64_t L = static_cast<int64_t>(cu[s + 1]) - cu[s];
      n = static_cast<int>((L + Lc - 1) / Lc);
    }
    int m = n > 0 ? n - 1 : 0;
    // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int tn = __shfl_up(n, o, kWave);
      const int tm = __shfl_up(m, o, kWave);
      if (lane >= o) {
        n += tn;
        m += tm;
      }
    }
    if (lane == kWave - 1) {
      wsum[0][wv] = n;
      wsum[1][wv] = m;
    }
    __syncthreads();
    int pn = carry[0], pm = carry[1];
    for (int w = 0; w < wv; ++w) {
      pn += wsum[0][w];
      pm += wsum[1][w];
    }
    if (s < S) {
      off[s + 1] = pn + n;
      moff[s + 1] = pm + m;
    }
    __syncthreads();
    if (tid == kPlanThreads - 1) {
      carry[0] = pn + n;
      carry[1] = pm + m;
    }
    __syncthreads();
  }
}

// The chunk a workgroup owns.  k indexes chunks over all sequences (upper bound
// ceil(T/Lc) + S); workgroups past the real count see ok == false.
struct ChunkRef {
  bool ok;
  int s;           // sequence
  int j;           // chunk index within the sequence
  int ns;          // chunks of the sequence
  int64_t start;   // first token (global index)
  int64_t end;     // one past the last token
  int cidx;        // carry slot of this chunk (valid when j < ns - 1)
  int pidx;        // carry slot of the previous chunk (valid when j > 0)
};

__device__ __forceinline__ ChunkRef chunk_ref(const int32_t* __restrict__ cu, const int32_t* __restrict__ off,
                                              const int32_t* __restrict__ moff, int S, int64_t k, int64_t Lc) {
  ChunkRef r{};
  const int total = off[S];
  r.ok = k < total;
  if (!r.ok) return r;
  int lo = 0, hi = S - 1;  // largest s with off[s] <= k (skips empty sequences)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (static_cast<int64_t>(off[mid]) <= k) lo = mid; else hi = mid - 1;
  }
  r.s = lo;
  r.j = static_cast<int>(k - off[lo]);
  r.ns = off[lo + 1] - off[lo];
  const int64_t seq_start = cu[lo], seq_end = cu[lo + 1];
  r.start = seq_start + static_cast<int64_t>(r.j) * Lc;
  r.end = (r.start + Lc < seq_end) ? r.start + Lc : seq_end;
  r.cidx = moff[lo] + r.j;
  r.pidx = moff[lo] + r.j - 1;
  return r;
}

struct CarryWs {
  int32_t* off;    // [S+1]
  int32_t* moff;   // [S+1]
  float* a;        // [M*ksub][d]    sum(delta) of a pass-1 piece, -1 for a sequence's first piece
  float* b;        // [M*ksub][d][NMAX] piece-end state (local after pass 1; the lane engine's k_carry makes it true)
  float* stash;    // [M][d][NMAX+3] initial ssm then conv state of a multi-chunk sequence (at its first slot)
  int ksub;        // row engine: pass 1 scans each non-last chunk as ksub pieces of Lc / ksub tokens
  int inl;         // row engine: off / moff are computed by every workgroup (S <= kPlanInline), not read
};

// The chunk plan of at most kPlanInline sequences, computed by one 256-thread workgroup into
// its LDS arrays off[0..S], moff[0..S]: the sums of k_chunk_plan.  Saves that kernel's launch
// where every workgroup can afford S loads of cu_seqlens.
constexpr int kPlanInline = 256;
__device__ __forceinline__ void chunk_plan_inline(const int32_t* __restrict__ cu, int S, int64_t Lc, int32_t* off,
                                                  int32_t* moff, int32_t (&wsum)[2][kPlanInline / kWave]) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wv = t / kWave;
  int n = 0;
  if (t < S) {
    const int64_t L = static_cast<int64_t>(cu[t + 1]) - cu[t];
    n = static_cast<int>((L + Lc - 1) / Lc);
  }
  int m = n > 0 ? n - 1 : 0;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {  // inclusive scan within the wave
    const int tn = __shfl_up(n, o, kWave);
    const int tm = __shfl_up(m, o, kWave);
    if (lane >= o) {
      n += tn;
      m += tm;
    }
  }
  if (lane == kWave - 1) {
    wsum[0][wv] = n;
    wsum[1][wv] = m;
  }
  __syncthreads();
  for (int w = 0; w < wv; ++w) {
    n += wsum[0][w];
    m += wsum[1][w];
  }
  if (t < S) {
    off[t + 1] = n;
    moff[t + 1] = m;
  }
  if (t == 0) {
    off[0] = 0;
    moff[0] = 0;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- B/C packing

// rows: [Tpad][2][NMAX] (B_t then C_t, zero-padded past N and past T)
template <typename IO, int NMAX>
__global__ void __launch_bounds__(kBlock) k_pack_bc_rows(const IO* __restrict__ B, const IO* __restrict__ C,
                                                        float* __restrict__ bc, int64_t T, int64_t Tpad, int N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= Tpad * 2 * NMAX) return;
  const int n = static_cast<int>(i % NMAX);
  const int which = static_cast<int>((i / NMAX) & 1);
  const int64_t g = i / (2 * NMAX);
  float v = 0.0f;
  if (n < N && g < T) v = ld_io(which ? C : B, g * N + n);
  bc[i] = v;
}

// ---------------------------------------------------------------- lane engine

// The three raw inputs before token g of sequence s (positions before its start
// come from the sequence's initial conv state `cs0`).
template <typename IO>
__device__ __forceinline__ void window_before(float (&win)[kKS], const IO* __restrict__ x, int64_t g,
                                              int64_t seq_start, int c, int d, const float* cs0) {
#pragma unroll
  for (int k = 0; k < kKS; ++k) {
    const int64_t q = g - kKS + k;
    win[k] = (q >= seq_start) ? ld_io(x, q * d + c) : cs0[kKS + (q - seq_start)];
  }
}

// Pass 1, lane engine: (sum(delta), local end state) of every non-last chunk.
template <typename IO, int NMAX>
__global__ void __launch_bounds__(kBlock) k_lane_agg(
    const IO* __restrict__ x, const IO* __restrict__ dt, const float* __restrict__ bc,
    const float* __restrict__ A_log, const float* __restrict__ D, const float* __restrict__ dt_bias,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b, const int32_t* __restrict__ cu,
    const float* __restrict__ conv_state, const float* __restrict__ ssm_state, CarryWs ws, int S, int d, int N,
    int64_t Lc) {
  const int nb = (d + kBlock - 1) / kBlock;
  const int64_t k = blockIdx.x / nb;
  const int c = static_cast<int>(blockIdx.x % nb) * kBlock + threadIdx.x;
  const ChunkRef r = chunk_ref(cu, ws.off, ws.moff, S, k, Lc);
  if (!r.ok || r.j == r.ns - 1 || c >= d) return;
  const int64_t sc = static_cast<int64_t>(r.s) * d + c;
  const int64_t pc = static_cast<int64_t>(r.cidx) * d + c;
  float h[NMAX];
  float win[kKS];
  if (r.j == 0) {  // first chunk of a multi-chunk sequence: start from the slot, and stash it
    float* st = ws.stash + pc * (NMAX + kKS);
#pragma unroll
    for (int n = 0; n < NMAX; ++n) {
      h[n] = (n < N) ? ssm_state[sc * N + n] : 0.0f;
      st[n] = h[n];
    }
#pragma unroll
    for (int q = 0; q < kKS; ++q) {
      win[q] = conv_state[sc * kKS + q];
      st[NMAX + q] = win[q];
    }
  } else {
#pragma unroll
    for (int n = 0; n < NMAX; ++n) h[n] = 0.0f;
    window_before(win, x, r.start, cu[r.s], c, d, conv_state + sc * kKS);
  }
  Chan<NMAX> ch;
  load_chan(ch, c, N, A_log, D, dt_bias, conv_w, conv_b);
  float dsum = 0.0f;
  scan_range<IO, NMAX, false>(ch, r.start, r.end, c, d, x, x, dt, bc, nullptr, win, h, dsum);
  ws.a[pc] = (r.j == 0) ? -1.0f : dsum;
#pragma unroll
  for (int n = 0; n < NMAX; ++n) ws.b[pc * NMAX + n] = h[n];
}

// Pass 2, lane engine: scan each chunk from its carry-in; y; final states.
template <typename IO, int NMAX>
__global__ void __launch_bounds__(kBlock) k_lane_final(
    const IO* __restrict__ x, const IO* __restrict__ z, const IO* __restrict__ dt, const float* __restrict__ bc,
    const float* __restrict__ A_log, const float* __restrict__ D, const float* __restrict__ dt_bias,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b, const int32_t* __restrict__ cu,
    float* __restrict__ conv_state, float* __restrict__ ssm_state, IO* __restrict__ y, CarryWs ws, int S, int d,
    int N, int64_t Lc) {
  const int nb = (d + kBlock - 1) / kBlock;
  const int64_t k = blockIdx.x / nb;
  const int c = static_cast<int>(blockIdx.x % nb) * kBlock + threadIdx.x;
  const ChunkRef r = chunk_ref(cu, ws.off, ws.moff, S, k, Lc);
  if (!r.ok || c >= d) return;
  const int64_t sc = static_cast<int64_t>(r.s) * d + c;
  float h[NMAX];
  float win[kKS];
  if (r.j == 0) {
    if (r.ns > 1) {  // the slot is written by this sequence's last chunk: read the stashed copy
      const float* st = ws.stash + (static_cast<int64_t>(r.cidx) * d + c) * (NMAX + kKS);
#pragma unroll
      for (int n = 0; n < NMAX; ++n) h[n] = st[n];
#pragma unroll
      for (int q = 0; q < kKS; ++q) win[q] = st[NMAX + q];
    } else {
#pragma unroll
      for (int n = 0; n < NMAX; ++n) h[n] = (n < N) ? ssm_state[sc * N + n] : 0.0f;
#pragma unroll
      for (int q = 0; q < kKS; ++q) win[q] = conv_state[sc * kKS + q];
    }
  } else {
    const float* hb = ws.b + (static_cast<int64_t>(r.pidx) * d + c) * NMAX;
#pragma unroll
    for (int n = 0; n < NMAX; ++n) h[n] = hb[n];
    window_before(win, x, r.start, cu[r.s], c, d, conv_state + sc * kKS);  // start >= seq start + Lc >= 3
  }
  Chan<NMAX> ch;
  load_chan(ch, c, N, A_log, D, dt_bias, conv_w, conv_b);
  float dsum = 0.0f;
  scan_range<IO, NMAX, true>(ch, r.start, r.end, c, d, x, z, dt, bc, y, win, h, dsum);
  if (r.j == r.ns - 1) {
#pragma unroll
    for (int q = 0; q < kKS; ++q) conv_state[sc * kKS + q] = win[q];
#pragma unroll
    for (int n = 0; n < NMAX; ++n)
      if (n < N) ssm_state[sc * N + n] = h[n];
  }
}

// Fold the chunk pairs of every multi-chunk sequence in order, in place:
// b[first] is already true (it started from the slot); b[i] = exp(A sum_i) b[i-1] + b[i].
// One thread per (channel, state entry).
template <int NMAX>
__global__ void __launch_bounds__(kBlock) k_carry(CarryWs ws, const float* __restrict__ A_log, int S, int d, int N) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (q >= static_cast<int64_t>(d) * NMAX) return;
  const int c = static_cast<int>(q / NMAX);
  const int n = static_cast<int>(q % NMAX);
  const float A2 = (n < N) ? -exp2_hw(A_log[static_cast<int64_t>(c) * N + n] * kLog2e) * kLog2e : 0.0f;
  for (int s = 0; s < S; ++s) {
    const int m0 = ws.moff[s], m1 = ws.moff[s + 1];
    if (m1 - m0 < 2) continue;  // zero or one non-last chunk: nothing to fold
    float cur = ws.b[static_cast<int64_t>(m0) * d * NMAX + q];
    for (int i = m0 + 1; i < m1; ++i) {
      const int64_t o = static_cast<int64_t>(i) * d;
      const float a = exp2_hw(A2 * ws.a[o + c]);
      cur = __builtin_fmaf(a, cur, ws.b[o * NMAX + q]);
      ws.b[o * NMAX + q] = cur;
    }
  }
}

}  // namespace mm
