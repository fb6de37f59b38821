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
//  * lane engine (k_lane_*): one lane per channel with all N state entries in
//    registers; 64 channels of one token per wave, so B_t/C_t are wave-uniform and
//    come through the scalar unit.  Most efficient per token; needs many
//    (chunk, channel block) pairs to fill the GPU.
//  * split engine (k_split): the N state entries of a 64-channel block are split
//    across the NMAX/NPW waves of one workgroup (NPW entries per wave).  The waves
//    share the per-token work through LDS: each computes the conv/SiLU/softplus of
//    its own tokens of a tile, all of them scan their state entries over the tile,
//    and the readout partial sums are added across waves.  Up to 16x more waves than
//    the lane engine for the same chunks, at the cost of LDS traffic and barriers.
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
  float* a;        // [M][d]         sum(delta) of a non-last chunk, -1 for a sequence's first chunk
  float* b;        // [M][d][NMAX]   chunk-end state (local after pass 1, true after k_carry)
  float* stash;    // [M][d][NMAX+3] initial ssm then conv state of a multi-chunk sequence (at its first slot)
};

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

// transposed: [2][NMAX][Tpad] (row n of B^T then of C^T), zero-padded
template <typename IO, int NMAX>
__global__ void __launch_bounds__(kBlock) k_pack_bc_cols(const IO* __restrict__ B, const IO* __restrict__ C,
                                                        float* __restrict__ bct, int64_t T, int64_t Tpad, int N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= Tpad * 2 * NMAX) return;
  // i = ((which * NMAX) + n) * Tpad + g; read B/C rows in the natural order to keep loads coalesced
  const int64_t g = i / (2 * NMAX);
  const int r = static_cast<int>(i % (2 * NMAX));
  const int which = r / NMAX;
  const int n = r % NMAX;
  float v = 0.0f;
  if (n < N && g < T) v = ld_io(which ? C : B, g * N + n);
  bct[(static_cast<int64_t>(which) * NMAX + n) * Tpad + g] = v;
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

// ---------------------------------------------------------------- split engine

// Workgroup = NW = NMAX/NPW waves over the same 64 channels; wave w owns state
// entries [w*NPW, (w+1)*NPW).  Tokens are processed in tiles of TILE = NW tokens
// with one barrier per tile; wave w computes the per-token work of token w of
// each tile (one tile ahead of the scan) and finishes its output (one tile behind).
//
// LDS per workgroup: pro[2][TILE][64] float2 (delta, delta*u), plus, for the final
// pass, yp[2][TILE][NW][64] readout partials.
template <int NMAX, int NPW, bool FINAL>
struct SplitShared {
  static constexpr int NW = NMAX / NPW;
  static constexpr int TILE = NW;
  float2 pro[2][TILE][kWave];
  float yp[FINAL ? 2 : 1][FINAL ? TILE : 1][FINAL ? NW : 1][kWave];
};

template <typename IO, int NMAX, int NPW, bool FINAL>
__global__ void __launch_bounds__(kWave * (NMAX / NPW)) k_split(
    const IO* __restrict__ x, const IO* __restrict__ z, const IO* __restrict__ dt, const float* __restrict__ bct,
    int64_t Tpad, const float* __restrict__ A_log, const float* __restrict__ D, const float* __restrict__ dt_bias,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b, const int32_t* __restrict__ cu,
    float* __restrict__ conv_state, float* __restrict__ ssm_state, IO* __restrict__ y, CarryWs ws, int S, int d,
    int N, int64_t Lc) {
  using SH = SplitShared<NMAX, NPW, FINAL>;
  constexpr int NW = SH::NW;
  constexpr int TILE = SH::TILE;
  __shared__ SH sh;
  const int nb = (d + kWave - 1) / kWave;
  const int64_t k = blockIdx.x / nb;
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int c = static_cast<int>(blockIdx.x % nb) * kWave + lane;
  const bool cval = c < d;
  const int cc = cval ? c : d - 1;  // clamped channel for parameter reads
  const ChunkRef r = chunk_ref(cu, ws.off, ws.moff, S, k, Lc);
  if (!r.ok) return;
  if (!FINAL && r.j == r.ns - 1) return;
  const int64_t seq_start = cu[r.s];
  const int64_t sc = static_cast<int64_t>(r.s) * d + cc;
  const int64_t len = r.end - r.start;
  const int ntiles = static_cast<int>((len + TILE - 1) / TILE);

  // per-channel constants
  const float dtb = dt_bias[cc];
  const float Dc = D[cc];
  const float cb = conv_b[cc];
  float w[kK];
#pragma unroll
  for (int q = 0; q < kK; ++q) w[q] = conv_w[static_cast<int64_t>(cc) * kK + q];
  float A2[NPW];
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int n = wv * NPW + i;
    A2[i] = (n < N) ? -exp2_hw(A_log[static_cast<int64_t>(cc) * N + n] * kLog2e) * kLog2e : 0.0f;
  }

  // initial state of this chunk and the conv state before its first token
  float h[NPW];
  const float* cs0;  // initial conv state of the sequence (used for its first three tokens only)
  const int64_t pc = static_cast<int64_t>(r.cidx) * d + cc;
  if (r.j == 0) {
    const bool multi = r.ns > 1;
    float* st = ws.stash + pc * (NMAX + kKS);
    if (FINAL && multi) {
      cs0 = st + NMAX;
#pragma unroll
      for (int i = 0; i < NPW; ++i) h[i] = st[wv * NPW + i];
    } else {
      cs0 = conv_state + sc * kKS;
#pragma unroll
      for (int i = 0; i < NPW; ++i) {
        const int n = wv * NPW + i;
        h[i] = (n < N) ? ssm_state[sc * N + n] : 0.0f;
      }
      if (!FINAL && cval) {  // pass 1 of a multi-chunk sequence: stash the initial state
#pragma unroll
        for (int i = 0; i < NPW; ++i) st[wv * NPW + i] = h[i];
        if (wv == 0) {
#pragma unroll
          for (int q = 0; q < kKS; ++q) st[NMAX + q] = cs0[q];
        }
      }
    }
  } else {
    cs0 = conv_state + sc * kKS;  // not read: the chunk starts >= Lc >= 3 tokens into the sequence
    if (FINAL) {
      const float* hb = ws.b + (static_cast<int64_t>(r.pidx) * d + cc) * NMAX;
#pragma unroll
      for (int i = 0; i < NPW; ++i) h[i] = hb[wv * NPW + i];
    } else {
#pragma unroll
      for (int i = 0; i < NPW; ++i) h[i] = 0.0f;
    }
  }

  // the sequence's initial conv state, for the conv windows of its first three tokens
  float cs0v[kKS];
#pragma unroll
  for (int k2 = 0; k2 < kKS; ++k2) cs0v[k2] = cs0[k2];

  // Token inputs of this wave's token (token wv) of a tile, loaded raw three tiles
  // ahead of their use so the HBM latency hides behind the scans of the tiles
  // between.  The loads are unconditional at clamped (always valid) addresses;
  // widening and the choice between x and the initial conv state happen at use.
  struct Pre {
    IO xr[kK];  // x of the token and of the three before it (clamped into the sequence)
    IO dtr, zr;
  };
  auto issue = [&](int tile) {
    Pre q;
    const int64_t g = r.start + static_cast<int64_t>(tile) * TILE + wv;
    const int64_t gl = g < r.end ? g : r.end - 1;
#pragma unroll
    for (int k2 = 0; k2 < kK; ++k2) {
      const int64_t gq = gl - (kK - 1) + k2;
      q.xr[k2] = x[(gq < seq_start ? seq_start : gq) * d + cc];
    }
    q.dtr = dt[gl * d + cc];
    if constexpr (FINAL) q.zr = z[gl * d + cc];
    else q.zr = q.dtr;
    return q;
  };
  // per-token work: delta and delta*u to LDS for the scans; D*u and SiLU(z) stay in
  // registers of this wave, which finishes the token two iterations later
  auto prologue = [&](int tile, int buf, const Pre& q, float2& fin) {
    const int64_t g = r.start + static_cast<int64_t>(tile) * TILE + wv;
    float delta = 0.0f, u = 0.0f;
    if (g < r.end) {
      float xc = cb;
#pragma unroll
      for (int k2 = 0; k2 < kK; ++k2) {
        const int64_t pos = g - (kK - 1) + k2 - seq_start;  // position in the sequence
        const float from_state = pos == -3 ? cs0v[0] : (pos == -2 ? cs0v[1] : cs0v[2]);
        const float xv = pos >= 0 ? ld_io(q.xr, k2) : from_state;
        xc = __builtin_fmaf(w[k2], xv, xc);
      }
      u = silu(xc);
      delta = softplus(ld_io(&q.dtr, 0) + dtb);
    }
    sh.pro[buf][wv][lane] = make_float2(delta, delta * u);
    if constexpr (FINAL) fin = make_float2(Dc * u, silu(ld_io(&q.zr, 0)));
  };

  // finish token wv of tile `tile`: y, and the final conv state at the sequence end
  auto epilogue = [&](int tile, int buf, float2 fin) {
    if constexpr (!FINAL) return;
    const int64_t g = r.start + static_cast<int64_t>(tile) * TILE + wv;
    if (g < r.end && cval) {
      float part[NW];
#pragma unroll
      for (int v = 0; v < NW; ++v) part[v] = sh.yp[buf][wv][v][lane];
#pragma unroll
      for (int w2 = 1; w2 < NW; w2 <<= 1)  // pairwise tree over the waves' partial readouts
#pragma unroll
        for (int v = 0; v + w2 < NW; v += 2 * w2) part[v] += part[v + w2];
      st_io(y, g * d + c, (part[0] + fin.x) * fin.y);
      if (g == r.end - 1 && r.j == r.ns - 1) {  // last token of the sequence: new conv state
        float nw[kKS];
#pragma unroll
        for (int k2 = 0; k2 < kKS; ++k2) {
          const int64_t gq = g - (kKS - 1) + k2;
          nw[k2] = (gq >= seq_start) ? ld_io(x, gq * d + c) : cs0[kKS + (gq - seq_start)];
        }
#pragma unroll
        for (int k2 = 0; k2 < kKS; ++k2) conv_state[sc * kKS + k2] = nw[k2];
      }
    }
  };

  float dsum = 0.0f;
  float2 fin_prev = make_float2(0.0f, 0.0f), fin_cur = make_float2(0.0f, 0.0f);

  // one tile: refill `fill` with tile it+3, finish tile it-1, scan tile it, and do the
  // per-token work of tile it+1 from `use` (loaded two iterations earlier)
  auto body = [&](int it, Pre& fill, const Pre& use) {
    const int buf = it & 1;
    fill = issue(it + 3);
    // B/C of this tile for this wave's state entries: wave-uniform scalar loads, issued
    // before the barrier so their latency overlaps the wait and the epilogue
    const int64_t g0 = r.start + static_cast<int64_t>(it) * TILE;
    float bb[NPW][TILE], cc2[NPW][TILE];
#pragma unroll
    for (int i2 = 0; i2 < NPW; ++i2) {
      const int n = wv * NPW + i2;
#pragma unroll
      for (int t = 0; t < TILE; ++t) {
        bb[i2][t] = bct[static_cast<int64_t>(n) * Tpad + g0 + t];
        if constexpr (FINAL) cc2[i2][t] = bct[static_cast<int64_t>(NMAX + n) * Tpad + g0 + t];
        else cc2[i2][t] = 0.0f;
      }
    }
    __syncthreads();
    if (it > 0) epilogue(it - 1, buf ^ 1, fin_prev);
    float2 pv[TILE];
#pragma unroll
    for (int t = 0; t < TILE; ++t) pv[t] = sh.pro[buf][t][lane];
    float yacc[TILE];
#pragma unroll
    for (int t = 0; t < TILE; ++t) yacc[t] = 0.0f;
#pragma unroll
    for (int i2 = 0; i2 < NPW; ++i2) {
      float hi = h[i2];
#pragma unroll
      for (int t = 0; t < TILE; ++t) {
        const float a = exp2_hw(pv[t].x * A2[i2]);
        hi = __builtin_fmaf(a, hi, pv[t].y * bb[i2][t]);
        if constexpr (FINAL) yacc[t] = __builtin_fmaf(hi, cc2[i2][t], yacc[t]);
      }
      h[i2] = hi;
    }
    if constexpr (!FINAL) {
      if (wv == 0) {
#pragma unroll
        for (int t = 0; t < TILE; ++t) dsum += pv[t].x;
      }
    } else {
#pragma unroll
      for (int t = 0; t < TILE; ++t) sh.yp[buf][t][wv][lane] = yacc[t];
    }
    float2 fin_next = make_float2(0.0f, 0.0f);
    if (it + 1 < ntiles) prologue(it + 1, buf ^ 1, use, fin_next);
    fin_prev = fin_cur;
    fin_cur = fin_next;
  };

  // three-slot ring of prefetched token inputs: tile t lives in slot t % 3; the loop is
  // unrolled by three so every slot is a fixed set of registers (no copies of loads in flight)
  Pre qa = issue(0), qb = issue(1), qc = issue(2);
  prologue(0, 0, qa, fin_cur);
  for (int it = 0; it < ntiles; it += 3) {
    body(it, qa, qb);
    if (it + 1 < ntiles) body(it + 1, qb, qc);
    if (it + 2 < ntiles) body(it + 2, qc, qa);
  }
  __syncthreads();
  if constexpr (FINAL) {
    if (ntiles > 0) epilogue(ntiles - 1, (ntiles - 1) & 1, fin_prev);
    if (r.j == r.ns - 1 && cval) {
#pragma unroll
      for (int i = 0; i < NPW; ++i) {
        const int n = wv * NPW + i;
        if (n < N) ssm_state[sc * N + n] = h[i];
      }
    }
  } else if (cval) {
    if (wv == 0) ws.a[pc] = (r.j == 0) ? -1.0f : dsum;
#pragma unroll
    for (int i = 0; i < NPW; ++i) ws.b[pc * NMAX + wv * NPW + i] = h[i];
  }
}

}  // namespace mm
