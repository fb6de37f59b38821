// Row engine of the prefill: one channel per 16-lane row of a wave, one state
// entry per lane (N <= 16, zero-padded), cross-lane exchange through DPP.
//
// Why: with few sequences the lane engine (one lane per channel) has too few
// waves to fill the GPU without cutting sequences into chunks that are scanned
// twice.  Spreading a channel's 16 state entries over 16 lanes gives 16x more
// waves from the same chunks.
//
// A workgroup (4 waves, 16 rows) owns 16 consecutive channels of one chunk and
// walks it in blocks of 16 tokens; blocks are aligned to multiples of 16 in the
// packed token stream.  Per block:
//  * the workgroup stages the block's x, z, dt tiles ([16 tokens][16 channels])
//    and the B, C tiles ([16 tokens][N], contiguous in memory) from HBM into LDS
//    with coalesced loads, two blocks ahead of their use, and writes y back from
//    an LDS tile one block behind -- every global access is a run of whole rows;
//  * lane j of a row does the per-token work of token j for the row's channel:
//    the causal conv (the three older inputs come from lanes j-1..j-3 or from the
//    previous block by DPP row shifts), SiLU, softplus, delta * u, D * u and
//    SiLU(z).  Tokens outside the chunk get delta = 0, which makes their step the
//    identity (exp(0) = 1, nothing added);
//  * the 16 recurrence steps: step i broadcasts delta and delta * u of token i from
//    lane i to the row (DPP row_newbcast, folded into the multiply that uses it);
//    lane n updates h_n = exp(delta A_n) h_n + (delta u) B_n and forms C_n h_n;
//  * a 16x16 transposing butterfly over the row (DPP row rotations and quad
//    permutes) sums C_n h_n over n for all 16 tokens at once and leaves token j's
//    sum in lane j, which finishes y for its token.
// One barrier per block.  The chunk plan, carries and stash are those of the
// other engines (mm_prefill.h); with one chunk per sequence ("whole" mode) the
// workgroup's chunk is simply its sequence and no plan is needed.
#pragma once

#include <utility>

#include "mm_prefill.h"

namespace mm {

constexpr int kRow = 16;                               // lanes per row = state entries = tokens per block
constexpr int kRowWaves = 4;                           // waves per workgroup
constexpr int kRowThreads = kRowWaves * kWave;         // 256
constexpr int kRowChans = kRowWaves * (kWave / kRow);  // 16 channels per workgroup
constexpr int kRowGroup = 4;                           // workgroups sharing 128-byte lines of bf16 io
constexpr int kXcds = 8;                               // MI355X: workgroup w runs on XCD w % 8

// ---------------------------------------------------------------- DPP helpers
// DPP controls (gfx9 encoding): quad_perm 0x00-0xFF, row_shr:k 0x110+k,
// row_ror:k 0x120+k (lane j of a row reads lane (j-k) mod 16), row_newbcast:k
// 0x150+k (every lane of a row reads lane k of the row).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_amdgcn_update_dpp(0.0f, v, CTRL, 0xF, 0xF, true);
}
// lane j reads lane j-k of the row; lanes j < k keep `old`
template <int K>
__device__ __forceinline__ float shr_or(float old, float v) {
  return __builtin_amdgcn_update_dpp(old, v, 0x110 + K, 0xF, 0xF, false);
}
template <int I>
__device__ __forceinline__ float bcast(float v) { return dpp<0x150 + I>(v); }

constexpr int kXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRor4 = 0x124;  // reads lane j-4: partner of lanes with bit 2 set
constexpr int kRor8 = 0x128;  // reads lane j^8
constexpr int kRor12 = 0x12C; // reads lane j+4: partner of lanes with bit 2 clear

__device__ __forceinline__ float comp(const float4& v, int e) {
  return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

// One recurrence step: token I of the block.
template <int I, bool READOUT>
__device__ __forceinline__ void row_step(float delta, float du, float A2, const float4 (&Bq)[4],
                                         const float4 (&Cq)[4], float& h, float (&p)[kRow]) {
  const float a = exp2_hw(bcast<I>(delta) * A2);
  h = __builtin_fmaf(a, h, bcast<I>(du) * comp(Bq[I >> 2], I & 3));
  if (READOUT) p[I] = comp(Cq[I >> 2], I & 3) * h;
}

template <bool READOUT, int... I>
__device__ __forceinline__ void row_steps(std::integer_sequence<int, I...>, float delta, float du, float A2,
                                          const float4 (&Bq)[4], const float4 (&Cq)[4], float& h, float (&p)[kRow]) {
  (row_step<I, READOUT>(delta, du, A2, Bq, Cq, h, p), ...);
}

// p[i] in lane n holds term n of token i; returns sum_n p[j] in lane j.
// Each stage halves the registers: lanes on one side of the stage's lane bit keep
// the lower half of the tokens, the others the upper half, each summed with the
// partner lane across that bit.
__device__ __forceinline__ float row_transpose_sum(const float (&p)[kRow], int j) {
  // keep the products C_n h_n separate from these sums, so that the lane exchange
  // folds into the adds (an fma would need the exchanged operand in a register)
#pragma clang fp contract(off)
  float q[8], r[4], s[2];
  const bool b3 = (j & 8) != 0, b2 = (j & 4) != 0, b1 = (j & 2) != 0, b0 = (j & 1) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float lo = p[i] + dpp<kRor8>(p[i]);
    const float hi = p[i + 8] + dpp<kRor8>(p[i + 8]);
    q[i] = b3 ? hi : lo;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = q[i] + dpp<kRor12>(q[i]);
    const float hi = q[i + 4] + dpp<kRor4>(q[i + 4]);
    r[i] = b2 ? hi : lo;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float lo = r[i] + dpp<kXor2>(r[i]);
    const float hi = r[i + 2] + dpp<kXor2>(r[i + 2]);
    s[i] = b1 ? hi : lo;
  }
  const float lo = s[0] + dpp<kXor1>(s[0]);
  const float hi = s[1] + dpp<kXor1>(s[1]);
  return b0 ? hi : lo;
}

// sum over the 16 lanes of the row, in every lane
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<kRor8>(v);
  v += dpp<kRor4>(v);
  v += dpp<kXor2>(v);
  v += dpp<kXor1>(v);
  return v;
}

__device__ __forceinline__ float io_f32(float v) { return v; }
__device__ __forceinline__ float io_f32(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

// ---------------------------------------------------------------- LDS tiles
// [token][channel] tiles are padded to 17 columns; the B/C tile is laid out
// [which][q][n] float4 holding tokens 4q..4q+3, so lane n reads B (or C) of 4
// tokens as one float4.
struct RowTiles {
  float x[2][kRow][kRowChans + 1];
  float z[2][kRow][kRowChans + 1];
  float dt[2][kRow][kRowChans + 1];
  float4 bc[2][2][4][kRow];
  float y[2][kRow][kRowChans + 1];
};

// One thread's share of a block's global inputs: element (token i/16, channel i%16)
// of the x/z/dt tiles, and element i of the contiguous [16][N] B and C tiles.
template <typename IO>
struct RowStage {
  IO x, z, dt, B, C;
};

template <typename IO, bool FINAL>
__device__ __forceinline__ void row_stage_load(RowStage<IO>& r, const IO* __restrict__ x, const IO* __restrict__ z,
                                               const IO* __restrict__ dt, const IO* __restrict__ B,
                                               const IO* __restrict__ C, int64_t tb, int T, int d, int N, int c0) {
  const int i = threadIdx.x;
  const uint32_t tmax = static_cast<uint32_t>(T - 1);
  uint32_t t = static_cast<uint32_t>(tb) + static_cast<uint32_t>(i >> 4);  // T <= INT32_MAX: no wrap
  t = t < tmax ? t : tmax;
  int c = c0 + (i & (kRowChans - 1));
  c = c < d ? c : d - 1;
  const int64_t o = static_cast<int64_t>(t) * static_cast<uint32_t>(d) + c;
  r.x = x[o];
  r.dt = dt[o];
  if (FINAL) r.z = z[o];
  if (i < kRow * N) {
    const int64_t last = static_cast<int64_t>(T) * N - 1;
    int64_t e = tb * N + i;
    e = e < last ? e : last;
    r.B = B[e];
    if (FINAL) r.C = C[e];
  }
}

template <typename IO, bool FINAL>
__device__ __forceinline__ void row_stage_store(const RowStage<IO>& r, RowTiles& L, int buf, int N) {
  const int i = threadIdx.x;
  const int tt = i >> 4, ch = i & (kRowChans - 1);
  L.x[buf][tt][ch] = io_f32(r.x);
  L.dt[buf][tt][ch] = io_f32(r.dt);
  if (FINAL) L.z[buf][tt][ch] = io_f32(r.z);
  if (i < kRow * N) {
    const int t = i / N, n = i - t * N;
    reinterpret_cast<float*>(&L.bc[buf][0][t >> 2][n])[t & 3] = io_f32(r.B);
    if (FINAL) reinterpret_cast<float*>(&L.bc[buf][1][t >> 2][n])[t & 3] = io_f32(r.C);
  }
}

// Workgroup -> (chunk, 16-channel block).  Groups of kRowGroup consecutive channel
// blocks of one chunk read the same cache lines of x/z/dt/y, so they are placed
// on the same XCD (same w % 8).  The grid is padded to a multiple of 32.
__device__ __forceinline__ void row_work(int64_t w, int ncg, int64_t& k, int& cb) {
  const int64_t item = (w / (kXcds * kRowGroup)) * kXcds + (w % kXcds);
  const int m = static_cast<int>((w / kXcds) % kRowGroup);
  k = item / ncg;
  cb = static_cast<int>(item % ncg) * kRowGroup + m;
}

// FINAL = false: pass 1 (sum(delta) and local end state of every non-last chunk).
// FINAL = true: pass 2 (y, and the final states at a sequence's last chunk).
// CKPT = true: also write the state before every 16-token block to ckpt, [rows][d][16],
// the block starting at token tb of sequence s at row s + tb / 16.  With FINAL = false
// (whole sequences only) that is all the pass writes: the checkpoint pass of the
// backward.  With FINAL = true it is the forward of a training step; a continuing
// chunk leaves a block it shares with the chunk before to that chunk.
// whole != 0: one chunk per sequence, workgroup chunk index = sequence (no plan).
template <typename IO, bool FINAL, bool CKPT = false>
__global__ void __launch_bounds__(kRowThreads) k_row(
    const IO* __restrict__ x, const IO* __restrict__ z, const IO* __restrict__ dt, const IO* __restrict__ B,
    const IO* __restrict__ C, const float* __restrict__ A_log, const float* __restrict__ D,
    const float* __restrict__ dt_bias, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    const int32_t* __restrict__ cu, float* __restrict__ conv_state, float* __restrict__ ssm_state,
    IO* __restrict__ y, CarryWs ws, int S, int64_t T, int d, int N, int64_t Lc, int whole,
    float* __restrict__ ckpt) {
  constexpr int NMAX = kRow;
  constexpr int64_t kMask = ~static_cast<int64_t>(kRow - 1);
  __shared__ RowTiles L;
  int64_t k;
  int cb;
  const int nchb = (d + kRowChans - 1) / kRowChans;
  row_work(blockIdx.x, (nchb + kRowGroup - 1) / kRowGroup, k, cb);
  if (cb >= nchb) return;
  ChunkRef R;
  if (whole) {
    if (k >= S) return;
    R.ok = true;
    R.s = static_cast<int>(k);
    R.j = 0;
    R.ns = 1;
    R.start = cu[R.s];
    R.end = cu[R.s + 1];
    if (R.end <= R.start) return;  // empty sequence: its slot stays as it is
    R.cidx = R.pidx = 0;
  } else {
    R = chunk_ref(cu, ws.off, ws.moff, S, k, Lc);
    if (!R.ok) return;
  }
  if (!FINAL && !CKPT && R.j == R.ns - 1) return;

  const int j = threadIdx.x & (kRow - 1);             // state entry in the scan; token of the block in the per-token work
  const int ch = static_cast<int>(threadIdx.x >> 4);  // row = channel within the workgroup
  const int c0 = cb * kRowChans;
  const int c = c0 + ch;
  const bool cvalid = c < d;
  const int cc = cvalid ? c : d - 1;  // rows past d compute on a valid channel and store nothing
  const int64_t sc = static_cast<int64_t>(R.s) * d + cc;
  const int64_t seq_start = cu[R.s];

  const float A2 = (j < N) ? -exp2_hw(A_log[static_cast<int64_t>(cc) * N + j] * kLog2e) * kLog2e : 0.0f;
  const float w0 = conv_w[cc * kK + 0], w1 = conv_w[cc * kK + 1], w2 = conv_w[cc * kK + 2];
  const float w3 = conv_w[cc * kK + 3];
  const float cbias = conv_b[cc], dtb = dt_bias[cc];
  const float Dc = FINAL ? D[cc] : 0.0f;

  // initial SSM state, and the sequence's initial conv state cs0 (pass 2 reads the
  // stashed copies of a multi-chunk sequence: its last chunk rewrites the slot)
  const bool multi = R.ns > 1;
  const float* cs0 = conv_state + sc * kKS;
  float h = 0.0f;
  if (!FINAL && !CKPT) {
    if (R.j == 0) {
      h = (j < N) ? ssm_state[sc * N + j] : 0.0f;
      if (cvalid) {
        float* stash = ws.stash + (static_cast<int64_t>(R.cidx) * d + c) * (NMAX + kKS);
        stash[j] = h;
        if (j < kKS) stash[NMAX + j] = cs0[j];
      }
    }
  } else {
    const float* st0 = multi ? ws.stash + (static_cast<int64_t>(ws.moff[R.s]) * d + cc) * (NMAX + kKS) : nullptr;
    if (multi) cs0 = st0 + NMAX;
    if (R.j == 0) {
      h = multi ? st0[j] : ((j < N) ? ssm_state[sc * N + j] : 0.0f);
    } else {
      h = ws.b[(static_cast<int64_t>(R.pidx) * d + cc) * NMAX + j];
    }
  }

  // raw input of token t of this sequence; positions before its start come from cs0
  auto hist = [&](int64_t t) -> float {
    if (t >= seq_start) return io_f32(x[t * d + cc]);
    const int64_t q = t - seq_start + kKS;
    return q >= 0 ? cs0[q] : 0.0f;
  };
  const int64_t tb0 = R.start & kMask;
  const int64_t tlast = (R.end - 1) & kMask;
  // lanes 13..15 of prev stand for the three tokens before the first block
  float prev = (j >= kRow - kKS) ? hist(tb0 - kRow + j) : 0.0f;
  const float hist0 = (tb0 + j < seq_start) ? hist(tb0 + j) : 0.0f;

  // B/C entries past N stay zero: the staging only writes n < N
  if (N < kRow) {
    float* bcf = reinterpret_cast<float*>(&L.bc[0][0][0][0]);
    for (int i = threadIdx.x; i < 2 * 2 * 4 * kRow * 4; i += kRowThreads) bcf[i] = 0.0f;
    __syncthreads();
  }

  const int nb = static_cast<int>((tlast - tb0) >> 4) + 1;
  const int T32 = static_cast<int>(T);
  RowStage<IO> stg{};
  row_stage_load<IO, FINAL>(stg, x, z, dt, B, C, tb0, T32, d, N, c0);
  row_stage_store<IO, FINAL>(stg, L, 0, N);
  if (nb > 1) row_stage_load<IO, FINAL>(stg, x, z, dt, B, C, tb0 + kRow, T32, d, N, c0);
  __syncthreads();

  float p[kRow];
  float dsum = 0.0f;
  float xv = 0.0f, x1 = 0.0f, x2 = 0.0f;
  const int64_t d64 = d;
  const int yt = threadIdx.x >> 4, ych = threadIdx.x & (kRowChans - 1);  // y tile element this thread stores
  const bool ych_ok = c0 + ych < d;

  for (int ib = 0; ib < nb; ++ib) {
    const int buf = ib & 1;
    const int64_t tb = tb0 + static_cast<int64_t>(ib) * kRow;
    if (CKPT && cvalid && (ib > 0 || tb0 == R.start || R.j == 0))  // the state before this block
      ckpt[((static_cast<int64_t>(tb >> 4) + R.s) * d + c) * NMAX + j] = h;
    {
      const int64_t t = tb + j;
      const bool act = t >= R.start && t < R.end;
      xv = (t < seq_start) ? hist0 : L.x[buf][j][ch];
      // the window: inputs of tokens t-1, t-2, t-3 from the lanes below, or from prev
      x1 = shr_or<1>(dpp<0x121>(prev), xv);
      x2 = shr_or<2>(dpp<0x122>(prev), xv);
      const float x3 = shr_or<3>(dpp<0x123>(prev), xv);
      float xc = cbias;
      xc = __builtin_fmaf(w0, x3, xc);
      xc = __builtin_fmaf(w1, x2, xc);
      xc = __builtin_fmaf(w2, x1, xc);
      xc = __builtin_fmaf(w3, xv, xc);
      const float u = silu(xc);
      // computed for every lane and masked with a multiply: no branch around softplus
      const float delta = softplus(L.dt[buf][j][ch] + dtb) * (act ? 1.0f : 0.0f);
      const float du = delta * u;
      if (!FINAL) dsum += delta;
      float4 Bq[4], Cq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        Bq[q] = L.bc[buf][0][q][j];
        Cq[q] = FINAL ? L.bc[buf][1][q][j] : Bq[q];
      }
      row_steps<FINAL>(std::make_integer_sequence<int, kRow>{}, delta, du, A2, Bq, Cq, h, p);
      if (FINAL) {
        const float s = row_transpose_sum(p, j);
        L.y[buf][j][ch] = __builtin_fmaf(Dc, u, s) * silu(L.z[buf][j][ch]);
      }
      prev = xv;
    }
    // stage block ib+1 (loaded one iteration ago), prefetch block ib+2, write y of block ib-1
    if (ib + 1 < nb) row_stage_store<IO, FINAL>(stg, L, buf ^ 1, N);
    if (ib + 2 < nb) row_stage_load<IO, FINAL>(stg, x, z, dt, B, C, tb + 2 * kRow, T32, d, N, c0);
    if (FINAL && ib > 0) {
      const int64_t t = tb - kRow + yt;
      if (t >= R.start && t < R.end && ych_ok) st_io(y, t * d64 + c0 + ych, L.y[buf ^ 1][yt][ych]);
    }
    __syncthreads();
  }
  if (FINAL) {
    const int64_t t = tb0 + static_cast<int64_t>(nb - 1) * kRow + yt;
    if (t >= R.start && t < R.end && ych_ok) st_io(y, t * d64 + c0 + ych, L.y[(nb - 1) & 1][yt][ych]);
  }

  if (CKPT && !FINAL) return;
  if (!FINAL) {
    const float ds = row_sum(dsum);
    if (cvalid) {
      const int64_t pc = static_cast<int64_t>(R.cidx) * d + c;
      if (j == 0) ws.a[pc] = (R.j == 0) ? -1.0f : ds;
      ws.b[pc * NMAX + j] = h;
    }
  } else if (R.j == R.ns - 1 && cvalid) {
    if (j < N) ssm_state[sc * N + j] = h;
    if (j == static_cast<int>((R.end - 1) & (kRow - 1))) {  // the lane of the sequence's last token
      conv_state[sc * kKS + 0] = x2;
      conv_state[sc * kKS + 1] = x1;
      conv_state[sc * kKS + 2] = xv;
    }
  }
}

}  // namespace mm
