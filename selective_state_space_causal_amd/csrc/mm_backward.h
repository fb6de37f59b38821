// Backward of the prefill over packed sequences: the gradients of a loss, given
// dL/dy, with respect to every input of the mixer, its parameters and the initial
// conv / SSM states.  This is the reverse mode of the step the forward kernels run
// (the one-token Mamba step of the TensorRT tensor-parallel builder,
// _add_mamba_tp_layer), sequence by sequence, with no gradient crossing a
// cu_seqlens boundary (PackMamba, abstract).  With g = SiLU(z), p = C.h + D u,
// y = p g, a = exp(delta A) and lambda_t = dL/dh_t (the adjoint of the state after
// token t):
//   dp = dy g,  dz = dy p SiLU'(z),  lambda_t = dp_t C_t + a_{t+1} lambda_{t+1},
//   dC_t += dp_t h_t,  dB_t += lambda_t delta_t u_t          (summed over channels)
//   du = dp D + delta S1,  ddelta = u S1 + S2,  S1 = sum_n lambda_n B_n,
//   S2 = sum_n lambda_n h_{t-1,n} a_n A_n,  dA += lambda h_{t-1} a delta,
//   ddt = ddelta sigmoid(dt + dt_bias),  dxc = du SiLU'(xc), and the conv taps
//   spread dxc back over the inputs (or the initial conv state) they read;
//   dh_init = a_0 lambda_0.
//
// Three steps, all in the row layout of the forward (one channel per 16-lane row,
// one state entry per lane, 16-token blocks aligned in the packed stream):
//  1. the forward pass in checkpoint mode (k_row<IO, false, true>) stores the state
//     before every block -- 64 bytes per (block, channel);
//  2. k_row_bwd walks each sequence's blocks in reverse.  Per block it recomputes
//     the 16 states from the block's checkpoint (the forward's operations in the
//     forward's order), the readout p by the transposing butterfly, then runs the
//     adjoint recurrence backwards over the 16 tokens; the sums over the state
//     index (S1, S2) go through the same butterfly, so the per-token tail (lane j =
//     token j) needs no further exchange.  dB and dC are sums over channels: the 16
//     rows of a workgroup are summed through LDS, and each 16-channel block writes
//     one partial [T][N] slice.  Parameter gradients are summed in registers over
//     all tokens of the workgroup's sequences (a workgroup takes every G-th
//     sequence) and written as one partial per workgroup row;
//  3. two small kernels sum the partials in a fixed order (the result does not
//     depend on scheduling) and round dB / dC to the io type.
#pragma once

#include "mm_row.h"

namespace mm {

constexpr int kPrm = kRow + 3 + kK;  // partial parameter gradients per channel: dA_log[16], dD, ddt_bias, dconv_b, dconv_w[4]

// lane j reads lane (j + K) mod 16 of the row (row_ror by 16 - K)
template <int K>
__device__ __forceinline__ float rol(float v) { return dpp<0x120 + (kRow - K)>(v); }
// lane j reads lane j + K of the row; lanes j >= 16 - K keep `old` (row_shl)
template <int K>
__device__ __forceinline__ float shl_or(float old, float v) {
  return __builtin_amdgcn_update_dpp(old, v, 0x100 + K, 0xF, 0xF, false);
}

__device__ __forceinline__ float sigmoid_hw(float v) { return rcp_hw(1.0f + exp2_hw(-v * kLog2e)); }
// d SiLU(v) / dv from s = sigmoid(v)
__device__ __forceinline__ float dsilu_s(float v, float s) { return s * __builtin_fmaf(v, 1.0f - s, 1.0f); }

// one row's dB or dC terms [token][n]; the padding puts the four rows of a wave on
// different LDS banks
struct RedRow {
  float v[kRow][kRow];
  float pad[kRow];
};

struct BwdTiles {
  float x[2][kRow][kRowChans + 1];
  float z[2][kRow][kRowChans + 1];
  float dt[2][kRow][kRowChans + 1];
  float dy[2][kRow][kRowChans + 1];
  float4 bc[2][2][4][kRow];
  float o[3][kRow][kRowChans + 1];      // dx, dz, ddt of the block, [token][channel]
  RedRow red[2][kRowChans];  // dB, dC terms [row][token][n] before the sum over rows
};

template <typename IO>
struct BwdStage {
  IO x, z, dt, dy, B, C;
};

// thread i: element (token i/16, channel i%16) of the [16][16] tiles, element i of
// the contiguous [16][N] B and C tiles; indices clamped into the arrays
template <typename IO>
__device__ __forceinline__ void bwd_stage_load(BwdStage<IO>& r, const IO* __restrict__ x, const IO* __restrict__ z,
                                               const IO* __restrict__ dt, const IO* __restrict__ dy,
                                               const IO* __restrict__ B, const IO* __restrict__ C, int64_t tb, int T,
                                               int d, int N, int c0) {
  const int i = threadIdx.x;
  const uint32_t tmax = static_cast<uint32_t>(T - 1);
  uint32_t t = static_cast<uint32_t>(tb) + static_cast<uint32_t>(i >> 4);
  t = t < tmax ? t : tmax;
  int c = c0 + (i & (kRowChans - 1));
  c = c < d ? c : d - 1;
  const int64_t o = static_cast<int64_t>(t) * static_cast<uint32_t>(d) + c;
  r.x = x[o];
  r.z = z[o];
  r.dt = dt[o];
  r.dy = dy[o];
  if (i < kRow * N) {
    const int64_t last = static_cast<int64_t>(T) * N - 1;
    int64_t e = tb * N + i;
    e = e < last ? e : last;
    r.B = B[e];
    r.C = C[e];
  }
}

template <typename IO>
__device__ __forceinline__ void bwd_stage_store(const BwdStage<IO>& r, BwdTiles& L, int buf, int N) {
  const int i = threadIdx.x;
  const int tt = i >> 4, ch = i & (kRowChans - 1);
  L.x[buf][tt][ch] = io_f32(r.x);
  L.z[buf][tt][ch] = io_f32(r.z);
  L.dt[buf][tt][ch] = io_f32(r.dt);
  L.dy[buf][tt][ch] = io_f32(r.dy);
  if (i < kRow * N) {
    const int t = i / N, n = i - t * N;
    reinterpret_cast<float*>(&L.bc[buf][0][t >> 2][n])[t & 3] = io_f32(r.B);
    reinterpret_cast<float*>(&L.bc[buf][1][t >> 2][n])[t & 3] = io_f32(r.C);
  }
}

// forward recompute, token I of the block: decay, state after the token, readout term
template <int I>
__device__ __forceinline__ void bwd_fwd_step(float delta, float du, float A2, const float4 (&Bq)[4],
                                             const float4 (&Cq)[4], float& h, float* hsl, float* asl,
                                             float (&pr)[kRow]) {
  const float a = exp2_hw(bcast<I>(delta) * A2);
  h = __builtin_fmaf(a, h, bcast<I>(du) * comp(Bq[I >> 2], I & 3));
  hsl[I * kRow] = h;
  asl[I * kRow] = a;
  pr[I] = comp(Cq[I >> 2], I & 3) * h;
}

template <int... I>
__device__ __forceinline__ void bwd_fwd_steps(std::integer_sequence<int, I...>, float delta, float du, float A2,
                                              const float4 (&Bq)[4], const float4 (&Cq)[4], float& h,
                                              float* hsl, float* asl, float (&pr)[kRow]) {
  (bwd_fwd_step<I>(delta, du, A2, Bq, Cq, h, hsl, asl, pr), ...);
}

// adjoint step, token I of the block (called for I = 15 down to 0).  lam holds
// lambda of token I+1 on entry and of token I on exit; anext the decay of token I+1
// on entry and of token I on exit; hcur the state after token I on entry and the
// state before it on exit.  The forward phase left the state h_I in rC[I] and the
// decay a_I in rB[I]; each slot is read before it is overwritten with the dC or dB
// term (slot I-1 is read at step I, one step before step I-1 overwrites it).
// lambda a_I h_{I-1} is formed as a product of the three: the equal difference
// lambda (h_I - du_I B_I) cancels where a_I h_{I-1} is small beside du_I B_I (large
// delta |A|), and that error is then scaled by delta A.
template <int I>
__device__ __forceinline__ void bwd_rev_step(float dp, float du, float delta, float An,
                                             const float4 (&Bq)[4], const float4 (&Cq)[4],
                                             float& lam, float& anext, float& accA,
                                             float (&s1)[kRow], float (&s2)[kRow], float (&rB)[kRow][kRow],
                                             float (&rC)[kRow][kRow], int j, float& hcur, float h0) {
  const float dpi = bcast<I>(dp);
  lam = __builtin_fmaf(anext, lam, dpi * comp(Cq[I >> 2], I & 3));
  const float hI = hcur;                            // the state after token I
  const float hprev = I > 0 ? rC[I - 1][j] : h0;    // the state before token I
  rC[I][j] = dpi * hI;
  const float dui = bcast<I>(du);
  const float aI = rB[I][j];
  rB[I][j] = lam * dui;
  const float sb = lam * comp(Bq[I >> 2], I & 3);
  s1[I] = sb;
  const float q = lam * (aI * hprev);
  s2[I] = q * An;
  accA = __builtin_fmaf(bcast<I>(delta), q, accA);
  anext = aI;
  hcur = hprev;
}

template <int... I>
__device__ __forceinline__ void bwd_rev_steps(std::integer_sequence<int, I...>, float dp, float du, float delta,
                                              float An, const float4 (&Bq)[4], const float4 (&Cq)[4],
                                              float& lam,
                                              float& anext, float& accA, float (&s1)[kRow], float (&s2)[kRow],
                                              float (&rB)[kRow][kRow], float (&rC)[kRow][kRow], int j, float h0) {
  float hcur = rC[kRow - 1][j];  // the state after the block's last token
  (bwd_rev_step<kRow - 1 - I>(dp, du, delta, An, Bq, Cq, lam, anext, accA, s1, s2, rB, rC, j, hcur, h0), ...);
}

// The reverse pass.  Workgroup (k, cb) takes channels 16 cb .. 16 cb + 15 of
// sequences k, k + G, k + 2G, ...  ckpt: [rows][d][16], block ib of sequence s at
// row (cu[s] >> 4) + s + ib.  Outputs: dx, dz, ddt [T][d] (io); dcs [S][d][3] and
// dss [S][d][N], the gradients of the initial states; pbc [nchb][2][T][N], the dB
// and dC sums over each 16-channel block; pprm [G][kPrm][d], the parameter
// gradients summed over each workgroup row's sequences.
template <typename IO>
__global__ void __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(3))) k_row_bwd(
    const IO* __restrict__ x, const IO* __restrict__ z, const IO* __restrict__ dt, const IO* __restrict__ B,
    const IO* __restrict__ C, const IO* __restrict__ dy, const float* __restrict__ A_log,
    const float* __restrict__ D, const float* __restrict__ dt_bias, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, const int32_t* __restrict__ cu, const float* __restrict__ conv_state,
    const float* __restrict__ ckpt, IO* __restrict__ dx, IO* __restrict__ dz, IO* __restrict__ ddt,
    float* __restrict__ dcs, float* __restrict__ dss, float* __restrict__ pbc, float* __restrict__ pprm, int S,
    int64_t T, int d, int N, int G) {
  constexpr int64_t kMask = ~static_cast<int64_t>(kRow - 1);
  __shared__ BwdTiles L;
  int64_t k;
  int cb;
  const int nchb = (d + kRowChans - 1) / kRowChans;
  row_work(blockIdx.x, (nchb + kRowGroup - 1) / kRowGroup, k, cb);
  if (cb >= nchb || k >= G) return;

  const int j = threadIdx.x & (kRow - 1);
  const int ch = static_cast<int>(threadIdx.x >> 4);
  const int c0 = cb * kRowChans;
  const int c = c0 + ch;
  const bool cvalid = c < d;
  const int cc = cvalid ? c : d - 1;  // rows past d compute on a valid channel with dy = 0 and store nothing
  const int64_t d64 = d;

  const float An = (j < N) ? -exp2_hw(A_log[static_cast<int64_t>(cc) * N + j] * kLog2e) : 0.0f;
  const float A2 = An * kLog2e;  // the forward's exponent scale, bit for bit
  const float w0 = conv_w[cc * kK + 0], w1 = conv_w[cc * kK + 1], w2 = conv_w[cc * kK + 2];
  const float w3 = conv_w[cc * kK + 3];
  const float cbias = conv_b[cc], dtb = dt_bias[cc], Dc = D[cc];

  if (N < kRow) {  // B/C entries past N stay zero: the staging only writes n < N
    float* bcf = reinterpret_cast<float*>(&L.bc[0][0][0][0]);
    for (int i = threadIdx.x; i < 2 * 2 * 4 * kRow * 4; i += kRowThreads) bcf[i] = 0.0f;
    __syncthreads();
  }

  // parameter gradients of this row's channel, summed over tokens: accA per state
  // entry (lane n), the others per token lane (summed over the row at the end)
  float accA = 0.0f, accD = 0.0f, accT = 0.0f, accCb = 0.0f;
  float accW[kK] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int T32 = static_cast<int>(T);

  for (int64_t s = k; s < S; s += G) {
    const int64_t start = cu[s], end = cu[s + 1];
    const int64_t sc = s * d64 + cc;
    if (end <= start) {  // nothing depends on an empty sequence's initial state
      if (cvalid) {
        if (j < N) dss[sc * N + j] = 0.0f;
        if (j < kKS) dcs[sc * kKS + j] = 0.0f;
      }
      continue;
    }
    const float* cs0 = conv_state + sc * kKS;
    auto hist = [&](int64_t t) -> float {
      if (t >= start) return io_f32(x[t * d64 + cc]);
      const int64_t q = t - start + kKS;
      return q >= 0 ? cs0[q] : 0.0f;
    };
    const int64_t tb0 = start & kMask;
    const int64_t tlast = (end - 1) & kMask;
    const int nb = static_cast<int>((tlast - tb0) >> 4) + 1;
    const int64_t crow0 = (start >> 4) + s;
    const float hist0 = (tb0 + j < start) ? hist(tb0 + j) : 0.0f;

    BwdStage<IO> stg{};
    bwd_stage_load<IO>(stg, x, z, dt, dy, B, C, tlast, T32, d, N, c0);
    bwd_stage_store<IO>(stg, L, (nb - 1) & 1, N);
    if (nb > 1) bwd_stage_load<IO>(stg, x, z, dt, dy, B, C, tlast - kRow, T32, d, N, c0);
    float h0 = ckpt[((crow0 + nb - 1) * d64 + cc) * kRow + j];
    float prev = (j >= kRow - kKS) ? hist(tlast - kRow + j) : 0.0f;
    __syncthreads();

    float lam = 0.0f, anext = 0.0f;  // adjoint of the state after the block, decay of the token after it
    float nxt = 0.0f;                // dxc of the block after (lane j: its token j)
    for (int ib = nb - 1; ib >= 0; --ib) {
      const int buf = ib & 1;
      const int64_t tb = tb0 + static_cast<int64_t>(ib) * kRow;
      const int64_t t = tb + j;
      const bool act = t >= start && t < end;
      // Staging and loads, at the top of the block so that they have its whole arithmetic
      // to arrive: block ib-1 (loaded an iteration ago) into the other buffer, whose block
      // ib+1 was last read before the previous iteration's barriers; the next (earlier)
      // block's checkpoint and conv look-back, loaded as raw values whatever the lane and
      // block (the indices clamped into range) and resolved at the end of the block; then
      // the loads of block ib-2.  The first use of any of them is then past the block's
      // arithmetic: the compiler waits for every outstanding load at a use (the stores in
      // the loop make it treat the counter as unordered), and an early use would stall on
      // the staging loads.
      if (ib >= 1) bwd_stage_store<IO>(stg, L, buf ^ 1, N);
      const float h0n = ckpt[((crow0 + (ib > 0 ? ib - 1 : 0)) * d64 + cc) * kRow + j];
      // look-back token of lane j >= 13, relative to the sequence start (chunks < 2^31 tokens)
      const int prel = static_cast<int>(tb - start) - 2 * kRow + j;
      const IO praw = x[(start + (prel > 0 ? prel : 0)) * d64 + cc];
      const float pcs = cs0[min(max(prel + kKS, 0), kKS - 1)];
      if (ib >= 2) bwd_stage_load<IO>(stg, x, z, dt, dy, B, C, tb - 2 * kRow, T32, d, N, c0);

      // per-token forward quantities (lane j = token j)
      const float xv = (t < start) ? hist0 : L.x[buf][j][ch];
      const float x1 = shr_or<1>(dpp<0x121>(prev), xv);
      const float x2 = shr_or<2>(dpp<0x122>(prev), xv);
      const float x3 = shr_or<3>(dpp<0x123>(prev), xv);
      float xc = cbias;
      xc = __builtin_fmaf(w0, x3, xc);
      xc = __builtin_fmaf(w1, x2, xc);
      xc = __builtin_fmaf(w2, x1, xc);
      xc = __builtin_fmaf(w3, xv, xc);
      const float sx = sigmoid_hw(xc);
      const float u = silu(xc);
      const float v = L.dt[buf][j][ch] + dtb;
      const float delta = softplus(v) * (act ? 1.0f : 0.0f);
      const float du = delta * u;
      const float zv = L.z[buf][j][ch];
      const float dyv = (act && cvalid) ? L.dy[buf][j][ch] : 0.0f;
      float4 Bq[4], Cq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        Bq[q] = L.bc[buf][0][q][j];
        Cq[q] = L.bc[buf][1][q][j];
      }

      __builtin_amdgcn_sched_barrier(0);
      // the block's states from its checkpoint, and the readout p
      // issue priority rises through the block (forward recompute 1, adjoint 2, tail 3) and
      // drops after the block's last barrier: the SIMD issues first for the wave nearest the
      // barriers its workgroup waits at (the waves sharing a SIMD belong to other workgroups)
      __builtin_amdgcn_s_setprio(1);
      float pr[kRow];
      float h = h0;
      bwd_fwd_steps(std::make_integer_sequence<int, kRow>{}, delta, du, A2, Bq, Cq, h, &L.red[1][ch].v[0][j],
                    &L.red[0][ch].v[0][j], pr);
      const float pt = __builtin_fmaf(Dc, u, row_transpose_sum(pr, j));
      const float sz = sigmoid_hw(zv);
      const float dp = dyv * (zv * sz);
      const float dzv = dyv * pt * dsilu_s(zv, sz);

      __builtin_amdgcn_sched_barrier(0);
      // the adjoint recurrence over the block, last token first.  The reverse broadcasts
      // from copies the compiler cannot merge with the forward's: a merged broadcast has
      // several uses, cannot fold into them and stays live across both phases.
      float s1[kRow], s2[kRow];
      float du_r = du, delta_r = delta, dp_r = dp;
      int lz = 0;  // a zero the compiler cannot see: the LDS reads below are not merged with earlier ones
      asm volatile("" : "+v"(du_r), "+v"(delta_r), "+v"(dp_r), "+v"(lz));
      const int jz = j + lz;
      // B and C again from LDS rather than kept in registers across the forward phase, and
      // the states from LDS where the forward phase left them
      float4 Br[4], Cr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        Br[q] = L.bc[buf][0][q][jz];
        Cr[q] = L.bc[buf][1][q][jz];
      }
      float(&rB)[kRow][kRow] = L.red[0][ch].v;
      float(&rC)[kRow][kRow] = L.red[1][ch].v;
      __builtin_amdgcn_s_setprio(2);
      bwd_rev_steps(std::make_integer_sequence<int, kRow>{}, dp_r, du_r, delta_r, An, Br, Cr, lam, anext,
                    accA, s1, s2, rB, rC, jz, h0);
      __builtin_amdgcn_sched_barrier(0);
      const float S1 = row_transpose_sum(s1, j);
      const float S2 = row_transpose_sum(s2, j);

      __builtin_amdgcn_sched_barrier(0);
      // per-token tail
      __builtin_amdgcn_s_setprio(3);
      const float dut = __builtin_fmaf(dp, Dc, delta * S1);
      const float ddel = __builtin_fmaf(u, S1, S2);
      const float dv = act ? ddel * sigmoid_hw(v) : 0.0f;
      const float dxc = act ? dut * dsilu_s(xc, sx) : 0.0f;
      accD = __builtin_fmaf(dp, u, accD);
      accT += dv;
      accCb += dxc;
      accW[0] = __builtin_fmaf(dxc, x3, accW[0]);
      accW[1] = __builtin_fmaf(dxc, x2, accW[1]);
      accW[2] = __builtin_fmaf(dxc, x1, accW[2]);
      accW[3] = __builtin_fmaf(dxc, xv, accW[3]);
      // input t is read by tap 3 of token t, tap 2 of t+1, tap 1 of t+2, tap 0 of t+3
      const float e1 = shl_or<1>(rol<1>(nxt), dxc);
      const float e2 = shl_or<2>(rol<2>(nxt), dxc);
      const float e3 = shl_or<3>(rol<3>(nxt), dxc);
      float dX = w3 * dxc;
      dX = __builtin_fmaf(w2, e1, dX);
      dX = __builtin_fmaf(w1, e2, dX);
      dX = __builtin_fmaf(w0, e3, dX);
      if (ib == 0 && cvalid && t < start && t >= start - kKS) dcs[sc * kKS + (t - start + kKS)] = dX;
      nxt = dxc;
      L.o[0][j][ch] = dX;
      L.o[1][j][ch] = dzv;
      L.o[2][j][ch] = dv;
      h0 = h0n;
      prev = (ib > 0 && j >= kRow - kKS) ? (prel >= 0 ? io_f32(praw) : (prel + kKS >= 0 ? pcs : 0.0f)) : 0.0f;

      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      {  // sums over the workgroup's 16 channels, and the io outputs of the block
        const int tt = threadIdx.x >> 4, n = threadIdx.x & (kRow - 1);
        const int64_t tg = tb + tt;
        float sB = 0.0f, sC = 0.0f;
#pragma unroll
        for (int r = 0; r < kRowChans; ++r) {
          sB += L.red[0][r].v[tt][n];
          sC += L.red[1][r].v[tt][n];
        }
        if (tg >= start && tg < end) {
          if (n < N) {
            pbc[((static_cast<int64_t>(cb) * 2 + 0) * T + tg) * N + n] = sB;
            pbc[((static_cast<int64_t>(cb) * 2 + 1) * T + tg) * N + n] = sC;
          }
          if (c0 + n < d) {
            const int64_t o = tg * d64 + c0 + n;
            st_io(dx, o, L.o[0][tt][n]);
            st_io(dz, o, L.o[1][tt][n]);
            st_io(ddt, o, L.o[2][tt][n]);
          }
        }
      }
      __syncthreads();
      __builtin_amdgcn_s_setprio(0);
    }

    // gradient of the initial SSM state: the adjoint carried through the block's first token
    if (cvalid && j < N) dss[sc * N + j] = anext * lam;
    // initial conv-state entries read from before block 0 (lanes 13..15 of the block before it)
    {
      const float r1 = rol<1>(nxt), r2 = rol<2>(nxt), r3 = rol<3>(nxt);
      float dX = (j >= kRow - 1) ? w2 * r1 : 0.0f;
      dX = __builtin_fmaf(w1, (j >= kRow - 2) ? r2 : 0.0f, dX);
      dX = __builtin_fmaf(w0, (j >= kRow - 3) ? r3 : 0.0f, dX);
      const int64_t t = tb0 - kRow + j;
      if (cvalid && t < start && t >= start - kKS) dcs[sc * kKS + (t - start + kKS)] = dX;
    }
  }

  const float sD = row_sum(accD), sT = row_sum(accT), sCb = row_sum(accCb);
  float sW[kK];
#pragma unroll
  for (int i = 0; i < kK; ++i) sW[i] = row_sum(accW[i]);
  if (cvalid) {
    float* P = pprm + k * kPrm * d64 + c;
    if (j < N) P[j * d64] = accA * An;  // dA_log = dA * A
    if (j == 0) {
      P[(kRow + 0) * d64] = sD;
      P[(kRow + 1) * d64] = sT;
      P[(kRow + 2) * d64] = sCb;
#pragma unroll
      for (int i = 0; i < kK; ++i) P[(kRow + 3 + i) * d64] = sW[i];
    }
  }
}

// dB, dC = the sums of the per-channel-block partials, in block order
template <typename IO>
__global__ void __launch_bounds__(kBlock) k_bwd_sum_bc(const float* __restrict__ pbc, IO* __restrict__ dB,
                                                     IO* __restrict__ dC, int64_t TN, int nchb) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= 2 * TN) return;
  const int q = i >= TN ? 1 : 0;
  const int64_t e = i - q * TN;
  const float* p = pbc + q * TN + e;
  const int64_t stride = 2 * TN;
  // sixteen partials loaded at once, added in block order (the same order as one at a time)
  float s = 0.0f;
  int b = 0;
  for (; b + 16 <= nchb; b += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = p[(b + u) * stride];
#pragma unroll
    for (int u = 0; u < 16; ++u) s += v[u];
  }
  for (; b < nchb; ++b) s += p[b * stride];
  st_io(q ? dC : dB, e, s);
}

// parameter gradients = the sums of the per-workgroup-row partials, in row order
__global__ void __launch_bounds__(kBlock) k_bwd_sum_params(const float* __restrict__ pprm, float* __restrict__ dA_log,
                                                         float* __restrict__ dD, float* __restrict__ ddt_bias,
                                                         float* __restrict__ dconv_b, float* __restrict__ dconv_w,
                                                         int d, int N, int G) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t d64 = d;
  if (i >= kPrm * d64) return;
  const int q = static_cast<int>(i / d64);
  const int c = static_cast<int>(i - q * d64);
  if (q < kRow && q >= N) return;
  float s = 0.0f;
  for (int g = 0; g < G; ++g) s += pprm[(static_cast<int64_t>(g) * kPrm + q) * d64 + c];
  if (q < kRow) dA_log[static_cast<int64_t>(c) * N + q] = s;
  else if (q == kRow) dD[c] = s;
  else if (q == kRow + 1) ddt_bias[c] = s;
  else if (q == kRow + 2) dconv_b[c] = s;
  else dconv_w[static_cast<int64_t>(c) * kK + (q - kRow - 3)] = s;
}

}  // namespace mm
