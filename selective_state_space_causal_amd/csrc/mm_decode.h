// Decode kernels: one token for each of Bs rows, state updated in place.
#pragma once

#include "mm_device.h"

namespace mm {

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

}  // namespace mm
