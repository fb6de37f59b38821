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
// direction; it is stored with nontemporal stores (it is not reused by this kernel)
// and loaded with plain loads (measured faster here than nontemporal ones).  The readout is summed across
// the G lanes of a channel with lane exchanges.  Requires N == NMAX, 16-byte aligned
// ssm_state, A_log and conv_w, and B/C rows aligned for 4-element vector loads.

__device__ __forceinline__ void ld4_io(const float* p, float (&o)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void ld4_io(const uint16_t* p, float (&o)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xFFFF0000u);
  o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xFFFF0000u);
}

// broadcast lane q of each group of G consecutive lanes (G = 1, 2 or 4) to its group
template <int G, int Q>
__device__ __forceinline__ float group_bcast(float v) {
  if constexpr (G == 1) return v;
  constexpr int ctrl = G == 4 ? Q * 0x55 : (Q | Q << 2 | (Q + 2) << 4 | (Q + 2) << 6);
  return __builtin_amdgcn_update_dpp(0.0f, v, ctrl, 0xF, 0xF, true);
}

template <typename IO, int NMAX, int G, int I>
__device__ __forceinline__ void decode_row_update(float delta, float du, const float (&A2)[4], const float (&bq)[4],
                                                  const float (&cq)[4], float (&h)[4], float& yp) {
  const float di = group_bcast<G, I>(delta), dui = group_bcast<G, I>(du);
  yp = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = exp2_hw(di * A2[e]);
    h[e] = __builtin_fmaf(a, h[e], dui * bq[e]);
    yp = __builtin_fmaf(h[e], cq[e], yp);
  }
  if constexpr (G >= 2) yp += __shfl_xor(yp, 1);
  if constexpr (G >= 4) yp += __shfl_xor(yp, 2);
}

// G = NMAX/4 lanes per channel and G rows per block: lane q of a channel's group does
// the per-token work (conv, SiLU, softplus, SiLU(z)) of row r0+q only and hands delta
// and delta*u to the group by DPP, so that work is not repeated across the lanes
// that share a channel; every load of the G rows is issued before any arithmetic.
template <typename IO, int NMAX>
__global__ void __launch_bounds__(kBlock) k_decode_vec(
    const IO* __restrict__ x, const IO* __restrict__ z, const IO* __restrict__ dt, const IO* __restrict__ B,
    const IO* __restrict__ C, const float* __restrict__ A_log, const float* __restrict__ D,
    const float* __restrict__ dt_bias, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    float* __restrict__ conv_state, float* __restrict__ ssm_state, IO* __restrict__ y, int Bs, int d) {
  constexpr int G = NMAX / 4;      // lanes per channel = rows per block
  constexpr int CPB = kBlock / G;  // channels per block
  const int nb = (d + CPB - 1) / CPB;
  const int r0 = static_cast<int>(blockIdx.x / nb) * G;
  const int q = static_cast<int>(threadIdx.x) % G;
  const int c = static_cast<int>(blockIdx.x % nb) * CPB + static_cast<int>(threadIdx.x) / G;
  if (c >= d) return;
  float h[G][4], bq[G][4], cq[G][4];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int r = (r0 + i < Bs) ? r0 + i : Bs - 1;  // rows past Bs load a valid row and store nothing
    const float* srow = ssm_state + (static_cast<int64_t>(r) * d + c) * NMAX + 4 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[i][e] = srow[e];
    ld4_io(B + static_cast<int64_t>(r) * NMAX + 4 * q, bq[i]);
    ld4_io(C + static_cast<int64_t>(r) * NMAX + 4 * q, cq[i]);
  }
  // this lane's own row r0+q: token inputs and conv state
  const bool own_ok = r0 + q < Bs;
  const int64_t orc = static_cast<int64_t>(own_ok ? r0 + q : Bs - 1) * d + c;
  float win[kKS];
#pragma unroll
  for (int k = 0; k < kKS; ++k) win[k] = nt_load(conv_state + orc * kKS + k);
  const float xv = ld_io(x, orc), zv = ld_io(z, orc), dtv = ld_io(dt, orc);
  const float4 w = reinterpret_cast<const float4*>(conv_w)[c];
  const float4 al = reinterpret_cast<const float4*>(A_log + static_cast<int64_t>(c) * NMAX)[q];
  const float alv[4] = {al.x, al.y, al.z, al.w};
  float A2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) A2[e] = -exp2_hw(alv[e] * kLog2e) * kLog2e;
  float xc = conv_b[c];
  xc = __builtin_fmaf(w.x, win[0], xc);
  xc = __builtin_fmaf(w.y, win[1], xc);
  xc = __builtin_fmaf(w.z, win[2], xc);
  xc = __builtin_fmaf(w.w, xv, xc);
  const float u = silu(xc);
  const float delta = softplus(dtv + dt_bias[c]);
  const float du = delta * u;
  float yp[G];
  decode_row_update<IO, NMAX, G, 0>(delta, du, A2, bq[0], cq[0], h[0], yp[0]);
  if constexpr (G >= 2) decode_row_update<IO, NMAX, G, 1>(delta, du, A2, bq[1], cq[1], h[1], yp[1]);
  if constexpr (G >= 4) {
    decode_row_update<IO, NMAX, G, 2>(delta, du, A2, bq[2], cq[2], h[2], yp[2]);
    decode_row_update<IO, NMAX, G, 3>(delta, du, A2, bq[3], cq[3], h[3], yp[3]);
  }
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (r0 + i < Bs) {
      float* srow = ssm_state + (static_cast<int64_t>(r0 + i) * d + c) * NMAX + 4 * q;
#pragma unroll
      for (int e = 0; e < 4; ++e) nt_store(h[i][e], srow + e);
    }
  }
  if (own_ok) {
    float ypo = yp[0];
#pragma unroll
    for (int i = 1; i < G; ++i) ypo = (q == i) ? yp[i] : ypo;
    st_io(y, orc, __builtin_fmaf(D[c], u, ypo) * silu(zv));
    // new conv state = [win1, win2, x]
    nt_store(win[1], conv_state + orc * kKS + 0);
    nt_store(win[2], conv_state + orc * kKS + 1);
    nt_store(xv, conv_state + orc * kKS + 2);
  }
}

// Replay decode ("ReplaySSM: Cache SSM Inputs, Not State", abstract): the state of
// each row is a checkpoint (the conv and SSM state before window step 0) plus the raw
// inputs x, dt, B of the window steps since it, kept by the caller in ring slots
// [W][Bs][...].  Step k replays steps 0..k-1 in registers and takes step k, so the
// fp32 state is read every step but written only when the window closes (commit).
// The per-step arithmetic is that of k_decode_vec (same operations in the same
// order, including the grouping of the readout sum), so a replayed step reproduces
// the eager step bit for bit.
//
// The same kernel also serves speculative decoding: one call can emit the outputs of
// several window steps (draft tokens) without writing any state, and commit the state
// after any of them (the accepted prefix); a rejected draft is dropped by moving the
// caller's ring position back.
//
// Layout: one lane per channel with its 16 state entries in registers, 256 channels
// of one row per block.  x and dt of every window step are one coalesced load per
// row; B and C of a row are the same for every lane, so they come through the
// scalar unit; the state moves as four 16-byte loads per lane.  Few, wide vector
// loads per (row, channel) keep this kernel on the HBM roofline where a
// lanes-per-channel layout spent its time issuing small loads.  W <= 4, N = 16.
// Window steps 0..k1 are taken from the checkpoint; steps k0..k1 write their output
// (z, C and y of step t at slot t - k0 of the z/C/y arrays, slot strides zs, cs_, ys);
// if 0 <= cstep <= k1 the state after step cstep becomes the checkpoint.
template <typename IO>
__global__ void __launch_bounds__(kBlock) k_decode_replay(
    const IO* __restrict__ x_ring, const IO* __restrict__ dt_ring, const IO* __restrict__ B_ring,
    const IO* __restrict__ z, const IO* __restrict__ C, const float* __restrict__ A_log,
    const float* __restrict__ D, const float* __restrict__ dt_bias, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, float* __restrict__ conv_state, float* __restrict__ ssm_state,
    IO* __restrict__ y, int Bs, int d, int k0, int k1, int cstep, int64_t zs, int64_t cst, int64_t ys) {
  constexpr int NMAX = 16;
  constexpr int W = 4;  // ring slots read at most
  const int nb = (d + kBlock - 1) / kBlock;
  const int r = static_cast<int>(blockIdx.x / nb);
  const int c = static_cast<int>(blockIdx.x % nb) * kBlock + static_cast<int>(threadIdx.x);
  // B of the window steps and C of the output steps: the same for every lane of the
  // block (scalar loads, all issued before any store)
  const int64_t bslot = static_cast<int64_t>(Bs) * NMAX;  // ring slot stride of B
  float bv[W][NMAX], cvv[W][NMAX];
#pragma unroll
  for (int t = 0; t < W; ++t) {
    const int tb = t <= k1 ? t : k1;
    const int tc = (t >= k0 ? t : k0) - k0;
    const IO* bt = B_ring + tb * bslot + static_cast<int64_t>(r) * NMAX;
    const IO* ct = C + (tc <= k1 - k0 ? tc : k1 - k0) * cst + static_cast<int64_t>(r) * NMAX;
#pragma unroll
    for (int v = 0; v < NMAX / 4; ++v) {
      float o[4], oc[4];
      ld4_io(bt + 4 * v, o);  // rows are aligned to four elements
      ld4_io(ct + 4 * v, oc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bv[t][4 * v + e] = o[e];
        cvv[t][4 * v + e] = oc[e];
      }
    }
  }
  if (c >= d) return;
  const int64_t slot = static_cast<int64_t>(Bs) * d;  // ring slot stride of x and dt
  const int64_t rc = static_cast<int64_t>(r) * d + c;
  float h[NMAX], cs[kKS], xs[W], ds[W], zv[W];
  const float4* srow = reinterpret_cast<const float4*>(ssm_state + rc * NMAX);
#pragma unroll
  for (int v = 0; v < NMAX / 4; ++v) {
    const float4 t = srow[v];
    h[4 * v] = t.x; h[4 * v + 1] = t.y; h[4 * v + 2] = t.z; h[4 * v + 3] = t.w;
  }
#pragma unroll
  for (int m = 0; m < kKS; ++m) cs[m] = conv_state[rc * kKS + m];
#pragma unroll
  for (int t = 0; t < W; ++t) {  // slots past k1 are not read
    xs[t] = (t <= k1) ? ld_io(x_ring, t * slot + rc) : 0.0f;
    ds[t] = (t <= k1) ? ld_io(dt_ring, t * slot + rc) : 0.0f;
    zv[t] = (t >= k0 && t <= k1) ? ld_io(z, (t - k0) * zs + rc) : 0.0f;
  }
  const float4 w = reinterpret_cast<const float4*>(conv_w)[c];
  const float cb = conv_b[c], dtb = dt_bias[c], Dc = D[c];
  float A2[NMAX];
#pragma unroll
  for (int v = 0; v < NMAX / 4; ++v) {
    const float4 al = reinterpret_cast<const float4*>(A_log + static_cast<int64_t>(c) * NMAX)[v];
    A2[4 * v] = -exp2_hw(al.x * kLog2e) * kLog2e;
    A2[4 * v + 1] = -exp2_hw(al.y * kLog2e) * kLog2e;
    A2[4 * v + 2] = -exp2_hw(al.z * kLog2e) * kLog2e;
    A2[4 * v + 3] = -exp2_hw(al.w * kLog2e) * kLog2e;
  }
  // X(m) = x of window step m (m >= 0) or checkpoint conv entry 3+m (m < 0)
  auto X = [&](int m) -> float { return m >= 0 ? xs[m] : cs[kKS + m]; };
#pragma unroll
  for (int t = 0; t < W; ++t) {
    if (t > k1) break;  // k0, k1 and cstep are uniform
    float xc = cb;
    xc = __builtin_fmaf(w.x, X(t - 3), xc);
    xc = __builtin_fmaf(w.y, X(t - 2), xc);
    xc = __builtin_fmaf(w.z, X(t - 1), xc);
    xc = __builtin_fmaf(w.w, xs[t], xc);
    const float u = silu(xc);
    const float delta = softplus(ds[t] + dtb);
    const float du = delta * u;
#pragma unroll
    for (int n = 0; n < NMAX; ++n) {
      const float a = exp2_hw(delta * A2[n]);
      h[n] = __builtin_fmaf(a, h[n], du * bv[t][n]);
    }
    if (t >= k0) {
      // readout, summed as the four-lane decode sums it: per group of four entries in
      // order, then (g0 + g1) + (g2 + g3)
      float g[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        g[v] = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) g[v] = __builtin_fmaf(h[4 * v + e], cvv[t][4 * v + e], g[v]);
      }
      const float yp = (g[0] + g[1]) + (g[2] + g[3]);
      st_io(y, (t - k0) * ys + rc, __builtin_fmaf(Dc, u, yp) * silu(zv[t]));
    }
    if (t == cstep) {  // the state after step t becomes the checkpoint
      float* so = ssm_state + rc * NMAX;
#pragma unroll
      for (int n = 0; n < NMAX; ++n) nt_store(h[n], so + n);
#pragma unroll
      for (int m = 0; m < kKS; ++m) conv_state[rc * kKS + m] = X(t - 2 + m);  // [X(t-2), X(t-1), X(t)]
    }
  }
}

}  // namespace mm
