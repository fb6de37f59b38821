// Decode kernels: one token for each of Bs rows, state updated in place.
#pragma once

#include "mm_device.h"

namespace mm {

typedef float f32x2_lo __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_lo __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_lo __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_lo __attribute__((ext_vector_type(2)));
typedef float f32x4_lo __attribute__((ext_vector_type(4)));
constexpr int kRpStride = 20;  // floats per channel row of the replay's LDS tile (16 + 4: rows 4 banks apart)

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
// direction, with nontemporal loads and stores (it is not reused by this kernel).  In a
// stream of back-to-back steps the nontemporal loads are the faster choice (measured at batch
// 256, d_inner 8192: 61.8 against 67.7 us per step in a HIP graph), though a single step
// after a cache flush is about 5% slower with them.  The readout is summed across
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
    for (int e = 0; e < 4; ++e) h[i][e] = nt_load(srow + e);
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
  const float cbv = conv_b[c], dtbv = dt_bias[c], Dv = D[c];
  // Every load of the step in flight together (the four rows' state, B and C, the own row's conv
  // state and inputs, the channel's parameters), consumed by empty asm statements: one wait for
  // all of them here.  Left to itself the compiler issued the later rows' state loads only as
  // earlier ones were consumed (reusing their registers), two or three round trips to memory
  // per step (63.0 -> 60.8 us per flushed step at batch 256, d_inner 8192).
  {
    f32x4_lo hv[G], bv[G], cv[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      hv[i] = f32x4_lo{h[i][0], h[i][1], h[i][2], h[i][3]};
      bv[i] = f32x4_lo{bq[i][0], bq[i][1], bq[i][2], bq[i][3]};
      cv[i] = f32x4_lo{cq[i][0], cq[i][1], cq[i][2], cq[i][3]};
    }
    const f32x4_lo ow = {win[0], win[1], win[2], xv};
    const f32x4_lo wv = {w.x, w.y, w.z, w.w};
    const f32x4_lo av = {al.x, al.y, al.z, al.w};
    const f32x4_lo pv = {zv, dtv, cbv, dtbv};
    asm volatile("" ::"v"(ow), "v"(wv), "v"(av), "v"(pv), "v"(Dv));
    if constexpr (G == 4)
      asm volatile("" ::"v"(hv[0]), "v"(hv[1]), "v"(hv[2]), "v"(hv[3]), "v"(bv[0]), "v"(bv[1]), "v"(bv[2]),
                   "v"(bv[3]), "v"(cv[0]), "v"(cv[1]), "v"(cv[2]), "v"(cv[3]));
    else if constexpr (G == 2)
      asm volatile("" ::"v"(hv[0]), "v"(hv[1]), "v"(bv[0]), "v"(bv[1]), "v"(cv[0]), "v"(cv[1]));
    else
      asm volatile("" ::"v"(hv[0]), "v"(bv[0]), "v"(cv[0]));
  }
  const float alv[4] = {al.x, al.y, al.z, al.w};
  float A2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) A2[e] = -exp2_hw(alv[e] * kLog2e) * kLog2e;
  float xc = cbv;
  xc = __builtin_fmaf(w.x, win[0], xc);
  xc = __builtin_fmaf(w.y, win[1], xc);
  xc = __builtin_fmaf(w.z, win[2], xc);
  xc = __builtin_fmaf(w.w, xv, xc);
  const float u = silu(xc);
  const float delta = softplus(dtv + dtbv);
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
    st_io(y, orc, __builtin_fmaf(Dv, u, ypo) * silu(zv));
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
// scalar unit; the block's checkpoint rows, one contiguous run, move between memory and
// an LDS tile in coalesced 16-byte pieces, and each lane takes its channel's 16 entries
// from the tile.  The per-step arithmetic stays in one lane, as in the eager step's
// order (a layout of several lanes per channel spent its time on the exchanges).
// W <= 4, N = 16.
// Window steps 0..k1 are taken from the checkpoint; steps k0..k1 write their output
// (z, C and y of step t at slot t - k0 of the z/C/y arrays, slot strides zs, cs_, ys);
// if 0 <= cstep <= k1 the state after step cstep becomes the checkpoint.
//
// Dual-precision checkpoint (the same page: a low-precision checkpoint serves the outputs of
// most steps, a higher-precision one the recurrent updates): with LO, the checkpoint is read
// from its bf16 copy (ssm_lo [Bs][d][16], conv_lo [Bs][d][4], entry 3 unused), 40 bytes per
// (row, channel) instead of 76; such a call commits nothing.  A committing call reads the
// fp32 checkpoint and, when ssm_lo_out is given, also writes the new checkpoint's bf16 copy
// (rounded to nearest even).
template <typename IO, bool LO>
__global__ void __launch_bounds__(kBlock) k_decode_replay(
    const IO* __restrict__ x_ring, const IO* __restrict__ dt_ring, const IO* __restrict__ B_ring,
    const IO* __restrict__ z, const IO* __restrict__ C, const float* __restrict__ A_log,
    const float* __restrict__ D, const float* __restrict__ dt_bias, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, float* __restrict__ conv_state, float* __restrict__ ssm_state,
    IO* __restrict__ y, int Bs, int d, int k0, int k1, int cstep, int64_t zs, int64_t cst, int64_t ys,
    const uint16_t* __restrict__ ssm_lo, const uint16_t* __restrict__ conv_lo, uint16_t* __restrict__ ssm_lo_out,
    uint16_t* __restrict__ conv_lo_out) {
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
  // Threads past d compute on channel d - 1 and store nothing (every thread takes the block's
  // barriers).
  const bool live = c < d;
  const int cl = live ? c : d - 1;
  const int64_t slot = static_cast<int64_t>(Bs) * d;  // ring slot stride of x and dt
  const int64_t rc = static_cast<int64_t>(r) * d + cl;
  // The block's checkpoint rows are one contiguous run of its channels' states: the threads load
  // it together in 16-byte pieces (consecutive lanes, consecutive pieces) and pass it through an
  // LDS tile [256 channels][kRpStride floats], from which each lane takes its own channel (a lane
  // loading its own 64 bytes would make every load instruction touch 64 separate pieces).  The
  // committing step returns the new state the same way.
  __shared__ __align__(16) float tile[kBlock * kRpStride];
  const int c0 = static_cast<int>(blockIdx.x % nb) * kBlock;
  const int nvalid = d - c0 < kBlock ? d - c0 : kBlock;  // the block's channels
  const int64_t rc0 = static_cast<int64_t>(r) * d + c0;
  constexpr int kPieces = LO ? NMAX / 8 : NMAX / 4;  // 16-byte pieces per channel
  u32x4_lo sp[kPieces];
#pragma unroll
  for (int k = 0; k < kPieces; ++k) {
    int i = static_cast<int>(threadIdx.x) + kBlock * k;  // piece i: channel i / kPieces
    if (i >= nvalid * kPieces) i = nvalid * kPieces - 1;  // (a valid piece, loaded again)
    sp[k] = LO ? reinterpret_cast<const u32x4_lo*>(ssm_lo + rc0 * NMAX)[i]
               : reinterpret_cast<const u32x4_lo*>(ssm_state + rc0 * NMAX)[i];
  }
  uint32_t cw[kKS];  // the conv entries: 3 fp32, or with LO their bf16 copy in cw[0], cw[1]
  if (LO) {
    const uint2 c2 = reinterpret_cast<const uint2*>(conv_lo)[rc];
    cw[0] = c2.x; cw[1] = c2.y; cw[2] = 0u;
  } else {
#pragma unroll
    for (int m = 0; m < kKS; ++m) cw[m] = __float_as_uint(conv_state[rc * kKS + m]);
  }
  uint32_t xr[W], dr[W], zr[W];  // raw io words
  // Every slot index is clamped into the call's range instead of skipping loads: the loads are
  // then unconditional and all in flight together (a load under a branch is waited for before
  // the next one issues).  Values of steps past k1 and z of steps before k0 are never used.
#pragma unroll
  for (int t = 0; t < W; ++t) {
    const int tx = t <= k1 ? t : k1;
    const int tz = (t >= k0 ? (t <= k1 ? t : k1) : k0) - k0;
    xr[t] = ld_io_raw(x_ring, tx * slot + rc);
    dr[t] = ld_io_raw(dt_ring, tx * slot + rc);
    zr[t] = ld_io_raw(z, tz * zs + rc);
  }
  const float4 w = reinterpret_cast<const float4*>(conv_w)[cl];
  const float cb = conv_b[cl], dtb = dt_bias[cl], Dc = D[cl];
  float4 al[NMAX / 4];
#pragma unroll
  for (int v = 0; v < NMAX / 4; ++v) al[v] = reinterpret_cast<const float4*>(A_log + static_cast<int64_t>(cl) * NMAX)[v];
  // Every value loaded above is consumed here at once (an empty asm), so all the loads are in
  // flight together and the lane waits once: otherwise the compiler sinks the ring loads into
  // the steps that use them, behind the first step's waits (more round trips to memory).
  asm volatile("" ::"v"(sp[0]), "v"(sp[1]), "v"(sp[kPieces - 1]), "v"(cw[0]), "v"(cw[1]), "v"(cw[2]), "v"(xr[0]),
               "v"(xr[1]), "v"(xr[2]), "v"(xr[3]), "v"(dr[0]), "v"(dr[1]), "v"(dr[2]), "v"(dr[3]), "v"(zr[0]),
               "v"(zr[1]), "v"(zr[2]), "v"(zr[3]));
  asm volatile("" ::"v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w), "v"(cb), "v"(dtb), "v"(Dc), "v"(al[0].x), "v"(al[0].y),
               "v"(al[0].z), "v"(al[0].w), "v"(al[1].x), "v"(al[1].y), "v"(al[1].z), "v"(al[1].w), "v"(al[2].x),
               "v"(al[2].y), "v"(al[2].z), "v"(al[2].w), "v"(al[3].x), "v"(al[3].y), "v"(al[3].z), "v"(al[3].w));
  // the checkpoint pieces into the tile, then this lane's channel out of it
#pragma unroll
  for (int k = 0; k < kPieces; ++k) {
    const int i = static_cast<int>(threadIdx.x) + kBlock * k;
    if (i < nvalid * kPieces)
      *reinterpret_cast<u32x4_lo*>(tile + (i / kPieces) * kRpStride + (i % kPieces) * 4) = sp[k];
  }
  __syncthreads();
  uint32_t hw[NMAX];
#pragma unroll
  for (int k = 0; k < kPieces; ++k) {
    const u32x4_lo v = *reinterpret_cast<const u32x4_lo*>(tile + static_cast<int>(threadIdx.x) * kRpStride + 4 * k);
    hw[4 * k] = v[0]; hw[4 * k + 1] = v[1]; hw[4 * k + 2] = v[2]; hw[4 * k + 3] = v[3];
  }
  float h[NMAX], cs[kKS], xs[W], ds[W], zv[W];
#pragma unroll
  for (int t = 0; t < W; ++t) {
    xs[t] = io_value<IO>(xr[t]);
    ds[t] = io_value<IO>(dr[t]);
    zv[t] = io_value<IO>(zr[t]);
  }
  if (LO) {  // bf16 -> fp32: the value in the upper half of the word (words 0..7 hold the state)
#pragma unroll
    for (int i = 0; i < NMAX / 2; ++i) {
      h[2 * i] = __uint_as_float(hw[i] << 16);
      h[2 * i + 1] = __uint_as_float(hw[i] & 0xFFFF0000u);
    }
    cs[0] = __uint_as_float(cw[0] << 16);
    cs[1] = __uint_as_float(cw[0] & 0xFFFF0000u);
    cs[2] = __uint_as_float(cw[1] << 16);
  } else {
#pragma unroll
    for (int n = 0; n < NMAX; ++n) h[n] = __uint_as_float(hw[n]);
#pragma unroll
    for (int m = 0; m < kKS; ++m) cs[m] = __uint_as_float(cw[m]);
  }
  float A2[NMAX];
#pragma unroll
  for (int v = 0; v < NMAX / 4; ++v) {
    A2[4 * v] = -exp2_hw(al[v].x * kLog2e) * kLog2e;
    A2[4 * v + 1] = -exp2_hw(al[v].y * kLog2e) * kLog2e;
    A2[4 * v + 2] = -exp2_hw(al[v].z * kLog2e) * kLog2e;
    A2[4 * v + 3] = -exp2_hw(al[v].w * kLog2e) * kLog2e;
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
      if (live) st_io(y, (t - k0) * ys + rc, __builtin_fmaf(Dc, u, yp) * silu(zv[t]));
    }
    if (!LO && t == cstep) {  // the state after step t becomes the checkpoint (uniform branch)
      // this lane's channel into its own tile row (the row it read the checkpoint from), then the
      // block's rows out together in 16-byte pieces, with their bf16 copy when one is kept
#pragma unroll
      for (int k = 0; k < NMAX / 4; ++k)
        *reinterpret_cast<f32x4_lo*>(tile + static_cast<int>(threadIdx.x) * kRpStride + 4 * k) =
            f32x4_lo{h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]};
      if (live) {
#pragma unroll
        for (int m = 0; m < kKS; ++m) conv_state[rc * kKS + m] = X(t - 2 + m);  // [X(t-2), X(t-1), X(t)]
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NMAX / 4; ++k) {
        const int i = static_cast<int>(threadIdx.x) + kBlock * k;  // piece i: channel i / 4
        if (i < nvalid * 4) {
          const f32x4_lo v = *reinterpret_cast<const f32x4_lo*>(tile + (i / 4) * kRpStride + (i % 4) * 4);
          nt_store(v, reinterpret_cast<f32x4_lo*>(ssm_state + rc0 * NMAX) + i);
          if (ssm_lo_out != nullptr) {
            const f32x2_lo p0 = {v[0], v[1]}, p1 = {v[2], v[3]};
            nt_store(u32x2_lo{__builtin_bit_cast(uint32_t, __builtin_convertvector(p0, bf16x2_lo)),
                              __builtin_bit_cast(uint32_t, __builtin_convertvector(p1, bf16x2_lo))},
                     reinterpret_cast<u32x2_lo*>(ssm_lo_out + rc0 * NMAX) + i);
          }
        }
      }
      if (ssm_lo_out != nullptr && live) {
        const f32x2_lo c01 = {X(t - 2), X(t - 1)}, c2z = {X(t), 0.0f};
        nt_store(u32x2_lo{__builtin_bit_cast(uint32_t, __builtin_convertvector(c01, bf16x2_lo)),
                          __builtin_bit_cast(uint32_t, __builtin_convertvector(c2z, bf16x2_lo))},
                 reinterpret_cast<u32x2_lo*>(conv_lo_out) + rc);
      }
    }
  }
}

// The bf16 copy of a replay checkpoint (rounded to nearest even): one thread per (row,
// channel) converts its 16 state entries and 3 conv entries (entry 3 of conv_lo is zero).
__global__ void __launch_bounds__(kBlock) k_checkpoint_lo(const float* __restrict__ conv_state,
                                                         const float* __restrict__ ssm_state,
                                                         uint16_t* __restrict__ conv_lo, uint16_t* __restrict__ ssm_lo,
                                                         int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= n) return;
  const float4* s4 = reinterpret_cast<const float4*>(ssm_state + i * 16);
  uint4* o4 = reinterpret_cast<uint4*>(ssm_lo + i * 16);
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const float4 a = s4[2 * v], b = s4[2 * v + 1];
    const f32x2_lo p0 = {a.x, a.y}, p1 = {a.z, a.w}, p2 = {b.x, b.y}, p3 = {b.z, b.w};
    o4[v] = make_uint4(__builtin_bit_cast(uint32_t, __builtin_convertvector(p0, bf16x2_lo)),
                       __builtin_bit_cast(uint32_t, __builtin_convertvector(p1, bf16x2_lo)),
                       __builtin_bit_cast(uint32_t, __builtin_convertvector(p2, bf16x2_lo)),
                       __builtin_bit_cast(uint32_t, __builtin_convertvector(p3, bf16x2_lo)));
  }
  const f32x2_lo c01 = {conv_state[i * kKS], conv_state[i * kKS + 1]}, c2z = {conv_state[i * kKS + 2], 0.0f};
  reinterpret_cast<uint2*>(conv_lo)[i] = make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(c01, bf16x2_lo)),
                                                    __builtin_bit_cast(uint32_t, __builtin_convertvector(c2z, bf16x2_lo)));
}

}  // namespace mm
