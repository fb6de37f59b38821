// Device helpers shared by the libmambamix kernels (gfx950, wave64): element I/O,
// hardware transcendentals, SiLU / softplus, the per-channel constants and the
// one-token mixer step of the TensorRT Mamba tensor-parallel builder
// (_add_mamba_tp_layer), and the sequential token loop built on it.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mambamix.h"

namespace mm {

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
// the same in two halves: the raw word as loaded, then its value
__device__ __forceinline__ uint32_t ld_io_raw(const float* p, int64_t i) { return __float_as_uint(p[i]); }
__device__ __forceinline__ uint32_t ld_io_raw(const uint16_t* p, int64_t i) { return p[i]; }
template <typename IO>
__device__ __forceinline__ float io_value(uint32_t raw) {
  return std::is_same<IO, float>::value ? __uint_as_float(raw) : __uint_as_float(raw << 16);
}
__device__ __forceinline__ void st_io(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_io(uint16_t* p, int64_t i, float v) {
  // float32 -> bfloat16 by the hardware conversion (round to nearest even, NaN stays NaN)
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// ---------------------------------------------------------------- scalar-base access
// Global-memory access from a wave-uniform base held as an opaque value in scalar
// registers: the compiler can then neither fold a thread's offset into a 64-bit
// vector address nor split the base into per-thread induction variables, so the
// access takes the scalar-base plus 32-bit vector-offset form (off < 2^32).
template <typename IO>
using gmem = __attribute__((address_space(1))) IO;

// p as an opaque value: the compiler keeps it in scalar registers (it is wave-uniform)
// and cannot reassociate it with a per-thread offset
template <typename P>
__device__ __forceinline__ P sreg(P p) {
  uint64_t v = reinterpret_cast<uint64_t>(p);
  asm volatile("" : "+s"(v));
  return reinterpret_cast<P>(v);
}
template <typename IO>
__device__ __forceinline__ gmem<IO>* sbase(IO* p) {
  return sreg(reinterpret_cast<gmem<IO>*>(reinterpret_cast<uint64_t>(p)));
}
template <typename IO>
__device__ __forceinline__ IO ld_at(gmem<const IO>* p, uint32_t off) {
  return *reinterpret_cast<gmem<const IO>*>(reinterpret_cast<gmem<const char>*>(p) + off);
}
template <typename IO>
__device__ __forceinline__ gmem<IO>* at(gmem<IO>* p, uint32_t off) {
  return reinterpret_cast<gmem<IO>*>(reinterpret_cast<gmem<char>*>(p) + off);
}
__device__ __forceinline__ void st_g(gmem<float>* p, float v) { *p = v; }
__device__ __forceinline__ void st_g(gmem<uint16_t>* p, float v) {
  *p = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // round to nearest even
}

// ---------------------------------------------------------------- math
// v_exp_f32 / v_log_f32 / v_rcp_f32 are the hardware base-2 exponential, base-2
// logarithm and reciprocal (about 1 ulp).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// x * sigmoid(x)
__device__ __forceinline__ float silu(float x) { return x * rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// softplus(v) = log(1 + e^v) = log(u) + log(1 + (1 + e - u) / u) with u = 1 + e rounded to
// float.  u - 1 is exact, and so is the rounding error d = e - (u - 1); log(u) + d differs
// from log(1 + e) by about d * e, under 2^-24 of the result, where log(u) alone would lose
// up to 2^-24 / log(1 + e) relative for small e.  The hardware log2 keeps ~1e-7 relative
// accuracy for u just above 1.  softplus(v) > v everywhere, and past v = 20 it exceeds v by
// less than 2.1e-9: the result is the larger of v and the value at min(v, 20).
__device__ __forceinline__ float softplus(float v) {
  const float e = exp2_hw(fminf(v, 20.0f) * kLog2e);
  const float u = 1.0f + e;
  const float d = e - (u - 1.0f);
  return fmaxf(v, __builtin_fmaf(log2_hw(u), kLn2, d));
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


template <typename T>
__device__ __forceinline__ T nt_load(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void nt_store(T v, T* p) { __builtin_nontemporal_store(v, p); }

}  // namespace mm
