// The input-dependent projections ahead of the scan, on the matrix cores (gfx950 MFMA), in
// the layer order of the TensorRT Mamba tensor-parallel builder (_add_mamba_tp_layer):
//   u     = SiLU(conv_b + sum_k conv_w[k] * window[k])        (the mixer's conv activation)
//   [dt_in | B | C] = u x w_x,  w_x = [w_dt_in | w_B | w_C]   ([d, R + 2N], input-major)
//   dt    = dt_in x w_dt_out                                   ([R, d])
// dt is the dt-projection output before dt_proj_bias, which the mixer core adds (dt_bias)
// before its softplus; B and C are the scan's input and readout vectors.  Both products are
// dense contractions, so they run as bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32
// accumulation.  The weights and x are bf16 already; the computed operands u and dt_in are
// split into a bf16 high part and a bf16 low part (v = hi + lo to 2^-16 relative) and enter
// two MFMAs each, so the products carry fp32-quality operands -- the builder computes in
// fp32 -- and the only rounding of note is that of the outputs to bf16.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies row l % 16 of A and
// column l % 16 of B, each with the 8 consecutive K indices 8 (l / 16) .. 8 (l / 16) + 7; the
// result leaves rows 4 (l / 16) .. 4 (l / 16) + 3 of column l % 16 in lane l.
//
// Memory access: the vector L1 looks up one cache line per 16-lane quarter of a wave and line,
// so operand loads in the MFMA layout (16 lanes = 16 rows of a row-major matrix) cost 16
// lookups per quarter.  Hence:
//  * k_proj_pack re-lays the weights once per call in the operands' own order, w_x as
//    [K step][K group][column][8] and w_dt as [K step][K group][channel][8], zero-padded to
//    Pp = P rounded up to 16 columns, dk = d rounded up to 32, Rp = R rounded up to 32: a
//    quarter wave then reads 256 contiguous bytes;
//  * x and the conv parameters are read with row-contiguous loads into a per-wave LDS tile and
//    taken from there in the operand layout.
// k_project: a workgroup of 8 waves takes 32 tokens (two 16-token row tiles):
//  1. wave w takes row tile w % 2 and the K quarter w / 2 of d: per K step of 32 channels it
//     stages the x rows t-3 .. t of its 16 tokens and the 32 channels' conv parameters, each
//     lane computes u for its token and 8 channels (rows before a sequence from the initial
//     conv state), and the wave issues the MFMAs of all output columns.  Splitting K four ways
//     gives four waves per SIMD at the 130m shape (a wave per 16 tokens alone would give one);
//  2. the quarters' accumulators are summed through LDS in quarter order (deterministic); B and
//     C leave from the sums, dt_in goes to LDS as bf16 high and low parts;
//  3. the eight waves split dt's 16-channel tiles: A = dt_in from LDS (both row tiles), B =
//     the re-laid w_dt.
#pragma once

#include <type_traits>

#include "mm_device.h"

namespace mm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kProjTokens = 32;  // tokens per workgroup
constexpr int kProjMaxP = 288;   // R + 2N, rounded up to 16
constexpr int kProjMaxR = 256;
constexpr int kProjK = 32;       // K per MFMA
constexpr int kProjWaves = 8;
constexpr int kProjThreads = kProjWaves * kWave;
constexpr int kProjRowTiles = kProjTokens / 16;          // 16-token row tiles per workgroup
constexpr int kProjKSplit = kProjWaves / kProjRowTiles;  // K quarters
constexpr int kProjXRows = 16 + kKS;                     // staged x rows per wave: t-3 .. t+15
constexpr int kProjXStride = kProjK + 8;                 // bf16 per staged row (padded)

__device__ __forceinline__ uint16_t bf16_bits(float v) {
  const __bf16 b = static_cast<__bf16>(v);
  return __builtin_bit_cast(uint16_t, b);
}

// wxP[ks][g][j][e] = w_x[32 ks + 8 g + e][j] (zero past P and past d);
// wdtP[kk][g][c][e] = w_dt[32 kk + 8 g + e][c] (zero past R)
__global__ void __launch_bounds__(kBlock) k_proj_pack(const uint16_t* __restrict__ w_x,
                                                      const uint16_t* __restrict__ w_dt, uint16_t* __restrict__ wxP,
                                                      uint16_t* __restrict__ wdtP, int d, int P, int Pp, int dk, int R,
                                                      int Rp) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t nx = static_cast<int64_t>(Pp) * dk;
  if (i < nx) {
    const int e = static_cast<int>(i & 7);
    const int64_t q = i >> 3;  // (ks * 4 + g) * Pp + j
    const int j = static_cast<int>(q % Pp);
    const int k = static_cast<int>(q / Pp) * 8 + e;
    wxP[i] = (j < P && k < d) ? w_x[static_cast<int64_t>(k) * P + j] : static_cast<uint16_t>(0);
    return;
  }
  const int64_t i2 = i - nx;
  if (i2 >= static_cast<int64_t>(d) * Rp) return;
  const int e = static_cast<int>(i2 & 7);
  const int64_t q = i2 >> 3;  // (kk * 4 + g) * d + c
  const int c = static_cast<int>(q % d);
  const int r = static_cast<int>(q / d) * 8 + e;
  wdtP[i2] = r < R ? w_dt[static_cast<int64_t>(r) * d + c] : static_cast<uint16_t>(0);
}

// LDS (dynamic, sized per call): a first region that holds, in turn, per wave two staging
// buffers (double-buffered across K steps), each the x rows [kProjXRows][kProjXStride] bf16 and
// conv parameters [40] float4 (32 channels' weights, then 8 x 4 biases); the K quarters' partial
// accumulators [row tile][quarter 1..3][Pp / 16][64 lanes] floatx4; and per wave the dt output
// tile.  After it, dt_in's high and low bf16 parts [kProjTokens][Rp + 8] (rows padded to keep
// the 16-byte reads aligned).
constexpr int kProjOStride = 32 + 8;  // bf16 per row of a wave's dt output tile [32 tokens][32 channels]
constexpr size_t kProjStageBytes = kProjXRows * kProjXStride * 2 + 40 * 16;  // one staging buffer
constexpr size_t kProjWaveBytes = (2 * kProjStageBytes > kProjTokens * kProjOStride * 2)
                                      ? 2 * kProjStageBytes
                                      : kProjTokens * kProjOStride * 2;
__host__ __device__ inline size_t proj_red_bytes(int Pp) {
  return static_cast<size_t>(kProjRowTiles) * (kProjKSplit - 1) * (Pp / 16) * kWave * 16;
}
__host__ __device__ inline size_t proj_region_bytes(int Pp) {
  const size_t a = kProjWaves * kProjWaveBytes, b = proj_red_bytes(Pp);
  return a > b ? a : b;
}
inline size_t proj_lds_bytes(int Pp, int Rp) {
  return proj_region_bytes(Pp) + static_cast<size_t>(2) * kProjTokens * (Rp + 8) * 2;
}

// split v into bf16 parts with hi + lo = v to about 2^-16 relative
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(v);
  lo = static_cast<__bf16>(v - static_cast<float>(hi));
}

// NT = Pp / 16 output column tiles of the first product, at most MAXNT (6, 12 or 18: the
// accumulators of MAXNT tiles stay in registers); Rp / 32 K steps of the second, at most MAXKR
// (2, 4 or 8: the w_dt operands of a tile pair stay in registers)
template <int MAXNT, int MAXKR>
__global__ void __launch_bounds__(kProjThreads) __attribute__((amdgpu_waves_per_eu(MAXNT <= 6 ? 4 : (MAXNT <= 12 ? 3 : 2)))) k_project(
    const uint16_t* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    const int32_t* __restrict__ cu, const float* __restrict__ conv_state, const uint16_t* __restrict__ wxP,
    const uint16_t* __restrict__ wdtP, uint16_t* __restrict__ dt, uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    int S, int64_t T, int d, int N, int R, int dk, int Rp, int NT) {
  constexpr int kMaxNT = MAXNT;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Pp = NT * 16;
  const int dstride = Rp + 8;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);  // wave-uniform
  auto xt = [&](int b) {  // staged x rows of buffer b, [kProjXRows][kProjXStride]
    return reinterpret_cast<uint16_t*>(smem + w * kProjWaveBytes + b * kProjStageBytes);
  };
  auto cpar = [&](int b) {  // conv parameters of buffer b, [40]
    return reinterpret_cast<float4*>(smem + w * kProjWaveBytes + b * kProjStageBytes + kProjXRows * kProjXStride * 2);
  };
  floatx4_t* red = reinterpret_cast<floatx4_t*>(smem);  // over the staging buffers, after the K loops
  uint16_t* dh = reinterpret_cast<uint16_t*>(smem + proj_region_bytes(Pp));
  uint16_t* dl = dh + static_cast<size_t>(kProjTokens) * dstride;
  const int mt = w % kProjRowTiles;  // row tile
  const int kq = w / kProjRowTiles;  // K quarter
  const int row = lane & 15;  // token row within the tile (A operand), column within a tile (B operand)
  const int kg = lane >> 4;   // 8-wide K group
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kProjTokens;
  const int64_t tw = t0 + mt * 16;  // the wave's first token
  const int64_t d64 = d;

  // this lane's token and its sequence
  int64_t t = tw + row;
  if (t >= T) t = T - 1;  // rows past T compute on a valid token and store nothing
  const int s = seq_of(cu, S, t);
  const int64_t back = t - cu[s];  // tokens of the sequence before t
  const float* cs = conv_state + static_cast<int64_t>(s) * d64 * kKS;

  floatx4_t acc[kMaxNT];
#pragma unroll
  for (int j = 0; j < kMaxNT; ++j) acc[j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // this lane's staging loads: 16 bytes (part lane % 4) of staged row lane / 4, and of row
  // 16 + lane / 4 for lanes < 12; the conv parameters for lanes < 40
  const int q4 = lane & 3;
  auto xsrc = [&](int rr) {  // staged row rr holds token tw - 3 + rr (clamped into 0 .. T-1)
    int64_t tok = tw - kKS + rr;
    tok = tok < 0 ? 0 : (tok >= T ? T - 1 : tok);
    return x + tok * d64 + q4 * 8;
  };
  const uint16_t* xa = xsrc(lane >> 2);
  const uint16_t* xb = xsrc(16 + ((lane >> 2) < kKS ? (lane >> 2) : 0));

  const int nks = dk / kProjK;
  const int ks0 = kq * nks / kProjKSplit, ks1 = (kq + 1) * nks / kProjKSplit;
  // A wave holding one of a sequence's first three tokens takes the loop that reads the conv
  // state; every other wave runs the loop without that branch.
  // the staging loads of K step ks: x rows and conv parameters (channels past d read valid
  // ones; their u is 0), issued one step ahead of their use
  uint4 pva, pvb;  // prefetched staging data
  float4 pvp;
  auto step_load = [&](int ks) {
    const int c0 = ks * kProjK;
    const int cx = c0 + q4 * 8 < d ? c0 : d - 8 - q4 * 8;
    pva = *reinterpret_cast<const uint4*>(xa + cx);
    pvb = *reinterpret_cast<const uint4*>(xb + cx);
    const int pc = lane < kProjK ? c0 + lane : c0 + (lane - kProjK) * 4;  // weight channel, or first bias
    const float* psrc = lane < kProjK ? conv_w + static_cast<int64_t>(pc < d ? pc : d - 1) * kK
                                      : conv_b + (pc < d ? pc : d - 4);
    pvp = *reinterpret_cast<const float4*>(psrc);
  };
  auto stage_write = [&](int b) {
    *reinterpret_cast<uint4*>(xt(b) + (lane >> 2) * kProjXStride + q4 * 8) = pva;
    if (lane < 4 * kKS) *reinterpret_cast<uint4*>(xt(b) + (16 + (lane >> 2)) * kProjXStride + q4 * 8) = pvb;
    if (lane < 40) cpar(b)[lane] = pvp;
  };
  // Per K step: the staging buffer of step ks was written at the end of the previous step (its
  // global loads issued a step before that), so neither the loads nor the LDS round trip stall
  // the step's arithmetic.
  auto kloop = [&](auto state) {
    constexpr bool STATE = decltype(state)::value;
    step_load(ks0 < ks1 ? ks0 : 0);
    stage_write(0);
    step_load(ks0 + 1 < ks1 ? ks0 + 1 : ks0);
    for (int ks = ks0; ks < ks1; ++ks) {
      const int c0 = ks * kProjK;
      const int b = (ks - ks0) & 1;
      // this step's w_x operands, used after the u arithmetic
      uint4 wb[kMaxNT];
      const uint16_t* wk = wxP + (static_cast<int64_t>(ks * 4 + kg) * Pp + row) * 8;
#pragma unroll
      for (int j = 0; j < kMaxNT; ++j)
        if (j < NT) wb[j] = *reinterpret_cast<const uint4*>(wk + j * 16 * 8);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's staging writes before its reads
      const int c = c0 + kg * 8;
      const bool live = c < d;
      float xr[4][8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint4 v = *reinterpret_cast<const uint4*>(xt(b) + (row + r) * kProjXStride + kg * 8);
        const uint32_t pv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xr[r][2 * e] = __uint_as_float(pv[e] << 16);
          xr[r][2 * e + 1] = __uint_as_float(pv[e] & 0xFFFF0000u);
        }
      }
      if (STATE && back < kKS && live) {  // older rows from the initial conv state, or 0 before it
#pragma unroll
        for (int r = 0; r < kKS; ++r) {
          const int64_t col = back - (3 - r) + kKS;
          if (back - (3 - r) < 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) xr[r][e] = col >= 0 ? cs[static_cast<int64_t>(c + e) * kKS + col] : 0.0f;
          }
        }
      }
      const float4 b0 = cpar(b)[kProjK + kg * 2], b1 = cpar(b)[kProjK + kg * 2 + 1];
      const float bias[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      bf16x8_t ua, ul;  // u's high and low parts
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 wv = cpar(b)[kg * 8 + e];
        float xc = bias[e];
        xc = __builtin_fmaf(wv.x, xr[0][e], xc);
        xc = __builtin_fmaf(wv.y, xr[1][e], xc);
        xc = __builtin_fmaf(wv.z, xr[2][e], xc);
        xc = __builtin_fmaf(wv.w, xr[3][e], xc);
        __bf16 hi, lo;
        split_bf16(live ? silu(xc) : 0.0f, hi, lo);
        ua[e] = hi;
        ul[e] = lo;
      }
      // the high parts over all column tiles, then the low parts: consecutive MFMAs are independent
#pragma unroll
      for (int j = 0; j < kMaxNT; ++j)
        if (j < NT) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, __builtin_bit_cast(bf16x8_t, wb[j]), acc[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < kMaxNT; ++j)
        if (j < NT) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ul, __builtin_bit_cast(bf16x8_t, wb[j]), acc[j], 0, 0, 0);
      if (ks + 1 < ks1) stage_write(b ^ 1);  // step ks + 1; that buffer was last read in step ks - 1
      step_load(ks + 2 < ks1 ? ks + 2 : ks);  // near the end a harmless repeat
    }
  };
  if (__any(back < kKS)) kloop(std::true_type{});
  else kloop(std::false_type{});

  // sum the K quarters in order: quarters 1..3 leave their accumulators in LDS, quarter 0 adds
  // them (fully unrolled loops with guards: a loop the compiler cannot unroll would index acc at
  // run time and move it to scratch memory)
  auto red_at = [&](int q, int j) {
    return red + ((static_cast<size_t>(mt) * (kProjKSplit - 1) + (q - 1)) * NT + j) * kWave + lane;
  };
  __syncthreads();  // every wave's K loop done: the staging buffers become the partial sums
  if (kq > 0) {
#pragma unroll
    for (int j = 0; j < kMaxNT; ++j)
      if (j < NT) *red_at(kq, j) = acc[j];
  }
  __syncthreads();
  const int P = R + 2 * N;
  if (kq == 0) {
#pragma unroll
    for (int j = 0; j < kMaxNT; ++j) {
      if (j < NT) {
#pragma unroll
        for (int q = 1; q < kProjKSplit; ++q) acc[j] += *red_at(q, j);
        const int col = j * 16 + row;
        // B, C out; dt_in to LDS.  acc[j][i]: token 16 mt + 4 kg + i, output column 16 j + row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tl = mt * 16 + kg * 4 + i;
          const int64_t tg = t0 + tl;
          const float v = acc[j][i];
          if (col < R) {
            __bf16 hi, lo;
            split_bf16(v, hi, lo);
            dh[tl * dstride + col] = __builtin_bit_cast(uint16_t, hi);
            dl[tl * dstride + col] = __builtin_bit_cast(uint16_t, lo);
          } else if (col < P && tg < T) {
            if (col < R + N) B[tg * N + (col - R)] = bf16_bits(v);
            else C[tg * N + (col - R - N)] = bf16_bits(v);
          }
        }
      }
    }
  }
  for (int i = threadIdx.x; i < kProjTokens * (Rp - R); i += kProjThreads) {  // zero K padding of dt_in
    const int tl = i / (Rp - R), r = R + i % (Rp - R);
    dh[tl * dstride + r] = 0;
    dl[tl * dstride + r] = 0;
  }
  __syncthreads();

  // dt = dt_in x w_dt: wave w takes a contiguous run of 16-channel tiles, two at a time; the
  // 32 tokens x 32 channels of a tile pair go through the wave's LDS area so that they leave as
  // 16-byte row pieces (a quarter wave writes four 64-byte row segments)
  constexpr int kMaxKR = MAXKR;
  const int nkr = Rp / kProjK;
  const int ntiles = d / 16;
  const int per_wave = (ntiles + kProjWaves - 1) / kProjWaves;
  const int nt_lo = w * per_wave;
  const int nt_hi = nt_lo + per_wave < ntiles ? nt_lo + per_wave : ntiles;
  uint16_t* ot = reinterpret_cast<uint16_t*>(smem + w * kProjWaveBytes);  // [kProjTokens][kProjOStride]
  // the w_dt operands of a tile pair (a lone last tile is taken twice and stored once), loaded a
  // pair ahead of their use
  bf16x8_t wv[2][kMaxKR];
  auto wdt_load = [&](int nt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ntile = nt + h < nt_hi ? nt + h : nt;
      const int64_t base = static_cast<int64_t>(ntile * 16 + row) * 8;
#pragma unroll
      for (int kk = 0; kk < kMaxKR; ++kk)
        if (kk < nkr)
          wv[h][kk] = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const uint4*>(wdtP + static_cast<int64_t>(kk * 4 + kg) * d * 8 + base));
    }
  };
  if (nt_lo < nt_hi) wdt_load(nt_lo);
  for (int nt = nt_lo; nt < nt_hi; nt += 2) {
    bf16x8_t wc[2][kMaxKR];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kk = 0; kk < kMaxKR; ++kk) wc[h][kk] = wv[h][kk];
    wdt_load(nt + 2 < nt_hi ? nt + 2 : nt);  // on the last pair a harmless repeat
    // four independent accumulations (two tiles x two row tiles), interleaved
    floatx4_t a[2][kProjRowTiles];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int m = 0; m < kProjRowTiles; ++m) a[h][m] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < kMaxKR; ++kk) {
      if (kk < nkr) {
        bf16x8_t ah[kProjRowTiles], al[kProjRowTiles];
#pragma unroll
        for (int m = 0; m < kProjRowTiles; ++m) {
          const size_t o = static_cast<size_t>(m * 16 + row) * dstride + kk * kProjK + kg * 8;
          ah[m] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(dh + o));
          al[m] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(dl + o));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int m = 0; m < kProjRowTiles; ++m) a[h][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], wc[h][kk], a[h][m], 0, 0, 0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int m = 0; m < kProjRowTiles; ++m) a[h][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[m], wc[h][kk], a[h][m], 0, 0, 0);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int m = 0; m < kProjRowTiles; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) ot[(m * 16 + kg * 4 + i) * kProjOStride + h * 16 + row] = bf16_bits(a[h][m][i]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile written before this wave reads it
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int tl = half * 16 + (lane >> 2), part = lane & 3;
      const int64_t tg = t0 + tl;
      const int ch = nt * 16 + part * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(ot + tl * kProjOStride + part * 8);
      if (tg < T && ch < nt_hi * 16) *reinterpret_cast<uint4*>(dt + tg * d64 + ch) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile read before the next pair overwrites it
  }
}

}  // namespace mm
