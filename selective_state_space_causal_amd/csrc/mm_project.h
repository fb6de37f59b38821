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
// The two products have opposite memory profiles, so each has a kernel of its own:
//  * k_proj_in reads x (T d bf16, the layer's large input) and writes only R + 2N values per
//    token: a read-streaming kernel.  A workgroup takes 64 tokens: four 16-token row tiles times
//    KP parts of the K range (four parts, 16 waves, up to 160 output columns; two beyond).  Per
//    K stage the workgroup's threads load the x rows its tokens need (t-3 .. t) with
//    row-contiguous 16-byte loads, the stage's conv parameters and its w_x operands, several
//    stages ahead of their use, into a double-buffered LDS area; each lane then computes u for
//    its token and 8 channels per MFMA K step and issues the MFMAs of all output columns.  The parts' sums are added in a fixed order through LDS
//    (deterministic).  B and C go to their outputs, dt_in to the workspace as bf16 high and low
//    parts [T][Rp] (zero past R).
//  * k_proj_dt writes dt (T d bf16) from dt_in (T Rp, small): a write-streaming kernel with
//    one workgroup per 64 tokens x 128 channels, far more workgroups than token tiles.  A wave
//    takes 16 tokens x 128 channels (8 column tiles); its output tile goes through LDS so
//    that it leaves as 16-byte row pieces.
//  * k_proj_pack re-lays the weights once per call in the operands' own order (a quarter wave
//    then reads 256 contiguous bytes): w_x as [K step][K group][column][8], w_dt as
//    [K step][K group][channel][8], zero-padded to Pp = R + 2N rounded up to 16 columns,
//    dk = d rounded up to 32 and Rp = R rounded up to 32.
#pragma once

#include <type_traits>

#include "mm_device.h"

namespace mm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProjMaxP = 288;  // R + 2N, rounded up to 16
constexpr int kProjMaxR = 256;
constexpr int kProjK = 32;      // K per MFMA

// k_proj_in
constexpr int kPinRT = 4;                      // 16-token row tiles per workgroup
constexpr int kPinTok = 16 * kPinRT;           // tokens per workgroup
constexpr int kPinPartThreads = kPinRT * kWave;  // threads per K part (one wave per row tile)
constexpr int kPinXRows = kPinTok + kKS;       // staged x rows: t-3 .. t+63

// Stage geometry of k_proj_in for NT output column tiles.  The K range is split into KP parts,
// each taken by kPinRT waves (one per 16-token row tile): four parts up to 10 column tiles
// (16 waves per workgroup, four per SIMD), two for the widest outputs, whose operands would not
// fit four times in LDS.  A stage holds KC channels (32 with four parts, whose neighbouring
// pieces make whole 128-byte lines of x; 64 with two, a whole line each, or 32 for the widest
// outputs) for each part: x
// [kPinXRows][KC + 8] bf16, the conv weights [KC] float4 and biases [KC] float of those
// channels, the KC / 32 MFMA K steps' w_x operands [K step][4 K groups][Pp][8] bf16, then the
// initial conv state [MS][KC][3] float of the workgroup's first MS sequences (the sequence of
// its first token and the next ones), which the first three tokens of a sequence read in place
// of x rows from before the sequence.
template <int NT>
struct PinGeo {
  static constexpr int Pp = NT * 16;
  static constexpr int KP = NT <= 10 ? 4 : 2;              // K parts
  static constexpr int THREADS = KP * kPinPartThreads;
  static constexpr int KC = KP == 4 ? 32 : (NT <= 12 ? 64 : 32);
  static constexpr int SUB = KC / kProjK;                  // MFMA K steps per stage
  static constexpr int XSTRIDE = KC + 8;                   // bf16 per staged x row
  static constexpr int XP = kPinXRows * KC / 8;            // 16-byte pieces per part: x,
  static constexpr int CWP = KC;                           // conv weights,
  static constexpr int CBP = KC / 4;                       // biases,
  static constexpr int WP = SUB * 4 * Pp;                  // w_x operands,
  static constexpr int CSP = KC * kKS / 4;                 // and per staged sequence, its conv state
  static constexpr int HP0 = XP + CWP + CBP + WP;
  static constexpr int L = (HP0 + kPinPartThreads - 1) / kPinPartThreads;  // loads per thread and stage
  // sequences whose initial conv state is staged: as many (up to 3) as fit in the load slots
  // the other pieces leave free
  static constexpr int MS0 = (L * kPinPartThreads - HP0) / CSP;
  static constexpr int MS = MS0 < 3 ? MS0 : 3;
  static constexpr int HP = HP0 + MS * CSP;
  static constexpr int CWOFF = kPinXRows * XSTRIDE * 2;    // byte offsets within a part
  static constexpr int CBOFF = CWOFF + KC * 16;
  static constexpr int WOFF = CBOFF + KC * 4;
  static constexpr int CSOFF = WOFF + WP * 16;
  static constexpr int HB = CSOFF + MS * KC * kKS * 4;     // bytes per part
  static constexpr int D = KP == 2 && NT <= 6 ? 4 : 1;     // stages in flight
};
template <int NT>
inline size_t pin_lds_bytes_t() {  // two stage buffers (+ a dummy slot); the parts' sums reuse them
  const size_t stage = static_cast<size_t>(2) * PinGeo<NT>::KP * PinGeo<NT>::HB + 16;
  const size_t red = static_cast<size_t>(kPinRT) * NT * kWave * 16;
  return stage > red ? stage : red;
}
// row stride (floats) of k_proj_in's output tile: room for the Pp output columns and for the Rp
// columns that dt_in's pieces read, plus 4 (rows start 4 banks apart)
__host__ __device__ inline int pin_out_stride(int Pp, int Rp) { return (Pp > Rp ? Pp : Rp) + 4; }
inline size_t pin_out_bytes(int Pp, int Rp) { return static_cast<size_t>(kPinTok) * pin_out_stride(Pp, Rp) * 4; }

// k_proj_dt
constexpr int kPdtWaves = 4;
constexpr int kPdtThreads = kPdtWaves * kWave;
constexpr int kPdtCh = 128;                // channels per workgroup (8 column tiles)
constexpr int kPdtTiles = kPdtCh / 16;
constexpr int kPdtOStride = kPdtCh + 8;    // bf16 per row of a wave's output tile (272 bytes)
constexpr int kPdtWGs = 768;               // about three workgroups per CU
// a raw buffer resource's fourth word on gfx9-family targets (32-bit data format, no swizzle,
// range checked against the byte count), and a store offset past any range k_proj_dt makes
// (ranges stay below 16 rows x 2^22 channels x 2 bytes = 2^27)
constexpr int kBufWord3 = 0x00020000;
constexpr int kBufPastEnd = 0x7FFFFFF0;
// cache-policy operand of the buffer stores: nontemporal (dt is written once and not read back
// by this call; the hint saved 5-10% of k_proj_dt's time)
constexpr int kBufNontemporal = 2;
inline size_t pdt_lds_bytes(int KR) {      // the block's w_dt operands, then per wave an output tile
  return static_cast<size_t>(KR) * 4 * kPdtCh * 16 + static_cast<size_t>(kPdtWaves) * 16 * kPdtOStride * 2;
}

__device__ __forceinline__ uint16_t bf16_bits(float v) {
  const __bf16 b = static_cast<__bf16>(v);
  return __builtin_bit_cast(uint16_t, b);
}

// every lane of a 16-lane row reads lane I of the row (DPP row_newbcast:I); float in, float out
template <int I>
__device__ __forceinline__ float pj_bcast(float v) {
  return __builtin_amdgcn_update_dpp(0.0f, v, 0x150 + I, 0xF, 0xF, true);
}
// lane j of a row reads lane j - K (row_shr:K) or j + K (row_shl:K, CTRL 0x100); lanes with no
// such lane in the row get 0
template <int CTRL>
__device__ __forceinline__ uint32_t pj_shift(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
}

// split v into bf16 parts with hi + lo = v to about 2^-16 relative
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(v);
  lo = static_cast<__bf16>(v - static_cast<float>(hi));
}

// One thread per 8-element output piece:
//   wxP[q][j][e] = w_x[8 q + e][j]   (q < dk / 8, j < Pp; zero past P and past d)
//   wdtP[q][c][e] = w_dt[8 q + e][c] (q < Rp / 8, c < d;  zero past R)
// Consecutive threads take consecutive j (or c): their reads of one row are contiguous and
// their 16-byte writes follow one another.
__global__ void __launch_bounds__(kBlock) k_proj_pack(const uint16_t* __restrict__ w_x,
                                                      const uint16_t* __restrict__ w_dt, uint16_t* __restrict__ wxP,
                                                      uint16_t* __restrict__ wdtP, int d, int P, int Pp, int dk, int R,
                                                      int Rp) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t nx = static_cast<int64_t>(dk / 8) * Pp;
  uint16_t v[8];
  if (i < nx) {
    const int q = static_cast<int>(i / Pp), j = static_cast<int>(i % Pp);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 8 * q + e;
      v[e] = (j < P && k < d) ? w_x[static_cast<int64_t>(k) * P + j] : static_cast<uint16_t>(0);
    }
    *reinterpret_cast<uint4*>(wxP + i * 8) = *reinterpret_cast<const uint4*>(v);
    return;
  }
  const int64_t i2 = i - nx;
  if (i2 >= static_cast<int64_t>(Rp / 8) * d) return;
  const int q = static_cast<int>(i2 / d), c = static_cast<int>(i2 % d);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = 8 * q + e;
    v[e] = r < R ? w_dt[static_cast<int64_t>(r) * d + c] : static_cast<uint16_t>(0);
  }
  *reinterpret_cast<uint4*>(wdtP + i2 * 8) = *reinterpret_cast<const uint4*>(v);
}

// [dt_in | B | C] = u x w_x for 64 tokens per workgroup, NT = Pp / 16 output column tiles (a
// template argument: the MFMAs run without guards); nks = dk / 32 MFMA K steps, grouped in
// stages of G::SUB.  Wave w takes row tile w % 4 and K part w / 4 (its share of the K range, as
// laid out below).  Stage g holds, for each part, everything its g-th stage needs (see PinGeo);
// the four waves of a part share its w_x operands.  The workgroup's threads load stage g + D
// into registers while stage g runs; those are the only global loads of the loop (bar the
// conv state of a sequence's first tokens), so waiting for stage g, which was issued first,
// never waits for a later one.  Two LDS stage buffers and one barrier per stage.  LDS
// (dynamic): the stage buffers; after the K loop, one part's accumulators
// [row tile][NT][64 lanes] floatx4.
template <int NT>
__global__ void __launch_bounds__(PinGeo<NT>::THREADS) k_proj_in(
    const uint16_t* __restrict__ x, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    const int32_t* __restrict__ cu, const float* __restrict__ conv_state, const uint16_t* __restrict__ wxP,
    uint16_t* __restrict__ dth, uint16_t* __restrict__ dtl, uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    int S, int64_t T, int d, int N, int R, int Rp, int nks, const float* __restrict__ cs_stage, int cs16) {
  extern __shared__ __align__(16) unsigned char smem[];
  using G = PinGeo<NT>;
  constexpr int Pp = G::Pp, HB = G::HB, HP = G::HP, L = G::L, D = G::D, SUB = G::SUB, KC = G::KC, KP = G::KP;
  constexpr int THREADS = G::THREADS;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int rt = w % kPinRT, h = w / kPinRT;
  const int row = lane & 15;  // token row of the tile (A operand) / column within a tile (B operand)
  const int kg = lane >> 4;   // 8-wide K group
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kPinTok;
  const int64_t d64 = d;
  // The nstg units of KC channels (SUB MFMA K steps each) are grouped by 128-byte line of x: U
  // units per line (two of 32 channels, or one of 64).  The lines split into GR = KP / U
  // consecutive runs of H lines, one per group of U parts, and part q takes unit q % U of each
  // line of run q / U: at stage g, line g of its run.  So the U parts of a group read the two
  // halves of a line at the same stage (one part running through a range of its own would
  // read them one stage apart, and at row strides of a power of two the line is then often
  // gone from the L2: 1.5x the algorithmic HBM bytes at d_inner 4096), while the GR runs keep
  // the workgroup's reads at GR places of the rows (one place, all parts side by side, was 5%
  // slower at d_inner 4096).  The loop runs nst = H stages.
  const int nstg = (nks + SUB - 1) / SUB;
  constexpr int U = KC == 32 ? 2 : 1;  // units per 128-byte line of x
  constexpr int GR = KP / U;           // line streams
  const int nl = (nstg + U - 1) / U;
  const int H = (nl + GR - 1) / GR;    // lines per stream
  auto part_len = [&](int q) {
    const int n = (nstg - q % U + U - 1) / U - (q / U) * H;
    return n < 0 ? 0 : (n < H ? n : H);
  };
  auto part_unit0 = [&](int q) { return (q / U) * H * U + q % U; };
  const int nst = H;
  const int slen = part_len(h);
  const int u0 = part_unit0(h);

  // this lane's token and its sequence (rows past T compute on a valid token and store nothing)
  int64_t t = t0 + rt * 16 + row;
  if (t >= T) t = T - 1;
  const int s = seq_of(cu, S, t);
  const int64_t back = t - cu[s];  // tokens of the sequence before t
  const float* cs = conv_state + static_cast<int64_t>(s) * d64 * kKS;
  // the staged conv states are those of sequences s_first .. s_first + MS - 1, loaded from
  // cs_stage: conv_state when it is 16-byte aligned (cs16), else conv_state rounded down to 16
  // bytes (in the same 16-byte block, so mapped) and not used; a wave whose lanes before the
  // fourth token of their sequence all have theirs staged reads them from LDS, any other wave
  // from global memory
  const int s_first = seq_of(cu, S, t0);
  const bool cs_lds = G::MS > 0 && cs16 != 0 && !__any(back < kKS && s - s_first >= G::MS);
  const int js = s - s_first;

  // The four waves of part q stage part q's pieces, so that a thread's stage index is
  // wave-uniform.  The pieces of thread i of a part are p = i + 256 k (k < L): the x
  // pieces (staged row p / (KC/8) = token t0 - 3 + p / (KC/8) clamped into 0 .. T-1, channels
  // 8 (p % (KC/8)) .. of the stage), KC conv weight rows (float4), KC / 4 pieces of four biases,
  // the staged sequences' conv state pieces (KC channels x 3 floats each, contiguous), and the
  // stage's w_x operand pieces (contiguous; last, so that the load slots that hold only w_x
  // pieces keep wave-uniform bases and steps).  Each piece keeps a 64-bit base, the byte
  // offset of its part's first stage, the bytes it advances per stage and the largest offset it
  // may read: channels past d read clamped, valid addresses (their u is forced to 0); slots past
  // the part's pieces load a valid address and go to a dummy slot.  (Offsets fit 32 bits for
  // d <= 2^22, which the host checks.)
  const int hs = w / kPinRT;                       // the part this wave stages (wave-uniform)
  const int ht = tid - hs * kPinPartThreads;
  const unsigned char* pbase[L];
  uint32_t poff[L], pinc[L], plim[L];
  int pdst[L];
  {
    const int kb = part_unit0(hs) * KC;  // the part's first channel
#pragma unroll
    for (int k = 0; k < L; ++k) {
      const int q = ht + kPinPartThreads * k;
      const bool real = q < HP;
      constexpr int P_CS = G::XP + G::CWP + G::CBP, P_W = P_CS + G::MS * G::CSP;
      const int p = real ? q : P_W;  // a w_x piece
      pdst[k] = hs * HB;
      if (p < G::XP) {
        int64_t tok = t0 - kKS + p / (KC / 8);
        tok = tok < 0 ? 0 : (tok >= T ? T - 1 : tok);
        pbase[k] = reinterpret_cast<const unsigned char*>(x + tok * d64);
        poff[k] = static_cast<uint32_t>(kb + 8 * (p % (KC / 8))) * 2u;
        pinc[k] = U * KC * 2;
        plim[k] = static_cast<uint32_t>(d - 8) * 2u;
        pdst[k] += (p / (KC / 8)) * G::XSTRIDE * 2 + (p % (KC / 8)) * 16;
      } else if (p < G::XP + G::CWP) {
        pbase[k] = reinterpret_cast<const unsigned char*>(conv_w);
        poff[k] = static_cast<uint32_t>(kb + (p - G::XP)) * 16u;
        pinc[k] = U * KC * 16;
        plim[k] = static_cast<uint32_t>(d - 1) * 16u;
        pdst[k] += G::CWOFF + (p - G::XP) * 16;
      } else if (p < P_CS) {
        pbase[k] = reinterpret_cast<const unsigned char*>(conv_b);
        poff[k] = static_cast<uint32_t>(kb + 4 * (p - G::XP - G::CWP)) * 4u;
        pinc[k] = U * KC * 4;
        plim[k] = static_cast<uint32_t>(d - 4) * 4u;
        pdst[k] += G::CBOFF + (p - G::XP - G::CWP) * 16;
      } else if (p < P_W) {  // conv state: sequence s_first + jj (clamped to S - 1), 4 floats
        const int jj = (p - P_CS) / G::CSP, pp = (p - P_CS) % G::CSP;
        const int sj = s_first + jj < S ? s_first + jj : S - 1;
        pbase[k] = reinterpret_cast<const unsigned char*>(cs_stage) + static_cast<int64_t>(sj) * d64 * kKS * 4;
        poff[k] = static_cast<uint32_t>(kb * kKS + 4 * pp) * 4u;
        pinc[k] = U * KC * kKS * 4;
        plim[k] = static_cast<uint32_t>(d * kKS - 4) * 4u;
        pdst[k] += G::CSOFF + (p - P_CS) * 16;
      } else {  // w_x: a stage's operands are SUB * 4 Pp contiguous pieces
        const int pw = p - P_W;
        pbase[k] = reinterpret_cast<const unsigned char*>(wxP);
        poff[k] = static_cast<uint32_t>(kb / kProjK * 4 * Pp + pw) * 16u;
        pinc[k] = U * SUB * 4 * Pp * 16;
        plim[k] = static_cast<uint32_t>(nks * 4 * Pp - 1) * 16u;  // the last operand piece
        pdst[k] += G::WOFF + pw * 16;
      }
      if (!real) pdst[k] = -1;  // staged nowhere
    }
  }
  // stage g of a part of len stages (clamped to its last stage)
  auto rel_stage = [&](int g, int len) { return len > 0 ? (g < len ? g : len - 1) : 0; };
  const int hlen = part_len(hs);
  auto load_stage = [&](int g, u32x4_t (&pf)[L]) {
    const uint32_t rel = static_cast<uint32_t>(rel_stage(g, hlen));  // wave-uniform
#pragma unroll
    for (int k = 0; k < L; ++k) {
      const uint32_t o = __umul24(rel, pinc[k]) + poff[k];
      pf[k] = *reinterpret_cast<const u32x4_t*>(pbase[k] + (o < plim[k] ? o : plim[k]));
    }
  };
  // (pieces past a part's own go to a 16-byte slot after the two stage buffers: no branch, so the
  // compiler's count of outstanding loads stays exact)
  unsigned char* dummy = smem + 2 * KP * HB;
  auto write_stage = [&](unsigned char* buf, const u32x4_t (&pf)[L]) {
#pragma unroll
    for (int k = 0; k < L; ++k) *reinterpret_cast<u32x4_t*>(pdst[k] >= 0 ? buf + pdst[k] : dummy) = pf[k];
  };

  floatx4_t acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // MFMA K step ks, the sub-th of the stage in buf (this wave's part)
  auto kstep = [&](const unsigned char* buf, int ks, int sub, auto state) {
    constexpr bool STATE = decltype(state)::value;
    const unsigned char* hb = buf + h * HB;
    const int c = ks * kProjK + kg * 8;
    const bool live = c < d;
    // x of tokens t-3 .. t: four row reads (the LDS has room to spare; the VALU has none)
    const int xo = sub * kProjK * 2 + kg * 16;
    float xr[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(hb + (rt * 16 + row + r) * G::XSTRIDE * 2 + xo);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xr[r][2 * e] = __uint_as_float(v[e] << 16);
        xr[r][2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
      }
    }
    if (STATE && back < kKS && live) {  // rows before the sequence: its initial conv state
      if (cs_lds) {
        // one lane offset per row, made opaque so that the eight channels' reads keep it and
        // differ only in their immediate offsets (hoisted per channel, the offsets would take
        // 24 registers)
#pragma unroll
        for (int r = 0; r < kKS; ++r) {
          if (back - (kKS - r) < 0) {
            int lo = ((js * KC + sub * kProjK + kg * 8) * kKS + static_cast<int>(back) + r) * 4;
            asm volatile("" : "+v"(lo));
#pragma unroll
            for (int e = 0; e < 8; ++e) xr[r][e] = *reinterpret_cast<const float*>(hb + G::CSOFF + lo + e * kKS * 4);
          }
        }
      } else {  // (the same opaque per-row address)
#pragma unroll
        for (int r = 0; r < kKS; ++r) {
          if (back - (kKS - r) < 0) {
            const float* gp = cs + (static_cast<int64_t>(c) * kKS + back + r);
            asm volatile("" : "+v"(gp));
#pragma unroll
            for (int e = 0; e < 8; ++e) xr[r][e] = gp[e * kKS];
          }
        }
      }
    }
    // the conv parameters of the lane's 8 channels (the 16 lanes of a K group read the same ones)
    const float4* cwp = reinterpret_cast<const float4*>(hb + G::CWOFF) + sub * kProjK + kg * 8;
    const float4* cbp = reinterpret_cast<const float4*>(hb + G::CBOFF + (sub * kProjK + kg * 8) * 4);
    const float4 b0 = cbp[0], b1 = cbp[1];
    const float bias[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    bf16x8_t ua, ul;  // u's high and low parts
    auto conv_e = [&](auto ec) {
      constexpr int e = decltype(ec)::value;
      const float4 wv = cwp[e];
      float xc = bias[e];
      xc = __builtin_fmaf(wv.x, xr[0][e], xc);
      xc = __builtin_fmaf(wv.y, xr[1][e], xc);
      xc = __builtin_fmaf(wv.z, xr[2][e], xc);
      xc = __builtin_fmaf(wv.w, xr[3][e], xc);
      const float uv = silu(xc);  // computed for every lane (no branch), then zeroed past d
      __bf16 hi, lo;
      split_bf16(live ? uv : 0.0f, hi, lo);
      ua[e] = hi;
      ul[e] = lo;
    };
    conv_e(std::integral_constant<int, 0>{});
    conv_e(std::integral_constant<int, 1>{});
    conv_e(std::integral_constant<int, 2>{});
    conv_e(std::integral_constant<int, 3>{});
    conv_e(std::integral_constant<int, 4>{});
    conv_e(std::integral_constant<int, 5>{});
    conv_e(std::integral_constant<int, 6>{});
    conv_e(std::integral_constant<int, 7>{});
    const u32x4_t* wo = reinterpret_cast<const u32x4_t*>(hb + G::WOFF) + (sub * 4 + kg) * Pp + row;
    if constexpr (KP == 2) {
      u32x4_t wb[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) wb[j] = wo[j * 16];
      // the high parts over all column tiles, then the low parts: consecutive MFMAs are independent
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, __builtin_bit_cast(bf16x8_t, wb[j]), acc[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ul, __builtin_bit_cast(bf16x8_t, wb[j]), acc[j], 0, 0, 0);
    } else {
      // four waves per SIMD leave 128 VGPRs: each column tile's operands are held for two MFMAs
      // only, the high part of tile j issued between the two of tile j - 1
      u32x4_t wp = wo[0];
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, __builtin_bit_cast(bf16x8_t, wp), acc[0], 0, 0, 0);
#pragma unroll
      for (int j = 1; j < NT; ++j) {
        const u32x4_t wn = wo[j * 16];
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, __builtin_bit_cast(bf16x8_t, wn), acc[j], 0, 0, 0);
        acc[j - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ul, __builtin_bit_cast(bf16x8_t, wp), acc[j - 1], 0, 0, 0);
        wp = wn;
      }
      acc[NT - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ul, __builtin_bit_cast(bf16x8_t, wp), acc[NT - 1], 0, 0, 0);
    }
  };

  // A wave holding one of a sequence's first three tokens takes the loop that reads the conv state.
  // The D register sets are written out one after another (not a loop the compiler may roll
  // back up: rotating registers that still wait for loads would wait for them at once).
  auto kloop = [&](auto state) {
    u32x4_t pf[D][L];
#pragma unroll
    for (int u = 0; u < D; ++u) load_stage(u, pf[u]);
    // (stages past the last one repeat it without computing: the loads, writes and barriers stay
    // unconditional and in a fixed order)
    auto stage = [&](int g0, auto uc) {
      constexpr int u = decltype(uc)::value;
      const int g = g0 + u;
      unsigned char* buf = smem + (g & 1) * (KP * HB);
      write_stage(buf, pf[u]);  // waits for stage g's loads only (the earliest outstanding)
      load_stage(g + D, pf[u]);  // near the end a harmless repeat (clamped)
      __syncthreads();  // stage g visible; every wave done with stage g - 1 (the other buffer)
      if (g < slen) {
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub) {
          const int ks = (u0 + g * U) * SUB + sub;
          if (ks < nks) kstep(buf, ks, sub, state);
        }
      }
    };
    for (int g0 = 0; g0 < nst; g0 += D) {
      stage(g0, std::integral_constant<int, 0>{});
      if constexpr (D > 1) stage(g0, std::integral_constant<int, 1>{});
      if constexpr (D > 2) {
        stage(g0, std::integral_constant<int, 2>{});
        stage(g0, std::integral_constant<int, 3>{});
      }
    }
  };
  if (__any(back < kKS)) kloop(std::true_type{});
  else kloop(std::false_type{});

  // The parts' sums, in a fixed order through one LDS area: the last part leaves its
  // accumulators there, each part before it adds its own to them and leaves the sum, and the
  // first part ends with (((part KP-1 + part KP-2) + ...) + part 0).  The sums then go through a
  // float tile [64 tokens][OS] in LDS, so that every output leaves in contiguous runs: the
  // workgroup's 64 rows of B, of C and of dt_in's two parts are each one contiguous block.
  floatx4_t* red = reinterpret_cast<floatx4_t*>(smem);
  for (int q = KP - 1; q >= 0; --q) {
    __syncthreads();  // the K loop done (first pass), or part q + 1's sums written
    if (h == q) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        floatx4_t& r = red[(static_cast<size_t>(rt) * NT + j) * kWave + lane];
        if (q < KP - 1) acc[j] += r;
        if (q > 0) r = acc[j];
      }
    }
  }
  __syncthreads();  // the partial sums are read: the area becomes the output tile
  const int OS = pin_out_stride(Pp, Rp);
  float* ot = reinterpret_cast<float*>(smem);
  if (h == 0) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) ot[(rt * 16 + kg * 4 + i) * OS + j * 16 + row] = acc[j][i];  // token row, column
  }
  __syncthreads();
  const int64_t nrows = T - t0 < kPinTok ? T - t0 : kPinTok;  // the workgroup's tokens
  // dt_in: 8 columns per piece (Rp is a multiple of 32), high and low parts, zero past R
  {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const int npc = Rp / 8;
    uint16_t* hb = dth + t0 * Rp;
    uint16_t* lb = dtl + t0 * Rp;
    for (int e = tid; e < nrows * npc; e += THREADS) {
      const int r = e / npc, c = (e % npc) * 8;
      const float4 a = *reinterpret_cast<const float4*>(ot + r * OS + c);
      const float4 b = *reinterpret_cast<const float4*>(ot + r * OS + c + 4);
      const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v0 = c + 2 * q < R ? v[2 * q] : 0.0f, v1 = c + 2 * q + 1 < R ? v[2 * q + 1] : 0.0f;
        const f32x2_t f = {v0, v1};
        const bf16x2_t hi = __builtin_convertvector(f, bf16x2_t);
        const f32x2_t hf = __builtin_convertvector(hi, f32x2_t);
        wh[q] = __builtin_bit_cast(uint32_t, hi);
        wl[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f - hf, bf16x2_t));
      }
      *reinterpret_cast<u32x4_t*>(hb + static_cast<int64_t>(e) * 8) = u32x4_t{wh[0], wh[1], wh[2], wh[3]};
      *reinterpret_cast<u32x4_t*>(lb + static_cast<int64_t>(e) * 8) = u32x4_t{wl[0], wl[1], wl[2], wl[3]};
    }
  }
  // B and C: the workgroup's rows are N contiguous values each
  {
    uint16_t* bb = B + t0 * N;
    uint16_t* cb_ = C + t0 * N;
    for (int e = tid; e < nrows * N; e += THREADS) {
      const int r = e / N, c = e % N;
      bb[e] = bf16_bits(ot[r * OS + R + c]);
      cb_[e] = bf16_bits(ot[r * OS + R + N + c]);
    }
  }
}

// dt = dt_in x w_dt.  Workgroup (cb, g) of ncb x G (g fastest) takes channels 128 cb .. 128 cb + 127
// and the 16-token tiles g * per .. (g + 1) * per - 1; wave w takes every fourth of them.  The block's
// w_dt operands (KR = Rp / 32 K steps, a template argument) are staged in LDS once, zero past
// d; per token tile a wave loads dt_in's high and low parts (prefetched one tile ahead: they
// are the only global loads of the loop), runs 8 x KR x 2 MFMAs and writes the 16 x 128 tile
// through its LDS tile as 16-byte row pieces.
template <int KR>
__global__ void __launch_bounds__(kPdtThreads) k_proj_dt(const uint16_t* __restrict__ dth,
                                                         const uint16_t* __restrict__ dtl,
                                                         const uint16_t* __restrict__ wdtP, uint16_t* __restrict__ dt,
                                                         int64_t T, int d, int ncb, int per) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int Rp = KR * kProjK;
  u32x4_t* wl = reinterpret_cast<u32x4_t*>(smem);  // [KR * 4][kPdtCh] pieces of 8 bf16
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  uint16_t* o = reinterpret_cast<uint16_t*>(smem + static_cast<size_t>(KR) * 4 * kPdtCh * 16) + w * 16 * kPdtOStride;
  const int row = lane & 15, kg = lane >> 4;
  // workgroups that run at the same time take different token ranges (they would otherwise all
  // read the same dt_in rows at once)
  const int64_t ngr = gridDim.x / ncb;
  const int cb = static_cast<int>(blockIdx.x / ngr);
  const int64_t g = blockIdx.x % ngr;
  const int c0 = cb * kPdtCh;
  const int64_t d64 = d;
  // the block's operands: piece (q, c) = wdtP[q][c0 + c][0..7] for q < KR * 4 (zero past d)
  for (int i = threadIdx.x; i < KR * 4 * kPdtCh; i += kPdtThreads) {
    const int q = i / kPdtCh, c = i % kPdtCh;
    wl[i] = c0 + c < d ? *reinterpret_cast<const u32x4_t*>(wdtP + (static_cast<int64_t>(q) * d + c0 + c) * 8)
                       : u32x4_t{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  const int64_t ntt = (T + 15) / 16;  // token tiles
  const int64_t tt0 = g * per;
  const int64_t tt1 = tt0 + per < ntt ? tt0 + per : ntt;
  auto load_a = [&](int64_t tt, u32x4_t (&a)[2 * KR]) {
    int64_t tk = tt * 16 + row;
    if (tk >= T) tk = T - 1;
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) {
      a[kk] = *reinterpret_cast<const u32x4_t*>(dth + tk * Rp + kk * kProjK + kg * 8);
      a[KR + kk] = *reinterpret_cast<const u32x4_t*>(dtl + tk * Rp + kk * kProjK + kg * 8);
    }
  };
  u32x4_t acur[2 * KR], anxt[2 * KR];
  int64_t tt = tt0 + w;
  load_a(tt < tt1 ? tt : tt0, acur);
  for (; tt < tt1; tt += kPdtWaves) {
    load_a(tt + kPdtWaves < tt1 ? tt + kPdtWaves : tt, anxt);  // past the last tile a harmless repeat
    floatx4_t acc[kPdtTiles];
#pragma unroll
    for (int j = 0; j < kPdtTiles; ++j) acc[j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KR; ++kk) {
      u32x4_t wv[kPdtTiles];
#pragma unroll
      for (int j = 0; j < kPdtTiles; ++j) wv[j] = wl[(kk * 4 + kg) * kPdtCh + j * 16 + row];
      const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, acur[kk]), al = __builtin_bit_cast(bf16x8_t, acur[KR + kk]);
#pragma unroll
      for (int j = 0; j < kPdtTiles; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv[j]), ah, acc[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < kPdtTiles; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv[j]), al, acc[j], 0, 0, 0);
    }
    // The MFMAs form the transposed tile (w_dt^T x dt_in^T): acc[j][i] is channel c0 + 16 j +
    // 4 kg + i of token 16 tt + row, so each lane writes four consecutive channels of one token
    // to the wave's LDS tile as 8 bytes; the tile then leaves as 16-byte row pieces.
    {
      typedef float f32x2_t __attribute__((ext_vector_type(2)));
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int j = 0; j < kPdtTiles; ++j) {
        const f32x2_t lo2 = {acc[j][0], acc[j][1]}, hi2 = {acc[j][2], acc[j][3]};
        *reinterpret_cast<u32x2_t*>(o + row * kPdtOStride + j * 16 + 4 * kg) =
            u32x2_t{__builtin_bit_cast(uint32_t, __builtin_convertvector(lo2, bf16x2_t)),
                    __builtin_bit_cast(uint32_t, __builtin_convertvector(hi2, bf16x2_t))};
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's tile written before it reads it
    {
      // buffer stores over the tile's rows: the hardware drops the stores of rows past T (past
      // the range) and of lanes past d (sent past it).  With no branch around them, the
      // compiler's count of outstanding memory operations stays exact, so its wait for the next
      // tile's dt_in loads does not also wait for these stores to complete.
      const int64_t r0 = tt * 16;
      const int nr = T - r0 < 16 ? static_cast<int>(T - r0) : 16;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(dt + r0 * d64, 0, nr * d * 2, kBufWord3);
#pragma unroll
      for (int k = 0; k < 16 * kPdtCh / 8 / kWave; ++k) {
        const int i = lane + kWave * k;
        const int r = i / (kPdtCh / 8), part = i % (kPdtCh / 8);
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(o + r * kPdtOStride + part * 8);
        const int off = c0 + part * 8 < d ? (r * d + c0 + part * 8) * 2 : kBufPastEnd;
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, kBufNontemporal);
      }
    }
#pragma unroll
    for (int k = 0; k < 2 * KR; ++k) acur[k] = anxt[k];
  }
}

}  // namespace mm
