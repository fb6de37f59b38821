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
//    with coalesced loads issued two blocks before the tiles go to LDS (three
//    blocks before their use), and writes y back from an LDS tile one block
//    behind -- every global access is a run of whole rows;
//  * lane j of a row does the per-token work of token j for the row's channel:
//    the causal conv (its window of inputs t-3 .. t comes from the x tile, whose
//    three front rows hold the previous block's last inputs), SiLU, softplus,
//    delta * u, D * u and SiLU(z).  Tokens outside the chunk get delta = 0, which makes their step the
//    identity (exp(0) = 1, nothing added);
//  * the 16 recurrence steps: step i broadcasts delta and delta * u of token i from
//    lane i to the row (DPP row_newbcast, folded into the multiply that uses it);
//    lane n updates h_n = exp(delta A_n) h_n + (delta u) B_n and forms C_n h_n;
//  * a 16x16 transposing butterfly over the row (DPP row rotations and quad
//    permutes) sums C_n h_n over n for all 16 tokens at once and leaves token j's
//    sum in lane j, which finishes y for its token.
// One barrier per block.  A block's four waves meet at that barrier, so a workgroup
// advances at the pace of its slowest wave, and the waves that share a SIMD belong
// to different workgroups.  Each wave therefore raises its issue priority step by
// step as it works through the block's recurrence and drops it after the barrier:
// the SIMD issues first for the wave nearest its barrier, and waves just past
// theirs (staging, LDS reads) fill the gaps.
// The chunk plan, carries and stash are those of the other engines (mm_prefill.h);
// with one chunk per sequence ("whole" mode) the workgroup's chunk is simply its
// sequence and no plan is needed.
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
constexpr int kRowMaxD = MM_ROW_MAX_D;                 // channel limit of the row layout (32-bit tile offsets)
static_assert(MM_ROW_MAX_D <= (1 << 22), "per-thread tile offsets must stay below 2^32");

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

__device__ __forceinline__ float comp(const float4& v, int e) {
  return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

// One recurrence step: token I of the block.  Steps 2, 8 and 13 raise the wave's issue
// priority to 1, 2 and 3 (k_row drops it to 0 after the block's barrier).
template <int I, bool READOUT>
__device__ __forceinline__ void row_step(float delta, float du, float A2, const float4 (&Bq)[4],
                                         const float4 (&Cq)[4], float& h, float (&p)[kRow]) {
  if (I == 2) __builtin_amdgcn_s_setprio(1);
  if (I == 8) __builtin_amdgcn_s_setprio(2);
  if (I == 13) __builtin_amdgcn_s_setprio(3);
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
// partner lane across that bit.  The stages across lane bits 3 and 2 split the row
// by DPP bank masks (banks of 4 lanes): per pair of registers one masked add writes
// the lanes that keep the lower token and one the lanes that keep the upper, in
// place of two adds and a select.  The masked adds sit in one asm block; its
// leading and trailing `s_nop 1` give the two wait states a DPP read needs after
// a VALU write of its source, which the compiler's hazard check does not see
// across the asm boundary.  Bits 1 and 0 (within a bank) use adds and selects.
__device__ __forceinline__ float row_transpose_sum(const float (&p)[kRow], int j) {
#pragma clang fp contract(off)
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = p[i];
  // bit 3: banks 0-1 (j < 8) keep token i, banks 2-3 token i + 8; partner j ^ 8 = ror 8.
  // bit 2: banks 0, 2 keep token i (partner j + 4 = ror 12), banks 1, 3 token i + 4 (ror 4).
  asm(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %2, %2 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %3, %3 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %4, %4, %4 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %4, %12, %12 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %5, %5, %5 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %5, %13, %13 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %6, %6, %6 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %6, %14, %14 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %7, %7, %7 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %7, %15, %15 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %4, %4 row_ror:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %1, %5, %5 row_ror:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %2, %2, %2 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %2, %6, %6 row_ror:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %3, %3, %3 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %3, %7, %7 row_ror:4 row_mask:0xf bank_mask:0xa\n\t"
      "s_nop 1"
      : "+&v"(q[0]), "+&v"(q[1]), "+&v"(q[2]), "+&v"(q[3]), "+&v"(q[4]), "+&v"(q[5]), "+&v"(q[6]), "+&v"(q[7])
      : "v"(p[8]), "v"(p[9]), "v"(p[10]), "v"(p[11]), "v"(p[12]), "v"(p[13]), "v"(p[14]), "v"(p[15]));
  // q[i], i < 4: token i + 4 b2 + 8 b3, summed over lane bits 3 and 2
  const bool b1 = (j & 2) != 0, b0 = (j & 1) != 0;
  float s[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float lo = q[i] + dpp<kXor2>(q[i]);
    const float hi = q[i + 2] + dpp<kXor2>(q[i + 2]);
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
// A block's tiles sit in one of three slots: block b in slot b % 3.  [token][channel]
// tiles are padded to 18 columns (no LDS bank conflicts for either the row or the
// column access); the B/C tile is laid out [which][q][n] float4 holding tokens
// 4q..4q+3, so lane n reads B (or C) of 4 tokens as one float4.  The x tile has three
// more rows in front, the raw inputs of the three tokens before the block (the conv
// window): the stager of block b also writes its last three rows there in block
// b + 1's slot.  With bf16 io the stager writes the 16 raw bits of dt, z, B and C into
// the upper half of their float (the lower halves are zeroed once), which is the
// float32 value without a conversion instruction.
constexpr int kTS = kRowChans + 2;  // tile row stride (floats)
struct RowSlot {
  float x[kKS + kRow][kTS];
  float z[kRow][kTS];
  float dt[kRow][kTS];
  float y[kRow][kTS];  // the block's outputs, from its scan until they are stored
  float4 bc[2][4][kRow];
};
constexpr int kSlots = 3;
struct RowTiles {
  RowSlot slot[kSlots];
};
constexpr uint32_t kSlotBytes = sizeof(RowSlot);

__device__ __forceinline__ RowSlot& slot_at(RowTiles& L, uint32_t off) {
  return *reinterpret_cast<RowSlot*>(reinterpret_cast<char*>(&L.slot[0]) + off);
}

// One thread's share of a block's global inputs: element (token i/16, channel i%16)
// of the x/z/dt tiles, and element i of the contiguous [16][N] B and C tiles.
template <typename IO>
struct RowStage {
  IO x, z, dt, B, C;
};

// Global pointers of one staged block: the x/z/dt tiles from channel c0 of its first
// token, the contiguous B/C tiles (wave-uniform, in scalar registers)
template <typename IO>
struct RowSrc {
  gmem<const IO>*x, *z, *dt, *B, *C;
};

// Loads a block's share of this thread: its byte offsets o in the [16][d] x/z/dt
// tiles and ob in the [16][N] B/C tiles (in the tensors' last block both are clamped
// to the last element, so only valid memory is read; the clamped values only feed
// tokens past the end of the chunk).
template <typename IO, bool FINAL>
__device__ __forceinline__ void row_stage_load(RowStage<IO>& r, const RowSrc<IO>& g, uint32_t o, uint32_t ob) {
  r.x = ld_at(g.x, o);
  r.dt = ld_at(g.dt, o);
  if (FINAL) r.z = ld_at(g.z, o);
  r.B = ld_at(g.B, ob);
  if (FINAL) r.C = ld_at(g.C, ob);
}

// A staging thread's byte offsets within a slot: element (token row tt, channel ch) of
// the [token][channel] tiles (x from its first block row) and its element of the B/C
// tile.
struct RowStOff {
  uint32_t tc;  // (tt * kTS + ch) * 4
  uint32_t bc;  // of B; C is one [4][16] float4 tile further
};

__device__ __forceinline__ void st_lds(char* p, float v) { *reinterpret_cast<float*>(p) = v; }
__device__ __forceinline__ void st_lds(char* p, uint16_t v) { *reinterpret_cast<uint16_t*>(p + 2) = v; }

// Writes a staged block into LDS: into the slot at byte offset sb, and the last three
// token rows of x also into the front rows of the slot at sn (the next block's).
template <typename IO, bool FINAL>
__device__ __forceinline__ void row_stage_store(const RowStage<IO>& r, RowTiles& L, uint32_t sb, uint32_t sn,
                                                const RowStOff& o, int N) {
  constexpr uint32_t kX = offsetof(RowSlot, x) + kKS * kTS * 4, kZ = offsetof(RowSlot, z),
                     kDt = offsetof(RowSlot, dt), kB = offsetof(RowSlot, bc), kC = kB + sizeof(float4) * 4 * kRow;
  constexpr int kFront = static_cast<int>(offsetof(RowSlot, x)) - (kRow - kKS) * kTS * 4;  // row tt - 13, next slot
  const int tt = threadIdx.x >> 4;
  char* base = reinterpret_cast<char*>(&L.slot[0]);
  char* t = base + sb + o.tc;
  const float xv = io_f32(r.x);
  st_lds(t + kX, xv);
  if (tt >= kRow - kKS) st_lds(base + sn + (static_cast<int>(o.tc) + kFront), xv);
  st_lds(t + kDt, r.dt);
  if (FINAL) st_lds(t + kZ, r.z);
  if (static_cast<int>(threadIdx.x) < kRow * N) {
    char* b = base + sb + o.bc;
    st_lds(b + kB, r.B);
    if (FINAL) st_lds(b + kC, r.C);
  }
}

// ---------------------------------------------------------------- vector staging
// With N = 16, d % 4 == 0 and io aligned to 4 elements, a workgroup stages each tile
// with one 4-element load per lane of one wave: wave 0 loads the x tile, wave 1 dt,
// wave 2 z and wave 3 B and C (pass 2), or waves 0..2 x, dt and B (pass 1).  Lane l
// takes row l / 4, channels 4 (l % 4) .. + 3 of a [16][d] tile, or elements 4 l .. 4 l + 3
// (token l / 4, states 4 (l % 4) .. + 3) of the [16][16] B or C tile; wave 1 stores the
// y tile the same way.  A block then costs 5 vector loads and one vector store per
// workgroup instead of 5 loads and one store per wave.
constexpr int kKindX = 0, kKindDt = 1, kKindZ = 2, kKindBC = 3, kKindNone = 4;

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <typename IO>
struct Vec4T;
template <>
struct Vec4T<uint16_t> {
  using T = u32x2_t;
};
template <>
struct Vec4T<float> {
  using T = f32x4_t;
};
template <typename IO>
using Vec4 = typename Vec4T<IO>::T;

template <typename IO>
__device__ __forceinline__ Vec4<IO> ld4(gmem<const IO>* p, uint32_t off) {
  return *reinterpret_cast<gmem<const Vec4<IO>>*>(reinterpret_cast<gmem<const char>*>(p) + off);
}
// the four elements into LDS floats S bytes apart (bf16: the raw bits into their upper halves)
template <int S>
__device__ __forceinline__ void st_lds4(char* p, const u32x2_t& v) {
  *reinterpret_cast<uint16_t*>(p + 2) = static_cast<uint16_t>(v.x);
  *reinterpret_cast<uint16_t*>(p + S + 2) = static_cast<uint16_t>(v.x >> 16);
  *reinterpret_cast<uint16_t*>(p + 2 * S + 2) = static_cast<uint16_t>(v.y);
  *reinterpret_cast<uint16_t*>(p + 3 * S + 2) = static_cast<uint16_t>(v.y >> 16);
}
template <int S>
__device__ __forceinline__ void st_lds4(char* p, const f32x4_t& v) {
  *reinterpret_cast<float*>(p) = v.x;
  *reinterpret_cast<float*>(p + S) = v.y;
  *reinterpret_cast<float*>(p + 2 * S) = v.z;
  *reinterpret_cast<float*>(p + 3 * S) = v.w;
}
// the four elements as floats, into 16 contiguous 8-byte aligned LDS bytes
__device__ __forceinline__ void st_lds4f(char* p, const u32x2_t& v) {
  float2* q = reinterpret_cast<float2*>(p);
  q[0] = make_float2(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u));
  q[1] = make_float2(__uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
}
__device__ __forceinline__ void st_lds4f(char* p, const f32x4_t& v) {
  float2* q = reinterpret_cast<float2*>(p);
  q[0] = make_float2(v.x, v.y);
  q[1] = make_float2(v.z, v.w);
}
// four floats stored as io (bf16: rounded to nearest even)
__device__ __forceinline__ void st_g4(gmem<uint16_t>* p, uint32_t off, const f32x4_t& v) {
  const f32x2_t fa = {v.x, v.y}, fb = {v.z, v.w};
  const bf16x2_t ha = __builtin_convertvector(fa, bf16x2_t), hb = __builtin_convertvector(fb, bf16x2_t);
  const u32x2_t u = {__builtin_bit_cast(uint32_t, ha), __builtin_bit_cast(uint32_t, hb)};
  *reinterpret_cast<gmem<u32x2_t>*>(reinterpret_cast<gmem<char>*>(p) + off) = u;
}
__device__ __forceinline__ void st_g4(gmem<float>* p, uint32_t off, const f32x4_t& v) {
  *reinterpret_cast<gmem<f32x4_t>*>(reinterpret_cast<gmem<char>*>(p) + off) = v;
}
// The same stores, and a one-float store, written as assembly.  The compiler then does not
// count them among the outstanding vector-memory operations: with stores among them it
// takes the counter as unordered and waits for zero before using any loaded register,
// which would drain the staging loads that are meant to stay in flight across two
// blocks.  Not counting the stores only makes its waits longer than needed, never short:
// loads complete in the order they were issued, so while a load is outstanding so are
// the loads after it.  The stores' addresses and data are read at issue; a store of
// more than 8 bytes needs one wait state before its data registers are written again.
__device__ __forceinline__ void st_g4_uncounted(gmem<uint16_t>* p, uint32_t off, const f32x4_t& v) {
  const f32x2_t fa = {v.x, v.y}, fb = {v.z, v.w};
  const bf16x2_t ha = __builtin_convertvector(fa, bf16x2_t), hb = __builtin_convertvector(fb, bf16x2_t);
  const u32x2_t u = {__builtin_bit_cast(uint32_t, ha), __builtin_bit_cast(uint32_t, hb)};
  asm volatile("global_store_dwordx2 %0, %1, %2" ::"v"(off), "v"(u), "s"(p) : "memory");
}
__device__ __forceinline__ void st_g4_uncounted(gmem<float>* p, uint32_t off, const f32x4_t& v) {
  asm volatile("global_store_dwordx4 %0, %1, %2\n\ts_nop 0" ::"v"(off), "v"(v), "s"(p) : "memory");
}
__device__ __forceinline__ void st_g_uncounted(gmem<float>* p, uint32_t off, float v) {
  asm volatile("global_store_dword %0, %1, %2" ::"v"(off), "v"(v), "s"(p) : "memory");
}

// a workgroup-uniform 64-bit value held in vector registers, moved to scalar registers
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// the lane mask that holds lanes j of every row with bit j of m16 set
__device__ __forceinline__ uint64_t row_mask(uint32_t m16) {
  const uint32_t m32 = m16 | (m16 << 16);
  return (static_cast<uint64_t>(m32) << 32) | m32;
}
// tokens [lo, hi) of a 16-token block (lo <= 15, hi >= 1, either may lie outside 0..16)
__device__ __forceinline__ uint32_t token_bits(int lo, int hi) {
  const uint32_t mlo = lo <= 0 ? 0u : (1u << lo) - 1u;
  const uint32_t mhi = hi >= kRow ? 0xFFFFu : (1u << hi) - 1u;
  return mhi & ~mlo;
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

// FINAL = false: pass 1 (sum(delta) and local end state of every piece of a non-last
// chunk: each such chunk is scanned as ws.ksub pieces of Lc / ksub tokens, so that the
// pass has enough workgroups; a sequence's first piece starts from its slot).
// FINAL = true: pass 2 (y, and the final states at a sequence's last chunk); a chunk's
// carry-in is the fold of the pieces before it, done by the chunk's own workgroup.
// With ws.inl every workgroup computes the chunk plan itself (no k_chunk_plan launch).
// CKPT = true: also write the state before every 16-token block to ckpt, [rows][d][16],
// the block starting at token tb of sequence s at row s + tb / 16.  With FINAL = false
// (whole sequences only) that is all the pass writes: the checkpoint pass of the
// backward.  With FINAL = true it is the forward of a training step; a continuing
// chunk leaves a block it shares with the chunk before to that chunk.
// whole != 0: one chunk per sequence, workgroup chunk index = sequence (no plan).
// d <= kRowMaxD keeps every per-thread offset within a block's tiles below 2^32.
// VEC: vector staging (N = 16, d % 4 == 0, io aligned to 4 elements).
template <typename IO, bool FINAL, bool CKPT, bool VEC>
__global__ void __launch_bounds__(kRowThreads) k_row(
    const IO* __restrict__ x, const IO* __restrict__ z, const IO* __restrict__ dt, const IO* __restrict__ B,
    const IO* __restrict__ C, const float* __restrict__ A_log, const float* __restrict__ D,
    const float* __restrict__ dt_bias, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    const int32_t* __restrict__ cu, float* __restrict__ conv_state, float* __restrict__ ssm_state,
    IO* __restrict__ y, CarryWs ws, int S, int64_t T, int d, int N, int64_t Lc, int whole,
    float* __restrict__ ckpt) {
  constexpr int NMAX = kRow;
  constexpr int64_t kMask = ~static_cast<int64_t>(kRow - 1);
  constexpr uint32_t es = sizeof(IO);
  __shared__ RowTiles L;
  __shared__ int32_t plan_l[2][kPlanInline + 1];
  __shared__ int32_t plan_w[2][kPlanInline / kWave];
  int64_t k;
  int cb;
  const int nchb = (d + kRowChans - 1) / kRowChans;
  row_work(blockIdx.x, (nchb + kRowGroup - 1) / kRowGroup, k, cb);
  if (cb >= nchb) return;  // (uniform over the workgroup)
  ChunkRef R;
  int64_t slot = 0;  // pass 1: this piece's carry slot
  int stash_i = 0;   // the sequence's stash slot (multi-chunk sequences)
  const int32_t* offp = ws.off;
  const int32_t* moffp = ws.moff;
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
    if (!FINAL && !CKPT) return;
  } else {
    if (ws.inl) {  // (uniform)
      chunk_plan_inline(cu, S, Lc, plan_l[0], plan_l[1], plan_w);
      offp = plan_l[0];
      moffp = plan_l[1];
    }
    if (!FINAL && !CKPT) {
      // pass 1: piece k of the non-last chunks, each chunk scanned as ksub pieces of Lc / ksub
      // tokens (pieces of non-last chunks are full); its sequence is the largest s with
      // moff[s] <= k / ksub
      const int64_t q = k / ws.ksub;
      if (q >= moffp[S]) return;
      int lo = 0, hi = S - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(moffp[mid]) <= q) lo = mid; else hi = mid - 1;
      }
      R.ok = true;
      R.s = lo;
      R.j = static_cast<int>(k - static_cast<int64_t>(ws.ksub) * moffp[lo]);  // piece within the sequence
      R.ns = offp[lo + 1] - offp[lo];
      R.start = cu[lo] + static_cast<int64_t>(R.j) * (Lc / ws.ksub);
      R.end = R.start + Lc / ws.ksub;
      R.cidx = R.pidx = 0;
      slot = k;
    } else {
      R = chunk_ref(cu, offp, moffp, S, k, Lc);
      if (!R.ok) return;
    }
    stash_i = moffp[R.s];
    // read from LDS, these workgroup-uniform values sit in vector registers: into scalar ones
    R.s = __builtin_amdgcn_readfirstlane(R.s);
    R.j = __builtin_amdgcn_readfirstlane(R.j);
    R.ns = __builtin_amdgcn_readfirstlane(R.ns);
    R.start = uniform64(R.start);
    R.end = uniform64(R.end);
    stash_i = __builtin_amdgcn_readfirstlane(stash_i);
  }

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

  // initial SSM state; the sequence's initial conv state comes from its slot or, in
  // pass 2 of a multi-chunk sequence, from the stash (its last chunk rewrites the slot)
  const bool multi = R.ns > 1;
  const bool from_stash = (FINAL || CKPT) && multi;
  float h = 0.0f;
  if (!FINAL && !CKPT) {
    if (R.j == 0) {
      h = (j < N) ? ssm_state[sc * N + j] : 0.0f;
      if (cvalid) {
        float* stash = ws.stash + (static_cast<int64_t>(stash_i) * d + c) * (NMAX + kKS);
        stash[j] = h;
        if (j < kKS) stash[NMAX + j] = conv_state[sc * kKS + j];
      }
    }
  } else if (R.j == 0) {
    h = from_stash ? ws.stash[(static_cast<int64_t>(stash_i) * d + cc) * (NMAX + kKS) + j]
                   : ((j < N) ? ssm_state[sc * N + j] : 0.0f);
  } else {
    // the carry-in: pass 1's pieces of the chunks before this one, folded in order with
    // (a, b) o (a', b') = (a a', a' b + b'), a piece's decay product being exp(A sum(delta)).
    // The first piece started from the slot, so its state is already true.  The loads of a
    // group of eight pieces are issued before their arithmetic.
    const int64_t m0 = static_cast<int64_t>(ws.ksub) * stash_i;
    const int64_t m1 = m0 + static_cast<int64_t>(R.j) * ws.ksub;
    const float* pa = ws.a + cc;
    const float* pb = ws.b + static_cast<int64_t>(cc) * NMAX + j;
    const int64_t sa = d, sb = static_cast<int64_t>(d) * NMAX;
    float cur = pb[m0 * sb];
    for (int64_t i = m0 + 1; i < m1; i += 8) {
      float av[8], bv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t iu = i + u < m1 ? i + u : m1 - 1;
        av[u] = pa[iu * sa];
        bv[u] = pb[iu * sb];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i + u < m1) cur = __builtin_fmaf(exp2_hw(A2 * av[u]), cur, bv[u]);
    }
    h = cur;
  }

  const int64_t tb0 = R.start & kMask;
  const int64_t tlast = (R.end - 1) & kMask;
  const int nb = static_cast<int>((tlast - tb0) >> 4) + 1;
  // token indices fit in 32 bits (T <= INT32_MAX)
  const int T32 = static_cast<int>(T), tb0i = static_cast<int>(tb0);
  const int rs = static_cast<int>(R.start), re = static_cast<int>(R.end);

  // the staging thread's element: token row srow, channel c0 + sch (clamped to d - 1)
  const int srow = static_cast<int>(threadIdx.x >> 4), sch = static_cast<int>(threadIdx.x & (kRowChans - 1));
  const int schc = c0 + sch < d ? sch : d - 1 - c0;
  const uint32_t xo = static_cast<uint32_t>(srow * d + schc) * es;
  const uint32_t bco = static_cast<uint32_t>(min(static_cast<int>(threadIdx.x), kRow * N - 1)) * es;
  const uint32_t yo = static_cast<uint32_t>(srow * d + sch) * es;  // the y element this thread stores
  // the tensors' last block (T - Tl < 16 tokens): its loads are clamped to valid memory
  const int Tl = (T32 - 1) & ~(kRow - 1);
  const int remT = T32 - Tl;
  const uint32_t xlim = static_cast<uint32_t>(remT * d - 1 - c0) * es;
  const uint32_t blim = static_cast<uint32_t>(remT * N - 1) * es;
  auto lim_x = [&](int tb) { return tb == Tl ? xlim : UINT32_MAX; };
  auto lim_b = [&](int tb) { return tb == Tl ? blim : UINT32_MAX; };

  RowStOff so;
  so.tc = static_cast<uint32_t>(srow * kTS + sch) * 4u;
  {
    const int i = min(static_cast<int>(threadIdx.x), kRow * N - 1), t = i / N, n = i - t * N;
    so.bc = static_cast<uint32_t>(((t >> 2) * kRow + n) * 16 + (t & 3) * 4);
  }

  // vector staging: this wave's tile kind and the lane's offsets (see above)
  const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int kind = FINAL ? wv : (wv == 2 ? kKindBC : (wv == 3 ? kKindNone : wv));
  const int vr = lane >> 2, vcg = lane & 3;
  uint32_t vo = 0, vo_t = 0, vl = 0;
  if (VEC) {
    if (kind == kKindBC || kind == kKindNone) {
      vo = static_cast<uint32_t>(4 * lane) * es;
      vo_t = static_cast<uint32_t>(min(4 * lane, remT * kRow - 4)) * es;
      vl = static_cast<uint32_t>(offsetof(RowSlot, bc) + (((vr >> 2) * kRow + 4 * vcg) * 16 + (vr & 3) * 4));
    } else {
      vo = static_cast<uint32_t>(vr * d + 4 * vcg) * es;
      vo_t = static_cast<uint32_t>(min(vr, remT - 1) * d + 4 * vcg) * es;
      const uint32_t rc = static_cast<uint32_t>(vr * kTS + 4 * vcg) * 4u;
      vl = rc + (kind == kKindX ? offsetof(RowSlot, x) + kKS * kTS * 4
                                : (kind == kKindDt ? offsetof(RowSlot, dt) : offsetof(RowSlot, z)));
    }
  }
  // x rows 13..15 also go to the next slot's front rows
  const int vfront = static_cast<int>(offsetof(RowSlot, x)) + ((vr - (kRow - kKS)) * kTS + 4 * vcg) * 4;
  const uint32_t vy = static_cast<uint32_t>(offsetof(RowSlot, y)) + static_cast<uint32_t>(vr * kTS + 4 * vcg) * 4u;
  const uint32_t vyo = static_cast<uint32_t>(vr * d + 4 * vcg) * es;

  // B/C entries past N stay zero (the staging only writes n < N), and so do the lower
  // halves of bf16 values
  if (sizeof(IO) == 2 || N < kRow) {
    float4* f = reinterpret_cast<float4*>(&L.slot[0]);
    for (int i = threadIdx.x; i < static_cast<int>(sizeof(L) / sizeof(float4)); i += kRowThreads)
      f[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    __syncthreads();
  }

  const int64_t sx = static_cast<int64_t>(kRow) * d, sb = static_cast<int64_t>(kRow) * N;  // elements per block
  RowSrc<IO> g;
  gmem<const IO>* gv = nullptr;  // vector staging: this wave's tensor at the block loaded next
  gmem<const IO>* gv_last = nullptr;
  auto set_src = [&](int tb) {
    const int64_t e0 = static_cast<int64_t>(tb) * d + c0, b0 = static_cast<int64_t>(tb) * N;
    if (VEC) {
      const IO* t = kind == kKindX ? x + e0 : (kind == kKindDt ? dt + e0 : (kind == kKindZ ? z + e0 : B + b0));
      gv = sbase(t);
      if (FINAL) g.C = sbase(C + b0);
    } else {
      g.x = sbase(x + e0);
      g.dt = sbase(dt + e0);
      if (FINAL) g.z = sbase(z + e0);
      g.B = sbase(B + b0);
      if (FINAL) g.C = sbase(C + b0);
    }
  };
  const int64_t vstride = (kind == kKindBC || kind == kKindNone) ? sb : sx;
  // Two sets of staging registers: a block's loads are issued two iterations before its
  // tiles go to LDS, blocks of even index (relative to the chunk's first block) through
  // the first set, odd ones through the second; the loop body is written out twice, so
  // that no registers move between the sets.  With vector staging every wave issues the
  // same two loads per block, whatever its tile kind and whether the block exists (the
  // second is C for the B/C wave and a repeat of the first for the others; past the
  // chunk's last block both re-read that block), so that the compiler's count of
  // outstanding loads is the same on every path and its waits only drain the loads of
  // the block being stored.
  struct StageRegs {
    RowStage<IO> r;
    Vec4<IO> a, b;
  };
  StageRegs q0{}, q1{};
  auto load = [&](int tb, StageRegs& q) {
    if (VEC) {
      const uint32_t o = tb == Tl ? vo_t : vo;
      q.a = ld4(gv, o);
      q.b = ld4(FINAL && kind == kKindBC ? g.C : gv, o);
    } else {
      row_stage_load<IO, FINAL>(q.r, g, min(xo, lim_x(tb)), min(bco, lim_b(tb)));
    }
  };
  // the staged block into the slot at byte offset sl; x rows 13..15 also into the slot at sn
  auto store = [&](uint32_t sl, uint32_t sn, const StageRegs& q) {
    if (VEC) {
      char* base = reinterpret_cast<char*>(&L.slot[0]);
      if (kind == kKindX) {
        st_lds4f(base + sl + vl, q.a);
        if (vr >= kRow - kKS) st_lds4f(base + sn + vfront, q.a);
      } else if (kind == kKindDt || kind == kKindZ) {
        st_lds4<4>(base + sl + vl, q.a);
      } else if (kind == kKindBC) {
        st_lds4<16>(base + sl + vl, q.a);
        if (FINAL) st_lds4<16>(base + sl + vl + sizeof(float4) * 4 * kRow, q.b);
      }
    } else {
      row_stage_store<IO, FINAL>(q.r, L, sl, sn, so, N);
    }
  };
  // blocks 0 and 1 staged, blocks 2 and 3 loaded
  set_src(tb0i);
  load(tb0i, q0);
  store(0, kSlotBytes, q0);
  if (VEC) __syncthreads();  // the history below overwrites x values other waves staged
  {
    // raw input of token t for the staging channel; tokens before the sequence's start
    // come from its initial conv state (zero before that)
    const int cs = c0 + schc;
    const float* cs0 = from_stash ? ws.stash + (static_cast<int64_t>(stash_i) * d + cs) * (NMAX + kKS) + NMAX
                                  : conv_state + (static_cast<int64_t>(R.s) * d + cs) * kKS;
    auto hist = [&](int64_t t) -> float {
      if (t >= seq_start) return io_f32(x[t * d + cs]);
      const int64_t q = t - seq_start + kKS;
      return q >= 0 ? cs0[q] : 0.0f;
    };
    if (srow < kKS) L.slot[0].x[srow][sch] = hist(tb0 - kKS + srow);  // the window before the first block
    const int64_t t = tb0 + srow;
    if (t < seq_start) {  // the first block starts in the sequence before: its tokens there are history
      const float v = hist(t);
      L.slot[0].x[kKS + srow][sch] = v;
      if (srow >= kRow - kKS) L.slot[1].x[srow - (kRow - kKS)][sch] = v;
    }
  }
  if (nb > 1) {
    set_src(tb0i + kRow);
    load(tb0i + kRow, q1);
    store(kSlotBytes, 2 * kSlotBytes, q1);
  }
  // blocks 2 and 3 (or the last block again), loaded
  const int tlasti = static_cast<int>(tlast);
  set_src(min(tb0i + 2 * kRow, tlasti));
  load(min(tb0i + 2 * kRow, tlasti), q0);
  set_src(min(tb0i + 3 * kRow, tlasti));
  load(min(tb0i + 3 * kRow, tlasti), q1);
  __syncthreads();

  // the lanes of the chunk's tokens in the first and the last block (all lanes between)
  const uint64_t mfirst = row_mask(token_bits(rs - tb0i, re - tb0i));
  const uint64_t mlast = row_mask(token_bits(rs - tlasti, re - tlasti));

  // The per-token work of a block (conv, SiLU, softplus, SiLU(z)) runs one iteration
  // ahead of its scan, so each iteration's scan and readout of block ib overlap the
  // per-token work of block ib+1: two independent dependency chains.
  struct Tok {
    float delta, du, u, zs;
  };
  auto token_work = [&](float x3, float x2, float x1, float xv, float dtv, float zv, uint64_t m) -> Tok {
    Tok o;
    float xc = cbias;
    xc = __builtin_fmaf(w0, x3, xc);
    xc = __builtin_fmaf(w1, x2, xc);
    xc = __builtin_fmaf(w2, x1, xc);
    xc = __builtin_fmaf(w3, xv, xc);
    o.u = silu(xc);
    // tokens outside the chunk get delta = 0: their step is the identity.  softplus is
    // computed on every lane (the empty asm keeps the select from becoming a branch around
    // it), then selected: one instruction, and a non-finite dt of a token outside the
    // chunk cannot reach the chunk's state through a multiply by zero
    float sp = softplus(dtv + dtb);
    asm volatile("" : "+v"(sp));
    o.delta = __builtin_amdgcn_inverse_ballot_w64(m) ? sp : 0.0f;
    o.du = o.delta * o.u;
    o.zs = FINAL ? silu(zv) : 0.0f;
    return o;
  };
  Tok tk;
  {
    const float* xr = &L.slot[0].x[j][ch];
    tk = token_work(xr[0], xr[kTS], xr[2 * kTS], xr[3 * kTS], L.slot[0].dt[j][ch], FINAL ? L.slot[0].z[j][ch] : 0.0f,
                    mfirst);
  }
  __syncthreads();  // the first iteration's staging rewrites the front rows of slot 0 read just above

  float p[kRow];
  float dsum = 0.0f;
  const uint32_t span = static_cast<uint32_t>(R.end - R.start);
  const uint32_t cko = static_cast<uint32_t>(c * NMAX + j) * 4u;
  // scalar loop state: the slots of blocks ib, ib+1, ib+2 (byte offsets), the block
  // loaded next, and the y / checkpoint rows of the previous / this block
  uint32_t s0 = 0, s1 = kSlotBytes, s2 = 2 * kSlotBytes;
  int tbl = tb0i + 4 * kRow;
  set_src(min(tbl, tlasti));
  // the source pointers of the chunk's last block (the loads past it re-read it)
  const RowSrc<IO> g_last = [&] {
    const RowSrc<IO> gs = g;
    gmem<const IO>* const gvs = gv;
    set_src(tlasti);
    const RowSrc<IO> gl = g;
    gv_last = gv;
    g = gs;
    gv = gvs;
    return gl;
  }();
  gmem<IO>* py = sbase(y + static_cast<int64_t>(tb0i - kRow) * d + c0);
  gmem<float>* pck = CKPT ? sbase(ckpt + (static_cast<int64_t>(tb0 >> 4) + R.s) * d * NMAX) : nullptr;
  int yrel = tb0i - kRow - rs;  // first token of the previous block relative to the chunk start
  // The lanes that store y of a block whose first token is rel tokens past the chunk
  // start: those of token rows t with 0 <= t + rel < span, on channels below d.  Element
  // staging: every wave, token rows 4 w + r in lanes 16 r .. 16 r + 15.  Vector staging:
  // wave 1, token row r in lanes 4 r .. 4 r + 3 (one lane per 4 channels).
  const int w4 = 4 * wv;
  const uint64_t ych_lanes = VEC ? 0x1111111111111111ull * ((1ull << min((d - c0) / 4, 4)) - 1ull)
                                 : row_mask(d - c0 >= kRowChans ? 0xFFFFu : (1u << (d - c0)) - 1u);
  auto y_lanes = [&](int rel) -> uint64_t {
    if (VEC) {
      const int lo = min(max(-rel, 0), kRow), hi = min(max(static_cast<int>(span) - rel, 0), kRow);
      const uint64_t mhi = hi >= kRow ? ~0ull : (1ull << (4 * hi)) - 1ull;
      const uint64_t mlo = lo >= kRow ? ~0ull : (1ull << (4 * lo)) - 1ull;
      return mhi & ~mlo & ych_lanes;
    }
    const int lo = min(max(-rel - w4, 0), 4), hi = min(max(static_cast<int>(span) - rel - w4, 0), 4);
    const uint64_t mhi = hi >= 4 ? ~0ull : (1ull << (16 * hi)) - 1ull;
    const uint64_t mlo = lo >= 4 ? ~0ull : (1ull << (16 * lo)) - 1ull;
    return mhi & ~mlo & ych_lanes;
  };
  // per-lane LDS offsets within a slot, held opaque so that each block's address is one add
  // of the slot's (scalar) offset rather than a rebuilt index expression
  uint32_t lx = static_cast<uint32_t>(offsetof(RowSlot, x) + (j * kTS + ch) * 4);   // x[j][ch]
  uint32_t lyw = static_cast<uint32_t>(offsetof(RowSlot, y) + (j * kTS + ch) * 4);  // y[j][ch]
  uint32_t lyr = VEC ? vy : static_cast<uint32_t>(offsetof(RowSlot, y)) + so.tc;    // y read for the store
  asm volatile("" : "+v"(lx), "+v"(lyw), "+v"(lyr));
  // y of the slot at sl, read from LDS (vector staging: four channels per lane) and then
  // stored to the rows of the lane mask m.  With vector staging only wave 1 stores, but every
  // wave reads (the same valid tile addresses): a read on one wave alone would leave the other
  // waves a value to set on every block, which costs more issue slots than the read.
  auto read_y = [&](uint32_t sl) -> f32x4_t {
    const char* yb = reinterpret_cast<const char*>(&L.slot[0]) + (sl + lyr);
    if (VEC) {
      const float2* q = reinterpret_cast<const float2*>(yb);
      const float2 a = q[0], b = q[1];
      return f32x4_t{a.x, a.y, b.x, b.y};
    }
    return f32x4_t{*reinterpret_cast<const float*>(yb), 0.0f, 0.0f, 0.0f};
  };
  auto write_y = [&](const f32x4_t& v, uint64_t m) {
    if (VEC) {
      if (wv == kKindDt && __builtin_amdgcn_inverse_ballot_w64(m)) {
        uint32_t o = vyo;
        asm volatile("" : "+v"(o));
        st_g4_uncounted(py, o, v);
      }
    } else if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      uint32_t o = yo;
      asm volatile("" : "+v"(o));
      st_g(at(py, o), v.x);
    }
  };
  // blocks between the first and the last are inside the chunk: all their rows store
  const uint64_t yfirst = y_lanes(tb0i - rs);

  auto block = [&](int ib, StageRegs& q) {
    // First the staging: block ib+2 (loaded two iterations ago) into its slot, the loads of
    // block ib+4 into the registers that held it, and y of block ib-1 out of LDS, so that
    // their latencies run under the arithmetic below.  Block ib+2's slot last held block
    // ib-1, whose tiles were last read in the iteration before (its y area is not written
    // here); the front rows go to block ib+3's slot, block ib's, whose x was read in the
    // iteration before as well.
    if (ib + 2 < nb) store(s2, s0, q);
    if (VEC || ib + 4 < nb) {
      const bool past = ib + 4 >= nb;
      const RowSrc<IO> gn = g;
      gmem<const IO>* const gvn = gv;
      if (past) {
        g = g_last;
        gv = gv_last;
      }
      load(past ? tlasti : tbl, q);
      g = gn;
      gv = gvn;
    }
    // the state before this block, stored after the staging: the hardware counts the store
    // among the outstanding accesses, so issued before the staging's waits it would make
    // them wait for it too
    if (CKPT && cvalid && (ib > 0 || tb0 == R.start || R.j == 0)) {
      uint32_t o = cko;
      asm volatile("" : "+v"(o));
      st_g_uncounted(pck, o, h);
    }
    const f32x4_t yv = FINAL ? read_y(s2) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    {
      const RowSlot& Sc = slot_at(L, s0);
      const RowSlot& Sn = slot_at(L, s1);
      float4 Bq[4], Cq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        Bq[q] = Sc.bc[0][q][j];
        Cq[q] = FINAL ? Sc.bc[1][q][j] : Bq[q];
      }
      // block ib+1's conv window (inputs of tokens t-3 .. t: rows j .. j+3), dt and z
      // (past the last block these are stale values, computed on and not used)
      const float* xr = reinterpret_cast<const float*>(reinterpret_cast<const char*>(&L.slot[0]) + (s1 + lx));
      const float x3 = xr[0], x2 = xr[kTS], x1 = xr[2 * kTS], xv = xr[3 * kTS];
      // dt[j][ch] and z[j][ch] at fixed distances from x[j][ch]
      const float dtv = xr[(offsetof(RowSlot, dt) - offsetof(RowSlot, x)) / 4];
      const float zv = FINAL ? xr[(offsetof(RowSlot, z) - offsetof(RowSlot, x)) / 4] : 0.0f;
      // all of the block's LDS reads are in flight before the arithmetic starts
      __builtin_amdgcn_sched_barrier(0);
      const Tok tn = token_work(x3, x2, x1, xv, dtv, zv, ib + 1 == nb - 1 ? mlast : ~0ull);
      if (!FINAL) dsum += tk.delta;
      row_steps<FINAL>(std::make_integer_sequence<int, kRow>{}, tk.delta, tk.du, A2, Bq, Cq, h, p);
      if (FINAL) {
        const float s = row_transpose_sum(p, j);
        *reinterpret_cast<float*>(reinterpret_cast<char*>(&L.slot[0]) + (s0 + lyw)) = __builtin_fmaf(Dc, tk.u, s) * tk.zs;
      }
      tk = tn;
    }
    if (FINAL && ib > 0) write_y(yv, ib == 1 ? yfirst : ych_lanes);
    // advance the scalar state
    const uint32_t st = s0;
    s0 = s1;
    s1 = s2;
    s2 = st;
    tbl += kRow;
    if (VEC) {
      gv = sreg(gv + vstride);
      if (FINAL) g.C = sreg(g.C + sb);
    } else {
      g.x = sreg(g.x + sx);
      g.dt = sreg(g.dt + sx);
      if (FINAL) g.z = sreg(g.z + sx);
      g.B = sreg(g.B + sb);
      if (FINAL) g.C = sreg(g.C + sb);
    }
    if (FINAL) py = sreg(py + sx);
    if (CKPT) pck = sreg(pck + static_cast<int64_t>(d) * NMAX);
    yrel += kRow;
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
  };
  for (int ib = 0; ib < nb; ib += 2) {
    block(ib, q0);
    if (ib + 1 < nb) block(ib + 1, q1);
  }
  const uint32_t xl = s2;  // slot of the last block (the rotation has moved it two places on)
  if (FINAL) write_y(read_y(xl), y_lanes(yrel));

  if (CKPT && !FINAL) return;
  if (!FINAL) {
    const float ds = row_sum(dsum);
    if (cvalid) {
      const int64_t pc = slot * d + c;
      if (j == 0) ws.a[pc] = (R.j == 0) ? -1.0f : ds;
      ws.b[pc * NMAX + j] = h;
    }
  } else if (R.j == R.ns - 1 && cvalid) {
    if (j < N) ssm_state[sc * N + j] = h;
    const int jl = static_cast<int>((R.end - 1) & (kRow - 1));  // the lane of the sequence's last token
    if (j < kKS) conv_state[sc * kKS + j] = slot_at(L, xl).x[jl + 1 + j][ch];
  }
}

}  // namespace mm
