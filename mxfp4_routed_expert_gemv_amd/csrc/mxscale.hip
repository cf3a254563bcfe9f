// Routed expert FFN for large batches on the scaled MXFP4 matrix-core
// instruction of gfx950 (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// The pages' expert FFN (kimi-k3-in-c review, "KDA/MLA/MoE" table;
// explainer page, "reduction one") multiplies E2M1 weight codes, each 32 of
// them sharing one E8M0 exponent, by activations that are never quantised.
// Once tokens are grouped by expert this is two GEMMs per expert,
// H = silu(X Wg^T) * (X Wu^T) and Y = H Wd^T, and the matrix core takes the
// MXFP4 weight bytes exactly as stored: one lane's B operand is one 16-byte
// MX block of one weight row (32 codes, low nibble first) and its scale byte.
//
// The A operand (activations) is E4M3 with one E8M0 scale per 32 elements.
// To keep the activations exact, each activation block is split into passes
// a = sum_p q_p 2^(s_0 - 127 - 5p), every q_p an E4M3 value rounded to
// nearest even from what the earlier passes left; each pass is one more MFMA
// on the same weights.  The first scale puts the block's largest magnitude in
// [2^7, 2^8); each rounding leaves at most half a unit of the 4-bit
// significand, which the next pass, 2^5 finer, holds again below 2^8.  Hence:
//   * x (bf16, 8 significant bits): 2 passes are exact for every element
//     within 2^-13 of its block's largest; smaller ones err by at most
//     2^-22 of it;
//   * h (fp32, from the gate/up epilogue): 3 passes leave a relative error of
//     at most 2^-14 per element.
// A block holding NaN or an infinity is written as E4M3 NaN codes, so every
// output that contracts over it is NaN.
//
// Tiling (wave = 64 lanes, MFMA 16 x 16 x 128):
//   * a stage is 128 contraction elements = 4 MX blocks;
//   * A lane (row i = lane % 16, group g = lane / 16) holds bytes
//     [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16) of its row's stage, and
//     the E8M0 scale of block g of its row; B lane (column j, group g) holds MX
//     block g of weight row j and its scale.  (Checked on the GPU against an
//     exact host product.)
//   * items are (m-tile, n-tile) pairs over the expert-sorted rows; stages
//     stream into LDS rings by LDS-DMA (see the grouped GEMM below).
// Every (row, output) sum runs over stages, then passes, then the matrix
// core's own order inside one instruction, none of which depends on the other
// rows of the tile: a token's bits do not depend on the batch around it.
#include <type_traits>

#include "internal.h"
#include "kern_common.h"
#include "grouped.h"

namespace k3 {
namespace {

using namespace grouped;

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kBK = 128;        // contraction elements per stage
constexpr int kPassStep = 5;    // scale exponent step between passes

// A step of a weight stream that moves 128 bytes (two 128-element stages) of
// each row at once (the one-token kernels; the grouped GEMMs with pair-wide
// weight copies): one copy instruction covers 8 rows (lane L: row
// L / 8 of the 8, 16-byte unit (L % 8) ^ swz(row)).  A row's 128 bytes sit
// at row * 128 in the slot, unit u at position u ^ swz(row): the 16 lanes
// that read one block of 16 consecutive rows then hit 16 distinct 4-bank
// groups of LDS.
__device__ __forceinline__ int step_swz(int row) { return (row >> 1) & 7; }

// LDS offset (within a step slot) of the block the lane feeds to the
// instruction for stage q (0, 1) of the step: row rw, block 4q + lg.
__device__ __forceinline__ int step_block_off(int rw, int q, int lg) {
  return rw * 128 + (((4 * q + lg) ^ step_swz(rw)) << 4);
}


// First-pass scale byte of a block from the bits of its largest magnitude
// (finite): puts that magnitude in [2^7, 2^8); blocks below 2^-110 keep the
// smallest byte for which every pass's byte is >= 0.
template <int NP>
__device__ __forceinline__ uint32_t first_scale(uint32_t max_bits) {
  const int s = (int)(max_bits >> 23) - 7;
  return (uint32_t)(s > kPassStep * (NP - 1) ? s : kPassStep * (NP - 1));
}

// The pass codes of values of a block with first scale byte sb0: v = a /
// 2^(sb0 - 127) (exact), then per pass the E4M3 code of v rounded to nearest
// even and v = (v - its value) * 32.  Every |v| met here is at most 256
// (the first pass's largest is below 2^8, a remainder is at most half a
// rounding step of 2^4, times 32), where the hardware conversion
// (v_cvt_pk_fp8_f32: OCP E4M3, round to nearest even) and its inverse equal
// a software encoder bit for bit (checked exhaustively on gfx950 over every
// such float).
// Four bf16 values (w0 low, w0 high, w1 low, w1 high): per pass one word of
// 4 codes in element order.
template <int NP>
__device__ __forceinline__ void split4(uint32_t w0, uint32_t w1, uint32_t sb0,
                                       uint32_t (&code)[NP]) {
  const float m = __uint_as_float((254u - sb0) << 23);
  float v[4] = {__uint_as_float(w0 << 16) * m, __uint_as_float(w0 & 0xFFFF0000u) * m,
                __uint_as_float(w1 << 16) * m, __uint_as_float(w1 & 0xFFFF0000u) * m};
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], pk, true);
    code[p] = (uint32_t)pk;
    if (p + 1 < NP) {
      v[0] = (v[0] - __builtin_amdgcn_cvt_f32_fp8(pk, 0)) * 32.0f;
      v[1] = (v[1] - __builtin_amdgcn_cvt_f32_fp8(pk, 1)) * 32.0f;
      v[2] = (v[2] - __builtin_amdgcn_cvt_f32_fp8(pk, 2)) * 32.0f;
      v[3] = (v[3] - __builtin_amdgcn_cvt_f32_fp8(pk, 3)) * 32.0f;
    }
  }
}
// Two fp32 values: per pass their codes in the low two bytes (a0 first).
template <int NP>
__device__ __forceinline__ void split2(float a0, float a1, uint32_t sb0, uint32_t (&code)[NP]) {
  const float m = __uint_as_float((254u - sb0) << 23);
  float v0 = a0 * m, v1 = a1 * m;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    code[p] = (uint32_t)pk & 0xFFFFu;
    if (p + 1 < NP) {
      v0 = (v0 - __builtin_amdgcn_cvt_f32_fp8(pk, 0)) * 32.0f;
      v1 = (v1 - __builtin_amdgcn_cvt_f32_fp8(pk, 1)) * 32.0f;
    }
  }
}

constexpr uint32_t kNaNCode = 0x7Fu;
constexpr uint32_t kAbsInf = 0x7F800000u;

// ------------------------------------------------------------ x quantisation
// One 32-element block of bf16 x (64 bytes at src) -> its 2 pass code words
// (pass p, elements 4i .. 4i+3 in word i, element order within the word)
// and its first-pass scale byte.
__device__ __forceinline__ uint32_t quant_xblock(const uint16_t* src, uint32_t (&packed)[2][8]) {
  constexpr int NP = 2;
  uint32_t w[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = reinterpret_cast<const uint4*>(src)[q];
    w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
  }
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    mb = max(mb, (w[i] << 16) & 0x7FFFFFFFu);
    mb = max(mb, w[i] & 0x7FFF0000u);
  }
  const bool bad = mb >= kAbsInf;
  const uint32_t sb0 = bad ? 127u + kPassStep * (NP - 1) : first_scale<NP>(mb);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t c[NP];
    split4<NP>(w[2 * i], w[2 * i + 1], sb0, c);
#pragma unroll
    for (int p = 0; p < NP; ++p) packed[p][i] = bad ? kNaNCode * 0x01010101u : c[p];
  }
  return sb0;
}

// Writes one quantised block into a stage record (272 bytes: pass 0 codes,
// pass 1 codes, scale unit) at `row`; lanes 4m .. 4m+3 hold the 4 blocks of
// one stage (blk = lane % 4) and are all active.
__device__ __forceinline__ void store_xblock(uint8_t* row, int blk, const uint32_t (&packed)[2][8],
                                             uint32_t sb0, bool write) {
  constexpr int NP = 2;
  uint32_t sc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const uint32_t mine = sb0 - kPassStep * p;
    const int l0 = threadIdx.x & ~3;
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) v |= (__shfl(mine, (l0 + q) & 63, 64) & 0xFFu) << (8 * q);
    sc[p] = v;
  }
  if (write) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uint4* dst = reinterpret_cast<uint4*>(row + p * 128 + blk * 32);
      dst[0] = uint4{packed[p][0], packed[p][1], packed[p][2], packed[p][3]};
      dst[1] = uint4{packed[p][4], packed[p][5], packed[p][6], packed[p][7]};
    }
    if (blk == 0) *reinterpret_cast<uint4*>(row + NP * 128) = uint4{sc[0], sc[1], 0u, 0u};
  }
}

// x [T][d] bf16 -> xq [T][d/128][17 units of 16 bytes]: per stage, the codes
// of pass 0 (128 bytes, element order), of pass 1, then one unit whose byte
// 4p + b is the scale of pass p, block b (bytes 8..15 zero).  One thread per
// 32-element block; the 4 threads of a stage are adjacent lanes.
__global__ __launch_bounds__(256) void quant_x(const uint16_t* __restrict__ x,
                                               uint8_t* __restrict__ xq, int64_t nblk, int d) {
  const int64_t gb = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = gb < nblk ? gb : nblk - 1;   // lanes past the end redo the last block
  uint32_t packed[2][8];
  const uint32_t sb0 = quant_xblock(x + b * 32, packed);
  const int nst = d / kBK;
  const int64_t nb_row = d / 32;
  const int64_t t = b / nb_row;
  const int j = (int)(b - t * nb_row), st = j >> 2, blk = j & 3;
  store_xblock(xq + ((size_t)t * nst + st) * (2 * 128 + 16), blk, packed, sb0, gb < nblk);
}

// ------------------------------------------- MXFP4 activations (one pass)
// The quantised-activation mode takes x and h as MXFP4 (OCP MX v1.0): per
// block of 32, scale byte s = e - 2 from the exponent field e of the block's
// largest magnitude X (so X / 2^(s-127) lies in [4, 8)), clamped to
// [0, 254] (X = 0 gives 0); each element the nearest E2M1 value of
// v / 2^(s-127), ties to the code with an even mantissa bit, above 6
// saturating to 6; a block holding a NaN or an infinity gets scale 255 and
// codes 0.  One pass, so the matrix core runs at its FP4 rate.  A record
// (a row's 128-element stage) is 5 units: 4 blocks of 16 code bytes (byte i
// = element 2i low nibble, 2i+1 high nibble, as the weights), then a unit
// whose byte b is block b's scale (bytes 4..15 unused).
constexpr int kQ4Units = 5;

// Scale byte of a block from the bits of its largest magnitude (finite).
__device__ __forceinline__ uint32_t q4_scale(uint32_t max_bits) {
  const int s = (int)(max_bits >> 23) - 2;
  return (uint32_t)(s < 0 ? 0 : (s > 254 ? 254 : s));
}
// E2M1 code of v under scale byte sb: a = |v| 2^(127 - sb) is exact, and the
// comparisons with the midpoints between E2M1 values alternate strict and
// non-strict so that ties go to the even code.
__device__ __forceinline__ uint32_t q4_code(float v, uint32_t sb) {
  const float a = ldexpf(fabsf(v), 127 - (int)sb);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// x [T][d] bf16 -> xq [T][d/128][kQ4Units units]: one thread per 32-element
// block; the 4 threads of a stage are adjacent lanes.
__global__ __launch_bounds__(256) void quant_x4(const uint16_t* __restrict__ x,
                                                uint8_t* __restrict__ xq, int64_t nblk, int d) {
  const int64_t gb = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = gb < nblk ? gb : nblk - 1;   // lanes past the end redo the last block
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
  uint32_t w[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = src[q];
    w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
  }
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    mb = max(mb, (w[i] << 16) & 0x7FFFFFFFu);
    mb = max(mb, w[i] & 0x7FFF0000u);
  }
  const bool bad = mb >= kAbsInf;
  const uint32_t sb = bad ? 255u : q4_scale(mb);
  uint32_t packed[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {   // word q: elements 8q .. 8q+7, two per byte
      const uint32_t wv = w[4 * q + h];
      const uint32_t lo = q4_code(__uint_as_float(wv << 16), sb);
      const uint32_t hi = q4_code(__uint_as_float(wv & 0xFFFF0000u), sb);
      word |= (lo | (hi << 4)) << (8 * h);
    }
    packed[q] = bad ? 0u : word;
  }
  const int nst = d / kBK;
  const int64_t nb_row = d / 32;
  const int64_t t = b / nb_row;
  const int j = (int)(b - t * nb_row), st = j >> 2, blk = j & 3;
  uint8_t* rec = xq + ((size_t)t * nst + st) * (kQ4Units * 16);
  const int l0 = threadIdx.x & ~3;
  uint32_t sc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) sc |= (__shfl(sb, (l0 + q) & 63, 64) & 0xFFu) << (8 * q);
  if (gb < nblk) {
    *reinterpret_cast<uint4*>(rec + blk * 16) = uint4{packed[0], packed[1], packed[2], packed[3]};
    if (blk == 0) *reinterpret_cast<uint4*>(rec + 64) = uint4{sc, 0u, 0u, 0u};
  }
}

// ---------------------------------------------------------- grouped GEMMs
// Tile of item `it` and its expert e.  Expert e owns items
// [s_mt[e] NT, s_mt[e+1] NT): its m-tiles times the NT n-tiles, so the
// expert of m-tile it / NT is the item's.  Within an expert the items run in
// blocks of G consecutive m-tiles, the n-tile slowest inside a block.
// Consecutive items run at the same time on the workgroups of one XCD, which
// then share each weight tile (up to G m-tiles of the expert) and each
// activation tile (consecutive n-tiles) through that XCD's L2.  G = 1 is
// m-tile-major: one search and no division beyond it / NT.
__device__ __forceinline__ int item_tile(const int* s_mt, int E, int it, int NT, int G, int& mt,
                                         int& nt) {
  const int mq = it / NT;
  const int e = __builtin_amdgcn_readfirstlane(mtile_expert(s_mt, E, mq));
  if (G == 1) {
    mt = mq;
    nt = it - mq * NT;
    return e;
  }
  const int m0 = s_mt[e], me = s_mt[e + 1] - m0;
  const int li = it - m0 * NT;
  const int blk = li / (G * NT);
  const int g0 = blk * G;
  const int gs = min(G, me - g0);
  const int r = li - blk * G * NT;
  nt = r / gs;
  mt = m0 + g0 + (r - nt * gs);
  return e;
}

// With pair-wide weight copies (PB), the copies a wave issues after the last
// copy that a stage needs, in the steady state, for either parity of the
// stage: per stage the wave issues NAW activation copies, then on every other
// stage nbc2 weight-code copies (two stages of its rows, 128 bytes each);
// the scale copies of every fourth stage are left out (fewer counted copies
// only make a wait stricter).
__host__ __device__ constexpr int newer_pairs(int RA, int RB, int NAW, int nbc2) {
  int best = 1 << 30;
  for (int par = 0; par < 2; ++par) {
    const int g = 2 * (RA + RB) + par;   // the awaited stage (any with full history)
    int na = 0, nb = 0;
    // A(g) was issued first in iteration g - RA + 1
    na += (((g - RA + 1) + RB - 1) % 2 == 0 ? nbc2 : 0);
    for (int i = g - RA + 2; i <= g - 1; ++i) na += NAW + ((i + RB - 1) % 2 == 0 ? nbc2 : 0);
    // the weight pair of stage g was issued in iteration 2 (g / 2) - RB + 1
    for (int i = 2 * (g / 2) - RB + 2; i <= g - 1; ++i)
      nb += NAW + ((i + RB - 1) % 2 == 0 ? nbc2 : 0);
    const int m = na < nb ? na : nb;
    best = m < best ? m : best;
  }
  return best;
}

// One workgroup of NC + 4 waves per CU: waves 0 .. NC-1 only compute (NC = 4
// or 8: one or two per SIMD), waves NC .. NC+3 only copy (one per SIMD), so a
// copy that stalls at issue (the memory pipeline's queues are full) does not
// hold back the matrix-core work of its SIMD.
//   * item = (m-tile of BM = 16 MF expert-sorted rows, n-tile of NC * 16 NF
//     weight rows); compute wave w computes all BM rows against weight rows
//     [16 NF w, 16 NF (w + 1)) of the n-tile;
//   * each stage (128 contraction elements) of A (activations, from L2) and
//     B (weight codes and scales, from HBM) is copied into LDS rings of RA
//     and RB slots by LDS-DMA, copy wave NC + q issuing quarter q of the
//     copies; the copy cursors run RA - 1 and RB - 1 stages ahead of the
//     compute and cross item boundaries, so the weight stream does not
//     drain between items;
//   * one s_barrier per stage, passed by both roles: before it a copy wave
//     waits for its own copies of the stage (a constant number of newer
//     copies may stay in flight; none near the end) and a compute wave for
//     its LDS reads of the previous stage; after it the copy waves refill
//     the slots of the previous stage.
// LDS layouts:
//   A slot: [BM rows][ULA = UA + 1 units of 16 bytes]: the source row's
//     stage (UA = 8 NP + 1 units) and one unused unit, padded to a whole
//     number of 256-unit copy rounds.  The 16-byte fragment reads of 16
//     rows run at the full LDS rate when the row pitch is an odd multiple
//     of 32 bytes (18 or 26 units), at half rate at 17 or 25 (measured);
//   B slot: codes [16 NF NC rows][4 MX blocks of 16 bytes], block b of row r at
//     position b ^ ((r >> 1) & 3), the swizzle of 64-byte rows that reads
//     at the full rate (with (r >> 2) & 3 it is half).  Local weight row r belongs to wave
//     r / (16 NF), fragment (r / 16) % NF, lane r % 16;
//   scale slot (a ring of SG): SGS / 4 halves of [16 NF NC rows][16 bytes],
//     half j holding the scales of stages 4 j .. 4 j + 3 of the group's SGS
//     consecutive stages (4 bytes a stage), as stored.  Copying a row's
//     scales several stages at a time keeps the copy requests per stage a
//     fraction of the rows (one 4-byte copy per row and stage halves the rate
//     at which the weight codes stream).  Each copy re-reads the row's
//     128-byte scale line, which the weight stream has usually pushed out of
//     the L2 since the row's previous copy, so 8-stage groups (SGS = 8) read
//     half the scale lines that 4-stage ones do.
// Gate/up (DOWN = false): A = xq rows gathered by token, NP = 2; wave w owns
//   the 8 NF features nt * 8 NF NC + w * 8 NF + [0, 8 NF): fragments
//   0 .. NF/2 - 1 are their gate rows, NF/2 .. NF - 1 their up rows; h is
//   written in 3 passes per 32-feature block (hq [P][f/128][25 units]).
// Down (DOWN = true): A = hq rows, NP = 3; wave w owns the 16 NF outputs
//   nt * 16 NF NC + w * 16 NF + [0, 16 NF); y fp32.
// A wave computes only the m-blocks (16 rows) that hold rows of the tile;
// with one compute wave per SIMD it reads the next m-block's A fragments
// before issuing this one's MFMAs.
// PB (pair-wide weight copies): every other stage, each weight row's next 128
// bytes (two stages) are copied at once, non-temporally, into a ring of
// (RB + 2) / 2 two-stage slots laid out as the one-token stream's steps:
// whole 128-byte lines per copy, each read once.
// Q4: the quantised-activation mode (A in MXFP4, one pass; gate/up writes h
// in MXFP4); otherwise A in exact E4M3 passes.
// SR: the weight scales bypass LDS: each compute wave loads its rows' 4 scale
// bytes of the next stage into registers (no scale ring, no scale copies).
template <int MF, int NF, int RA, int RB, bool DOWN, bool PB, bool Q4, int NC, bool SR = false,
          int SGS = 4, bool NT2 = false>
__global__ __launch_bounds__(64 * (NC + 4)) __attribute__((amdgpu_waves_per_eu(NC / 4 + 1, NC / 4 + 1))) void mx_gemm_scaled(
    const uint8_t* __restrict__ a_src, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ wsc, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, void* __restrict__ out, int d, int f, int E,
    int k, int G) {
  constexpr int NP = Q4 ? 1 : (DOWN ? 3 : 2);   // activation passes
  constexpr int NPH = 3;                        // passes of the h this kernel writes (exact)
  constexpr int UA = Q4 ? kQ4Units : NP * 8 + 1;   // units of a source row's stage
  constexpr int A_FMT = Q4 ? 4 : 0;             // A operand format: FP4 or E4M3
  constexpr int ULA = UA + 1;                   // units of an A row in LDS
  constexpr int BM = 16 * MF;
  constexpr int A_UNITS = (BM * ULA + 255) / 256 * 256;
  constexpr int A_SLOT = A_UNITS * 16;
  constexpr int NAW = A_UNITS / 256;            // A copies per wave per stage
  constexpr int WROWS = NF * 16;                // weight rows per wave
  constexpr int BROWS = NC * WROWS;             // weight rows per stage
  constexpr int FW = NF * 8;                    // gate/up: features per wave
  constexpr int B_SLOT = BROWS * 64;            // weight codes of one stage
  constexpr int S_SLOT = BROWS * 4 * SGS;       // weight scales of SGS stages (4 bytes a row and stage)
  constexpr int NBCW = BROWS * 4 / 256;         // B code copies per wave per stage
  constexpr int SCW = BROWS / 256 * (SGS / 4);  // scale copies per wave per group (SGS stages)
  // Scale groups in flight: compute stage c reads group c / SGS while the
  // copies of stage c + RB - 1 fill the group of stage c + RB + 3; a slot is
  // refilled only after its last stage was read (SG * SGS > RB + 6).
  constexpr int SG = (RB + 6) / SGS + 1;
  static_assert(SGS == 4 || SGS == 8, "scale groups of 4 or 8 stages");
  // Per stage the copies are issued A first, then B (then, on every fourth
  // stage, the scales, which are not counted below: fewer counted copies
  // only make a wait stricter).  When stage g is awaited, A(g) was followed
  // by B(g + RB - RA) and the copies of RA - 2 later stages, B(g) by the
  // copies of RB - 2 later stages.  The scales of a stage's group were copied
  // at least 4 stages before its codes.
  constexpr int NEWER_A = NBCW + (RA - 2) * (NAW + NBCW), NEWER_B = (RB - 2) * (NAW + NBCW);
  constexpr int RBP = (RB + 2) / 2;             // PB: two-stage weight slots
  constexpr int B_SLOT_P = BROWS * 128;
  constexpr int NBC = PB ? 2 * NBCW : NBCW;     // weight-code copies per wave per copy round
  constexpr int NEWER = PB ? newer_pairs(RA, RB, NAW, NBC)
                           : (NEWER_A < NEWER_B ? NEWER_A : NEWER_B);
  constexpr int RMAX = RA > RB ? RA : RB;
  static_assert(NF == 4 || NF == 8, "4 or 8 fragments per wave");
  static_assert(NC == 4 || NC == 8, "4 or 8 compute waves");
  static_assert(RA >= 2 && RB >= 2, "rings need two slots");
  static_assert((RA - 1) * NAW + (PB ? (RB / 2 + 1) * NBC : (RB - 1) * NBCW) + RB / 4 * SCW + SCW <= 63,
                "memory counter range");
  __shared__ __attribute__((aligned(16))) uint8_t sA[RA * A_SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t sB[PB ? RBP * B_SLOT_P : RB * B_SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t sS[SR ? 16 : SG * S_SLOT];
  __shared__ int s_mt[kMaxE + 1];
  __shared__ int s_wave[NC + 4];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const bool copier = wv >= NC;
  const int cq = wv & 3;                      // a copy wave's quarter of each stage's copies
  build_mtiles_n<64 * (NC + 4)>(offsets, E, BM, s_mt, s_wave);
  const int NT = DOWN ? d / BROWS : f / (NC * FW);
  const int nst = (DOWN ? f : d) / kBK;
  const ItemRange ir0 = item_range((long)s_mt[E] * NT);
  const int it_first = (int)ir0.first, it_end = (int)ir0.end, it_step = (int)ir0.step;
  const int n_items = it_first < it_end ? (it_end - it_first + it_step - 1) / it_step : 0;
  const int g_total = n_items * nst;            // stages this workgroup computes
  const size_t w_row = (size_t)(DOWN ? f : d) / 2, s_row = (size_t)(DOWN ? f : d) / 32;
  const size_t e_rows = DOWN ? (size_t)d : (size_t)2 * f;
  const size_t a_row = (size_t)nst * UA * 16;   // bytes per A source row

  // ---- copy cursors: A and B RA - 1 and RB - 1 stages ahead of the compute;
  // the scale cursor 4 stages ahead of B (a group of 4 stages' scales is
  // copied a quarter per stage, so each group has landed before its first
  // stage's codes)
  int a_it = it_first, b_it = it_first, s_it = it_first;
  int a_st = 0, b_st = 0, s_st = 4;
  if (s_st >= nst) {
    s_st -= nst;
    s_it += it_step;
  }
  int s_e = 0, s_nt = 0;
  const uint8_t* ap[NAW];
  const uint8_t* bp[NBC];
  // weight row of local row r of an n-tile
  auto grow = [&](int nt, int r) -> size_t {
    if (DOWN) return (size_t)nt * BROWS + r;
    const int cw = r / WROWS, nf = (r >> 4) % NF;
    return (size_t)((nf >= NF / 2 ? f : 0) + nt * (NC * FW) + cw * FW + (nf % (NF / 2)) * 16 +
                    (r & 15));
  };
  auto a_setup = [&]() {
    int mt, nt_unused;
    const int e = item_tile(s_mt, E, a_it, NT, G, mt, nt_unused);
    const int row0 = offsets[e] + (mt - s_mt[e]) * BM;
    const int rows = min(BM, offsets[e + 1] - row0);
#pragma unroll
    for (int q = 0; q < NAW; ++q) {
      const int unit = cq * (NAW * 64) + q * 64 + lane;
      int r = unit / ULA, u = unit - r * ULA;
      // padding units and the rows past the tile's last: all the same 16
      // bytes (the first row's first unit), so that their lanes' copies
      // merge into one request; those LDS rows are never stored from
      if (r >= rows || u >= UA) r = u = 0;
      const size_t src_row = DOWN ? (size_t)(row0 + r) : (size_t)(sorted_pair[row0 + r] / k);
      ap[q] = a_src + src_row * a_row + u * 16;
    }
  };
  auto b_setup = [&]() {
    int mt, nt;
    const int e = item_tile(s_mt, E, b_it, NT, G, mt, nt);
    const uint8_t* wbase = wq + (size_t)e * e_rows * w_row;
#pragma unroll
    for (int q = 0; q < NBC; ++q) {
      if constexpr (PB) {   // 8 rows per copy, 128 bytes each
        const int r = (cq * (NBC * 64) + q * 64 + lane) >> 3;
        bp[q] = wbase + grow(nt, r) * w_row + (((lane & 7) ^ step_swz(r)) << 4);
      } else {
        const int r = (cq * (NBCW * 64) + q * 64 + lane) >> 2;
        const int b = (lane & 3) ^ ((r >> 1) & 3);
        bp[q] = wbase + grow(nt, r) * w_row + b * 16;
      }
    }
  };
  auto s_setup = [&]() {
    int mt;
    s_e = item_tile(s_mt, E, s_it, NT, G, mt, s_nt);
  };
  const uint32_t sA_lds = lds_addr(sA), sB_lds = lds_addr(sB), sS_lds = lds_addr(sS);
  // Scales of group grp (SGS stages) of the scale cursor's item, every row of
  // the tile (4 SGS bytes a row), this wave's quarter of the rows, into scale
  // slot `slot`; one copy per 64 rows and half, on every SGS-th stage.  Past
  // the last item the copy repeats rows of expert 0 into a slot nobody reads.
  auto issue_scales = [&](int grp, int slot, bool valid) {
#pragma unroll
    for (int q = 0; q < BROWS / 256; ++q)
#pragma unroll
      for (int hf = 0; hf < SGS / 4; ++hf) {
        const int r0 = cq * (BROWS / 4) + q * 64, r = r0 + lane;
        const uint8_t* src = valid ? wsc + ((size_t)s_e * e_rows + grow(s_nt, r)) * s_row +
                                         grp * (4 * SGS) + hf * 16
                                   : wsc + (size_t)r * s_row + hf * 16;
        dma16_raw(src, sS_lds + (uint32_t)(slot * S_SLOT + hf * (BROWS * 16) + r0 * 16));
      }
  };
  auto issue_a = [&](int g) {
    if (a_it >= it_end) return;
    const uint32_t base = sA_lds + (uint32_t)((g % RA) * A_SLOT + cq * (NAW * 64) * 16);
#pragma unroll
    for (int q = 0; q < NAW; ++q) dma16_raw(ap[q] + (size_t)a_st * (UA * 16), base + q * 1024);
    if (++a_st == nst) {
      a_st = 0;
      a_it += it_step;
      if (a_it < it_end) a_setup();
    }
  };
  auto issue_b = [&](int g) {
    if (b_it >= it_end) return;
    if constexpr (PB) {
      if ((b_st & 1) == 0) {
        const uint32_t base = sB_lds + (uint32_t)(((g >> 1) % RBP) * B_SLOT_P);
#pragma unroll
        for (int q = 0; q < NBC; ++q) {
          // read once per m-tile: non-temporal, except with MXFP4 activations,
          // where the items of a block share each weight tile through the L2
          if constexpr (Q4)
            dma16_raw(bp[q] + (b_st >> 1) * kBK, base + (cq * (NBC * 64) + q * 64) * 16);
          else
            dma16_raw_nt(bp[q] + (b_st >> 1) * kBK, base + (cq * (NBC * 64) + q * 64) * 16);
        }
      }
    } else {
      const uint32_t base = sB_lds + (uint32_t)((g % RB) * B_SLOT);
      // NT2: the copy of a line's second half (odd stages) is non-temporal:
      // the line has served both its stages and leaves the L2 first
      if (NT2 && (b_st & 1)) {
#pragma unroll
        for (int q = 0; q < NBCW; ++q)
          dma16_raw_nt(bp[q] + b_st * (kBK / 2), base + (cq * (NBCW * 64) + q * 64) * 16);
      } else {
#pragma unroll
        for (int q = 0; q < NBCW; ++q)
          dma16_raw(bp[q] + b_st * (kBK / 2), base + (cq * (NBCW * 64) + q * 64) * 16);
      }
    }
    if (!SR && s_st % SGS == 0) issue_scales(s_st / SGS, (g / SGS + 1) % SG, s_it < it_end);
    if (++b_st == nst) {
      b_st = 0;
      b_it += it_step;
      if (b_it < it_end) b_setup();
    }
    if (++s_st == nst) {
      s_st = 0;
      s_it += it_step;
      if (s_it < it_end) s_setup();
    }
  };
  if (copier && a_it < it_end) {
    a_setup();
    b_setup();
    if (s_it < it_end) s_setup();
    // scales of the first item's first group (older than every counted copy)
    if constexpr (!SR) {
      int mt, nt;
      const int e = item_tile(s_mt, E, it_first, NT, G, mt, nt);
#pragma unroll
      for (int q = 0; q < BROWS / 256; ++q)
#pragma unroll
        for (int hf = 0; hf < SGS / 4; ++hf) {
          const int r0 = cq * (BROWS / 4) + q * 64;
          dma16_raw(wsc + ((size_t)e * e_rows + grow(nt, r0 + lane)) * s_row + hf * 16,
                    sS_lds + (uint32_t)(hf * (BROWS * 16) + r0 * 16));
        }
    }
  }
  if (copier) {
    // prologue, in the loop's order: virtual stage j issues A(j + RA - 1), B(j + RB - 1)
#pragma unroll
    for (int j = -(RMAX - 1); j < 0; ++j) {
      if (j + RA - 1 >= 0) issue_a(j + RA - 1);
      if (j + RB - 1 >= 0) issue_b(j + RB - 1);
    }
    // g_total stages, as many barriers as the compute waves pass: wait for
    // this stage's copies, barrier, copy ahead
#pragma unroll 1
    for (int g = 0; g < g_total; ++g) {
      if (g + RMAX - 2 < g_total) wait_vmem<NEWER>();
      else wait_vmem<0>();
      wg_barrier();
      issue_a(g + RA - 1);
      issue_b(g + RB - 1);
    }
    wait_vmem<0>();
    return;
  }

  int g = 0;   // global stage index of this workgroup
  // SR: each compute wave loads its own rows' scale words (4 bytes: a row's 4
  // blocks of one stage) straight into registers, one stage ahead; the
  // cursor crosses item boundaries.  Fragment nf's rows sit nf_off(nf) rows
  // after fragment 0's.
  int sc_it = it_first, sc_st = 0;
  const uint8_t* scp = nullptr;
  uint32_t sc_c[NF], sc_n[NF];
  auto nf_off = [&](int nf) -> int {
    return DOWN ? nf * 16 : (nf >= NF / 2 ? f : 0) + (nf % (NF / 2)) * 16;
  };
  auto sc_setup = [&]() {
    int mt, nt;
    const int e = item_tile(s_mt, E, sc_it, NT, G, mt, nt);
    scp = wsc + ((size_t)e * e_rows + grow(nt, wv * WROWS + ln)) * s_row;
  };
  auto sc_load = [&](uint32_t (&w)[NF]) {
    if (sc_it >= it_end) return;
#pragma unroll
    for (int nf = 0; nf < NF; ++nf)
      w[nf] = *reinterpret_cast<const uint32_t*>(scp + (size_t)nf_off(nf) * s_row + sc_st * 4);
    if (++sc_st == nst) {
      sc_st = 0;
      sc_it += it_step;
      if (sc_it < it_end) sc_setup();
    }
  };
  if constexpr (SR) {
    if (sc_it < it_end) sc_setup();
    sc_load(sc_c);
  }
  // One item with NMB m-blocks (16 rows each) holding rows of the tile: the
  // stage loop and epilogue are specialised on NMB, so the accumulators stay
  // in the matrix-core registers and no MFMA sits behind a branch.
  auto run_item = [&](auto nmb_c, int nt, int row0, int rows) {
    constexpr int NMB = decltype(nmb_c)::value;
    f32x4_t acc[NMB][NF];
#pragma unroll
    for (int i = 0; i < NMB; ++i)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) acc[i][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int s = 0; s < nst; ++s, ++g) {
      if constexpr (SR) sc_load(sc_n);
      wait_lds();
      wg_barrier();
      const uint8_t* abase = sA + (g % RA) * A_SLOT;
      const uint8_t* bbase = PB ? sB + ((g >> 1) % RBP) * B_SLOT_P : sB + (g % RB) * B_SLOT;
      const uint8_t* sbase =
          sS + ((g / SGS) % SG) * S_SLOT + ((g % SGS) >> 2) * (BROWS * 16) + (g & 3) * 4 + lg;
      i32x8_t bq[NF];
      int bs[NF];
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const int r = wv * WROWS + nf * 16 + ln;
        if constexpr (SR) bs[nf] = (int)((sc_c[nf] >> (8 * lg)) & 0xFFu);
        else bs[nf] = sbase[r * 16];
        const uint4 c = *reinterpret_cast<const uint4*>(
            PB ? bbase + step_block_off(r, g & 1, lg)
               : bbase + r * 64 + ((lg ^ ((r >> 1) & 3)) * 16));
        bq[nf] = i32x8_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
      }
      // A fragments of m-block i: pass p = bytes [16 lg, +16) and
      // [64 + 16 lg, +16) of the pass's 128, and the scale byte of block lg
      // two compute waves per SIMD (NC = 8) cover each other's LDS reads, so
      // an m-block's A fragments are read just before its MFMAs; with one,
      // the next block's are read ahead
      constexpr int NAB = NC == 8 ? 1 : 2;
      i32x8_t a[NAB][NP];
      int as[NAB][NP];
      auto load_a = [&](int i, i32x8_t (&av)[NP], int (&sv)[NP]) {
        const uint8_t* arow = abase + (i * 16 + ln) * (ULA * 16);
        if constexpr (Q4) {   // the lane's MX block of the row, as a weight lane
          const uint4 c = *reinterpret_cast<const uint4*>(arow + lg * 16);
          av[0] = i32x8_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
          sv[0] = arow[(UA - 1) * 16 + lg];
        } else {
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const uint4 lo = *reinterpret_cast<const uint4*>(arow + (p * 8 + lg) * 16);
            const uint4 hi = *reinterpret_cast<const uint4*>(arow + (p * 8 + 4 + lg) * 16);
            av[p] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                            (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            sv[p] = arow[(UA - 1) * 16 + p * 4 + lg];
          }
        }
      };
      if constexpr (NAB == 2) load_a(0, a[0], as[0]);
#pragma unroll
      for (int i = 0; i < NMB; ++i) {
        if constexpr (NAB == 2) {
          if (i + 1 < NMB) load_a(i + 1, a[(i + 1) & 1], as[(i + 1) & 1]);
        } else {
          load_a(i, a[0], as[0]);
        }
        const int ab = NAB == 2 ? (i & 1) : 0;
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            acc[i][nf] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a[ab][p], bq[nf], acc[i][nf], A_FMT, 4, 0, as[ab][p], 0, bs[nf]);
      }
      if constexpr (SR) {
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) sc_c[nf] = sc_n[nf];
      }
    }
    if (DOWN) {
      float* y = static_cast<float*>(out);
#pragma unroll
      for (int i = 0; i < NMB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = i * 16 + lg * 4 + r;
          if (m < rows) {
            float* yr = y + (size_t)(row0 + m) * d + nt * BROWS + wv * WROWS + ln;
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) yr[nf * 16] = acc[i][nf][r];
          }
        }
    } else if constexpr (Q4) {
      // h = silu(g) * u for this wave's 32-feature blocks, quantised to
      // MXFP4; a block's largest magnitude is reduced over the 16 lanes of the
      // row (lanes with the same lg), and two neighbouring lanes' codes share
      // a byte (every lane takes part in both exchanges).
      uint8_t* hq = static_cast<uint8_t*>(out);
      const size_t h_row = (size_t)(f / kBK) * (kQ4Units * 16);
#pragma unroll
      for (int hb = 0; hb < NF / 4; ++hb) {
        const int fb = (nt * (NC * FW) + wv * FW) / 32 + hb, hst = fb >> 2, blk = fb & 3;
#pragma unroll
        for (int i = 0; i < NMB; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = i * 16 + lg * 4 + r;
            const float h0 = silu_mul(acc[i][2 * hb][r], acc[i][2 * hb + NF / 2][r]);
            const float h1 = silu_mul(acc[i][2 * hb + 1][r], acc[i][2 * hb + 1 + NF / 2][r]);
            uint32_t mb =
                max(__float_as_uint(h0) & 0x7FFFFFFFu, __float_as_uint(h1) & 0x7FFFFFFFu);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, o, 64));
            const bool bad = mb >= kAbsInf;
            const uint32_t sb = bad ? 255u : q4_scale(mb);
            const uint32_t c0 = bad ? 0u : q4_code(h0, sb), c1 = bad ? 0u : q4_code(h1, sb);
            const uint32_t n0 = (uint32_t)__shfl_xor((int)c0, 1, 64);
            const uint32_t n1 = (uint32_t)__shfl_xor((int)c1, 1, 64);
            if (m < rows) {
              uint8_t* hr = hq + (size_t)(row0 + m) * h_row + (size_t)hst * (kQ4Units * 16);
              if ((ln & 1) == 0) {   // features ln, ln + 1 and 16 + ln, 17 + ln of the block
                hr[blk * 16 + (ln >> 1)] = (uint8_t)(c0 | (n0 << 4));
                hr[blk * 16 + 8 + (ln >> 1)] = (uint8_t)(c1 | (n1 << 4));
              }
              if (ln == 0) hr[64 + blk] = (uint8_t)sb;
            }
          }
      }
    } else {
      // h = silu(g) * u for this wave's 32-feature blocks, written as NPH
      // passes; a block's largest magnitude is reduced over the 16 lanes of
      // the row (lanes with the same lg), every lane taking part.
      uint8_t* hq = static_cast<uint8_t*>(out);
      const size_t h_row = (size_t)(f / kBK) * (NPH * 128 + 16);
#pragma unroll
      for (int hb = 0; hb < NF / 4; ++hb) {
        const int fb = (nt * (NC * FW) + wv * FW) / 32 + hb, hst = fb >> 2, blk = fb & 3;
#pragma unroll
        for (int i = 0; i < NMB; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = i * 16 + lg * 4 + r;
            const float h0 = silu_mul(acc[i][2 * hb][r], acc[i][2 * hb + NF / 2][r]);
            const float h1 = silu_mul(acc[i][2 * hb + 1][r], acc[i][2 * hb + 1 + NF / 2][r]);
            uint32_t mb =
                max(__float_as_uint(h0) & 0x7FFFFFFFu, __float_as_uint(h1) & 0x7FFFFFFFu);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, o, 64));
            const bool bad = mb >= kAbsInf;
            const uint32_t sb0 = bad ? 127u + kPassStep * (NPH - 1) : first_scale<NPH>(mb);
            uint32_t c01[NPH];
            split2<NPH>(h0, h1, sb0, c01);
            if (m < rows) {
              uint8_t* hr = hq + (size_t)(row0 + m) * h_row + (size_t)hst * (NPH * 128 + 16);
#pragma unroll
              for (int p = 0; p < NPH; ++p) {
                hr[p * 128 + blk * 32 + ln] = (uint8_t)(bad ? kNaNCode : c01[p]);
                hr[p * 128 + blk * 32 + 16 + ln] = (uint8_t)(bad ? kNaNCode : c01[p] >> 8);
              }
              if (ln == 0) {
#pragma unroll
                for (int p = 0; p < NPH; ++p)
                  hr[NPH * 128 + p * 4 + blk] = (uint8_t)(sb0 - kPassStep * p);
              }
            }
          }
      }
    }
  };
  for (int it = it_first; it < it_end; it += it_step) {
    int mt, nt;
    const int e = item_tile(s_mt, E, it, NT, G, mt, nt);
    const int row0 = offsets[e] + (mt - s_mt[e]) * BM;
    const int rows = min(BM, offsets[e + 1] - row0);
    // 1 .. MF live blocks (an m-tile holds 1 .. BM rows); clamped, so that
    // every item runs its nst stages and barriers
    const int nmb = max(1, min(MF, (rows + 15) >> 4));
    static_assert(MF <= 8, "item dispatch covers up to 8 m-blocks");
    switch (nmb) {
      case 1: run_item(std::integral_constant<int, 1>(), nt, row0, rows); break;
      case 2: if constexpr (MF >= 2) run_item(std::integral_constant<int, 2>(), nt, row0, rows); break;
      case 3: if constexpr (MF >= 3) run_item(std::integral_constant<int, 3>(), nt, row0, rows); break;
      case 4: if constexpr (MF >= 4) run_item(std::integral_constant<int, 4>(), nt, row0, rows); break;
      case 5: if constexpr (MF >= 5) run_item(std::integral_constant<int, 5>(), nt, row0, rows); break;
      case 6: if constexpr (MF >= 6) run_item(std::integral_constant<int, 6>(), nt, row0, rows); break;
      case 7: if constexpr (MF >= 7) run_item(std::integral_constant<int, 7>(), nt, row0, rows); break;
      default: if constexpr (MF >= 8) run_item(std::integral_constant<int, 8>(), nt, row0, rows); break;
    }
  }
}

// -------------------------------------------------------------- one token
// The decode batch of one token: each touched expert's weights are read once,
// so the product is bound by how fast they stream, and decoding E2M1 on the
// vector ALU (a quarter-rate conversion per two weights) costs about half the
// streaming time.  Here the weights go to the matrix core as stored, as in
// the grouped GEMM, and every wave streams only its own weight rows:
//   * the wave's rows are NF fragments of 16 rows; their codes stream through
//     a private LDS ring of D stages by LDS-DMA (issued D - 1 stages ahead,
//     the wave's own wait counts, no barrier inside the stream); their scales
//     for all stages sit in LDS (copied once, contiguous rows);
//   * the activation row (x in 2 passes, quantised in the workgroup by the
//     same code as quant_x; or the pair's h row in 3 passes) sits in LDS and
//     every lane reads its A operand from it, so all 16 rows of the product
//     are the token's (row 0 is stored); the raw row arrives by LDS-DMA
//     while the workgroup scans the offsets, and x is quantised while the
//     first weight stages fly;
//   * per output, stages then passes then the instruction's own order, as in
//     the grouped GEMM: the token's bits equal its row's bits there.
// One workgroup (4 waves) per (active expert, 128 features) for gate/up and
// per (active expert, 64 NF output rows) for down.  For one token an active
// expert has exactly one pair, at sorted position j = its rank.

// The expert whose range of sorted positions holds j, or -1.  Each thread
// checks 4 consecutive experts per round with all its loads issued at once,
// so the scan costs one memory latency for up to 1024 experts.
__device__ int expert_at(const int32_t* __restrict__ offsets, int E, int j, int* s_e) {
  const int t4 = threadIdx.x * 4;
  int o[5];
#pragma unroll
  for (int u = 0; u < 5; ++u) o[u] = offsets[min(t4 + u, E)];
  if (threadIdx.x == 0) *s_e = -1;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (t4 + u < E && o[u] <= j && o[u + 1] > j) *s_e = t4 + u;
  for (int b = t4 + 4 * (int)blockDim.x; b < E; b += 4 * (int)blockDim.x) {
#pragma unroll
    for (int u = 0; u < 5; ++u) o[u] = offsets[min(b + u, E)];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (b + u < E && o[u] <= j && o[u + 1] > j) *s_e = b + u;
  }
  __syncthreads();
  return *s_e;
}

constexpr int kDn1Ring = 2;
// One-token gate/up scales: a group is 16 stages (64 bytes) of each of the
// wave's 64 rows, read 4 lanes a row (16 rows and 16 to 32 cache lines per
// copy instruction; 16 bytes of each of 64 rows cost 64 lines per copy, which
// made the scale stream a tenth of the kernel's time); two group slots.
constexpr int kGu1ScaleGroup = 16, kGu1ScaleSlot = 64 * kGu1ScaleGroup * 4;

// Quantises one step of the token's row (stages 2t, 2t+1: 8 blocks of 32)
// into two stage records at rec (the layout quant_x writes) with one wave:
// lane l takes elements 4l .. 4l+3 of the step (8 bytes at src), the 8 lanes
// of a block reduce its largest magnitude, and every element goes through
// the same split as in quant_xblock, so the records equal quant_x's bit for
// bit.
__device__ __forceinline__ void quant_x_step(const uint8_t* src, uint8_t* rec, int lane) {
  constexpr int NP = 2, REC = (NP * 8 + 1) * 16;
  const uint2 raw = *reinterpret_cast<const uint2*>(src);
  const uint32_t w[2] = {raw.x, raw.y};
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    mb = max(mb, (w[i] << 16) & 0x7FFFFFFFu);
    mb = max(mb, w[i] & 0x7FFF0000u);
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, o, 64));
  const bool bad = mb >= kAbsInf;
  const uint32_t sb0 = bad ? 127u + kPassStep * (NP - 1) : first_scale<NP>(mb);
  uint32_t pk[NP];
  split4<NP>(w[0], w[1], sb0, pk);
#pragma unroll
  for (int p = 0; p < NP; ++p) pk[p] = bad ? kNaNCode * 0x01010101u : pk[p];
  uint8_t* r = rec + (lane >> 5) * REC;
#pragma unroll
  for (int p = 0; p < NP; ++p) *reinterpret_cast<uint32_t*>(r + p * 128 + (lane & 31) * 4) = pk[p];
  if ((lane & 7) == 0) {
    const int blk = (lane >> 3) & 3;
#pragma unroll
    for (int p = 0; p < NP; ++p) r[NP * 128 + 4 * p + blk] = (uint8_t)(sb0 - kPassStep * p);
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gateup_1tok(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ wsc, const int32_t* __restrict__ offsets,
    uint8_t* __restrict__ hq, int d, int f, int E) {
  constexpr int NF = 4, NP = 2, NPH = 3, UA = NP * 8 + 1, REC = UA * 16;
  constexpr int ROWS = NF * 16, SLOT = ROWS * 128, NCI = ROWS / 8;
  constexpr int GSTEPS = kGu1ScaleGroup / 2;    // steps per scale group
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int s_e;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ln = lane & 15, lg = lane >> 4;
  const int ngr = f / 128;
  const int j = blockIdx.x / ngr, nt = blockIdx.x - j * ngr;
  const int nst = d / kBK, nb = d / 32, nsp = nst / 2;
  const size_t w_row = (size_t)d / 2, s_row = (size_t)nb;
  const int x_pad = (2 * d + 1023) / 1024 * 1024;
  uint8_t* s_x = lds;                                        // the bf16 row
  uint8_t* s_xq = lds + x_pad + wv * 2 * (2 * REC);          // the wave's 2 step records
  uint8_t* s_sc = lds + x_pad + 8 * (2 * REC) + wv * 2 * kGu1ScaleSlot;
  uint8_t* s_ring = lds + x_pad + 8 * (2 * REC) + 4 * 2 * kGu1ScaleSlot + wv * D * SLOT;
  // the token's row by LDS-DMA (1 KB per instruction, the waves in turn),
  // beside the offsets scan
  {
    const int units = d / 8;
    const uint8_t* xs = reinterpret_cast<const uint8_t*>(x);
    for (int u = wv; u * 64 < units; u += 4)
      dma16_raw(xs + min(u * 64 + lane, units - 1) * 16, lds_addr(s_x) + (uint32_t)(u * 1024));
  }
  const int e = expert_at(offsets, E, j, &s_e);
  if (e < 0) {   // no expert at this rank: the row's copies land before the exit
    wait_vmem<0>();
    return;
  }
  // the wave's rows: 0 .. 31 gate rows F + r, 32 .. 63 the up rows; fragment
  // nf holds rows nf * 16 + [0, 16)
  const int F = nt * 128 + wv * 32;
  const size_t gate0 = (size_t)e * 2 * f + F, up0 = gate0 + f;
  auto wrow = [&](int r) { return r < 32 ? gate0 + r : up0 + (r - 32); };
  const uint8_t* cp[NCI];
#pragma unroll
  for (int i = 0; i < NCI; ++i) {
    const int r = i * 8 + (lane >> 3);
    cp[i] = wq + wrow(r) * w_row + (((lane & 7) ^ step_swz(r)) << 4);
  }
  // scales: group g (stages 16 g .. 16 g + 15) into slot g % 2 as
  // [row][64 bytes]; copy k covers rows 16 k .. 16 k + 15, lane l row
  // 16 k + l / 4, 16-byte unit l % 4 (clamped to the row's last unit past its
  // end: the last group of a row shorter than 64 bytes).  Group g + 1 is
  // copied as soon as group g - 1's slot is free: with the codes of the
  // step D - 1 after group g's first.
  const uint8_t* sp[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) sp[k] = wsc + wrow(16 * k + (lane >> 2)) * s_row;
  const uint32_t ring_l = lds_addr(s_ring), sc_l = lds_addr(s_sc);
  const int ngroups = (nsp + GSTEPS - 1) / GSTEPS;
  auto issue_group = [&](int g) {
    if (g >= ngroups) return;
    const int off = min(g * (kGu1ScaleGroup * 4) + (lane & 3) * 16, nb - 16);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      dma16_raw(sp[k] + off, sc_l + (uint32_t)((g & 1) * kGu1ScaleSlot + k * 1024));
  };
  issue_group(0);
  auto issue = [&](int t) {
    if (t >= nsp) return;
    if (t % GSTEPS == D - 1) issue_group(t / GSTEPS + 1);
    const uint32_t slot = ring_l + (uint32_t)((t % D) * SLOT);
#pragma unroll
    for (int i = 0; i < NCI; ++i) dma16_raw_nt(cp[i] + t * 128, slot + i * 1024);
  };
#pragma unroll
  for (int t = 0; t < D - 1; ++t) issue(t);
  // The row's copies are older than the 4 scale and (D - 1) NCI code copies
  // issued since (the weight stream starts without waiting for the row); the
  // barrier shares each wave's part of the row.
  if (nsp >= D - 1) wait_vmem<4 + (D - 1) * NCI>();
  else wait_vmem<0>();
  __syncthreads();
  // Each wave quantises the row itself, one step ahead of use, while its
  // copies fly (spread over the stream, the quantisation costs the stream
  // less than one pass over the whole row up front).
  quant_x_step(s_x + lane * 8, s_xq, lane);

  f32x4_t acc[NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) acc[nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int t = 0; t < nsp; ++t) {
    issue(t + D - 1);
    if (t + 1 < nsp) quant_x_step(s_x + (t + 1) * 512 + lane * 8, s_xq + ((t + 1) & 1) * (2 * REC), lane);
    // copies still allowed in flight: steps t+1 .. t+D-1, NCI each (the scale
    // copies issued with them are not counted: fewer counted copies only make
    // the wait stricter); a scale group was copied with codes of an earlier
    // step than its first, so that step's wait covers it
    static_assert(D >= 2 && D <= 4 && D - 1 < GSTEPS, "rings of 2 to 4 steps");
    if (t + D - 1 < nsp) wait_vmem<(D - 1) * NCI>();
    else wait_vmem<0>();
    const uint8_t* slot = s_ring + (t % D) * SLOT;
    const uint8_t* sc = s_sc + ((t / GSTEPS) & 1) * kGu1ScaleSlot;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      i32x8_t bq[NF];
      int bs[NF];
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const int rw = nf * 16 + ln;
        const uint4 c = *reinterpret_cast<const uint4*>(slot + step_block_off(rw, q, lg));
        bq[nf] = i32x8_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
        bs[nf] = sc[rw * (kGu1ScaleGroup * 4) + ((t % GSTEPS) * 2 + q) * 4 + lg];
      }
      const uint8_t* arow = s_xq + (t & 1) * (2 * REC) + q * REC;
      i32x8_t a[NP];
      int as[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint4 lo = *reinterpret_cast<const uint4*>(arow + (p * 8 + lg) * 16);
        const uint4 hi = *reinterpret_cast<const uint4*>(arow + (p * 8 + 4 + lg) * 16);
        a[p] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        as[p] = arow[(UA - 1) * 16 + p * 4 + lg];
      }
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
          acc[nf] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[p], bq[nf], acc[nf], 0, 4,
                                                                     0, as[p], 0, bs[nf]);
    }
  }
  // h of the token (row 0) for the wave's 32 features, in NPH passes, as in
  // the grouped GEMM's epilogue
  const size_t h_row = (size_t)(f / kBK) * (NPH * 128 + 16);
  const int fb = F / 32, hst = fb >> 2, blk = fb & 3;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = lg * 4 + r;
    const float h0 = silu_mul(acc[0][r], acc[2][r]);
    const float h1 = silu_mul(acc[1][r], acc[3][r]);
    uint32_t mb = max(__float_as_uint(h0) & 0x7FFFFFFFu, __float_as_uint(h1) & 0x7FFFFFFFu);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, o, 64));
    const bool bad = mb >= kAbsInf;
    const uint32_t sb0 = bad ? 127u + kPassStep * (NPH - 1) : first_scale<NPH>(mb);
    uint32_t c01[NPH];
    split2<NPH>(h0, h1, sb0, c01);
    if (m == 0) {
      uint8_t* hr = hq + (size_t)j * h_row + (size_t)hst * (NPH * 128 + 16);
#pragma unroll
      for (int p = 0; p < NPH; ++p) {
        hr[p * 128 + blk * 32 + ln] = (uint8_t)(bad ? kNaNCode : c01[p]);
        hr[p * 128 + blk * 32 + 16 + ln] = (uint8_t)(bad ? kNaNCode : c01[p] >> 8);
      }
      if (ln == 0) {
#pragma unroll
        for (int p = 0; p < NPH; ++p) hr[NPH * 128 + p * 4 + blk] = (uint8_t)(sb0 - kPassStep * p);
      }
    }
  }
}

template <int NF, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void down_1tok(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ wsc, const int32_t* __restrict__ offsets, float* __restrict__ y,
    int d, int f, int E, int cpe) {
  constexpr int NP = 3, UA = NP * 8 + 1;
  constexpr int ROWS = NF * 16, SLOT = ROWS * 128, NCI = ROWS / 8;
  static_assert((D - 1) * NCI <= 63, "copies in flight within the wait counter");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int s_e;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ln = lane & 15, lg = lane >> 4;
  const int j = blockIdx.x / cpe, c = blockIdx.x - j * cpe;
  const int nst = f / kBK, nb = f / 32, nsp = nst / 2;
  const size_t w_row = (size_t)f / 2, s_row = (size_t)nb;
  const int h_row = nst * UA * 16;
  const int h_pad = (h_row + 1023) / 1024 * 1024;
  const int sreg = (ROWS * nb + 1023) / 1024 * 1024;   // scales of the wave's rows, padded
  uint8_t* s_hq = lds;
  uint8_t* s_sc = lds + h_pad + wv * sreg;
  uint8_t* s_ring = lds + h_pad + 4 * sreg + wv * D * SLOT;
  // the pair's h row by LDS-DMA (1 KB per instruction, the waves in turn),
  // beside the offsets scan
  {
    const int units = h_row / 16;
    const uint8_t* hs = hq + (size_t)j * h_row;
    for (int u = wv; u * 64 < units; u += 4)
      dma16_raw(hs + min(u * 64 + lane, units - 1) * 16, lds_addr(s_hq) + (uint32_t)(u * 1024));
  }
  const int e = expert_at(offsets, E, j, &s_e);
  if (e < 0) {   // no expert at this rank: the row's copies land before the exit
    wait_vmem<0>();
    return;
  }
  const int o0 = c * (4 * ROWS) + wv * ROWS;   // the wave's first output row
  const size_t row0 = (size_t)e * d + o0;
  const uint8_t* cp[NCI];
#pragma unroll
  for (int i = 0; i < NCI; ++i) {
    const int r = i * 8 + (lane >> 3);
    cp[i] = wq + (row0 + r) * w_row + (((lane & 7) ^ step_swz(r)) << 4);
  }
  const uint32_t ring_l = lds_addr(s_ring);
  auto issue = [&](int t) {
    if (t >= nsp) return;
    const uint32_t slot = ring_l + (uint32_t)((t % D) * SLOT);
#pragma unroll
    for (int i = 0; i < NCI; ++i) dma16_raw_nt(cp[i] + t * 128, slot + i * 1024);
  };
  // scales of the wave's rows (ROWS rows of nb bytes, one contiguous run),
  // 1 KB per copy into [row][16-byte unit] with unit k of row r at position
  // (k + r / 4) mod (nb / 16): the 16 rows a scale read spans then sit in 16
  // distinct 4-bank groups (unrotated, rows 64 bytes apart alias onto 4)
  {
    const int ku = nb / 16, units = ROWS * ku;
    const uint8_t* sbase = wsc + row0 * s_row;
    for (int u = 0; u * 64 < units; ++u) {
      const int S = min(u * 64 + lane, units - 1);
      const int r = S / ku;
      int k = S - r * ku - (r >> 2) % ku;
      if (k < 0) k += ku;
      dma16_raw(sbase + (size_t)(r * ku + k) * 16, lds_addr(s_sc) + (uint32_t)(u * 1024));
    }
  }
#pragma unroll
  for (int t = 0; t < D - 1; ++t) issue(t);
  // The weight stream starts before the h row is awaited: the row's (and the
  // scales') copies are older than the first step's NCI code copies (when
  // nsp < D - 1 fewer were issued: wait for everything); the barrier shares
  // each wave's part of the row.
  if (nsp >= D - 1) wait_vmem<(D - 1) * NCI>();
  else wait_vmem<0>();
  __syncthreads();

  f32x4_t acc[NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) acc[nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int t = 0; t < nsp; ++t) {
    issue(t + D - 1);
    if (t + D - 1 < nsp) wait_vmem<(D - 1) * NCI>();
    else wait_vmem<0>();
    const uint8_t* slot = s_ring + (t % D) * SLOT;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int st = 2 * t + q;
      i32x8_t bq[NF];
      int bs[NF];
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const int rw = nf * 16 + ln;
        const uint4 cc = *reinterpret_cast<const uint4*>(slot + step_block_off(rw, q, lg));
        bq[nf] = i32x8_t{(int)cc.x, (int)cc.y, (int)cc.z, (int)cc.w, 0, 0, 0, 0};
        int kk = (st >> 2) + (rw >> 2) % (nb / 16);
        if (kk >= nb / 16) kk -= nb / 16;
        bs[nf] = s_sc[rw * nb + kk * 16 + (st & 3) * 4 + lg];
      }
      const uint8_t* arow = s_hq + st * (UA * 16);
      i32x8_t a[NP];
      int as[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint4 lo = *reinterpret_cast<const uint4*>(arow + (p * 8 + lg) * 16);
        const uint4 hi = *reinterpret_cast<const uint4*>(arow + (p * 8 + 4 + lg) * 16);
        a[p] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        as[p] = arow[(UA - 1) * 16 + p * 4 + lg];
      }
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
          acc[nf] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[p], bq[nf], acc[nf], 0, 4,
                                                                     0, as[p], 0, bs[nf]);
    }
  }
  if (lg == 0) {   // row 0 of every fragment: lanes 0 .. 15, element 0
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) y[(size_t)j * d + o0 + nf * 16 + ln] = acc[nf][0];
  }
}

// LDS bytes of the one-token kernels (0 when the shape does not fit).
int gateup_1tok_lds(const k3moe_shape& s, int ring) {
  const int n = (2 * s.d + 1023) / 1024 * 1024 + 8 * 2 * 272 + 4 * 2 * kGu1ScaleSlot +
                4 * ring * 64 * 128;
  return n <= 160 * 1024 - 256 ? n : 0;
}
// NF = fragments (16 output rows each) per wave.
int down_1tok_lds(const k3moe_shape& s, int NF) {
  const int nst = s.f / kBK, nb = s.f / 32;
  const int sreg = (16 * NF * nb + 1023) / 1024 * 1024;
  const int n = (nst * 25 * 16 + 1023) / 1024 * 1024 + 4 * sreg + 4 * kDn1Ring * NF * 16 * 128;
  return n <= 160 * 1024 - 256 && s.d % (64 * NF) == 0 ? n : 0;
}

}  // namespace

size_t xq_bytes(const k3moe_shape& s) {
  const size_t rec = s.act == K3MOE_ACT_MXFP4 ? kQ4Units * 16 : 2 * 128 + 16;
  return (size_t)s.T * (size_t)(s.d / kBK) * rec;
}

namespace {
// m-tiles per item block: with MXFP4 activations, blocks of 8 when an
// expert is expected to span several m-tiles (the weights of a block are then
// shared through the L2); the exact passes keep m-tile-major order, whose
// activation tiles (the larger stream there) are shared instead.
int pick_g(const k3moe_shape& s, int mf) {
  return s.act == K3MOE_ACT_MXFP4 && (double)s.T * s.k / s.E > 16.0 * mf ? 8 : 1;
}
// With MXFP4 activations the tall tiles are 128 rows instead of 96: the A
// slot of a stage is the same size (rows round up to whole copies), and a
// stage's matrix work (a quarter of the exact passes') grows by a third
// against the same copy latency (skewed prefill gate/up 9.37 -> 8.51 ms,
// down 5.85 -> 5.14 ms; uniform 4096-token batch 3.38 -> 3.32 and 1.95 ->
// 1.90 ms).
int q4_tile(const k3moe_shape& s, int mf) {
  return s.act == K3MOE_ACT_MXFP4 && mf > 3 ? 8 : mf;
}
}  // namespace

hipError_t launch_gateup_scaled(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                                const int32_t* offsets, const int32_t* sorted_pair, float* h,
                                uint8_t* xq, hipStream_t st) {
  const bool q4 = s.act == K3MOE_ACT_MXFP4;
  if (s.T == 1 && !q4) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint8_t* w = static_cast<const uint8_t*>(b.w13);
    const uint8_t* ws = static_cast<const uint8_t*>(b.w13_scale);
    uint8_t* hb = reinterpret_cast<uint8_t*>(h);
    const unsigned g1 = (unsigned)(s.k * (s.f / 128));
    if (const int lds = gateup_1tok_lds(s, 4)) {
      gateup_1tok<4><<<g1, 256, lds, st>>>(xb, w, ws, offsets, hb, s.d, s.f, s.E);
      return hipGetLastError();
    }
    if (const int lds = gateup_1tok_lds(s, 3)) {
      gateup_1tok<3><<<g1, 256, lds, st>>>(xb, w, ws, offsets, hb, s.d, s.f, s.E);
      return hipGetLastError();
    }
  }
  const int64_t nblk = s.T * (int64_t)(s.d / 32);
  if (q4)
    quant_x4<<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(static_cast<const uint16_t*>(x), xq,
                                                             nblk, s.d);
  else
    quant_x<<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(static_cast<const uint16_t*>(x), xq,
                                                            nblk, s.d);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const uint8_t* w = static_cast<const uint8_t*>(b.w13);
  const uint8_t* ws = static_cast<const uint8_t*>(b.w13_scale);
  const dim3 g(grouped_grid());   // one workgroup per CU
  const int mf = q4_tile(s, pick_mf(s, 6));
  const int G = pick_g(s, mf);
  const bool sg8 = (s.d / kBK) % 8 == 0;   // scale copies of 8 stages
#define K3_SC(MF, NF, RA, RB, PB, NC)                                                        \
  do {                                                                                        \
    if (q4)                                                                                   \
      mx_gemm_scaled<MF, NF, RA, RB, false, PB, true, NC><<<g, 64 * (NC + 4), 0, st>>>(       \
          xq, w, ws, offsets, sorted_pair, h, s.d, s.f, s.E, s.k, G);                         \
    else                                                                                      \
      mx_gemm_scaled<MF, NF, RA, RB, false, PB, false, NC><<<g, 64 * (NC + 4), 0, st>>>(      \
          xq, w, ws, offsets, sorted_pair, h, s.d, s.f, s.E, s.k, G);                         \
  } while (0)
  // Short m-tiles (weight-stream bound): pair-wide non-temporal weight copies
  // with deep rings on both operands (a wave waits for its copies in issue
  // order, so the activation ring's lead also bounds the weights').  Taller
  // ones: 96-row m-tiles, so that an expert's weights are streamed once for
  // up to 96 of its pairs.  Their gate/up takes 8 compute waves (n-tiles of
  // 512 weight rows), so each activation stage is copied for half as many
  // n-tiles; LDS then holds two one-stage weight slots (4.99 -> 4.85 ms on a
  // uniform 4096-token batch, 16.0 -> 14.8 ms on the Zipf-skewed 16384-token
  // one, against 4 compute waves with 4 weight slots; same bits).
  // With MXFP4 activations a stage holds a quarter of the matrix-core work
  // of the exact passes, so the tall tiles (128 rows, q4_tile) take deeper
  // rings (3 activation stages, 4 weight stages) to keep more copies in
  // flight; 8 compute waves, which leave room for 3 weight stages only, were
  // slower there (skewed batch 8.9 -> 11.3 ms).
  if (mf <= 1) K3_SC(1, 4, 4, 4, true, 4);
  else if (mf <= 3) K3_SC(3, 4, 2, 5, false, 4);
  else if (q4)
    mx_gemm_scaled<8, 4, 3, 4, false, true, true, 4><<<g, 512, 0, st>>>(
        xq, w, ws, offsets, sorted_pair, h, s.d, s.f, s.E, s.k, G);
  // The exact 96-row tiles copy each weight row's scales 8 stages at a time
  // where the stage count allows: every scale copy re-reads the row's
  // 128-byte scale line (the weight stream has pushed it out of the L2 since
  // the row's previous copy), so this halves those reads (a uniform
  // 4096-token batch reads 19.1 GB per launch instead of 22.7; 1-2% faster,
  // same bits).  The MXFP4-activation tiles keep 4-stage groups (8 were
  // slower on the skewed batch).  The tall exact tiles (gate/up and down)
  // copy the second half of each weight line non-temporally (NT2): the
  // line is then done with and leaves the L2 before the scale and
  // activation lines (gate/up 19.1 -> 18.3 GB, down 10.2 -> 9.1 GB per
  // launch at 4096 tokens; time unchanged to 2% faster, same bits).
  else if (sg8)
    mx_gemm_scaled<6, 4, 2, 2, false, false, false, 8, false, 8, true><<<g, 768, 0, st>>>(
        xq, w, ws, offsets, sorted_pair, h, s.d, s.f, s.E, s.k, G);
  else K3_SC(6, 4, 2, 2, false, 8);
#undef K3_SC
  return hipGetLastError();
}

hipError_t launch_down_scaled(const k3moe_shape& s, const k3moe_expert_bank& b, const float* h,
                              const int32_t* offsets, float* y, hipStream_t st) {
  const bool q4 = s.act == K3MOE_ACT_MXFP4;
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(h);
  const uint8_t* w = static_cast<const uint8_t*>(b.w2);
  const uint8_t* ws = static_cast<const uint8_t*>(b.w2_scale);
  if (s.T == 1 && !q4) {
    // 7 fragments per wave where d allows (d = 7168: 256 workgroups), else 8
    if (const int lds = down_1tok_lds(s, 7)) {
      const int cpe = s.d / (64 * 7);
      down_1tok<7, kDn1Ring><<<(unsigned)(s.k * cpe), 256, lds, st>>>(hb, w, ws, offsets, y, s.d,
                                                                      s.f, s.E, cpe);
      return hipGetLastError();
    }
    if (const int lds = down_1tok_lds(s, 8)) {
      const int cpe = s.d / (64 * 8);
      down_1tok<8, kDn1Ring><<<(unsigned)(s.k * cpe), 256, lds, st>>>(hb, w, ws, offsets, y, s.d,
                                                                      s.f, s.E, cpe);
      return hipGetLastError();
    }
  }
  const dim3 g(grouped_grid());
  const int mf = q4_tile(s, pick_mf(s, 6));
  const int G = pick_g(s, mf);
#define K3_SD(MF, NF, RA, RB, PB, NC)                                                        \
  do {                                                                                        \
    if (q4)                                                                                   \
      mx_gemm_scaled<MF, NF, RA, RB, true, PB, true, NC><<<g, 64 * (NC + 4), 0, st>>>(        \
          hb, w, ws, offsets, nullptr, y, s.d, s.f, s.E, s.k, G);                             \
    else                                                                                      \
      mx_gemm_scaled<MF, NF, RA, RB, true, PB, false, NC><<<g, 64 * (NC + 4), 0, st>>>(       \
          hb, w, ws, offsets, nullptr, y, s.d, s.f, s.E, s.k, G);                             \
  } while (0)
  // The same tiles as the gate/up.  The tall exact ones take 8 compute waves
  // with their weight scales in registers (SR): the 3-pass activation slots
  // leave no LDS for a scale ring beside 512-row weight stages (2.98 -> 2.67
  // ms on a uniform 4096-token batch, 10.75 -> 9.11 ms on the Zipf 16384-token
  // one, against 4 compute waves; same bits).  Scales in registers slow the
  // gate/up (4.83 -> 5.62 ms), whose LDS holds its scale ring.
  if (mf <= 1) K3_SD(1, 4, 4, 4, true, 4);
  else if (mf <= 3) K3_SD(3, 4, 2, 5, false, 4);
  else if (q4)
    mx_gemm_scaled<8, 4, 3, 4, true, true, true, 4><<<g, 512, 0, st>>>(
        hb, w, ws, offsets, nullptr, y, s.d, s.f, s.E, s.k, G);
  else
    mx_gemm_scaled<6, 4, 2, 2, true, false, false, 8, true, 4, true><<<g, 768, 0, st>>>(
        hb, w, ws, offsets, nullptr, y, s.d, s.f, s.E, s.k, G);
#undef K3_SD
  return hipGetLastError();
}

}  // namespace k3
