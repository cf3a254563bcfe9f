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

// E4M3 (OCP, bias 7, no infinities) encoding of v, |v| <= 256, rounded to
// nearest even; q receives the value the code stands for.
__device__ __forceinline__ uint32_t e4m3_rne(float v, float& q) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const uint32_t ua = __float_as_uint(v) & 0x7FFFFFFFu;
  uint32_t code;
  float qa;
  if (ua < 0x3C800000u) {   // below 2^-6: subnormal codes, steps of 2^-9
    const float n = __builtin_rintf(__uint_as_float(ua) * 512.0f);
    code = (uint32_t)n;     // 8 is the smallest normal, 2^-6
    qa = n * (1.0f / 512.0f);
  } else {
    const uint32_t ur = (ua + 0x7FFFFu + ((ua >> 20) & 1u)) & 0xFFF00000u;
    code = (((ur >> 23) - 120u) << 3) | ((ur >> 20) & 7u);
    qa = __uint_as_float(ur);
  }
  q = __uint_as_float(__float_as_uint(qa) | (sign << 24));
  return code | sign;
}

// First-pass scale byte of a block from the bits of its largest magnitude
// (finite): puts that magnitude in [2^7, 2^8); blocks below 2^-110 keep the
// smallest byte for which every pass's byte is >= 0.
template <int NP>
__device__ __forceinline__ uint32_t first_scale(uint32_t max_bits) {
  const int s = (int)(max_bits >> 23) - 7;
  return (uint32_t)(s > kPassStep * (NP - 1) ? s : kPassStep * (NP - 1));
}

// The NP pass codes of one value of a block with first scale byte sb0.
template <int NP>
__device__ __forceinline__ void split_passes(float a, uint32_t sb0, uint32_t (&code)[NP]) {
  float v = a * __uint_as_float((254u - sb0) << 23);   // a / 2^(sb0 - 127), exact
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float q;
    code[p] = e4m3_rne(v, q);
    v = (v - q) * 32.0f;
  }
}

constexpr uint32_t kNaNCode = 0x7Fu;
constexpr uint32_t kAbsInf = 0x7F800000u;

// ------------------------------------------------------------ x quantisation
// x [T][d] bf16 -> xq [T][d/128][17 units of 16 bytes]: per stage, the codes
// of pass 0 (128 bytes, element order), of pass 1, then one unit whose byte
// 4p + b is the scale of pass p, block b (bytes 8..15 zero).  One thread per
// 32-element block; the 4 threads of a stage are adjacent lanes.
__global__ __launch_bounds__(256) void quant_x(const uint16_t* __restrict__ x,
                                               uint8_t* __restrict__ xq, int64_t nblk, int d) {
  constexpr int NP = 2;
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
  const uint32_t sb0 = bad ? 127u + kPassStep * (NP - 1) : first_scale<NP>(mb);
  uint32_t packed[NP][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int p = 0; p < NP; ++p) packed[p][i] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t bits = e & 1 ? (w[2 * i + (e >> 1)] & 0xFFFF0000u) : (w[2 * i + (e >> 1)] << 16);
      uint32_t c[NP];
      split_passes<NP>(__uint_as_float(bits), sb0, c);
#pragma unroll
      for (int p = 0; p < NP; ++p) packed[p][i] |= (bad ? kNaNCode : c[p]) << (8 * e);
    }
  }
  const int nst = d / kBK;
  const int64_t nb_row = d / 32;
  const int64_t t = b / nb_row;
  const int j = (int)(b - t * nb_row), st = j >> 2, blk = j & 3;
  uint8_t* row = xq + ((size_t)t * nst + st) * (NP * 128 + 16);
  // scale unit: lane blk == 0 of the stage gathers its neighbours' bytes
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
  if (gb < nblk) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uint4* dst = reinterpret_cast<uint4*>(row + p * 128 + blk * 32);
      dst[0] = uint4{packed[p][0], packed[p][1], packed[p][2], packed[p][3]};
      dst[1] = uint4{packed[p][4], packed[p][5], packed[p][6], packed[p][7]};
    }
    if (blk == 0) *reinterpret_cast<uint4*>(row + NP * 128) = uint4{sc[0], sc[1], 0u, 0u};
  }
}

// ---------------------------------------------------------- grouped GEMMs
// One workgroup of 4 waves per CU, one wave per SIMD (so each wave may hold
// 512 registers).  Every wave both copies and computes:
//   * item = (m-tile of BM = 16 MF expert-sorted rows, n-tile of 4 * 16 NF
//     weight rows); wave w computes all BM rows against weight rows
//     [16 NF w, 16 NF (w + 1)) of the n-tile;
//   * each stage (128 contraction elements) of A (activations, from L2) and
//     B (weight codes and scales, from HBM) is copied into LDS rings of RA
//     and RB slots by LDS-DMA, each wave issuing a quarter of the copies;
//     the copy cursors run RA - 1 and RB - 1 stages ahead of the compute
//     and cross item boundaries, so the weight stream does not drain
//     between items;
//   * one s_barrier per stage: before it each wave waits for its own copies
//     of the stage (a constant number of newer copies may stay in flight;
//     none near the end) and for its LDS reads of the previous stage; after
//     it the slots of the previous stage are refilled.
// LDS layouts:
//   A slot: [BM rows][UA units of 16 bytes] exactly as the source row's
//     stage (UA = 8 NP + 1, odd, so the 16 rows of a fragment read fall on
//     distinct banks), padded to a whole number of 256-unit copy rounds;
//   B slot: codes [64 NF rows][4 MX blocks of 16 bytes], block b of row r at
//     position b ^ ((r >> 2) & 3).  Local weight row r belongs to wave
//     r / (16 NF), fragment (r / 16) % NF, lane r % 16;
//   scale slot (a ring of SG): [64 NF rows][16 bytes], the scales of 4
//     consecutive stages of the row (4 bytes a stage), as stored.  Copying a
//     row's scales 4 stages at a time keeps the copy requests per stage a
//     quarter of the rows; one 4-byte copy per row and stage halves the rate
//     at which the weight codes stream.
// Gate/up (DOWN = false): A = xq rows gathered by token, NP = 2; wave w owns
//   the 8 NF features nt * 32 NF + w * 8 NF + [0, 8 NF): fragments
//   0 .. NF/2 - 1 are their gate rows, NF/2 .. NF - 1 their up rows; h is
//   written in 3 passes per 32-feature block (hq [P][f/128][25 units]).
// Down (DOWN = true): A = hq rows, NP = 3; wave w owns the 16 NF outputs
//   nt * 64 NF + w * 16 NF + [0, 16 NF); y fp32.
// A wave computes only the m-blocks (16 rows) that hold rows of the tile,
// and reads the next m-block's A fragments before issuing this one's MFMAs.
template <int MF, int NF, int RA, int RB, bool DOWN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void mx_gemm_scaled(
    const uint8_t* __restrict__ a_src, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ wsc, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, void* __restrict__ out, int d, int f, int E,
    int k) {
  constexpr int NP = DOWN ? 3 : 2;              // activation passes
  constexpr int NPH = 3;                        // passes of the h this kernel writes
  constexpr int UA = NP * 8 + 1;
  constexpr int BM = 16 * MF;
  constexpr int A_UNITS = (BM * UA + 255) / 256 * 256;
  constexpr int A_SLOT = A_UNITS * 16;
  constexpr int NAW = A_UNITS / 256;            // A copies per wave per stage
  constexpr int WROWS = NF * 16;                // weight rows per wave
  constexpr int BROWS = 4 * WROWS;              // weight rows per stage
  constexpr int FW = NF * 8;                    // gate/up: features per wave
  constexpr int B_SLOT = BROWS * 64;            // weight codes of one stage
  constexpr int S_SLOT = BROWS * 16;            // weight scales of 4 stages (16 bytes a row)
  constexpr int NBCW = BROWS * 4 / 256;         // B code copies per wave per stage
  constexpr int NBW = NBCW + 1;                 // + one scale copy (a quarter group)
  constexpr int QR = BROWS / 16;                // scale rows per wave per stage
  // Scale groups in flight: compute stage c reads group c / 4 while the
  // copies of stage c + RB - 1 fill group (c + RB - 1) / 4 + 1; a slot is
  // refilled only after its last stage was read (SG * 4 > RB + 6).
  constexpr int SG = (RB + 6) / 4 + 1;
  // Per stage the copies are issued A first, then B.  When stage g is
  // awaited, A(g) was followed by B(g + RB - RA) and the copies of RA - 2
  // later stages, B(g) by the copies of RB - 2 later stages.
  constexpr int NEWER_A = NBW + (RA - 2) * (NAW + NBW), NEWER_B = (RB - 2) * (NAW + NBW);
  constexpr int NEWER = NEWER_A < NEWER_B ? NEWER_A : NEWER_B;
  constexpr int RMAX = RA > RB ? RA : RB;
  static_assert(NF == 4 || NF == 8, "4 or 8 fragments per wave");
  static_assert(RA >= 2 && RB >= 2, "rings need two slots");
  static_assert((RA - 1) * NAW + (RB - 1) * NBW <= 63, "memory counter range");
  __shared__ __attribute__((aligned(16))) uint8_t sA[RA * A_SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t sB[RB * B_SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t sS[SG * S_SLOT];
  __shared__ int s_mt[kMaxE + 1];
  __shared__ int s_wave[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  build_mtiles_n<256>(offsets, E, BM, s_mt, s_wave);
  const int NT = DOWN ? d / BROWS : f / (4 * FW);
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
  const uint8_t* bp[NBCW];
  // weight row of local row r of an n-tile
  auto grow = [&](int nt, int r) -> size_t {
    if (DOWN) return (size_t)nt * BROWS + r;
    const int cw = r / WROWS, nf = (r >> 4) % NF;
    return (size_t)((nf >= NF / 2 ? f : 0) + nt * (4 * FW) + cw * FW + (nf % (NF / 2)) * 16 +
                    (r & 15));
  };
  auto a_setup = [&]() {
    const int mt = a_it / NT;
    const int e = __builtin_amdgcn_readfirstlane(mtile_expert(s_mt, E, mt));
    const int row0 = offsets[e] + (mt - s_mt[e]) * BM;
    const int rows = min(BM, offsets[e + 1] - row0);
#pragma unroll
    for (int q = 0; q < NAW; ++q) {
      const int unit = wv * (NAW * 64) + q * 64 + lane;
      int r = unit / UA, u = unit - r * UA;
      if (r >= BM) r = u = 0;   // padding units: any valid source
      const int rr = min(r, rows - 1);
      const size_t src_row = DOWN ? (size_t)(row0 + rr) : (size_t)(sorted_pair[row0 + rr] / k);
      ap[q] = a_src + src_row * a_row + u * 16;
    }
  };
  auto b_setup = [&]() {
    const int mt = b_it / NT, nt = b_it - mt * NT;
    const int e = __builtin_amdgcn_readfirstlane(mtile_expert(s_mt, E, mt));
    const uint8_t* wbase = wq + (size_t)e * e_rows * w_row;
#pragma unroll
    for (int q = 0; q < NBCW; ++q) {
      const int r = (wv * (NBCW * 64) + q * 64 + lane) >> 2;
      const int b = (lane & 3) ^ ((r >> 2) & 3);
      bp[q] = wbase + grow(nt, r) * w_row + b * 16;
    }
  };
  auto s_setup = [&]() {
    const int mt = s_it / NT;
    s_nt = s_it - mt * NT;
    s_e = __builtin_amdgcn_readfirstlane(mtile_expert(s_mt, E, mt));
  };
  const uint32_t sA_lds = lds_addr(sA), sB_lds = lds_addr(sB), sS_lds = lds_addr(sS);
  // Scales of quarter q (rows [q BROWS / 4, (q + 1) BROWS / 4), this
  // wave's quarter of them) of group grp of the scale cursor's item, into scale
  // slot `slot` (16 bytes a row; lanes beyond the half stay idle).  Past the
  // last item the copy repeats a valid row into a slot nobody reads, so every
  // stage issues one copy.
  auto issue_scales = [&](int q, int grp, int slot, bool valid) {
    const int r0 = q * (BROWS / 4) + wv * QR;
    const int r = r0 + (lane < QR ? lane : 0);
    const uint8_t* src = valid ? wsc + ((size_t)s_e * e_rows + grow(s_nt, r)) * s_row + grp * 16
                               : wsc + (size_t)r * s_row;
    const uint32_t dst = sS_lds + (uint32_t)(slot * S_SLOT + r0 * 16);
    if (lane < QR) dma16_raw(src, dst);
  };
  auto issue_a = [&](int g) {
    if (a_it >= it_end) return;
    const uint32_t base = sA_lds + (uint32_t)((g % RA) * A_SLOT + wv * (NAW * 64) * 16);
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
    const uint32_t base = sB_lds + (uint32_t)((g % RB) * B_SLOT);
#pragma unroll
    for (int q = 0; q < NBCW; ++q)
      dma16_raw(bp[q] + b_st * (kBK / 2), base + (wv * (NBCW * 64) + q * 64) * 16);
    issue_scales(s_st & 3, s_st >> 2, (g / 4 + 1) % SG, s_it < it_end);
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
  if (a_it < it_end) {
    a_setup();
    b_setup();
    if (s_it < it_end) s_setup();
    // scales of the first item's first group (older than every counted copy)
    const int mt = it_first / NT, nt = it_first - mt * NT;
    const int e = __builtin_amdgcn_readfirstlane(mtile_expert(s_mt, E, mt));
#pragma unroll
    for (int q = 0; q < BROWS / 256; ++q) {
      const int r0 = wv * (BROWS / 4) + q * 64;
      dma16_raw(wsc + ((size_t)e * e_rows + grow(nt, r0 + lane)) * s_row,
                sS_lds + (uint32_t)(r0 * 16));
    }
  }
  // prologue, in the loop's order: virtual stage j issues A(j + RA - 1), B(j + RB - 1)
#pragma unroll
  for (int j = -(RMAX - 1); j < 0; ++j) {
    if (j + RA - 1 >= 0) issue_a(j + RA - 1);
    if (j + RB - 1 >= 0) issue_b(j + RB - 1);
  }

  int g = 0;   // global stage index of this workgroup
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
      if (g + RMAX - 2 < g_total) wait_vmem<NEWER>();
      else wait_vmem<0>();
      wait_lds();
      wg_barrier();
      issue_a(g + RA - 1);
      issue_b(g + RB - 1);
      const uint8_t* abase = sA + (g % RA) * A_SLOT;
      const uint8_t* bbase = sB + (g % RB) * B_SLOT;
      const uint8_t* sbase = sS + ((g / 4) % SG) * S_SLOT + (g & 3) * 4 + lg;
      i32x8_t bq[NF];
      int bs[NF];
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const int r = wv * WROWS + nf * 16 + ln;
        bs[nf] = sbase[r * 16];
        const uint4 c =
            *reinterpret_cast<const uint4*>(bbase + r * 64 + ((lg ^ ((r >> 2) & 3)) * 16));
        bq[nf] = i32x8_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
      }
      // A fragments of m-block i: pass p = bytes [16 lg, +16) and
      // [64 + 16 lg, +16) of the pass's 128, and the scale byte of block lg
      i32x8_t a[2][NP];
      int as[2][NP];
      auto load_a = [&](int i, i32x8_t (&av)[NP], int (&sv)[NP]) {
        const uint8_t* arow = abase + (i * 16 + ln) * (UA * 16);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const uint4 lo = *reinterpret_cast<const uint4*>(arow + (p * 8 + lg) * 16);
          const uint4 hi = *reinterpret_cast<const uint4*>(arow + (p * 8 + 4 + lg) * 16);
          av[p] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          sv[p] = arow[(UA - 1) * 16 + p * 4 + lg];
        }
      };
      load_a(0, a[0], as[0]);
#pragma unroll
      for (int i = 0; i < NMB; ++i) {
        if (i + 1 < NMB) load_a(i + 1, a[(i + 1) & 1], as[(i + 1) & 1]);
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            acc[i][nf] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a[i & 1][p], bq[nf], acc[i][nf], 0, 4, 0, as[i & 1][p], 0, bs[nf]);
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
    } else {
      // h = silu(g) * u for this wave's 32-feature blocks, written as NPH
      // passes; a block's largest magnitude is reduced over the 16 lanes of
      // the row (lanes with the same lg), every lane taking part.
      uint8_t* hq = static_cast<uint8_t*>(out);
      const size_t h_row = (size_t)(f / kBK) * (NPH * 128 + 16);
#pragma unroll
      for (int hb = 0; hb < NF / 4; ++hb) {
        const int fb = (nt * (4 * FW) + wv * FW) / 32 + hb, hst = fb >> 2, blk = fb & 3;
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
            uint32_t c0[NPH], c1[NPH];
            split_passes<NPH>(h0, sb0, c0);
            split_passes<NPH>(h1, sb0, c1);
            if (m < rows) {
              uint8_t* hr = hq + (size_t)(row0 + m) * h_row + (size_t)hst * (NPH * 128 + 16);
#pragma unroll
              for (int p = 0; p < NPH; ++p) {
                hr[p * 128 + blk * 32 + ln] = (uint8_t)(bad ? kNaNCode : c0[p]);
                hr[p * 128 + blk * 32 + 16 + ln] = (uint8_t)(bad ? kNaNCode : c1[p]);
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
    const int mt = it / NT, nt = it - mt * NT;
    const int e = __builtin_amdgcn_readfirstlane(mtile_expert(s_mt, E, mt));
    const int row0 = offsets[e] + (mt - s_mt[e]) * BM;
    const int rows = min(BM, offsets[e + 1] - row0);
    const int nmb = (rows + 15) >> 4;
    static_assert(MF <= 6, "item dispatch covers up to 6 m-blocks");
    switch (nmb) {
      case 1: run_item(std::integral_constant<int, 1>(), nt, row0, rows); break;
      case 2: if constexpr (MF >= 2) run_item(std::integral_constant<int, 2>(), nt, row0, rows); break;
      case 3: if constexpr (MF >= 3) run_item(std::integral_constant<int, 3>(), nt, row0, rows); break;
      case 4: if constexpr (MF >= 4) run_item(std::integral_constant<int, 4>(), nt, row0, rows); break;
      case 5: if constexpr (MF >= 5) run_item(std::integral_constant<int, 5>(), nt, row0, rows); break;
      default: if constexpr (MF >= 6) run_item(std::integral_constant<int, 6>(), nt, row0, rows); break;
    }
  }
  wait_vmem<0>();
}

}  // namespace

size_t xq_bytes(const k3moe_shape& s) {
  return (size_t)s.T * (size_t)(s.d / kBK) * (2 * 128 + 16);
}

hipError_t launch_gateup_scaled(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                                const int32_t* offsets, const int32_t* sorted_pair, float* h,
                                uint8_t* xq, hipStream_t st) {
  const int64_t nblk = s.T * (int64_t)(s.d / 32);
  quant_x<<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(static_cast<const uint16_t*>(x), xq,
                                                          nblk, s.d);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const uint8_t* w = static_cast<const uint8_t*>(b.w13);
  const uint8_t* ws = static_cast<const uint8_t*>(b.w13_scale);
  const dim3 g(mfma_grid() / 2);   // one workgroup per CU
#define K3_SC(MF, NF, RA, RB)                                                                \
  mx_gemm_scaled<MF, NF, RA, RB, false><<<g, dim3(256), 0, st>>>(xq, w, ws, offsets,         \
                                                                 sorted_pair, h, s.d, s.f, s.E, s.k)
  // Short m-tiles (weight-stream bound): a deep weight ring.  Taller ones:
  // 96-row m-tiles, so that an expert's weights are streamed once for up to
  // 96 of its pairs.
  const int mf = pick_mf(s, 6);
  if (mf <= 1) K3_SC(1, 4, 2, 7);
  else if (mf <= 3) K3_SC(3, 4, 2, 5);
  else K3_SC(6, 4, 2, 4);
#undef K3_SC
  return hipGetLastError();
}

hipError_t launch_down_scaled(const k3moe_shape& s, const k3moe_expert_bank& b, const float* h,
                              const int32_t* offsets, float* y, hipStream_t st) {
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(h);
  const uint8_t* w = static_cast<const uint8_t*>(b.w2);
  const uint8_t* ws = static_cast<const uint8_t*>(b.w2_scale);
  const dim3 g(mfma_grid() / 2);
#define K3_SD(MF, NF, RA, RB)                                                                 \
  mx_gemm_scaled<MF, NF, RA, RB, true><<<g, dim3(256), 0, st>>>(hb, w, ws, offsets, nullptr, y, \
                                                                s.d, s.f, s.E, s.k)
  const int mf = pick_mf(s, 6);
  if (mf <= 1) K3_SD(1, 4, 2, 7);
  else if (mf <= 3) K3_SD(3, 4, 2, 5);
  else K3_SD(6, 4, 2, 3);
#undef K3_SD
  return hipGetLastError();
}

}  // namespace k3
