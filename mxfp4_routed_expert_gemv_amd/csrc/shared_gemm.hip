// Shared (always-on) experts in the matrix-core class, and the router's bf16
// logits there: bf16 GEMMs on the matrix cores (v_mfma_f32_16x16x32_bf16)
// with both operands staged through LDS rings by LDS-DMA.
//
// The pages keep two shared experts beside the routed ones and run every
// token through both (the kimi-k3-in-c review, "at a glance" table; the
// README's shard census): S = sum_j Wd_j (silu(Wg_j x) * (Wu_j x)).  With
// bf16 weights and thousands of tokens these are two dense GEMMs:
//   gate/up: [T x d] . [d x 2 S fs]  ->  h = silu(g) * u      [T][S][fs]
//   down:    [T x S fs] . [S fs x d] ->  y                    [T][d]
//
// Structure (one workgroup of 8 waves per CU, two waves per SIMD):
//   * waves 0..3 only compute, waves 4..7 only copy: each stage (64
//     contraction elements) of the activation tile and of the weight tile is
//     copied into a ring of kRing LDS slots, copy wave 4 + q issuing quarter
//     q of the copies, kRing - 1 stages ahead of the compute; one s_barrier
//     per stage is passed by both roles (a copy wave first waits for its own
//     copies of that stage, a compute wave for its LDS reads of the previous
//     one), and after it the copy waves refill the previous stage's slot;
//   * items are (n-tile, m-tile of 128 tokens) in 8 contiguous ranges (one
//     per XCD), ordered so that the workgroups of an XCD work on 8 m-tiles x
//     4 n-tiles at a time and share both operands through their L2;
//   * LDS rows are 128 bytes (64 bf16); 16-byte unit u of row r sits at
//     position u ^ ((r >> 1) & 7), so the 16 rows that one fragment read
//     touches fall on 16 distinct 4-bank groups.
// Every (token, output) value is the chain of the other shared-expert
// kernels (stages of 64 elements in order, then the two 32-element halves
// of a stage, and in the down product the hi then the lo bf16 part of h):
// a token's bits do not depend on the batch or tile around it.
//   gate/up: waves side by side along the weights, each 128 tokens x 64
//     weight rows (32 gate rows and the matching 32 up rows); the epilogue
//     writes h already split for the down product: hi = bf16(h),
//     lo = bf16(h - hi), two [T][S fs] bf16 planes;
//   down: waves 2 x 2, each 64 tokens x 64 outputs; A = the hi and lo planes
//     of h, contracted over both experts in one chain; y fp32.
#include "internal.h"
#include "kern_common.h"
#include "grouped.h"

namespace k3 {
namespace {

using namespace grouped;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kBK = 64;        // contraction elements per stage
constexpr int kRing = 3;       // LDS slots per operand ring

__device__ __forceinline__ int row_swz(int r) { return (r >> 1) & 7; }

// Tile of item `it`: groups of kGM consecutive m-tiles, the m-tile fastest
// within a group, then the n-tile, so that 32 consecutive items (the ones the
// workgroups of one XCD run at the same time) are 8 m-tiles x 4 n-tiles and
// share both operands through that XCD's L2.
constexpr int kGM = 8;
__device__ __forceinline__ void item_tile(int it, int n_mt, int NT, int& mt, int& nt) {
  const int grp = it / (kGM * NT), first = grp * kGM;
  const int gsz = min(n_mt - first, kGM);
  const int r = it - grp * (kGM * NT);
  nt = r / gsz;
  mt = first + (r - nt * gsz);
}
// LDS byte offset of unit u (16 bytes: elements 8u .. 8u+7 of the stage) of row r
__device__ __forceinline__ int unit_off(int r, int u) { return r * 128 + ((u ^ row_swz(r)) << 4); }

__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* base, int r, int u) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(base + unit_off(r, u)));
}

// Tile shape: BM tokens per m-tile, WM compute waves along the tokens and
// 4 / WM along the weight rows, NF 16-row weight fragments per wave (gate/up:
// NF / 2 gate fragments, then the matching up fragments).
// The products this kernel runs: the shared experts' gate/up and down, and
// the router's bf16 logits (x [T][d] against w_router [E][d], fp32 out).
constexpr int kGateUp = 0, kDown = 1, kLogits = 2;

template <int MODE, int BM_, int WM_, int NF_, int NC_>
struct Tiles {
  static constexpr bool DOWN = MODE == kDown;
  static constexpr int BM = BM_, WM = WM_, NF = NF_;
  static constexpr int NPL = DOWN ? 2 : 1;        // activation planes (h hi, h lo)
  static constexpr int NC = NC_;                  // compute waves
  static constexpr int WN = NC / WM;
  static constexpr int MF = BM / 16 / WM;         // 16-row blocks per compute wave
  static constexpr int BN = WN * NF * 16;         // weight rows per n-tile
  static constexpr int FW = NF * 8;               // gate/up: features per wave
  static constexpr int A_SLOT = NPL * BM * 128;
  static constexpr int B_SLOT = BN * 128;
  static constexpr int NA = NPL * BM * 8 / 256;   // A copies per copy wave per stage
  static constexpr int NB = BN * 8 / 256;         // B copies per copy wave per stage
  static constexpr int NCP = NA + NB;
  static_assert(MF >= 1 && NA >= 1 && NB >= 1 && NA * 256 == NPL * BM * 8 && NB * 256 == BN * 8,
                "whole copy rounds");
  static_assert(MODE != kGateUp || NF % 2 == 0, "gate/up fragments come in gate/up pairs");
};

// x (gate/up, logits: [T][d] bf16) or h (down: hi and lo planes [T][S fs]
// bf16) times the weights (gate/up: w13 [S][2 fs][d]; down: w2 [S][d][fs];
// logits: w_router [E][d], rows past E read row E - 1 and are not stored).
template <int MODE, int BM, int WM, int NF, int NC = 4, int RING = kRing>
__global__ __launch_bounds__(64 * (NC + 4)) __attribute__((amdgpu_waves_per_eu(NC / 4 + 1, NC / 4 + 1))) void shared_gemm_lds(
    const uint16_t* __restrict__ a0, const uint16_t* __restrict__ a1,
    const uint16_t* __restrict__ w, void* __restrict__ out, int T, int d, int fs, int S, int E) {
  using C = Tiles<MODE, BM, WM, NF, NC>;
  constexpr bool DOWN = MODE == kDown;
  constexpr int MF = C::MF, kBM = BM, FW = C::FW;
  constexpr int kRing = RING;
  __shared__ __attribute__((aligned(16))) uint8_t sA[kRing * C::A_SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kRing * C::B_SLOT];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const bool copier = wv >= NC;
  const int K = DOWN ? S * fs : d;                // contraction length
  const int nst = K / kBK;
  const int nf_t = fs / (C::WN * FW);             // gate/up n-tiles per expert
  const int NT = DOWN ? d / C::BN : MODE == kLogits ? (E + C::BN - 1) / C::BN : S * nf_t;
  const int n_mt = (T + kBM - 1) / kBM;
  const ItemRange ir = item_range((long)NT * n_mt);
  const int it_first = (int)ir.first, it_end = (int)ir.end, it_step = (int)ir.step;
  const int n_items = it_first < it_end ? (it_end - it_first + it_step - 1) / it_step : 0;
  const int g_total = n_items * nst;
  const size_t a_row = (size_t)K;                 // elements per activation row (each plane)

  // weight row of local row r of n-tile nt (gate/up: wave r / (16 NF) owns
  // the gate rows of its FW features, then the matching up rows)
  auto wrow = [&](int nt, int r) -> size_t {
    if (DOWN) return (size_t)nt * C::BN + r;
    if (MODE == kLogits) return (size_t)min(nt * C::BN + r, E - 1);
    const int se = nt / nf_t, ntf = nt - se * nf_t;
    const int cw = r / (16 * NF), nf = (r >> 4) % NF;
    return (size_t)se * 2 * fs + (nf >= NF / 2 ? fs : 0) + ntf * (C::WN * FW) + cw * FW +
           (nf % (NF / 2)) * 16 + (r & 15);
  };

  if (copier) {
    const int cq = wv - NC;
    const uint16_t* ap[C::NA];
    const uint16_t* bp[C::NB];
    int c_it = it_first, c_st = 0;
    // per item: this wave's units' source rows (stage 0)
    auto setup = [&]() {
      int nt, mt;
      item_tile(c_it, n_mt, NT, mt, nt);
      const int row0 = mt * kBM, rows = min(kBM, T - row0);
#pragma unroll
      for (int c = 0; c < C::NA; ++c) {
        const int U = (cq * C::NA + c) * 64 + lane;
        const int pl = U / (kBM * 8), v = U - pl * (kBM * 8);
        const int r = v >> 3, u = (v & 7) ^ row_swz(r);
        ap[c] = (pl ? a1 : a0) + (size_t)(row0 + min(r, rows - 1)) * a_row + u * 8;
      }
#pragma unroll
      for (int c = 0; c < C::NB; ++c) {
        const int V = (cq * C::NB + c) * 64 + lane;
        const int r = V >> 3, u = (V & 7) ^ row_swz(r);
        bp[c] = w + wrow(nt, r) * (DOWN ? (size_t)fs : (size_t)d) + u * 8;
      }
    };
    auto issue = [&](int g) {
      if (c_it >= it_end) return;
      const uint32_t abase = lds_addr(sA) + (uint32_t)((g % kRing) * C::A_SLOT);
      const uint32_t bbase = lds_addr(sB) + (uint32_t)((g % kRing) * C::B_SLOT);
      const size_t ao = (size_t)c_st * kBK;
      // down: stage c_st of the chain is expert c_st / spe, elements (c_st % spe) * 64 of its rows
      const size_t bo = DOWN ? (size_t)(c_st * kBK / fs) * ((size_t)d * fs) + (size_t)(c_st * kBK % fs)
                             : (size_t)c_st * kBK;
#pragma unroll
      for (int c = 0; c < C::NA; ++c)
        dma16_raw(ap[c] + ao, abase + (uint32_t)((cq * C::NA + c) * 1024));
#pragma unroll
      for (int c = 0; c < C::NB; ++c)
        dma16_raw(bp[c] + bo, bbase + (uint32_t)((cq * C::NB + c) * 1024));
      if (++c_st == nst) {
        c_st = 0;
        c_it += it_step;
        if (c_it < it_end) setup();
      }
    };
    if (c_it < it_end) setup();
#pragma unroll
    for (int j = 0; j < kRing - 1; ++j) issue(j);
#pragma unroll 1
    for (int g = 0; g < g_total; ++g) {
      // the copies of stages g + 1 .. g + kRing - 2 may stay in flight
      if (g + kRing - 2 < g_total) wait_vmem<(kRing - 2) * C::NCP>();
      else wait_vmem<0>();
      wg_barrier();
      issue(g + kRing - 1);
    }
    wait_vmem<0>();
    return;
  }

  const int wm = wv / C::WN, wn = wv - wm * C::WN;
  int g = 0;
  for (int it = it_first; it < it_end; it += it_step) {
    int nt, mt;
    item_tile(it, n_mt, NT, mt, nt);
    const int row0 = mt * kBM, rows = min(kBM, T - row0);
    f32x4_t acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) acc[i][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int s = 0; s < nst; ++s, ++g) {
      wait_lds();
      wg_barrier();
      const uint8_t* abase = sA + (g % kRing) * C::A_SLOT;
      const uint8_t* bbase = sB + (g % kRing) * C::B_SLOT;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int u = 4 * j + lg;   // elements 32 j + 8 lg .. +8 of the stage
        bf16x8_t b[NF];
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) b[nf] = lds_frag(bbase, (wn * NF + nf) * 16 + ln, u);
        bf16x8_t a[2][C::NPL];
        auto load_a = [&](int i, bf16x8_t (&av)[C::NPL]) {
          const int r = (wm * MF + i) * 16 + ln;
#pragma unroll
          for (int p = 0; p < C::NPL; ++p) av[p] = lds_frag(abase + p * (kBM * 128), r, u);
        };
        load_a(0, a[0]);
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          if (i + 1 < MF) load_a(i + 1, a[(i + 1) & 1]);
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
#pragma unroll
            for (int p = 0; p < C::NPL; ++p)
              acc[i][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i & 1][p], b[nf], acc[i][nf],
                                                                   0, 0, 0);
        }
      }
    }
    if constexpr (MODE == kLogits) {
      float* l = static_cast<float*>(out);
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = (wm * MF + i) * 16 + lg * 4 + r;
          if (m < rows) {
            const int e0 = nt * C::BN + wn * (NF * 16) + ln;
            float* lr = l + (size_t)(row0 + m) * E + e0;
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
              if (e0 + nf * 16 < E) lr[nf * 16] = acc[i][nf][r];
          }
        }
    } else if constexpr (DOWN) {
      float* y = static_cast<float*>(out);
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = (wm * MF + i) * 16 + lg * 4 + r;
          if (m < rows) {
            float* yr = y + (size_t)(row0 + m) * d + nt * C::BN + wn * (NF * 16) + ln;
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) yr[nf * 16] = acc[i][nf][r];
          }
        }
    } else {
      // h = silu(g) * u of the wave's 32 features, as its hi and lo bf16 parts
      uint16_t* hh = static_cast<uint16_t*>(out);
      uint16_t* hl = hh + (size_t)T * S * fs;
      const int se = nt / nf_t, ntf = nt - se * nf_t;
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = (wm * MF + i) * 16 + lg * 4 + r;
          if (m < rows) {
            const size_t o = (size_t)(row0 + m) * S * fs + (size_t)se * fs + ntf * (C::WN * FW) +
                             wn * FW + ln;
#pragma unroll
            for (int q = 0; q < NF / 2; ++q) {
              const float hv = silu_mul(acc[i][q][r], acc[i][q + NF / 2][r]);
              const uint16_t hi = f32_to_bf16(hv);
              hh[o + q * 16] = hi;
              hl[o + q * 16] = f32_to_bf16(hv - __uint_as_float((uint32_t)hi << 16));
            }
          }
        }
    }
  }
}

// h: T * S * fs * 4 bytes, written by the gate/up as two bf16 planes and
// read back by the down.
// One (gate/up, down) pair of tile shapes: BM tokens per m-tile, WM waves
// along the tokens and NF weight fragments per wave for each, NC compute waves
// (4 or 8; with 8, the rings hold 2 stages instead of 3).
template <int BMG, int WMG, int NFG, int NCG, int BMD, int WMD, int NFD, int NCD, int RS = kRing>
hipError_t shared_lds_pair(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                           float* h, float* y, hipStream_t st) {
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* w13 = static_cast<const uint16_t*>(b.w13);
  const uint16_t* w2 = static_cast<const uint16_t*>(b.w2);
  const int T = (int)s.T, S = b.n_experts, fs = b.f;
  uint16_t* hh = reinterpret_cast<uint16_t*>(h);
  const dim3 g(grouped_grid());   // one workgroup per CU
  constexpr int RG = NCG == 8 ? 2 : RS, RD = NCD == 8 ? 2 : RS;
  shared_gemm_lds<kGateUp, BMG, WMG, NFG, NCG, RG><<<g, 64 * (NCG + 4), 0, st>>>(
      xb, nullptr, w13, hh, T, s.d, fs, S, 0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  shared_gemm_lds<kDown, BMD, WMD, NFD, NCD, RD><<<g, 64 * (NCD + 4), 0, st>>>(
      hh, hh + (size_t)T * S * fs, w2, y, T, s.d, fs, S, 0);
  return hipGetLastError();
}

}  // namespace

bool shared_lds_ok(const k3moe_shape& s) {
  return s.f_shared % 128 == 0 && s.d % 256 == 0;
}

// Tile shapes by batch (measured at d 7168, two experts of fs 2048; the
// shared FFN, gate/up + down):
//   T <= 64:   64-token tiles, the 4 waves splitting the tokens, n-tiles of
//              16 features / 32 outputs (256 and 224 items: the weights spread
//              over every CU), 4-slot rings: 42-44 us (50-53 us with 3 slots;
//              5 to 8 slots gain nothing more; the register-fed small-batch
//              kernels took 125-181 us);
//   T <= 256:  64-token tiles, waves 2 x 2: 69-79 us;
//   T <= 640:  128-token tiles, waves 2 x 2: 120-128 us at 384-512 tokens;
//   larger:    gate/up 128-token tiles with the waves side by side along the
//              weights; down 128-token tiles of 256 outputs on 8 compute waves
//              (2 x 4); from 2048 tokens the gate/up also takes 8 compute
//              waves on 256-token tiles (2 x 4, each wave 128 tokens x 64
//              rows).  0.22 ms at 1024 tokens, 0.90 ms at 4096, 3.2 ms at
//              16384 (0.24, 1.00 and 3.5 ms with 4 compute waves; same bits).
hipError_t launch_shared_lds(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                             float* h, float* y, hipStream_t st) {
  if (s.T <= 64) return shared_lds_pair<64, 4, 2, 4, 64, 4, 2, 4, 4>(s, b, x, h, y, st);
  if (s.T <= 256) return shared_lds_pair<64, 2, 4, 4, 64, 2, 4, 4>(s, b, x, h, y, st);
  if (s.T <= 640) return shared_lds_pair<128, 2, 4, 4, 128, 2, 4, 4>(s, b, x, h, y, st);
  if (s.T < 2048) return shared_lds_pair<128, 1, 4, 4, 128, 2, 4, 8>(s, b, x, h, y, st);
  return shared_lds_pair<256, 2, 4, 8, 128, 2, 4, 8>(s, b, x, h, y, st);
}

// The router's fp32 logits on the bf16 matrix cores: l[t][e] = x_t . w_e
// (their bound does not depend on the order of the sum).  64-token tiles up to
// 2048 tokens, 128 above (the whole route at 896 experts: 153 us at 512
// tokens, 189 at 2048, 332 at 4096, 1.30 ms at 16384, against 172, 352, 477
// and 1904 us with register-fed tiles; same ids and weights).
hipError_t launch_router_logits_lds(const uint16_t* x, const uint16_t* wr, float* l, int T, int d,
                                    int E, hipStream_t st) {
  const dim3 g(grouped_grid());
  if (T > 2048)
    shared_gemm_lds<kLogits, 128, 2, 4><<<g, 512, 0, st>>>(x, nullptr, wr, l, T, d, 0, 0, E);
  else
    shared_gemm_lds<kLogits, 64, 2, 4><<<g, 512, 0, st>>>(x, nullptr, wr, l, T, d, 0, 0, E);
  return hipGetLastError();
}

}  // namespace k3
