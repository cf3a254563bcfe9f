// Routed expert FFN for large batches: grouped GEMMs on bf16 MFMA.
//
// The pages' expert FFN (kimi-k3-in-c review, "KDA/MLA/MoE" table;
// explainer page, "reduction one": nibbles decoded against a shared block
// exponent, multiplied by unquantised activations) becomes, once tokens are grouped by expert, two GEMMs per
// expert: H = silu(X W_gate^T) * (X W_up^T) and Y = H W_down^T.  Activations
// stay exact: x is bf16, and the fp32 h is split into two bf16 terms
// (hi = RNE(h), lo = RNE(h - hi)) that both go through the matrix core.  The
// weights are decoded exactly (an E2M1 value times a power of two is a bf16
// number) by the scaled fp4 -> bf16 conversion, in registers.
//
// Tiling (wave = 64 lanes, MFMA 16x16x32 bf16 -> fp32):
//   * an m-tile is up to BM = 16 MF consecutive rows of one expert in the
//     expert-sorted pair order; every workgroup of 4 waves computes one
//     (m-tile, n-tile) item at a time and loops over items (persistent grid);
//     items are split into 8 contiguous ranges, one per XCD, so the
//     workgroups that share an m-tile's activations run on the same L2;
//   * the contraction runs in stages of 128 elements (4 MX blocks).  Lane
//     (n = lane % 16, g = lane / 16) loads the 16 bytes of MX block g of
//     weight row n straight from HBM, with its scale, and decodes them into
//     the B operand of 4 MFMA steps; step j consumes elements
//     g*32 + j*8 .. +8 of the stage.  The A operand (activations in LDS) is
//     read with the same element order, so every product pairs the right x
//     and w and the sum per (row, output) runs over stages, then steps j,
//     in a fixed order that does not depend on the other rows of the tile.
#include "internal.h"
#include "kern_common.h"

namespace k3 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kBK = 128;         // contraction elements per stage
constexpr int kThreads = 256;    // 4 waves
constexpr int kLdsRow = 272;     // bytes per LDS row: 128 bf16 + 16 pad (bank spread)
constexpr int kMaxE = 1024;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Exact decode of 8 E2M1 codes (one dword, low nibble first) times scale.
__device__ __forceinline__ bf16x8_t decode8(uint32_t w, float sc) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// m-tile schedule in LDS: s_mt[e] = index of expert e's first m-tile
// (exclusive scan of ceil(n_e / BM)), s_mt[E] = number of m-tiles.
__device__ void build_mtiles(const int32_t* __restrict__ offsets, int E, int BM, int* s_mt,
                             int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int c[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    c[j] = 0;
    if (e < E) {
      const int n = offsets[e + 1] - offsets[e];
      c[j] = n > 0 ? (n + BM - 1) / BM : 0;
    }
    sum += c[j];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == 63) s_wave[wv] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wv; ++w) base += s_wave[w];
  int ex = base + incl - sum;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    if (e < E) s_mt[e] = ex;
    ex += c[j];
  }
  if (tid == kThreads - 1) s_mt[E] = ex;   // ex = grand total after the last thread's experts
  __syncthreads();
}

// Expert owning m-tile mt: the last e with s_mt[e] <= mt (then s_mt[e+1] > mt).
__device__ __forceinline__ int mtile_expert(const int* s_mt, int E, int mt) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_mt[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// Item range of this workgroup: 8 contiguous ranges, range x served by the
// workgroups with blockIdx % 8 == x (one XCD each), strided by gridDim / 8.
struct ItemRange {
  long first, end, step;
};
__device__ __forceinline__ ItemRange item_range(long n_items) {
  const int x = blockIdx.x & 7;
  const long per = (n_items + 7) / 8;
  const long lo = x * per;
  long hi = lo + per;
  if (hi > n_items) hi = n_items;
  return ItemRange{lo + (blockIdx.x >> 3), hi, (long)(gridDim.x >> 3)};
}

// E8M0 byte -> fp32 scale 2^(s-127), branch-free (s = 0: 2^-127, s = 255: NaN).
__device__ __forceinline__ float e8m0_scale(uint32_t s) {
  uint32_t bits = s << 23;
  bits = s == 0u ? 0x00400000u : bits;
  bits = s == 255u ? 0x7FC00000u : bits;
  return __uint_as_float(bits);
}

// ------------------------------------------------------------------ gate/up
// Item = (m-tile, n-tile of 128 features); wave w owns features
// nt*128 + w*32 + [0, 32): B fragments nf = 0,1 are gate rows, 2,3 the up rows
// of the same features.  Output h [P][f] fp32 in sorted-pair order.
template <int MF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void gateup_mfma(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ w13s, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, float* __restrict__ h, int d, int f, int E, int k) {
  constexpr int BM = 16 * MF;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kLdsRow];
  __shared__ int s_mt[kMaxE + 1];
  __shared__ int s_wave[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  build_mtiles(offsets, E, BM, s_mt, s_wave);
  const int NT = f / 128;
  const ItemRange ir = item_range((long)s_mt[E] * NT);
  const int nst = d / kBK;
  const size_t w_row = (size_t)d / 2, s_row = (size_t)d / 32;

  for (long it = ir.first; it < ir.end; it += ir.step) {
    const int mt = (int)(it / NT), nt = (int)(it - (long)mt * NT);
    const int e = mtile_expert(s_mt, E, mt);
    const int row0 = offsets[e] + (mt - s_mt[e]) * BM;
    const int rows = min(BM, offsets[e + 1] - row0);

    // A loader: chunk q = tid % 16 (8 bf16) of rows tid/16 + 16 i.
    const uint16_t* xr[MF];
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int r = min((tid >> 4) + 16 * i, rows - 1);
      const int tok = sorted_pair[row0 + r] / k;
      xr[i] = x + (size_t)tok * d + (tid & 15) * 8;
    }
    // B loader: weight row of fragment nf for this lane, MX block lg.
    const uint8_t* wp[4];
    const uint8_t* sp[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const size_t row = (size_t)e * 2 * f + (nf >= 2 ? f : 0) + nt * 128 + wv * 32 +
                         (nf & 1) * 16 + ln;
      wp[nf] = w13 + row * w_row + lg * 16;
      sp[nf] = w13s + row * s_row;
    }

    f32x4_t acc[MF][4];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[i][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    __syncthreads();   // the previous item's last reads of sA are done
    uint4 av[MF];
    uint4 bq[4];
    uint32_t bs[4];
#pragma unroll
    for (int i = 0; i < MF; ++i) av[i] = ldg16(xr[i]);
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      bq[nf] = ldg16(wp[nf]);
      bs[nf] = *reinterpret_cast<const uint32_t*>(sp[nf]);
    }
#pragma unroll
    for (int i = 0; i < MF; ++i)
      *reinterpret_cast<uint4*>(&sA[0][((tid >> 4) + 16 * i) * kLdsRow + (tid & 15) * 16]) = av[i];
    __syncthreads();

#pragma unroll 1
    for (int s = 0; s < nst; ++s) {
      const int cur = s & 1;
      const int sn = min(s + 1, nst - 1);   // clamped prefetch (the last one is unused)
      uint4 bqn[4];
      uint32_t bsn[4];
#pragma unroll
      for (int i = 0; i < MF; ++i) av[i] = ldg16(xr[i] + sn * kBK);
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        bqn[nf] = ldg16(wp[nf] + sn * (kBK / 2));
        bsn[nf] = *reinterpret_cast<const uint32_t*>(sp[nf] + sn * 4);
      }
      float sc[4];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) sc[nf] = e8m0_to_f32((bs[nf] >> (8 * lg)) & 0xFFu);
      const uint8_t* abase = &sA[cur][ln * kLdsRow + lg * 64];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t b[4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const uint32_t wj = j == 0 ? bq[nf].x : j == 1 ? bq[nf].y : j == 2 ? bq[nf].z : bq[nf].w;
          b[nf] = decode8(wj, sc[nf]);
        }
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(abase + i * 16 * kLdsRow + j * 16));
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
            acc[i][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[nf], acc[i][nf], 0, 0, 0);
        }
      }
      if (s + 1 < nst) {
#pragma unroll
        for (int i = 0; i < MF; ++i)
          *reinterpret_cast<uint4*>(&sA[cur ^ 1][((tid >> 4) + 16 * i) * kLdsRow + (tid & 15) * 16]) = av[i];
      }
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) { bq[nf] = bqn[nf]; bs[nf] = bsn[nf]; }
      __syncthreads();
    }

    // Epilogue: lane holds rows i*16 + lg*4 + r, feature column ln of each
    // fragment; h = silu(gate) * up.
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = i * 16 + lg * 4 + r;
        if (m < rows) {
          float* hr = h + (size_t)(row0 + m) * f + nt * 128 + wv * 32 + ln;
          hr[0] = silu_mul(acc[i][0][r], acc[i][2][r]);
          hr[16] = silu_mul(acc[i][1][r], acc[i][3][r]);
        }
      }
  }
}

// ------------------------------------------- grouped GEMMs, producer/consumer
// The routed gate/up and down products with the loads taken off the critical
// path.  A workgroup has 8 waves:
//   * waves 0..3 (consumers) only read LDS, decode weights and issue MFMAs;
//   * waves 4,5 copy the activations of each stage (A: x rows gathered by
//     the expert-sorted pairs, or h rows) into an RA-slot LDS ring;
//   * waves 6,7 copy the weight codes and scales of each stage (B, streamed
//     from HBM) into an RB-slot LDS ring.
// Copies are LDS-DMA (global -> LDS without registers), issued R - 1 stages
// ahead; each copier wave has its own memory counter, so the HBM stream never
// waits behind the L2 stream.  One s_barrier per stage: before it every
// copier waits until the next stage's copies have landed (a constant count
// of newer copies may stay in flight; copies past the last stage repeat the
// last stage into a slot nobody reads), and every consumer waits for its LDS
// reads, so a slot is refilled only after it was read and read only after it
// was filled.  All roles run the same loops and barriers.
//
// LDS layouts (XOR placements spread the 16 rows a consumer fragment reads
// over all banks):
//   A slot: [BM rows][AU units of 16 bytes], unit u of row r at position
//     u ^ (r & 15).  Gate/up: AU = 16 units of 8 bf16.  Down: AU = 32, unit
//     2c = the 8 hi values of feature block c, 2c + 1 the 8 lo values.
//   B slot: codes [256 rows][4 MX blocks of 16 bytes], block b of row r at
//     position b ^ ((r >> 2) & 3); then scales [256 rows] one dword (the 4
//     block scales of the stage).  Local weight row r belongs to consumer
//     r / 64, fragment (r / 16) % 4, lane r % 16.
constexpr int kPcThreads = 512;

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// LDS-DMA copies: lane i's 16 (or 4) bytes from g land at lds_base + 16 i
// (or 4 i); lds_base must be the same for every lane of the wave.
__device__ __forceinline__ void dma16_to_lds(const void* g, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(const void* g, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, lds_base, 4, 0, 0);
}

// m-tile schedule for an NTH-thread workgroup (threads 0..255 own 4 experts each).
template <int NTH>
__device__ void build_mtiles_n(const int32_t* __restrict__ offsets, int E, int BM, int* s_mt,
                               int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int c[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    c[j] = 0;
    if (tid < 256 && e < E) {
      const int n = offsets[e + 1] - offsets[e];
      c[j] = n > 0 ? (n + BM - 1) / BM : 0;
    }
    sum += c[j];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == 63) s_wave[wv] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wv; ++w) base += s_wave[w];
  int ex = base + incl - sum;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    if (tid < 256 && e < E) s_mt[e] = ex;
    ex += c[j];
  }
  if (tid == NTH - 1) s_mt[E] = ex;
  __syncthreads();
}

// Gate/up (DOWN = false): item = (m-tile, 128 features); B fragments 0,1 are
// the gate rows and 2,3 the up rows of consumer w's features nt*128 + w*32 +
// [0, 32); output h as split pairs (8 hi, then 8 lo bf16 per 8 features).
// Down (DOWN = true): item = (m-tile, 256 outputs); consumer w owns outputs
// nt*256 + w*64 + [0, 64); A = split h; each step issues the hi product, then
// the lo product; output y fp32.
template <int MF, int RA, int RB, bool DOWN, int NC>
__global__ __launch_bounds__((NC + 4) * 64) void mx_gemm_pc(
    const uint8_t* __restrict__ a_src, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ wsc, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, float* __restrict__ out, int d, int f, int E,
    int k) {
  constexpr int BM = 16 * MF;
  constexpr int AU = DOWN ? 32 : 16;
  constexpr int A_SLOT = BM * AU * 16;
  constexpr int NTH = (NC + 4) * 64;
  constexpr int BROWS = NC * 64;                // weight rows per stage
  constexpr int B_CODES = BROWS * 64;
  constexpr int B_SLOT = B_CODES + BROWS * 4;
  constexpr int NA = BM * AU / 2 / 64;          // A copies per A wave per stage
  constexpr int NBC = BROWS * 4 / 2 / 64;       // B code copies per B wave per stage
  constexpr int NBS = BROWS / 2 / 64;           // B scale copies per B wave per stage
  constexpr int NB = NBC + NBS;
  static_assert(RA >= 2 && RB >= 2, "rings need two slots");
  // at most R - 1 stages of copies are in flight per copier wave; the memory
  // counter tracks 63
  static_assert((RA - 1) * NA <= 63 && (RB - 1) * NB <= 63, "memory counter range");
  __shared__ __attribute__((aligned(16))) uint8_t sA[RA * A_SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t sB[RB * B_SLOT];
  __shared__ int s_mt[kMaxE + 1];
  __shared__ int s_wave[NTH / 64];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const bool a_copier = wv == NC || wv == NC + 1, b_copier = wv >= NC + 2;
  const int pa = wv - NC, pb = wv - NC - 2;
  build_mtiles_n<NTH>(offsets, E, BM, s_mt, s_wave);
  const int NT = DOWN ? d / (NC * 64) : f / (NC * 32);
  const int nst = (DOWN ? f : d) / kBK;
  const ItemRange ir = item_range((long)s_mt[E] * NT);
  const size_t w_row = (size_t)(DOWN ? f : d) / 2, s_row = (size_t)(DOWN ? f : d) / 32;
  const size_t e_rows = DOWN ? (size_t)d : (size_t)2 * f;
  const size_t a_row = DOWN ? (size_t)f * 4 : (size_t)d * 2;   // bytes per A source row

  // Every role walks the same items and executes 1 + nst barriers per item
  // (one after the prologue, one per stage).
  if (a_copier) {
    for (long it = ir.first; it < ir.end; it += ir.step) {
      const int mt = (int)(it / NT);
      const int e = mtile_expert(s_mt, E, mt);
      const int row0 = offsets[e] + (mt - s_mt[e]) * BM;
      const int rows = min(BM, offsets[e + 1] - row0);
      const uint8_t* ap[NA];
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        const int unit = pa * (BM * AU / 2) + q * 64 + lane;
        const int r = unit / AU;
        const int u = (unit % AU) ^ (r & 15);
        const int rr = min(r, rows - 1);
        const size_t src_row = DOWN ? (size_t)(row0 + rr) : (size_t)(sorted_pair[row0 + rr] / k);
        ap[q] = a_src + src_row * a_row + u * 16;
      }
      auto issue_a = [&](int st, int slot) {
        uint8_t* base = sA + slot * A_SLOT + pa * (BM * AU / 2) * 16;
#pragma unroll
        for (int q = 0; q < NA; ++q) dma16_to_lds(ap[q] + (size_t)st * (AU * 16), base + q * 1024);
      };
#pragma unroll
      for (int q = 0; q < RA - 1; ++q) issue_a(min(q, nst - 1), q);
      wait_vmem<(RA - 2) * NA>();
      wg_barrier();
#pragma unroll 1
      for (int s = 0; s < nst; ++s) {
        issue_a(min(s + RA - 1, nst - 1), (s + RA - 1) % RA);
        wait_vmem<(RA - 2) * NA>();
        wg_barrier();
      }
      // copies past the last stage land before the next item refills the ring
      wait_vmem<0>();
    }
  } else if (b_copier) {
    for (long it = ir.first; it < ir.end; it += ir.step) {
      const int mt = (int)(it / NT), nt = (int)(it - (long)mt * NT);
      const int e = mtile_expert(s_mt, E, mt);
      auto grow = [&](int r) -> size_t {
        if (DOWN) return (size_t)nt * (NC * 64) + r;
        const int cw = r >> 6, nf = (r >> 4) & 3;
        return (size_t)((nf >= 2 ? f : 0) + nt * (NC * 32) + cw * 32 + (nf & 1) * 16 + (r & 15));
      };
      const uint8_t* wbase = wq + (size_t)e * e_rows * w_row;
      const uint8_t* sbase = wsc + (size_t)e * e_rows * s_row;
      const uint8_t* bp[NBC];
      const uint8_t* sp[NBS];
#pragma unroll
      for (int q = 0; q < NBC; ++q) {
        const int r = (pb * (NBC * 64) + q * 64 + lane) >> 2;
        const int b = (lane & 3) ^ ((r >> 2) & 3);
        bp[q] = wbase + grow(r) * w_row + b * 16;
      }
#pragma unroll
      for (int q = 0; q < NBS; ++q) sp[q] = sbase + grow(pb * (NBS * 64) + q * 64 + lane) * s_row;
      auto issue_b = [&](int st, int slot) {
        uint8_t* base = sB + slot * B_SLOT;
#pragma unroll
        for (int q = 0; q < NBC; ++q)
          dma16_to_lds(bp[q] + st * (kBK / 2), base + (pb * (NBC * 64) + q * 64) * 16);
#pragma unroll
        for (int q = 0; q < NBS; ++q)
          dma4_to_lds(sp[q] + st * 4, base + B_CODES + (pb * (NBS * 64) + q * 64) * 4);
      };
#pragma unroll
      for (int q = 0; q < RB - 1; ++q) issue_b(min(q, nst - 1), q);
      wait_vmem<(RB - 2) * NB>();
      wg_barrier();
#pragma unroll 1
      for (int s = 0; s < nst; ++s) {
        issue_b(min(s + RB - 1, nst - 1), (s + RB - 1) % RB);
        wait_vmem<(RB - 2) * NB>();
        wg_barrier();
      }
      wait_vmem<0>();
    }
  } else {
    for (long it = ir.first; it < ir.end; it += ir.step) {
      const int mt = (int)(it / NT), nt = (int)(it - (long)mt * NT);
      const int e = mtile_expert(s_mt, E, mt);
      const int row0 = offsets[e] + (mt - s_mt[e]) * BM;
      const int rows = min(BM, offsets[e + 1] - row0);
      f32x4_t acc[MF][4];
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[i][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      wg_barrier();
#pragma unroll 1
      for (int s = 0; s < nst; ++s) {
        const uint8_t* abase = sA + (s % RA) * A_SLOT;
        const uint8_t* bbase = sB + (s % RB) * B_SLOT;
        float sc[4];
        uint4 bq[4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const int r = wv * 64 + nf * 16 + ln;
          const uint32_t sw = *reinterpret_cast<const uint32_t*>(bbase + B_CODES + r * 4);
          sc[nf] = e8m0_scale((sw >> (8 * lg)) & 0xFFu);
          bq[nf] = *reinterpret_cast<const uint4*>(bbase + r * 64 + ((lg ^ ((r >> 2) & 3)) * 16));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x8_t b[4];
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) {
            const uint4& q = bq[nf];
            const uint32_t wj = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
            b[nf] = decode8(wj, sc[nf]);
          }
          const int c = lg * 4 + j;   // 8-element block of the stage this step reads
#pragma unroll
          for (int i = 0; i < MF; ++i) {
            const uint8_t* arow = abase + (i * 16 + ln) * (AU * 16);
            if (DOWN) {
              const bf16x8_t ah = as_bf16x8(*reinterpret_cast<const uint4*>(arow + (((2 * c) ^ ln) * 16)));
              const bf16x8_t al = as_bf16x8(*reinterpret_cast<const uint4*>(arow + (((2 * c + 1) ^ ln) * 16)));
#pragma unroll
              for (int nf = 0; nf < 4; ++nf) {
                acc[i][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b[nf], acc[i][nf], 0, 0, 0);
                acc[i][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b[nf], acc[i][nf], 0, 0, 0);
              }
            } else {
              const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(arow + ((c ^ ln) * 16)));
#pragma unroll
              for (int nf = 0; nf < 4; ++nf)
                acc[i][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[nf], acc[i][nf], 0, 0, 0);
            }
          }
        }
        wait_lds();
        wg_barrier();
      }
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = i * 16 + lg * 4 + r;
          if (m < rows) {
            if (DOWN) {
              float* yr = out + (size_t)(row0 + m) * d + nt * (NC * 64) + wv * 64 + ln;
#pragma unroll
              for (int nf = 0; nf < 4; ++nf) yr[nf * 16] = acc[i][nf][r];
            } else {
              uint16_t* hr = reinterpret_cast<uint16_t*>(out + (size_t)(row0 + m) * f);
#pragma unroll
              for (int half = 0; half < 2; ++half) {
                const float v = silu_mul(acc[i][half][r], acc[i][half + 2][r]);
                const uint16_t hi = f32_to_bf16(v);
                const uint16_t lo = f32_to_bf16(v - __uint_as_float((uint32_t)hi << 16));
                const int col = nt * (NC * 32) + wv * 32 + half * 16 + ln;
                hr[(col >> 3) * 16 + (col & 7)] = hi;
                hr[(col >> 3) * 16 + 8 + (col & 7)] = lo;
              }
            }
          }
        }
    }
  }
}

// --------------------------------------------------------------------- down
// Item = (m-tile, n-tile of 256 outputs); wave w owns outputs
// nt*256 + w*64 + [0, 64) as 4 fragments.  A = h rows of the m-tile (fp32,
// contiguous in sorted-pair order), stored in LDS as bf16 hi and lo parts;
// every step issues the hi product, then the lo product.
template <int MF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void down_mfma(
    const float* __restrict__ h, const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2s,
    const int32_t* __restrict__ offsets, float* __restrict__ y, int d, int f, int E) {
  constexpr int BM = 16 * MF;
  constexpr int PER = BM / 8;   // 16-byte h chunks per thread per stage
  __shared__ __attribute__((aligned(16))) uint8_t sH[2][BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t sL[2][BM * kLdsRow];
  __shared__ int s_mt[kMaxE + 1];
  __shared__ int s_wave[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  build_mtiles(offsets, E, BM, s_mt, s_wave);
  const int NT = d / 256;
  const ItemRange ir = item_range((long)s_mt[E] * NT);
  const int nst = f / kBK;
  const size_t w_row = (size_t)f / 2, s_row = (size_t)f / 32;
  const int q = tid & 31;   // 4-float chunk of the 128-element stage

  for (long it = ir.first; it < ir.end; it += ir.step) {
    const int mt = (int)(it / NT), nt = (int)(it - (long)mt * NT);
    const int e = mtile_expert(s_mt, E, mt);
    const int row0 = offsets[e] + (mt - s_mt[e]) * BM;
    const int rows = min(BM, offsets[e + 1] - row0);

    const float* hr[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int r = min((tid >> 5) + 8 * i, rows - 1);
      hr[i] = h + (size_t)(row0 + r) * f + q * 4;
    }
    const uint8_t* wp[4];
    const uint8_t* sp[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const size_t row = (size_t)e * d + nt * 256 + wv * 64 + nf * 16 + ln;
      wp[nf] = w2 + row * w_row + lg * 16;
      sp[nf] = w2s + row * s_row;
    }

    f32x4_t acc[MF][4];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[i][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // fp32 -> (hi, lo) bf16 pairs, written as 8 bytes each.
    auto split_store = [&](int buf, const uint4 (&v)[PER]) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const float fv[4] = {__uint_as_float(v[i].x), __uint_as_float(v[i].y),
                             __uint_as_float(v[i].z), __uint_as_float(v[i].w)};
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          hi[c] = f32_to_bf16(fv[c]);
          lo[c] = f32_to_bf16(fv[c] - __uint_as_float((uint32_t)hi[c] << 16));
        }
        const int off = ((tid >> 5) + 8 * i) * kLdsRow + q * 8;
        *reinterpret_cast<uint2*>(&sH[buf][off]) =
            make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
        *reinterpret_cast<uint2*>(&sL[buf][off]) =
            make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
      }
    };

    __syncthreads();
    uint4 hv[PER];
    uint4 bq[4];
    uint32_t bs[4];
#pragma unroll
    for (int i = 0; i < PER; ++i) hv[i] = ldg16(hr[i]);
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      bq[nf] = ldg16(wp[nf]);
      bs[nf] = *reinterpret_cast<const uint32_t*>(sp[nf]);
    }
    split_store(0, hv);
    __syncthreads();

#pragma unroll 1
    for (int s = 0; s < nst; ++s) {
      const int cur = s & 1;
      const int sn = min(s + 1, nst - 1);
      uint4 bqn[4];
      uint32_t bsn[4];
#pragma unroll
      for (int i = 0; i < PER; ++i) hv[i] = ldg16(hr[i] + sn * kBK);
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        bqn[nf] = ldg16(wp[nf] + sn * (kBK / 2));
        bsn[nf] = *reinterpret_cast<const uint32_t*>(sp[nf] + sn * 4);
      }
      float sc[4];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) sc[nf] = e8m0_to_f32((bs[nf] >> (8 * lg)) & 0xFFu);
      const int aoff = ln * kLdsRow + lg * 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t b[4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const uint32_t wj = j == 0 ? bq[nf].x : j == 1 ? bq[nf].y : j == 2 ? bq[nf].z : bq[nf].w;
          b[nf] = decode8(wj, sc[nf]);
        }
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          const int o = aoff + i * 16 * kLdsRow + j * 16;
          const bf16x8_t ah = as_bf16x8(*reinterpret_cast<const uint4*>(&sH[cur][o]));
          const bf16x8_t al = as_bf16x8(*reinterpret_cast<const uint4*>(&sL[cur][o]));
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) {
            acc[i][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b[nf], acc[i][nf], 0, 0, 0);
            acc[i][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b[nf], acc[i][nf], 0, 0, 0);
          }
        }
      }
      if (s + 1 < nst) split_store(cur ^ 1, hv);
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) { bq[nf] = bqn[nf]; bs[nf] = bsn[nf]; }
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = i * 16 + lg * 4 + r;
        if (m < rows) {
          float* yr = y + (size_t)(row0 + m) * d + nt * 256 + wv * 64 + ln;
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) yr[nf * 16] = acc[i][nf][r];
        }
      }
  }
}

// ----------------------------------------------------------- shared experts
// The always-on experts see every token, with bf16 weights: the same tiling
// with m-tiles of consecutive tokens, stages of 64 contraction elements, and
// the B fragments loaded as bf16 (lane (n, g) reads elements j*32 + g*8 .. +8
// of step j), with A read in the same order.
constexpr int kBKs = 64;
constexpr int kLdsRowS = 144;   // 64 bf16 + 16 pad

// Item = (m-tile, shared expert s, n-tile of 128 features); h [T][S][fs].
template <int MF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void gateup_shared_mfma(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13, float* __restrict__ h,
    int T, int d, int fs, int S) {
  constexpr int BM = 16 * MF;
  constexpr int PER = BM / 32;    // 16-byte x chunks per thread per stage
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kLdsRowS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int NT = fs / 128;
  const int n_mt = (T + BM - 1) / BM;
  const ItemRange ir = item_range((long)n_mt * S * NT);
  const int nst = d / kBKs;
  const int q = tid & 7;

  for (long it = ir.first; it < ir.end; it += ir.step) {
    const int mt = (int)(it / (S * NT));
    const int rem = (int)(it - (long)mt * S * NT);
    const int se = rem / NT, nt = rem - se * NT;
    const int row0 = mt * BM;
    const int rows = min(BM, T - row0);

    const uint16_t* xr[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
      xr[i] = x + (size_t)(row0 + min((tid >> 3) + 32 * i, rows - 1)) * d + q * 8;
    const uint16_t* wp[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const size_t row = (size_t)se * 2 * fs + (nf >= 2 ? fs : 0) + nt * 128 + wv * 32 +
                         (nf & 1) * 16 + ln;
      wp[nf] = w13 + row * d + lg * 8;
    }
    f32x4_t acc[MF][4];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[i][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    __syncthreads();
    uint4 av[PER];
    uint4 bq[4][2];
#pragma unroll
    for (int i = 0; i < PER; ++i) av[i] = ldg16(xr[i]);
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      bq[nf][0] = ldg16(wp[nf]);
      bq[nf][1] = ldg16(wp[nf] + 32);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      *reinterpret_cast<uint4*>(&sA[0][((tid >> 3) + 32 * i) * kLdsRowS + q * 16]) = av[i];
    __syncthreads();

#pragma unroll 1
    for (int s = 0; s < nst; ++s) {
      const int cur = s & 1;
      const int sn = min(s + 1, nst - 1);
      uint4 bn[4][2];
#pragma unroll
      for (int i = 0; i < PER; ++i) av[i] = ldg16(xr[i] + sn * kBKs);
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        bn[nf][0] = ldg16(wp[nf] + sn * kBKs);
        bn[nf][1] = ldg16(wp[nf] + sn * kBKs + 32);
      }
      const uint8_t* abase = &sA[cur][ln * kLdsRowS + lg * 16];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(abase + i * 16 * kLdsRowS + j * 64));
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
            acc[i][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(bq[nf][j]), acc[i][nf], 0, 0, 0);
        }
      if (s + 1 < nst) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
          *reinterpret_cast<uint4*>(&sA[cur ^ 1][((tid >> 3) + 32 * i) * kLdsRowS + q * 16]) = av[i];
      }
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) { bq[nf][0] = bn[nf][0]; bq[nf][1] = bn[nf][1]; }
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = i * 16 + lg * 4 + r;
        if (m < rows) {
          float* hr = h + ((size_t)(row0 + m) * S + se) * fs + nt * 128 + wv * 32 + ln;
          hr[0] = silu_mul(acc[i][0][r], acc[i][2][r]);
          hr[16] = silu_mul(acc[i][1][r], acc[i][3][r]);
        }
      }
  }
}

// Item = (m-tile, n-tile of 256 outputs); the contraction runs over the
// shared experts in order, then over each one's fs elements, so
// y = sum over s of h_s W2_s^T is one accumulation chain per output.
template <int MF, bool COMBINE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void down_shared_mfma(
    const float* __restrict__ h, const uint16_t* __restrict__ w2, float* __restrict__ y, int T,
    int d, int fs, int S, CombineArgs comb) {
  constexpr int BM = 16 * MF;
  constexpr int PER = BM / 16;    // 16-byte h chunks per thread per stage (16 per row)
  __shared__ __attribute__((aligned(16))) uint8_t sH[2][BM * kLdsRowS];
  __shared__ __attribute__((aligned(16))) uint8_t sL[2][BM * kLdsRowS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int NT = d / 256;
  const int n_mt = (T + BM - 1) / BM;
  const ItemRange ir = item_range((long)n_mt * NT);
  const int spe = fs / kBKs;       // stages per shared expert
  const int nst = S * spe;
  const int q = tid & 15;          // 4-float chunk of the 64-element stage
  const size_t hrow = (size_t)S * fs;

  for (long it = ir.first; it < ir.end; it += ir.step) {
    const int mt = (int)(it / NT), nt = (int)(it - (long)mt * NT);
    const int row0 = mt * BM;
    const int rows = min(BM, T - row0);
    const float* hr[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
      hr[i] = h + (size_t)(row0 + min((tid >> 4) + 16 * i, rows - 1)) * hrow + q * 4;
    const uint16_t* wp[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
      wp[nf] = w2 + (size_t)(nt * 256 + wv * 64 + nf * 16 + ln) * fs + lg * 8;
    const size_t wexp = (size_t)d * fs;   // elements per shared expert's w2

    f32x4_t acc[MF][4];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[i][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto split_store = [&](int buf, const uint4 (&v)[PER]) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const float fv[4] = {__uint_as_float(v[i].x), __uint_as_float(v[i].y),
                             __uint_as_float(v[i].z), __uint_as_float(v[i].w)};
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          hi[c] = f32_to_bf16(fv[c]);
          lo[c] = f32_to_bf16(fv[c] - __uint_as_float((uint32_t)hi[c] << 16));
        }
        const int off = ((tid >> 4) + 16 * i) * kLdsRowS + q * 8;
        *reinterpret_cast<uint2*>(&sH[buf][off]) =
            make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
        *reinterpret_cast<uint2*>(&sL[buf][off]) =
            make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
      }
    };
    // element offset of stage s in h's row and in each w2 row
    auto h_off = [&](int s) { return (size_t)(s / spe) * fs + (size_t)(s % spe) * kBKs; };
    auto w_off = [&](int s) { return (size_t)(s / spe) * wexp + (size_t)(s % spe) * kBKs; };

    __syncthreads();
    uint4 hv[PER];
    uint4 bq[4][2];
#pragma unroll
    for (int i = 0; i < PER; ++i) hv[i] = ldg16(hr[i]);
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      bq[nf][0] = ldg16(wp[nf]);
      bq[nf][1] = ldg16(wp[nf] + 32);
    }
    split_store(0, hv);
    __syncthreads();

#pragma unroll 1
    for (int s = 0; s < nst; ++s) {
      const int cur = s & 1;
      const int sn = min(s + 1, nst - 1);
      const size_t ho = h_off(sn), wo = w_off(sn);
      uint4 bn[4][2];
#pragma unroll
      for (int i = 0; i < PER; ++i) hv[i] = ldg16(hr[i] + ho);
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        bn[nf][0] = ldg16(wp[nf] + wo);
        bn[nf][1] = ldg16(wp[nf] + wo + 32);
      }
      const int aoff = ln * kLdsRowS + lg * 16;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          const int o = aoff + i * 16 * kLdsRowS + j * 64;
          const bf16x8_t ah = as_bf16x8(*reinterpret_cast<const uint4*>(&sH[cur][o]));
          const bf16x8_t al = as_bf16x8(*reinterpret_cast<const uint4*>(&sL[cur][o]));
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) {
            acc[i][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, as_bf16x8(bq[nf][j]), acc[i][nf], 0, 0, 0);
            acc[i][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, as_bf16x8(bq[nf][j]), acc[i][nf], 0, 0, 0);
          }
        }
      if (s + 1 < nst) split_store(cur ^ 1, hv);
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) { bq[nf][0] = bn[nf][0]; bq[nf][1] = bn[nf][1]; }
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = i * 16 + lg * 4 + r;
        if (m < rows) {
          const int t = row0 + m;
          const int o = nt * 256 + wv * 64 + ln;
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) {
            const size_t oi = (size_t)t * d + o + nf * 16;
            if (COMBINE) {
              const float v = combine_one(acc[i][nf][r], comb.y_perm, comb.pair_pos, comb.topk_w,
                                          t, comb.k, d, o + nf * 16);
              if (comb.out_bf16) static_cast<uint16_t*>(comb.out)[oi] = f32_to_bf16(v);
              else static_cast<float*>(comb.out)[oi] = v;
            } else {
              y[oi] = acc[i][nf][r];
            }
          }
        }
      }
  }
}

int mfma_grid() {
  static int g = 0;
  if (!g) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    g = ((cus * 2 + 7) / 8) * 8;   // two workgroups per CU, a multiple of the 8 XCDs
  }
  return g;
}

// Rows per m-tile from the expected pairs per expert (T k / E), with some
// headroom so that most experts fit one tile.
int pick_mf(const k3moe_shape& s, int max_mf) {
  const double ppe = (double)s.T * s.k / s.E * 1.15;
  int mf = (int)((ppe + 15.0) / 16.0);
  if (mf < 1) mf = 1;
  if (mf > max_mf) mf = max_mf;
  return mf;
}

}  // namespace

bool shared_mfma_ok(const k3moe_shape& s) {
  return s.T >= kMfmaMinT && s.x_dtype == K3MOE_BF16 && s.d % 256 == 0 && s.f_shared % 128 == 0;
}

hipError_t launch_shared_mfma(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                              float* h, float* y, hipStream_t st, const CombineArgs& comb) {
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* w13 = static_cast<const uint16_t*>(b.w13);
  const uint16_t* w2 = static_cast<const uint16_t*>(b.w2);
  const int T = (int)s.T, S = b.n_experts, fs = b.f;
  const dim3 g(mfma_grid()), blk(kThreads);
  if (T >= 1024) gateup_shared_mfma<8><<<g, blk, 0, st>>>(xb, w13, h, T, s.d, fs, S);
  else if (T >= 128) gateup_shared_mfma<4><<<g, blk, 0, st>>>(xb, w13, h, T, s.d, fs, S);
  else gateup_shared_mfma<2><<<g, blk, 0, st>>>(xb, w13, h, T, s.d, fs, S);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // (the combine stays a kernel of its own in this class: folded into this
  // epilogue its scattered reads cost more than they save)
  if (comb.y_perm) return hipErrorInvalidValue;
  if (T >= 128) down_shared_mfma<4, false><<<g, blk, 0, st>>>(h, w2, y, T, s.d, fs, S, comb);
  else down_shared_mfma<2, false><<<g, blk, 0, st>>>(h, w2, y, T, s.d, fs, S, comb);
  return hipGetLastError();
}

bool mfma_shape_ok(const k3moe_shape& s) {
  return s.x_dtype == K3MOE_BF16 && s.d % 512 == 0 && s.f % 256 == 0;
}

hipError_t launch_gateup_mfma(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                              const int32_t* offsets, const int32_t* sorted_pair, float* h,
                              hipStream_t st) {
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint8_t* w = static_cast<const uint8_t*>(b.w13);
  const uint8_t* ws = static_cast<const uint8_t*>(b.w13_scale);
  const dim3 g(mfma_grid()), blk(kThreads);
#define K3_GU(MF) gateup_mfma<MF><<<g, blk, 0, st>>>(xb, w, ws, offsets, sorted_pair, h, s.d, s.f, s.E, s.k)
  switch (pick_mf(s, 5)) {
    case 1: K3_GU(1); break;
    case 2: K3_GU(2); break;
    case 3: K3_GU(3); break;
    case 4: K3_GU(4); break;
    default: K3_GU(5); break;
  }
#undef K3_GU
  return hipGetLastError();
}

hipError_t launch_gateup_pc(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                            const int32_t* offsets, const int32_t* sorted_pair, float* h,
                            hipStream_t st) {
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const uint8_t* w = static_cast<const uint8_t*>(b.w13);
  const uint8_t* ws = static_cast<const uint8_t*>(b.w13_scale);
  const dim3 g(mfma_grid() / 2);   // one workgroup per CU
#define K3_PC(MF, RA, RB, NC)                                                               \
  mx_gemm_pc<MF, RA, RB, false, NC><<<g, dim3((NC + 4) * 64), 0, st>>>(xb, w, ws, offsets, \
                                                                      sorted_pair, h, s.d, s.f, s.E, s.k)
  // Four consumer waves (128 features per item) up to 96-row m-tiles; for
  // taller expected m-tiles, eight consumer waves (256 features per item,
  // half the activation re-reads) with 80-row m-tiles.
  const int mf = pick_mf(s, 8);
  if (mf <= 1) K3_PC(1, 3, 7, 4);
  else if (mf <= 2) K3_PC(2, 3, 7, 4);
  else if (mf <= 4) K3_PC(4, 3, 6, 4);
  else if (mf <= 6) K3_PC(6, 3, 4, 4);
  else K3_PC(5, 2, 3, 8);
#undef K3_PC
  return hipGetLastError();
}

hipError_t launch_down_pc(const k3moe_shape& s, const k3moe_expert_bank& b, const float* h,
                          const int32_t* offsets, float* y, hipStream_t st) {
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(h);
  const uint8_t* w = static_cast<const uint8_t*>(b.w2);
  const uint8_t* ws = static_cast<const uint8_t*>(b.w2_scale);
  const dim3 g(mfma_grid() / 2);
#define K3_DPC(MF, RA, RB, NC)                                                               \
  mx_gemm_pc<MF, RA, RB, true, NC><<<g, dim3((NC + 4) * 64), 0, st>>>(hb, w, ws, offsets, nullptr, \
                                                                     y, s.d, s.f, s.E, s.k)
  const int mf = pick_mf(s, 3);
  if (mf <= 1) K3_DPC(1, 3, 3, 8);
  else if (mf <= 2) K3_DPC(2, 3, 3, 8);
  else K3_DPC(3, 2, 3, 8);
#undef K3_DPC
  return hipGetLastError();
}

hipError_t launch_down_mfma(const k3moe_shape& s, const k3moe_expert_bank& b, const float* h,
                            const int32_t* offsets, float* y, hipStream_t st) {
  const uint8_t* w = static_cast<const uint8_t*>(b.w2);
  const uint8_t* ws = static_cast<const uint8_t*>(b.w2_scale);
  const dim3 g(mfma_grid()), blk(kThreads);
#define K3_DN(MF) down_mfma<MF><<<g, blk, 0, st>>>(h, w, ws, offsets, y, s.d, s.f, s.E)
  switch (pick_mf(s, 4)) {
    case 1: K3_DN(1); break;
    case 2: K3_DN(2); break;
    case 3: K3_DN(3); break;
    default: K3_DN(4); break;
  }
#undef K3_DN
  return hipGetLastError();
}

}  // namespace k3
