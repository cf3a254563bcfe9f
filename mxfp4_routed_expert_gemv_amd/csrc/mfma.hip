// Shared (always-on) experts for large batches: bf16 GEMMs on the matrix
// cores (v_mfma_f32_16x16x32_bf16).
//
// The pages keep two shared experts resident beside the routed ones (the
// kimi-k3-in-c review, "at a glance" table; the README's shard census); every
// token goes through both: S = sum_j Wd_j (silu(Wg_j x) * (Wu_j x)).  Their
// weights are bf16, so these are plain bf16 GEMMs over all T tokens:
//   * an m-tile is up to BM = 16 MF consecutive tokens; a persistent grid of
//     4-wave workgroups walks (m-tile, expert, n-tile) items, split into 8
//     contiguous ranges, one per XCD, so the workgroups that share an
//     m-tile's activations run on the same L2;
//   * the contraction runs in stages of 64 elements; lane (n = lane % 16,
//     g = lane / 16) loads 8 consecutive bf16 weights of row n for each
//     MFMA step j, and the A operand (activations in LDS) is read in the same
//     element order, so every (token, output) sum runs in a fixed order that
//     does not depend on the other tokens of the tile.
// Also here: the shape rule of the matrix-core path class, its persistent
// grid size and its m-tile height.
#include "internal.h"
#include "kern_common.h"
#include "grouped.h"

namespace k3 {
namespace {

using namespace grouped;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kThreads = 256;    // 4 waves

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
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

// Shared experts at small batches (up to 64 tokens): the weights dominate,
// and the tiled kernels above would give too few items to spread them over
// the CUs.  Here a workgroup takes 16 features (gate/up) or 16 outputs
// (down) of one expert for every token, its 4 waves splitting the tokens
// (wave w: tokens 16 w .. 16 w + 15), so that gate/up runs S fs / 16 and
// down d / 16 workgroups.  Operands come from memory straight into
// registers, PD - 1 stages ahead.  Each (token, output) value is the same chain
// as in the tiled kernels (stages of 64 elements, then the two 32-element
// halves, the down's hi then lo pass), so it has their bits.
template <int PD>
__global__ __launch_bounds__(kThreads) void gateup_shared_small(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w13,
                                                                float* __restrict__ h, int T,
                                                                int d, int fs, int S) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int ng = fs / 16;
  const int se = blockIdx.x / ng, g = blockIdx.x - se * ng;
  if (se >= S || 16 * wv >= T) return;   // no barrier below
  const int nst = d / kBKs;
  const uint16_t* ar = x + (size_t)min(16 * wv + ln, T - 1) * d + lg * 8;
  const uint16_t* gr = w13 + ((size_t)se * 2 * fs + g * 16 + ln) * d + lg * 8;
  const uint16_t* ur = gr + (size_t)fs * d;
  uint4 av[PD][2], gv[PD][2], uv[PD][2];
  auto load = [&](int st, int sl) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      av[sl][j] = ldg16(ar + st * kBKs + j * 32);
      gv[sl][j] = ldg16(gr + st * kBKs + j * 32);
      uv[sl][j] = ldg16(ur + st * kBKs + j * 32);
    }
  };
  f32x4_t acc_g = f32x4_t{0.f, 0.f, 0.f, 0.f}, acc_u = acc_g;
#pragma unroll
  for (int q = 0; q < PD - 1; ++q) load(min(q, nst - 1), q);
#pragma unroll 1
  for (int s0 = 0; s0 < nst; s0 += PD) {   // nst % PD == 0
#pragma unroll
    for (int q = 0; q < PD; ++q) {
      load(min(s0 + q + PD - 1, nst - 1), (q + PD - 1) % PD);   // past the end: a repeat
      __builtin_amdgcn_sched_barrier(0);   // keep the loads PD - 1 stages ahead
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8_t a = as_bf16x8(av[q][j]);
        acc_g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(gv[q][j]), acc_g, 0, 0, 0);
        acc_u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(uv[q][j]), acc_u, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * wv + lg * 4 + r;
    if (t < T) h[((size_t)t * S + se) * fs + g * 16 + ln] = silu_mul(acc_g[r], acc_u[r]);
  }
}

template <int PD>
__global__ __launch_bounds__(kThreads) void down_shared_small(const float* __restrict__ h,
                                                              const uint16_t* __restrict__ w2,
                                                              float* __restrict__ y, int T, int d,
                                                              int fs, int S) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int o0 = blockIdx.x * 16;
  if (o0 >= d || 16 * wv >= T) return;   // no barrier below
  const int spe = fs / kBKs, nst = S * spe;
  const float* hr = h + (size_t)min(16 * wv + ln, T - 1) * S * fs + lg * 8;
  const uint16_t* wr = w2 + (size_t)(o0 + ln) * fs + lg * 8;
  const size_t wexp = (size_t)d * fs;   // elements per shared expert's w2
  uint4 hv[PD][2][2], bv[PD][2];
  auto load = [&](int st, int sl) {
    const size_t ho = (size_t)(st / spe) * fs + (size_t)(st % spe) * kBKs;
    const size_t wo = (size_t)(st / spe) * wexp + (size_t)(st % spe) * kBKs;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      hv[sl][j][0] = ldg16(hr + ho + j * 32);
      hv[sl][j][1] = ldg16(hr + ho + j * 32 + 4);
      bv[sl][j] = ldg16(wr + wo + j * 32);
    }
  };
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < PD - 1; ++q) load(min(q, nst - 1), q);
#pragma unroll 1
  for (int s0 = 0; s0 < nst; s0 += PD) {   // nst % PD == 0
#pragma unroll
    for (int q = 0; q < PD; ++q) {
      load(min(s0 + q + PD - 1, nst - 1), (q + PD - 1) % PD);   // past the end: a repeat
      __builtin_amdgcn_sched_barrier(0);   // keep the loads PD - 1 stages ahead
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // h split into hi and lo bf16, as the tiled kernel does
        const float fv[8] = {__uint_as_float(hv[q][j][0].x), __uint_as_float(hv[q][j][0].y),
                             __uint_as_float(hv[q][j][0].z), __uint_as_float(hv[q][j][0].w),
                             __uint_as_float(hv[q][j][1].x), __uint_as_float(hv[q][j][1].y),
                             __uint_as_float(hv[q][j][1].z), __uint_as_float(hv[q][j][1].w)};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint16_t h0 = f32_to_bf16(fv[2 * c]), h1 = f32_to_bf16(fv[2 * c + 1]);
          const uint16_t l0 = f32_to_bf16(fv[2 * c] - __uint_as_float((uint32_t)h0 << 16));
          const uint16_t l1 = f32_to_bf16(fv[2 * c + 1] - __uint_as_float((uint32_t)h1 << 16));
          hi[c] = h0 | ((uint32_t)h1 << 16);
          lo[c] = l0 | ((uint32_t)l1 << 16);
        }
        const bf16x8_t ah = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
        const bf16x8_t al = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
        const bf16x8_t b = as_bf16x8(bv[q][j]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * wv + lg * 4 + r;
    if (t < T) y[(size_t)t * d + o0 + ln] = acc[r];
  }
}

}  // namespace

int mfma_grid() { return (cu_count() * 2 + 7) / 8 * 8; }
int grouped_grid() { return (cu_count() + 7) / 8 * 8; }

// Rows per m-tile from the expected pairs per expert (T k / E), with some
// headroom so that most experts fit one tile.
int pick_mf(const k3moe_shape& s, int max_mf) {
  const double ppe = (double)s.T * s.k / s.E * 1.15;
  int mf = (int)((ppe + 15.0) / 16.0);
  if (mf < 1) mf = 1;
  if (mf > max_mf) mf = max_mf;
  return mf;
}


// The shared experts take the matrix-core kernels only inside the MFMA path
// class (so a token's bits change at no other batch size than the class
// boundary), and only when their width fits the kernels' 128-feature tiles;
// otherwise they stay GEMVs at every batch size.
bool shared_mfma_ok(const k3moe_shape& s) { return use_mfma(s) && s.f_shared % 128 == 0; }

hipError_t launch_shared_mfma(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                              float* h, float* y, hipStream_t st, const CombineArgs& comb) {
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* w13 = static_cast<const uint16_t*>(b.w13);
  const uint16_t* w2 = static_cast<const uint16_t*>(b.w2);
  const int T = (int)s.T, S = b.n_experts, fs = b.f;
  const dim3 g(mfma_grid()), blk(kThreads);
  if (T <= 64 && fs % 16 == 0 && (s.d / kBKs) % 4 == 0 && (S * fs / kBKs) % 4 == 0 &&
      !comb.y_perm) {
    gateup_shared_small<4><<<(unsigned)(S * (fs / 16)), blk, 0, st>>>(xb, w13, h, T, s.d, fs, S);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    down_shared_small<4><<<(unsigned)(s.d / 16), blk, 0, st>>>(h, w2, y, T, s.d, fs, S);
    return hipGetLastError();
  }
  if (T >= 1024) gateup_shared_mfma<8><<<g, blk, 0, st>>>(xb, w13, h, T, s.d, fs, S);
  else if (T >= 128) gateup_shared_mfma<4><<<g, blk, 0, st>>>(xb, w13, h, T, s.d, fs, S);
  else gateup_shared_mfma<2><<<g, blk, 0, st>>>(xb, w13, h, T, s.d, fs, S);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // (the combine stays a kernel of its own in this class: folded into this
  // epilogue its scattered reads cost more than they save)
  if (comb.y_perm) return hipErrorInvalidValue;
  if (T >= 1024) down_shared_mfma<8, false><<<g, blk, 0, st>>>(h, w2, y, T, s.d, fs, S, comb);
  else if (T >= 128) down_shared_mfma<4, false><<<g, blk, 0, st>>>(h, w2, y, T, s.d, fs, S, comb);
  else down_shared_mfma<2, false><<<g, blk, 0, st>>>(h, w2, y, T, s.d, fs, S, comb);
  return hipGetLastError();
}

bool mfma_shape_ok(const k3moe_shape& s) {
  // the scaled-MXFP4 grouped GEMMs take 128-element stages in groups of 4
  return s.x_dtype == K3MOE_BF16 && s.d % 512 == 0 && s.f % 512 == 0;
}

}  // namespace k3
