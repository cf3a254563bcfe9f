// Shared (always-on) experts at small batches in the matrix-core path class:
// bf16 matrix-core kernels with operands straight into registers; larger
// batches take the LDS-ring GEMMs of shared_gemm.hip.
//
// The pages keep two shared experts resident beside the routed ones (the
// kimi-k3-in-c review, "at a glance" table; the README's shard census); every
// token goes through both: S = sum_j Wd_j (silu(Wg_j x) * (Wu_j x)).
// Also here: the shape rule of the matrix-core path class, the persistent
// grid sizes and the routed GEMMs' m-tile height.
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
// The always-on experts see every token, with bf16 weights.  Every
// (token, output) value runs in stages of 64 contraction elements, each the
// two 32-element halves in order, one v_mfma_f32_16x16x32_bf16 each: lane
// (n, g) of the instruction holds elements j*32 + g*8 .. +8 of half j of
// weight row n and of its token row.  The down product splits fp32 h into
// hi = bf16(h) and lo = bf16(h - hi) and contracts over both experts in one
// chain, hi then lo at each half.  The LDS-ring GEMMs (shared_gemm.hip)
// and the small-batch kernels here follow that one chain, so a token's bits
// do not depend on which of them runs it.
constexpr int kBKs = 64;

// Shared experts at small batches (up to 64 tokens): the weights dominate,
// and the LDS-ring GEMMs' 128-token tiles would give too few items to spread
// them over the CUs.  Here a workgroup takes 16 features (gate/up) or 16 outputs
// (down) of one expert for every token, its 4 waves splitting the tokens
// (wave w: tokens 16 w .. 16 w + 15), so that gate/up runs S fs / 16 and
// down d / 16 workgroups.  Operands come from memory straight into
// registers, PD - 1 stages ahead.  Each (token, output) value is the same chain
// as in the LDS-ring GEMMs (stages of 64 elements, then the two 32-element
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
  const dim3 blk(kThreads);
  if (T <= 64 && fs % 16 == 0 && (s.d / kBKs) % 4 == 0 && (S * fs / kBKs) % 4 == 0 &&
      !comb.y_perm) {
    gateup_shared_small<4><<<(unsigned)(S * (fs / 16)), blk, 0, st>>>(xb, w13, h, T, s.d, fs, S);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    down_shared_small<4><<<(unsigned)(s.d / 16), blk, 0, st>>>(h, w2, y, T, s.d, fs, S);
    return hipGetLastError();
  }
  // (in this class the combine stays a kernel of its own: folded into the
  // down's epilogue its scattered reads cost more than they save)
  if (comb.y_perm || !shared_lds_ok(s)) return hipErrorInvalidValue;
  return launch_shared_lds(s, b, x, h, y, st);
}

bool mfma_shape_ok(const k3moe_shape& s) {
  // the scaled-MXFP4 grouped GEMMs take 128-element stages in groups of 4
  return s.x_dtype == K3MOE_BF16 && s.d % 512 == 0 && s.f % 512 == 0;
}

}  // namespace k3
