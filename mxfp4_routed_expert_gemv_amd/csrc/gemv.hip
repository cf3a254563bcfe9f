// Decode-class expert FFN: matrix-vector kernels that stream each weight row
// once from HBM.
//
// The pages' engine multiplies the 4-bit experts directly instead of
// expanding them (kimi-k3-in-c review, "KDA/MLA/MoE" table; explainer page,
// "reduction one"); here each lane loads one 16-byte MX block (32 E2M1 codes)
// per row with a 128-bit load, turns each code byte into a bf16 (or fp32)
// pair in registers with v_cvt_scalef32_pk_*_fp4, reduces the block with
// dot2/FMA steps, applies the block's E8M0 scale, and the 64 lanes of the
// wave are combined by a fixed butterfly.  Every (token, output) reduction
// has the same order whatever else is in the batch.
//
// Work unit: one wave = (active expert, group of R output rows); the wave
// loops over that expert's tokens, MT at a time, so a weight row is fetched
// from HBM once per call however many tokens chose the expert.
#include "internal.h"
#include "kern_common.h"

namespace k3 {
namespace {

// ------------------------------------------------------------ active experts
// Experts with at least one pair, in ascending id; one workgroup (E <= 1024).
__global__ __launch_bounds__(1024) void build_active(const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ active,
                                                     int32_t* __restrict__ n_active, int E) {
  __shared__ int sums[1024];
  const int e = threadIdx.x;
  const int flag = (e < E && offsets[e + 1] > offsets[e]) ? 1 : 0;
  sums[e] = flag;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = (e >= o) ? sums[e - o] : 0;
    __syncthreads();
    sums[e] += add;
    __syncthreads();
  }
  if (flag) active[sums[e] - 1] = e;
  if (e == 1023) *n_active = sums[1023];
}

template <bool XF32>
struct XBlock;  // one 32-element activation block
template <>
struct XBlock<false> {
  uint4 v[4];
  __device__ __forceinline__ void load(const void* x, size_t elem) {
    const uint16_t* p = static_cast<const uint16_t*>(x) + elem;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ldg16(p + 8 * i);
  }
  __device__ __forceinline__ float dot(const uint4& c) const { return block_dot_bf16(c, v); }
};
template <>
struct XBlock<true> {
  uint4 v[8];
  __device__ __forceinline__ void load(const void* x, size_t elem) {
    const float* p = static_cast<const float*>(x) + elem;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ldg16(p + 4 * i);
  }
  __device__ __forceinline__ float dot(const uint4& c) const { return block_dot_f32(c, v); }
};

// ------------------------------------------------------ routed gate/up (MXFP4)
// h[p][j] = silu(g) * u for the R gate rows j = rg*R .. rg*R+R-1 of expert e
// and the matching up rows f + j, for every sorted pair p of e.
template <int R, int MT, int NU, bool XF32>
__global__ __launch_bounds__(256) void gemv_gateup_mxfp4(
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ w13s, const void* __restrict__ x,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active,
    float* __restrict__ h, int d, int f, int k, int rgroups) {
  constexpr int NR = 2 * R;
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int j = wid / rgroups, rg = wid - j * rgroups;
  if (j >= *n_active) return;
  const int e = active[j];
  const int p0 = offsets[e], p1 = offsets[e + 1];
  const int nb = d >> 5;
  const size_t rb = (size_t)(d >> 1), sb = (size_t)nb;
  const uint8_t* qe = w13 + (size_t)e * 2 * f * rb;
  const uint8_t* se = w13s + (size_t)e * 2 * f * sb;
  int rows[NR];
#pragma unroll
  for (int r = 0; r < R; ++r) { rows[r] = rg * R + r; rows[R + r] = f + rg * R + r; }

  for (int p = p0; p < p1; p += MT) {
    float acc[NR][MT];
    size_t xoff[MT];
    bool tv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      tv[mt] = p + mt < p1;
      xoff[mt] = tv[mt] ? (size_t)(sorted_pair[p + mt] / k) * d : 0;
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r][mt] = 0.0f;
    }
    for (int b0 = 0; b0 < nb; b0 += kWave * NU) {
      uint4 cq[NU][NR];
      uint32_t cs[NU][NR];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int b = b0 + lane + kWave * u;
        if (b < nb) {
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            cq[u][r] = ldg16(qe + rows[r] * rb + (size_t)b * 16);
            cs[u][r] = se[rows[r] * sb + b];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int b = b0 + lane + kWave * u;
        if (b < nb) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if (!tv[mt]) continue;
            XBlock<XF32> xb;
            xb.load(x, xoff[mt] + (size_t)b * 32);
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r][mt] = __builtin_fmaf(xb.dot(cq[u][r]), e8m0_to_f32(cs[u][r]), acc[r][mt]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[r][mt] = wave_sum(acc[r][mt]);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (lane == r * MT + mt && tv[mt])
          h[(size_t)(p + mt) * f + rg * R + r] = silu_mul(acc[r][mt], acc[R + r][mt]);
  }
}

// --------------------------------------------------------- routed down (MXFP4)
// y[p][o] = sum_j Wd[e][o][j] h[p][j] for rows o = rg*R .. rg*R+R-1.
template <int R, int MT, int NU>
__global__ __launch_bounds__(256) void gemv_down_mxfp4(
    const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2s, const float* __restrict__ h,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, float* __restrict__ y, int d, int f, int rgroups) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int j = wid / rgroups, rg = wid - j * rgroups;
  if (j >= *n_active) return;
  const int e = active[j];
  const int p0 = offsets[e], p1 = offsets[e + 1];
  const int nb = f >> 5;
  const size_t rb = (size_t)(f >> 1), sb = (size_t)nb;
  const uint8_t* qe = w2 + (size_t)e * d * rb;
  const uint8_t* se = w2s + (size_t)e * d * sb;
  const int o0 = rg * R;

  for (int p = p0; p < p1; p += MT) {
    float acc[R][MT];
    bool tv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      tv[mt] = p + mt < p1;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r][mt] = 0.0f;
    }
    for (int b0 = 0; b0 < nb; b0 += kWave * NU) {
      uint4 cq[NU][R];
      uint32_t cs[NU][R];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int b = b0 + lane + kWave * u;
        if (b < nb) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            cq[u][r] = ldg16(qe + (size_t)(o0 + r) * rb + (size_t)b * 16);
            cs[u][r] = se[(size_t)(o0 + r) * sb + b];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int b = b0 + lane + kWave * u;
        if (b < nb) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if (!tv[mt]) continue;
            XBlock<true> hb;
            hb.load(h, (size_t)(p + mt) * f + (size_t)b * 32);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][mt] = __builtin_fmaf(hb.dot(cq[u][r]), e8m0_to_f32(cs[u][r]), acc[r][mt]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[r][mt] = wave_sum(acc[r][mt]);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (lane == r * MT + mt && tv[mt]) y[(size_t)(p + mt) * d + o0 + r] = acc[r][mt];
  }
}

// ------------------------------------------------------- shared experts (bf16)
// 8-element chunk dot: acc += sum over the chunk in element order.
template <bool XF32>
__device__ __forceinline__ float chunk_dot(const uint4& w, const void* x, size_t elem, float acc) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  if (XF32) {
    const float* p = static_cast<const float*>(x) + elem;
    const uint4 a = ldg16(p), b = ldg16(p + 4);
    const uint32_t xx[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc = __builtin_fmaf(bf16_lo(ww[q]), __uint_as_float(xx[2 * q]), acc);
      acc = __builtin_fmaf(bf16_hi(ww[q]), __uint_as_float(xx[2 * q + 1]), acc);
    }
  } else {
    const uint4 a = ldg16(static_cast<const uint16_t*>(x) + elem);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ww[0]), as_bf16x2(a.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ww[1]), as_bf16x2(a.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ww[2]), as_bf16x2(a.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ww[3]), as_bf16x2(a.w), acc, false);
  }
  return acc;
}

// hs[t][s][j] = silu(g) * u for shared expert s, rows j = rg*R .. rg*R+R-1.
template <int R, int MT, int NU, bool XF32>
__global__ __launch_bounds__(256) void gemv_gateup_bf16(const uint16_t* __restrict__ w13,
                                                        const void* __restrict__ x,
                                                        float* __restrict__ hs, int T, int d,
                                                        int fs, int S, int rgroups) {
  constexpr int NR = 2 * R;
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int s = wid / rgroups, rg = wid - s * rgroups;
  if (s >= S) return;
  const int nc = d >> 3;
  const uint16_t* we = w13 + (size_t)s * 2 * fs * d;
  int rows[NR];
#pragma unroll
  for (int r = 0; r < R; ++r) { rows[r] = rg * R + r; rows[R + r] = fs + rg * R + r; }
  for (int t0 = 0; t0 < T; t0 += MT) {
    float acc[NR][MT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[r][mt] = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += kWave * NU) {
      uint4 wv[NU][NR];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int c = c0 + lane + kWave * u;
        if (c < nc)
#pragma unroll
          for (int r = 0; r < NR; ++r) wv[u][r] = ldg16(we + (size_t)rows[r] * d + (size_t)c * 8);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int c = c0 + lane + kWave * u;
        if (c < nc)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (t0 + mt < T)
#pragma unroll
              for (int r = 0; r < NR; ++r)
                acc[r][mt] = chunk_dot<XF32>(wv[u][r], x, (size_t)(t0 + mt) * d + (size_t)c * 8,
                                             acc[r][mt]);
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[r][mt] = wave_sum(acc[r][mt]);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (lane == r * MT + mt && t0 + mt < T)
          hs[((size_t)(t0 + mt) * S + s) * fs + rg * R + r] = silu_mul(acc[r][mt], acc[R + r][mt]);
  }
}

// y[t][o] = sum over shared experts s in order of (sum_j W2[s][o][j] hs[t][s][j]).
template <int R, int MT, int NU>
__global__ __launch_bounds__(256) void gemv_down_bf16(const uint16_t* __restrict__ w2,
                                                      const float* __restrict__ hs,
                                                      float* __restrict__ y, int T, int d, int fs,
                                                      int S, int rgroups) {
  const int lane = threadIdx.x & 63;
  const int rg = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rg >= rgroups) return;
  const int nc = fs >> 3;
  const int o0 = rg * R;
  for (int t0 = 0; t0 < T; t0 += MT) {
    float tot[R][MT];
    for (int s = 0; s < S; ++s) {
      const uint16_t* we = w2 + (size_t)s * d * fs;
      float acc[R][MT];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[r][mt] = 0.0f;
      for (int c0 = 0; c0 < nc; c0 += kWave * NU) {
        uint4 wv[NU][R];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int c = c0 + lane + kWave * u;
          if (c < nc)
#pragma unroll
            for (int r = 0; r < R; ++r) wv[u][r] = ldg16(we + (size_t)(o0 + r) * fs + (size_t)c * 8);
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int c = c0 + lane + kWave * u;
          if (c < nc)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              if (t0 + mt < T)
#pragma unroll
                for (int r = 0; r < R; ++r)
                  acc[r][mt] = chunk_dot<true>(wv[u][r], hs,
                                               ((size_t)(t0 + mt) * S + s) * fs + (size_t)c * 8,
                                               acc[r][mt]);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float v = wave_sum(acc[r][mt]);
          tot[r][mt] = (s == 0) ? v : tot[r][mt] + v;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (lane == r * MT + mt && t0 + mt < T) y[(size_t)(t0 + mt) * d + o0 + r] = tot[r][mt];
  }
}

inline unsigned blocks_for_waves(int64_t waves) { return (unsigned)((waves + 3) / 4); }

template <int MT>
hipError_t routed_launch(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                         const int32_t* offsets, const int32_t* sorted_pair, float* y,
                         const ExpertWs& ws, hipStream_t st) {
  constexpr int RG = 2, RD = 8;
  const int64_t P = s.T * s.k;
  const int64_t max_active = P < s.E ? P : s.E;
  const int rg_gu = s.f / RG, rg_dn = s.d / RD;
  const uint8_t* w13 = static_cast<const uint8_t*>(bank.w13);
  const uint8_t* w13s = static_cast<const uint8_t*>(bank.w13_scale);
  const uint8_t* w2 = static_cast<const uint8_t*>(bank.w2);
  const uint8_t* w2s = static_cast<const uint8_t*>(bank.w2_scale);
  const unsigned g1 = blocks_for_waves(max_active * rg_gu);
  if (s.x_dtype == K3MOE_F32)
    gemv_gateup_mxfp4<RG, MT, 4, true><<<g1, 256, 0, st>>>(w13, w13s, x, offsets, sorted_pair,
                                                           ws.active, ws.n_active, ws.h, s.d, s.f,
                                                           s.k, rg_gu);
  else
    gemv_gateup_mxfp4<RG, MT, 4, false><<<g1, 256, 0, st>>>(w13, w13s, x, offsets, sorted_pair,
                                                            ws.active, ws.n_active, ws.h, s.d,
                                                            s.f, s.k, rg_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned g2 = blocks_for_waves(max_active * rg_dn);
  gemv_down_mxfp4<RD, (MT > 2 ? 2 : MT), 1><<<g2, 256, 0, st>>>(
      w2, w2s, ws.h, offsets, ws.active, ws.n_active, y, s.d, s.f, rg_dn);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_ffn(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                             const int32_t* offsets, const int32_t* sorted_pair, float* y,
                             const ExpertWs& ws, hipStream_t st) {
  build_active<<<1, 1024, 0, st>>>(offsets, ws.active, ws.n_active, s.E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (s.T == 1) return routed_launch<1>(s, bank, x, offsets, sorted_pair, y, ws, st);
  return routed_launch<4>(s, bank, x, offsets, sorted_pair, y, ws, st);
}

hipError_t launch_shared_ffn(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                             float* y, const SharedWs& ws, hipStream_t st) {
  constexpr int RG = 2, RD = 4;
  const int S = bank.n_experts, fs = bank.f, T = (int)s.T;
  const uint16_t* w13 = static_cast<const uint16_t*>(bank.w13);
  const uint16_t* w2 = static_cast<const uint16_t*>(bank.w2);
  const int rg_gu = fs / RG, rg_dn = s.d / RD;
  const unsigned g1 = blocks_for_waves((int64_t)S * rg_gu);
  const bool xf32 = s.x_dtype == K3MOE_F32;
  if (T == 1) {
    if (xf32)
      gemv_gateup_bf16<RG, 1, 4, true><<<g1, 256, 0, st>>>(w13, x, ws.h, T, s.d, fs, S, rg_gu);
    else
      gemv_gateup_bf16<RG, 1, 4, false><<<g1, 256, 0, st>>>(w13, x, ws.h, T, s.d, fs, S, rg_gu);
  } else {
    if (xf32)
      gemv_gateup_bf16<RG, 4, 4, true><<<g1, 256, 0, st>>>(w13, x, ws.h, T, s.d, fs, S, rg_gu);
    else
      gemv_gateup_bf16<RG, 4, 4, false><<<g1, 256, 0, st>>>(w13, x, ws.h, T, s.d, fs, S, rg_gu);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned g2 = blocks_for_waves(rg_dn);
  if (T == 1)
    gemv_down_bf16<RD, 1, 2><<<g2, 256, 0, st>>>(w2, ws.h, y, T, s.d, fs, S, rg_dn);
  else
    gemv_down_bf16<RD, 2, 2><<<g2, 256, 0, st>>>(w2, ws.h, y, T, s.d, fs, S, rg_dn);
  return hipGetLastError();
}

}  // namespace k3
