// Device helpers shared by the gfx950 kernels of libk3moe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k3 {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 scale byte -> fp32 2^(s-127): s = 0 is the subnormal 2^-127, s = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return s == 0u ? __uint_as_float(0x00400000u)
                 : (s == 255u ? __uint_as_float(0x7FC00000u) : __uint_as_float(s << 23));
}

// Two E2M1 codes (byte `sel` of `w`: low nibble = even element) -> bf16 pair,
// exactly (E2M1 values have two significant bits).
template <int SEL>
__device__ __forceinline__ bf16x2_t e2m1x2_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}
template <int SEL>
__device__ __forceinline__ f32x2_t e2m1x2_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2_t, w);
}

// sum_{q < 16} code_pair(q) . x_pair(q) for one 32-element block: 16 dot2
// steps in a fixed order (the partial sum of one scale block).
__device__ __forceinline__ float block_dot_bf16(const uint4& c, const uint4 (&xv)[4]) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 xa = xv[q];
    // code dword q holds elements 8q .. 8q+7; x dwords 4q .. 4q+3 hold the
    // same elements as bf16 pairs.
    acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<0>(cw[q]), as_bf16x2(xa.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<1>(cw[q]), as_bf16x2(xa.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<2>(cw[q]), as_bf16x2(xa.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<3>(cw[q]), as_bf16x2(xa.w), acc, false);
  }
  return acc;
}

// Same block partial with fp32 activations (32 floats = 8 x uint4):
// sequential fused multiply-adds in element order.
__device__ __forceinline__ float block_dot_f32(const uint4& c, const uint4 (&xv)[8]) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 xa = xv[2 * q], xb = xv[2 * q + 1];
    f32x2_t w0 = e2m1x2_f32<0>(cw[q]), w1 = e2m1x2_f32<1>(cw[q]);
    f32x2_t w2 = e2m1x2_f32<2>(cw[q]), w3 = e2m1x2_f32<3>(cw[q]);
    acc = __builtin_fmaf(w0.x, __uint_as_float(xa.x), acc);
    acc = __builtin_fmaf(w0.y, __uint_as_float(xa.y), acc);
    acc = __builtin_fmaf(w1.x, __uint_as_float(xa.z), acc);
    acc = __builtin_fmaf(w1.y, __uint_as_float(xa.w), acc);
    acc = __builtin_fmaf(w2.x, __uint_as_float(xb.x), acc);
    acc = __builtin_fmaf(w2.y, __uint_as_float(xb.y), acc);
    acc = __builtin_fmaf(w3.x, __uint_as_float(xb.z), acc);
    acc = __builtin_fmaf(w3.y, __uint_as_float(xb.w), acc);
  }
  return acc;
}

// Butterfly sum over the 64 lanes; every lane ends with the same bits
// (each step adds the same two operands, in either order, on both partners).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_min(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmin(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  return v;
}

// DPP move of a 64-bit value (two 32-bit halves); lanes whose source lies
// outside the row, or whose row is masked off, read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK,
                                                            0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL,
                                                            ROW_MASK, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

// Maximum of an unsigned 64-bit value over the wave, returned to every lane
// (row_shr 1/2/4/8 within rows of 16, then row_bcast 15 and 31 carry the row
// maxima to lane 63; 0 is the identity).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0x111, 0xF>(v); v = o > v ? o : v;
  o = dpp_u64<0x112, 0xF>(v); v = o > v ? o : v;
  o = dpp_u64<0x114, 0xF>(v); v = o > v ? o : v;
  o = dpp_u64<0x118, 0xF>(v); v = o > v ? o : v;
  o = dpp_u64<0x142, 0xA>(v); v = o > v ? o : v;
  o = dpp_u64<0x143, 0xC>(v); v = o > v ? o : v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Order-preserving map of a non-NaN double to uint64 (a < b iff key(a) <
// key(b)); every key is > 0, so 0 can stand for "no value".
__device__ __forceinline__ uint64_t order_key(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double key_value(uint64_t k) {
  const uint64_t u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)u);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  // silu(g) * u with silu(g) = g / (1 + e^-g); for g < -88.7 e^-g is +inf
  // and the quotient is -0, never NaN.
  return (g / (1.0f + expf(-g))) * u;
}

// One output of the fixed-order combine: starting from the shared experts'
// fp32 value, the routed slots of token t in slot order (ascending expert
// id), skipping zero weights and dropped pairs.  The combine kernel and the
// fused shared-expert epilogues both call this, so they agree bit for bit.
__device__ __forceinline__ float combine_one(float acc, const float* __restrict__ y_perm,
                                             const int32_t* __restrict__ pair_pos,
                                             const float* __restrict__ topk_w, int64_t t, int k,
                                             int d, int o) {
  // groups of 8 slots: every load of a group is issued before its first
  // multiply-add (dropped pairs read row 0 and are skipped)
  constexpr int G = 8;
  for (int s0 = 0; s0 < k; s0 += G) {
    float w[G], v[G];
    int pp[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int s = min(s0 + u, k - 1);
      w[u] = topk_w[t * k + s];
      pp[u] = pair_pos[t * k + s];
    }
#pragma unroll
    for (int u = 0; u < G; ++u) v[u] = y_perm[(size_t)(pp[u] >= 0 ? pp[u] : 0) * d + o];
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (s0 + u < k && w[u] != 0.0f && pp[u] >= 0) acc = __builtin_fmaf(w[u], v[u], acc);
  }
  return acc;
}

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Copies n16 16-byte words (at most 2048) into LDS with a 256-thread
// workgroup; out-of-range threads rewrite the last word with its own value,
// so every load is issued before any wait.
__device__ __forceinline__ void stage_row(const uint4* __restrict__ src, int n16, uint4* dst) {
  constexpr int U = 8;  // up to 2048 words (32 KB)
  uint4 t[U];
#pragma unroll
  for (int u = 0; u < U; ++u) t[u] = src[min((int)threadIdx.x + 256 * u, n16 - 1)];
  // Out-of-range threads rewrite the last word with its own value: stores
  // stay unconditional, so the loads above are all issued before any wait.
#pragma unroll
  for (int u = 0; u < U; ++u) dst[min((int)threadIdx.x + 256 * u, n16 - 1)] = t[u];
}


}  // namespace k3
