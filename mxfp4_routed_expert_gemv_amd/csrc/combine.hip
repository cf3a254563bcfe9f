// Fixed-order combine: out[t] = shared_y[t] + sum over the token's slots in
// ascending expert id (the order route writes them) of w * y, skipping zero
// weights, with no atomics, so every output has one summation order.
#include "internal.h"
#include "kern_common.h"

namespace k3 {
namespace {

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ shared_y,
                                                      void* __restrict__ out, int64_t T, int d,
                                                      int k) {
  const int dq = d >> 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * dq) return;
  const int64_t t = i / dq;
  const int o = (int)(i - t * dq) * 4;
  float4 acc = shared_y ? *reinterpret_cast<const float4*>(shared_y + t * d + o)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
  // Slots in groups of 8: every load of a group is issued before the first
  // multiply-add (dropped pairs read row 0 and are skipped), so the k row
  // loads overlap instead of forming a chain.
  constexpr int G = 8;
  for (int s0 = 0; s0 < k; s0 += G) {
    float w[G];
    int pp[G];
    float4 v[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const bool in = s0 + u < k;
      w[u] = in ? topk_w[t * k + s0 + u] : 0.0f;
      pp[u] = in ? pair_pos[t * k + s0 + u] : -1;
    }
#pragma unroll
    for (int u = 0; u < G; ++u)
      v[u] = *reinterpret_cast<const float4*>(y_perm + (size_t)(pp[u] >= 0 ? pp[u] : 0) * d + o);
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (w[u] != 0.0f && pp[u] >= 0) {
        acc.x = __builtin_fmaf(w[u], v[u].x, acc.x);
        acc.y = __builtin_fmaf(w[u], v[u].y, acc.y);
        acc.z = __builtin_fmaf(w[u], v[u].z, acc.z);
        acc.w = __builtin_fmaf(w[u], v[u].w, acc.w);
      }
  }
  if (OUT_BF16) {
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
    pk.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + t * d + o) = pk;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + t * d + o) = acc;
  }
}

}  // namespace

hipError_t launch_combine(const k3moe_shape& s, const float* y_perm, const int32_t* pair_pos,
                          const float* topk_w, const float* shared_y, void* out, hipStream_t st) {
  const int64_t n = s.T * (s.d / 4);
  const unsigned g = (unsigned)((n + 255) / 256);
  if (s.out_dtype == K3MOE_BF16)
    combine_kernel<true><<<g, 256, 0, st>>>(y_perm, pair_pos, topk_w, shared_y, out, s.T, s.d, s.k);
  else
    combine_kernel<false><<<g, 256, 0, st>>>(y_perm, pair_pos, topk_w, shared_y, out, s.T, s.d,
                                             s.k);
  return hipGetLastError();
}

}  // namespace k3
