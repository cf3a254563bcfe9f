// One-token shared-expert gate/up, shared by the stand-alone kernel and the
// kernel that runs it beside the top-k selection.
#pragma once

#include "kern_common.h"

namespace k3 {

// d == kSgU * 8 * 64: every lane owns kSgU chunks of 8 bf16 of each row.
constexpr int kSgU = 14;

// Item = (shared expert se, feature j): its gate row and up row against x
// (staged in LDS as d / 8 uint4), all loads issued before any arithmetic; per
// row dot2 steps over the lane's chunks in order, then the fixed transposed
// butterfly; hs[se][j] = silu(g) * u.
__device__ __forceinline__ void shared_gateup_item(int item, const uint16_t* __restrict__ w13,
                                                   const uint4* xs, float* __restrict__ hs,
                                                   int d, int fs, int lane) {
  const int se = item / fs, j = item - se * fs;
  const uint16_t* gr = w13 + ((size_t)se * 2 * fs + j) * d;
  const uint16_t* ur = gr + (size_t)fs * d;
  uint4 g[kSgU], u[kSgU];
#pragma unroll
  for (int q = 0; q < kSgU; ++q) {
    const int c = lane + kWave * q;
    g[q] = ldg16(gr + (size_t)c * 8);
    u[q] = ldg16(ur + (size_t)c * 8);
  }
  __builtin_amdgcn_sched_barrier(0);   // every load above is issued before any arithmetic
  float v[2] = {0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < kSgU; ++q) {
    const uint4 xa = xs[lane + kWave * q];
    v[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(g[q].x), as_bf16x2(xa.x), v[0], false);
    v[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(g[q].y), as_bf16x2(xa.y), v[0], false);
    v[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(g[q].z), as_bf16x2(xa.z), v[0], false);
    v[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(g[q].w), as_bf16x2(xa.w), v[0], false);
    v[1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(u[q].x), as_bf16x2(xa.x), v[1], false);
    v[1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(u[q].y), as_bf16x2(xa.y), v[1], false);
    v[1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(u[q].z), as_bf16x2(xa.z), v[1], false);
    v[1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(u[q].w), as_bf16x2(xa.w), v[1], false);
  }
  // transposed butterfly (the same pairing tree as the other GEMV reductions)
  {
    const bool up = (lane & 32) != 0;
    const float send = up ? v[0] : v[1];
    const float keep = up ? v[1] : v[0];
    v[0] = keep + __shfl_xor(send, 32, kWave);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) v[0] = v[0] + __shfl_xor(v[0], o, kWave);
  }
  const float uval = __shfl_xor(v[0], 32, kWave);
  if (lane == 0) hs[(size_t)se * fs + j] = silu_mul(v[0], uval);
}

}  // namespace k3
