// Device helpers of the grouped (expert-sorted) GEMMs: the m-tile schedule
// over the experts' row ranges, the XCD-contiguous item split of a
// persistent grid, and the LDS-DMA / wait / barrier primitives of the
// producer/consumer kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k3 {
namespace grouped {

constexpr int kMaxE = 1024;   // experts the LDS m-tile table holds

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

// The same copies written as inline assembly, for waves that also read LDS:
// the compiler does not see them, so it does not wait for every copy in
// flight before each LDS read (it would, as a copy might write what the read
// reads); the caller's own s_waitcnt / s_barrier order the two instead.
// lds is the LDS byte address of lane 0's destination (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// (m0 is set inside the statement; the compiler reserves m0 and uses it for
// nothing else in these kernels, so listing it as clobbered only warns.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_raw(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
// The same copy for data read exactly once (a weight stream): non-temporal,
// so it does not push reusable lines (scales, activations) out of the L2.
__device__ __forceinline__ void dma16_raw_nt(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
// One byte per lane: lane i's byte lands in LDS dword i (zero-extended).
__device__ __forceinline__ void dma1_raw(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ubyte %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

// m-tile schedule for an NTH-thread workgroup: s_mt[e] = index of expert e's
// first m-tile (exclusive scan of ceil(n_e / BM)), s_mt[E] = number of
// m-tiles.  Threads 0..255 own 4 experts each.
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
    const int v = __shfl_up(incl, o, 64);
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

}  // namespace grouped
}  // namespace k3
