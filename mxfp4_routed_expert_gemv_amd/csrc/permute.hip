// Token -> expert counting sort, stable in pair order (pair p = t*k + slot).
//
// Three launches, all integer and exact:
//   chunk_hist    one workgroup per chunk of 256 tokens: per-expert pair
//                 counts of the chunk (LDS atomics; counts are order-free);
//   chunk_scan    one workgroup: per expert, exclusive scan over chunks; then
//                 an exclusive scan over experts gives offsets, and each chunk
//                 base becomes offsets[e] + pairs of e in earlier chunks;
//   chunk_scatter one workgroup per chunk: a token's rank among the chunk's
//                 tokens routed to e is the popcount of the lower token bits
//                 of e's 256-bit token mask, so every pair's sorted position
//                 is fixed without any ordering between threads.
// A token routes to k distinct experts, so "stable in pair order" is "tokens
// in ascending order within each expert".
#include "internal.h"
#include "kern_common.h"

namespace k3 {
namespace {

constexpr int kChunk = kPermChunk;  // tokens per chunk = threads per workgroup

// Slot s of a token takes part in the sort when its id is in [0, E) and no
// earlier slot of the same token holds the same id.
__device__ __forceinline__ bool valid_slot(const int32_t* row, int s, int E) {
  const int e = row[s];
  if (e < 0 || e >= E) return false;
  for (int q = 0; q < s; ++q)
    if (row[q] == e) return false;
  return true;
}

__global__ __launch_bounds__(kChunk) void chunk_hist(const int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ chunk_base,
                                                     int32_t* __restrict__ diag, int64_t T, int E,
                                                     int k) {
  __shared__ int cnt[1024];
  for (int e = threadIdx.x; e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kChunk + threadIdx.x;
  int bad = 0;
  if (t < T) {
    const int32_t* row = idx + t * k;
    for (int s = 0; s < k; ++s) {
      if (valid_slot(row, s, E)) atomicAdd(&cnt[row[s]], 1);
      else ++bad;
    }
  }
  if (bad && diag) atomicAdd(&diag[K3MOE_DIAG_BAD_EXPERT_IDS], bad);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunk)
    chunk_base[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of 1024 threads: thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void chunk_scan(int32_t* __restrict__ chunk_base,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets, int nchunks,
                                                   int E) {
  __shared__ int sums[1024];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      const int v = chunk_base[(size_t)c * E + e];
      chunk_base[(size_t)c * E + e] = run;
      run += v;
    }
    counts[e] = run;
  }
  // Exclusive scan of counts over experts (Hillis-Steele in LDS).
  sums[e] = (e < E) ? run : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = (e >= o) ? sums[e - o] : 0;
    __syncthreads();
    sums[e] += add;
    __syncthreads();
  }
  const int excl = sums[e] - ((e < E) ? run : 0);
  if (e < E) {
    offsets[e] = excl;
    for (int c = 0; c < nchunks; ++c) chunk_base[(size_t)c * E + e] += excl;
  }
  if (e == E - 1) offsets[E] = excl + run;
}

__global__ __launch_bounds__(kChunk) void chunk_scatter(const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ chunk_base,
                                                        const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted_pair,
                                                        int32_t* __restrict__ pair_pos,
                                                        int64_t T, int E, int k) {
  __shared__ unsigned long long mask[1024][kChunk / 64];
  for (int i = threadIdx.x; i < E * (kChunk / 64); i += kChunk) (&mask[0][0])[i] = 0ull;
  __syncthreads();
  const int lt = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * kChunk + lt;
  const int word = lt >> 6;
  const unsigned long long bit = 1ull << (lt & 63);
  if (t < T)
    for (int s = 0; s < k; ++s)
      if (valid_slot(idx + t * k, s, E)) atomicOr(&mask[idx[t * k + s]][word], bit);
  __syncthreads();
  if (t < T)
    for (int s = 0; s < k; ++s) {
      const int e = idx[t * k + s];
      const int64_t p = t * k + s;
      if (valid_slot(idx + t * k, s, E)) {
        int rank = __popcll(mask[e][word] & (bit - 1ull));
        for (int w = 0; w < word; ++w) rank += __popcll(mask[e][w]);
        const int pos = chunk_base[(size_t)blockIdx.x * E + e] + rank;
        sorted_pair[pos] = (int32_t)p;
        pair_pos[p] = pos;
      } else {
        pair_pos[p] = -1;
      }
    }
  // Positions past the last valid pair (only when ids were dropped) get -1.
  const int64_t P = T * k;
  const int valid = offsets[E];
  for (int64_t q = valid + (int64_t)blockIdx.x * kChunk + lt; q < P; q += (int64_t)gridDim.x * kChunk)
    sorted_pair[q] = -1;
}

}  // namespace

hipError_t launch_permute(const k3moe_shape& s, const int32_t* idx, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                          int32_t* diag, const PermuteWs& ws, hipStream_t st) {
  const int nchunks = (int)((s.T + kChunk - 1) / kChunk);
  chunk_hist<<<nchunks, kChunk, 0, st>>>(idx, ws.chunk_base, diag, s.T, s.E, s.k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  chunk_scan<<<1, 1024, 0, st>>>(ws.chunk_base, counts, offsets, nchunks, s.E);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  chunk_scatter<<<nchunks, kChunk, 0, st>>>(idx, ws.chunk_base, offsets, sorted_pair, pair_pos,
                                            s.T, s.E, s.k);
  return hipGetLastError();
}

}  // namespace k3
