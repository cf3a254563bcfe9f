// Token -> expert counting sort, stable in pair order (pair p = t*k + slot).
//
// Every result is integer and exact.  A token's rank among the tokens routed
// to expert e is the popcount of the lower token bits of e's token mask, so
// every pair's sorted position is fixed without any ordering between threads.
// Slot s of a token takes part only when its id is in [0, E) and no earlier
// slot of the token holds the same id; a token then routes to each expert at
// most once, and "stable in pair order" is "tokens ascending within an
// expert".
//
// Small batches (T <= 256, T*k <= 4096): one workgroup does everything in LDS.
// Larger batches, three launches over chunks of CH tokens:
//   chunk_hist    per-chunk, per-expert pair counts (LDS atomics);
//   chunk_scan    per expert, exclusive scan over chunks; exclusive scan over
//                 experts gives offsets; chunk bases become offsets[e] + pairs
//                 of e in earlier chunks;
//   chunk_scatter per chunk, positions = chunk base + rank from the masks.
#include "internal.h"
#include "kern_common.h"

namespace k3 {
namespace {

constexpr int kSmallT = 256, kSmallPairs = 4096;

__device__ __forceinline__ bool valid_slot(const int32_t* row, int s, int E) {
  const int e = row[s];
  if (e < 0 || e >= E) return false;
  for (int q = 0; q < s; ++q)
    if (row[q] == e) return false;
  return true;
}

// Block-wide exclusive scan of one int per thread (blockDim.x == 1024).
__device__ __forceinline__ int block_excl_scan_1024(int v, int* sums, int* total) {
  const int tid = threadIdx.x;
  sums[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = tid >= o ? sums[tid - o] : 0;
    __syncthreads();
    sums[tid] += add;
    __syncthreads();
  }
  const int incl = sums[tid];
  *total = sums[1023];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(1024) void permute_small(const int32_t* __restrict__ idx,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_pair,
                                                      int32_t* __restrict__ pair_pos,
                                                      int32_t* __restrict__ diag, int T, int E,
                                                      int k) {
  __shared__ int ids[kSmallPairs];
  __shared__ unsigned char valid[kSmallPairs];
  __shared__ int cnt[1024];
  __shared__ int sums[1024];
  __shared__ unsigned long long mask[1024][kSmallT / 64];
  const int tid = threadIdx.x;
  const int P = T * k;
  for (int p = tid; p < P; p += 1024) ids[p] = idx[p];
  cnt[tid] = 0;
  for (int i = tid; i < E * (kSmallT / 64); i += 1024) (&mask[0][0])[i] = 0ull;
  __syncthreads();
  int bad = 0;
  for (int p = tid; p < P; p += 1024) {
    const int t = p / k, s = p - t * k;
    const bool ok = valid_slot(ids + t * k, s, E);
    valid[p] = ok;
    if (ok) {
      atomicAdd(&cnt[ids[p]], 1);
      atomicOr(&mask[ids[p]][t >> 6], 1ull << (t & 63));
    } else {
      ++bad;
    }
  }
  if (bad && diag) atomicAdd(&diag[K3MOE_DIAG_BAD_EXPERT_IDS], bad);
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  int total;
  const int excl = block_excl_scan_1024(c, sums, &total);
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = excl;
    cnt[tid] = excl;  // cnt now holds each expert's first position
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  for (int p = tid; p < P; p += 1024) {
    if (valid[p]) {
      const int e = ids[p], t = p / k, w = t >> 6;
      int rank = __popcll(mask[e][w] & ((1ull << (t & 63)) - 1ull));
      for (int q = 0; q < w; ++q) rank += __popcll(mask[e][q]);
      const int pos = cnt[e] + rank;
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
    } else {
      pair_pos[p] = -1;
    }
  }
  for (int q = total + tid; q < P; q += 1024) sorted_pair[q] = -1;
}

// Chunked path.  CH tokens per chunk (one thread per token); the chunk's id
// rows are staged in LDS with coalesced loads.
template <int CH>
__global__ __launch_bounds__(256) void chunk_hist(const int32_t* __restrict__ idx,
                                                  int32_t* __restrict__ chunk_base,
                                                  int32_t* __restrict__ diag, int64_t T, int E,
                                                  int k) {
  __shared__ int rows[kSmallPairs];  // CH * k <= 4096
  __shared__ int cnt[1024];
  const int64_t t0 = (int64_t)blockIdx.x * CH;
  const int nt = (int)((T - t0) < CH ? (T - t0) : CH);
  for (int i = threadIdx.x; i < nt * k; i += 256) rows[i] = idx[t0 * k + i];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  int bad = 0;
  if ((int)threadIdx.x < nt)
    for (int s = 0; s < k; ++s) {
      if (valid_slot(rows + threadIdx.x * k, s, E)) atomicAdd(&cnt[rows[threadIdx.x * k + s]], 1);
      else ++bad;
    }
  if (bad && diag) atomicAdd(&diag[K3MOE_DIAG_BAD_EXPERT_IDS], bad);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_base[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of 1024 threads: thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void chunk_scan(int32_t* __restrict__ chunk_base,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets, int nchunks,
                                                   int E) {
  __shared__ int sums[1024];
  constexpr int B = 16;
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += B) {
      int v[B];
#pragma unroll
      for (int u = 0; u < B; ++u) v[u] = (c0 + u < nchunks) ? chunk_base[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (c0 + u < nchunks) {
          chunk_base[(size_t)(c0 + u) * E + e] = run;
          run += v[u];
        }
    }
  }
  int total;
  const int excl = block_excl_scan_1024(e < E ? run : 0, sums, &total);
  if (e < E) {
    counts[e] = run;
    offsets[e] = excl;
    for (int c = 0; c < nchunks; ++c) chunk_base[(size_t)c * E + e] += excl;
  }
  if (e == 0) offsets[E] = total;
}

template <int CH>
__global__ __launch_bounds__(256) void chunk_scatter(const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ chunk_base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted_pair,
                                                     int32_t* __restrict__ pair_pos, int64_t T,
                                                     int E, int k) {
  constexpr int NW = CH / 64;
  __shared__ int rows[kSmallPairs];  // CH * k <= 4096
  __shared__ int base[1024];
  __shared__ unsigned long long mask[1024][NW];
  const int64_t t0 = (int64_t)blockIdx.x * CH;
  const int nt = (int)((T - t0) < CH ? (T - t0) : CH);
  for (int i = threadIdx.x; i < nt * k; i += 256) rows[i] = idx[t0 * k + i];
  for (int e = threadIdx.x; e < E; e += 256) base[e] = chunk_base[(size_t)blockIdx.x * E + e];
  for (int i = threadIdx.x; i < E * NW; i += 256) (&mask[0][0])[i] = 0ull;
  __syncthreads();
  const int lt = threadIdx.x;
  const int word = lt >> 6;
  const unsigned long long bit = 1ull << (lt & 63);
  if (lt < nt)
    for (int s = 0; s < k; ++s)
      if (valid_slot(rows + lt * k, s, E)) atomicOr(&mask[rows[lt * k + s]][word], bit);
  __syncthreads();
  if (lt < nt)
    for (int s = 0; s < k; ++s) {
      const int64_t p = (t0 + lt) * k + s;
      if (valid_slot(rows + lt * k, s, E)) {
        const int e = rows[lt * k + s];
        int rank = __popcll(mask[e][word] & (bit - 1ull));
        for (int w = 0; w < word; ++w) rank += __popcll(mask[e][w]);
        const int pos = base[e] + rank;
        sorted_pair[pos] = (int32_t)p;
        pair_pos[p] = pos;
      } else {
        pair_pos[p] = -1;
      }
    }
  // Positions past the last valid pair (only when ids were dropped) get -1.
  const int64_t P = T * k;
  const int valid = offsets[E];
  for (int64_t q = valid + (int64_t)blockIdx.x * 256 + lt; q < P; q += (int64_t)gridDim.x * 256)
    sorted_pair[q] = -1;
}

template <int CH>
hipError_t chunked(const k3moe_shape& s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_pair, int32_t* pair_pos, int32_t* diag, const PermuteWs& ws,
                   hipStream_t st) {
  const int nchunks = (int)((s.T + CH - 1) / CH);
  chunk_hist<CH><<<nchunks, 256, 0, st>>>(idx, ws.chunk_base, diag, s.T, s.E, s.k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  chunk_scan<<<1, 1024, 0, st>>>(ws.chunk_base, counts, offsets, nchunks, s.E);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  chunk_scatter<CH><<<nchunks, 256, 0, st>>>(idx, ws.chunk_base, offsets, sorted_pair, pair_pos,
                                             s.T, s.E, s.k);
  return hipGetLastError();
}

}  // namespace

int permute_chunk_tokens(int k) { return k <= 16 ? 256 : 64; }

hipError_t launch_permute(const k3moe_shape& s, const int32_t* idx, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                          int32_t* diag, const PermuteWs& ws, hipStream_t st) {
  if (s.T <= kSmallT && s.T * s.k <= kSmallPairs) {
    permute_small<<<1, 1024, 0, st>>>(idx, counts, offsets, sorted_pair, pair_pos, diag,
                                      (int)s.T, s.E, s.k);
    return hipGetLastError();
  }
  if (s.k <= 16) return chunked<256>(s, idx, counts, offsets, sorted_pair, pair_pos, diag, ws, st);
  return chunked<64>(s, idx, counts, offsets, sorted_pair, pair_pos, diag, ws, st);
}

}  // namespace k3
