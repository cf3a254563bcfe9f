// Router logits, top-k and softmax weights.
//
// Routing follows the pages' MoE layer (16 of 896 experts per token —
// kimi-k3-in-c review, "at a glance" table) with softmax weights renormalised
// over the chosen experts.  The chosen SET must equal what an exact fp64
// evaluation of the logits in ascending-i order picks, bit for bit, so:
//   1. the logits are computed in fp64 (bf16 x bf16 and fp32 x bf16 products
//      are exact in fp64) together with a rigorous bound on their distance to
//      the sequential fp64 value;
//   2. the top-k kernel selects by (logit desc, id asc) and checks that every
//      chosen expert beats every other expert by more than the two bounds;
//      when that fails it re-evaluates the undecided experts sequentially in
//      fp64, ascending i — the exact same operations as the oracle, hence the
//      same bits — and selects among them.
// The pages' own K3 router (kimi-k3-in-c review page, "KDA/MLA/MoE" table)
// is the other mode: selection by sigmoid(l) + bias, where the bias bends
// only the selection, and weights from the unbiased sigmoid(l), raw or
// renormalised over the chosen.  Its selection key carries the logit's bound
// through the sigmoid (slope at most 1/4) plus the fp64 evaluation of the
// sigmoid and the bias addition on either side; after a recheck the logits
// are the oracle's bits and only the sigmoid evaluation can still separate
// the two sides, which is counted when it could decide the set.
#include "internal.h"
#include "kern_common.h"
#include "decode_t1.h"

#include <limits.h>

namespace k3 {
namespace {

// One wave per expert row; loops over tokens.  Per lane: 8-element chunks
// c = lane, lane+64, ..., up to 16 per pass, all loads of a pass issued before
// the arithmetic; fp64 sequential partial over the lane's chunks, then a
// fixed butterfly over the wave.
template <bool XF32>
__global__ __launch_bounds__(256) void router_gemv_f64(const void* __restrict__ x,
                                                       const uint16_t* __restrict__ wr,
                                                       double* __restrict__ logits,
                                                       float* __restrict__ lbound, int T, int d,
                                                       int E) {
  constexpr int U = 16;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int nc = d / 8;
  const uint16_t* wrow = wr + (size_t)e * d;
  for (int t = 0; t < T; ++t) {
    // Four independent fp64 partial sums per lane (chunk slot u mod 4), so
    // the multiply-add chains overlap; any fixed order is covered by the bound.
    double acc4[4] = {0.0, 0.0, 0.0, 0.0};
    float aabs = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += kWave * U) {
      uint4 wv[U], xa[U], xb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = min(c0 + lane + kWave * u, nc - 1);
        wv[u] = ldg16(wrow + (size_t)c * 8);
        if (XF32) {
          const float* xr = static_cast<const float*>(x) + (size_t)t * d + (size_t)c * 8;
          xa[u] = ldg16(xr);
          xb[u] = ldg16(xr + 4);
        } else {
          xa[u] = ldg16(static_cast<const uint16_t*>(x) + (size_t)t * d + (size_t)c * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = c0 + lane + kWave * u < nc;
        const uint32_t ww[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
        float xf[8];
        if (XF32) {
          xf[0] = __uint_as_float(xa[u].x); xf[1] = __uint_as_float(xa[u].y);
          xf[2] = __uint_as_float(xa[u].z); xf[3] = __uint_as_float(xa[u].w);
          xf[4] = __uint_as_float(xb[u].x); xf[5] = __uint_as_float(xb[u].y);
          xf[6] = __uint_as_float(xb[u].z); xf[7] = __uint_as_float(xb[u].w);
        } else {
          const uint32_t xw[4] = {xa[u].x, xa[u].y, xa[u].z, xa[u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) { xf[2 * q] = bf16_lo(xw[q]); xf[2 * q + 1] = bf16_hi(xw[q]); }
        }
        double a = acc4[u & 3];
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float w0 = bf16_lo(ww[q]), w1 = bf16_hi(ww[q]);
          a = __builtin_fma((double)xf[2 * q], (double)w0, a);      // exact product
          a = __builtin_fma((double)xf[2 * q + 1], (double)w1, a);
          s = s + fabsf(xf[2 * q] * w0) + fabsf(xf[2 * q + 1] * w1);
        }
        acc4[u & 3] = ok ? a : acc4[u & 3];
        aabs = ok ? aabs + s : aabs;
      }
    }
    double acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    acc = wave_sum(acc);
    aabs = wave_sum(aabs);
    if (lane == 0) {
      // |acc - exact| <= (d/64 + 8) u S (per-lane chains, 2 adds, 6 butterfly
      // levels) and |oracle - exact| <= d u S with u = 2^-53 and
      // S = sum|p| <= 1.01 aabs (aabs is an fp32 sum of rounded |products|,
      // d <= 16384).
      const double bnd = (2.0 * d + 64.0) * 0x1p-53 * (double)aabs * 1.02;
      logits[(size_t)t * E + e] = acc;
      lbound[(size_t)t * E + e] = (float)bnd;
    }
  }
}

// Large batches: the same fp64 logits on the fp64 matrix cores
// (MFMA 16x16x4).  A workgroup computes 16 TA tokens x 16 EB experts (TA,
// EB in {1, 2}: smaller tiles at small batches, so that enough workgroups
// share the fp64 matrix work); wave w covers the contraction slice
// [w d/4, (w+1) d/4), and the four partial sums are added in wave order.
// Each logit's arithmetic (its MFMA chain over the wave's slice, the
// partials' order, the norms of its two rows) does not depend on the tile
// shape, so neither do its bits.  Lane (i = lane % 16, c = lane / 16) holds
// elements c*8 .. c*8+7 of each 32-element group of its token row (A) and
// expert row (B); MFMA step q (0..7) takes element c*8 + q from every lane,
// so each product pairs x and w of the same element.  The bound uses
// sum|x_i w_i| <= |x| |w| (Cauchy-Schwarz), with the squared norms summed
// in fp64 (bf16 squares are exact) along the same pass.
typedef __attribute__((ext_vector_type(4))) double f64x4_t;

template <int TA, int EB>
__global__ __launch_bounds__(256) void router_mfma_f64(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ wr,
                                                       double* __restrict__ logits,
                                                       float* __restrict__ lbound, int T, int d,
                                                       int E) {
  constexpr int BT = 16 * TA, BE = 16 * EB;
  __shared__ double part[4][BT][BE + 1];
  __shared__ double nrm[4][2][32];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 15, lc = lane >> 4;
  const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE;
  const int kq = d / 4;                 // contraction slice per wave (multiple of 64)
  const int kbeg = wv * kq;
  const uint16_t* ar[TA];
  const uint16_t* br[EB];
#pragma unroll
  for (int f = 0; f < TA; ++f) ar[f] = x + (size_t)min(t0 + f * 16 + li, T - 1) * d + kbeg + lc * 8;
#pragma unroll
  for (int f = 0; f < EB; ++f) br[f] = wr + (size_t)min(e0 + f * 16 + li, E - 1) * d + kbeg + lc * 8;
  f64x4_t acc[TA][EB];
#pragma unroll
  for (int a = 0; a < TA; ++a)
#pragma unroll
    for (int b = 0; b < EB; ++b) acc[a][b] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  double sa[TA], sb[EB];
#pragma unroll
  for (int f = 0; f < TA; ++f) sa[f] = 0.0;
#pragma unroll
  for (int f = 0; f < EB; ++f) sb[f] = 0.0;

  // register ring of PD groups: group gi's loads are issued PD groups ahead
  // (small tiles, few waves per SIMD: 4; the 32 x 32 tile: 1, which keeps
  // its registers to 4 waves per SIMD)
  constexpr int PD = TA * EB == 4 ? 1 : 4;
  const int ng = kq / 32;
  uint4 av[PD][TA], bv[PD][EB];
  auto load = [&](int g, int slot) {
#pragma unroll
    for (int f = 0; f < TA; ++f) av[slot][f] = ldg16(ar[f] + g * 32);
#pragma unroll
    for (int f = 0; f < EB; ++f) bv[slot][f] = ldg16(br[f] + g * 32);
  };
#pragma unroll
  for (int q = 0; q < PD; ++q) load(min(q, ng - 1), q);
  // bf16 pair -> two fp64 values and their squares added to a norm, in order
  auto widen = [](const uint4& v, double (&o)[8], double& nsq) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      o[2 * u] = (double)bf16_lo(w[u]);
      o[2 * u + 1] = (double)bf16_hi(w[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) nsq = __builtin_fma(o[u], o[u], nsq);
  };
#pragma unroll 1
  for (int g0 = 0; g0 < ng; g0 += PD) {
#pragma unroll
    for (int q = 0; q < PD; ++q) {
      if (g0 + q < ng) {
        double xa[TA][8], wb[EB][8];
#pragma unroll
        for (int f = 0; f < TA; ++f) widen(av[q][f], xa[f], sa[f]);
#pragma unroll
        for (int f = 0; f < EB; ++f) widen(bv[q][f], wb[f], sb[f]);
        load(min(g0 + q + PD, ng - 1), q);   // past the end: a repeat, unused
        __builtin_amdgcn_sched_barrier(0);   // keep the loads PD groups ahead
#pragma unroll
        for (int qs = 0; qs < 8; ++qs)
#pragma unroll
          for (int a = 0; a < TA; ++a)
#pragma unroll
            for (int b = 0; b < EB; ++b)
              acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(xa[a][qs], wb[b][qs], acc[a][b], 0, 0,
                                                               0);
      }
    }
  }
  // Output element r of fragment (a, b): token a*16 + lc + 4 r, expert b*16 + li.
#pragma unroll
  for (int a = 0; a < TA; ++a)
#pragma unroll
    for (int b = 0; b < EB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wv][a * 16 + lc + 4 * r][b * 16 + li] = acc[a][b][r];
  // squared norms: the four lanes c of a row, in lane order
  auto lane_sum = [&](double v) {
    v += __shfl_xor(v, 16, kWave);
    return v + __shfl_xor(v, 32, kWave);
  };
#pragma unroll
  for (int f = 0; f < TA; ++f) {
    const double va = lane_sum(sa[f]);
    if (lc == 0) nrm[wv][0][f * 16 + li] = va;
  }
#pragma unroll
  for (int f = 0; f < EB; ++f) {
    const double vb = lane_sum(sb[f]);
    if (lc == 0) nrm[wv][1][f * 16 + li] = vb;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < (BT * BE + 255) / 256; ++u) {
    const int o = tid + 256 * u;
    const int tt = o / BE, ee = o % BE;
    const int t = t0 + tt, e = e0 + ee;
    if (tt < BT && t < T && e < E) {
      const double l = ((part[0][tt][ee] + part[1][tt][ee]) + part[2][tt][ee]) + part[3][tt][ee];
      const double nx = ((nrm[0][0][tt] + nrm[1][0][tt]) + nrm[2][0][tt]) + nrm[3][0][tt];
      const double nw = ((nrm[0][1][ee] + nrm[1][1][ee]) + nrm[2][1][ee]) + nrm[3][1][ee];
      // |l - exact| <= (d + 8) 2^-52 S for any internal order of the matrix
      // core (each step rounds once to fp64), |oracle - exact| <= d 2^-53 S,
      // S <= sqrt(nx nw) (1 + 2^-40) with the fp64 squared norms.
      const double bnd = (3.0 * d + 128.0) * 0x1p-53 * sqrt(nx * nw) * 1.02;
      logits[(size_t)t * E + e] = l;
      lbound[(size_t)t * E + e] = (float)bnd;
    }
  }
}

constexpr int kMaxJ = 16;  // E <= 1024 = 16 per lane

__device__ __forceinline__ bool better(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Exact sequential fp64 logit: the oracle's operation sequence (products are
// exact in fp64, so multiply-add fusion cannot change a bit).
template <bool XF32>
__device__ double exact_logit(const void* x, const uint16_t* wr, int t, int e, int d) {
  const uint16_t* wrow = wr + (size_t)e * d;
  double acc = 0.0;
  if (XF32) {
    const float* xr = static_cast<const float*>(x) + (size_t)t * d;
    for (int i = 0; i < d; ++i)
      acc = __builtin_fma((double)xr[i], (double)__uint_as_float((uint32_t)wrow[i] << 16), acc);
  } else {
    const uint16_t* xr = static_cast<const uint16_t*>(x) + (size_t)t * d;
    for (int i = 0; i < d; ++i)
      acc = __builtin_fma((double)__uint_as_float((uint32_t)xr[i] << 16),
                          (double)__uint_as_float((uint32_t)wrow[i] << 16), acc);
  }
  return acc;
}

// Lane-local best not-yet-taken entry by (key desc, j asc); jb = -1 if none.
__device__ __forceinline__ void lane_best(const uint64_t (&key)[kMaxJ], uint32_t taken,
                                          uint64_t& kb, int& jb) {
  kb = 0;
  jb = -1;
#pragma unroll
  for (int j = 0; j < kMaxJ; ++j)
    if (!((taken >> j) & 1u) && key[j] > kb) { kb = key[j]; jb = j; }
}

// The k-th largest (1 <= k <= popcount(active)) of the values v of the lanes
// in the wave-uniform mask active, counted with multiplicity: a descent over
// the bits from the top, keeping the lanes that agree with the answer on the
// bits above (set) and the answer's rank among them (need); it ends as soon
// as one lane is left.
__device__ __forceinline__ uint64_t kth_largest_u64(uint64_t v, uint64_t active, int k) {
  uint64_t set = active;
  int need = k;
  for (int b = 63; b >= 0 && __popcll(set) > 1; --b) {
    const uint64_t ones = __ballot((v >> b) & 1u) & set;
    const int c = __popcll(ones);
    if (c >= need) {
      set = ones;
    } else {
      need -= c;
      set &= ~ones;
    }
  }
  const int l = __ffsll((long long)set) - 1;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// LDS of one token's selection (one wave).
struct TopkLds {
  double candL[1024];
  int candId[1024];
  int candTaken[1024];
  int chosen[1024];
};

// Orders the wave's LDS accesses (the selection runs in a single wave, so no
// workgroup barrier is needed, nor allowed when it shares a workgroup).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Token t's selection by one wave.  Lane l holds experts l + 64 j as
// order-preserving 64-bit keys; each of k rounds takes the wave maximum with
// DPP, ties between lanes going to the lower expert id.
// fp64 sigmoid score, 1 / (1 + e^-l); the same formula as the oracle's.
__device__ __forceinline__ double sigmoid_score(double l) { return 1.0 / (1.0 + exp(-l)); }
// Relative bound on the difference between the two sides' fp64 selection
// scores for the same logit: each side's exp within 1 ulp, the sigmoid's add
// and divide and the bias add within half an ulp each, with margin.
constexpr double kScoreEps = 8.0 * 0x1p-53;

struct RouterMode {
  int mode = K3MOE_ROUTER_SOFTMAX;
  const float* bias = nullptr;   // [E] fp32 or nullptr (sigmoid modes only)
};

template <bool XF32>
__device__ void topk_token(int t, int lane, TopkLds& sm, const double* __restrict__ logits,
                           const float* __restrict__ lbound, const void* __restrict__ x,
                           const uint16_t* __restrict__ wr, int32_t* __restrict__ idx_out,
                           float* __restrict__ w_out, float* __restrict__ logits_out,
                           int32_t* __restrict__ diag, int d, int E, int k, const PermOut& perm,
                           const RouterMode rm) {
  const bool sig = rm.mode != K3MOE_ROUTER_SOFTMAX;
  double* candL = sm.candL;
  int* candId = sm.candId;
  int* candTaken = sm.candTaken;
  int* chosen = sm.chosen;
  const int nj = (E + kWave - 1) / kWave;
  const double* lrow = logits + (size_t)t * E;
  const float* brow = lbound + (size_t)t * E;

  uint64_t key[kMaxJ];
  float b[kMaxJ];
  int nonfin = 0;
  // Every load is issued (clamped index) before any is used.
  double lv[kMaxJ];
  float bias[kMaxJ];
#pragma unroll
  for (int j = 0; j < kMaxJ; ++j) {
    const int e = min(lane + kWave * j, E - 1);
    lv[j] = lrow[e];
    b[j] = brow[e];
    bias[j] = rm.bias ? rm.bias[e] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kMaxJ; ++j) {
    const int e = lane + kWave * j;
    const bool ok = j < nj && e < E;
    if (ok && !isfinite(lv[j])) ++nonfin;
    if (sig) {
      // selection score and its bound: the logit's bound through the slope
      // of the sigmoid (at most 1/4), plus the two sides' score evaluation
      const double sc = sigmoid_score(lv[j]) + (double)bias[j];
      key[j] = ok ? order_key(isnan(sc) ? -INFINITY : sc) : 0;
      b[j] = (float)((0.25 * (double)b[j] + kScoreEps * (1.0 + fabs((double)bias[j]))) *
                     (1.0 + 0x1p-20));
    } else {
      key[j] = ok ? order_key(isnan(lv[j]) ? -INFINITY : lv[j]) : 0;
    }
    // masked with bit operations so the loads above stay unconditional
    b[j] = __uint_as_float(__float_as_uint(b[j]) & (0u - (uint32_t)ok));
  }
  if (logits_out)
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j)
      if (j < nj && lane + kWave * j < E) logits_out[(size_t)t * E + lane + kWave * j] = (float)lv[j];
  nonfin = wave_sum(nonfin);
  if (lane == 0 && nonfin && diag) atomicAdd(&diag[K3MOE_DIAG_NONFINITE_LOGITS], nonfin);

  uint32_t taken = 0;
  uint64_t kb;
  int jb;
  int k_rounds = k;
  lane_best(key, taken, kb, jb);
  // Sample select: the k-th of the 64 lane maxima bounds the k-th key from
  // below (the k lanes with the largest maxima hold k keys at least as
  // large), so the chosen ones are among the keys at or above it, k of them
  // at least and usually a few more.  When at most 64, they are compacted one
  // per lane in ascending id, the k-th largest of them is found exactly, and
  // the chosen ones are those above it plus, among those equal to it, the
  // lowest ids (the order of k rounds of the wave maximum with the lowest id
  // on ties).
  {
    const uint64_t thr = kth_largest_u64(kb, __ballot(kb != 0), k);
    uint32_t cm = 0;
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j)
      if (key[j] != 0 && key[j] >= thr) cm |= 1u << j;
    const int nc = wave_sum((int)__popc(cm));
    if (nc <= kWave) {
      // compaction: j-major, then lane, which is ascending id
      uint64_t ck = 0;
      int ci = -1, n = 0;
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) {
        const bool mine = (cm >> j) & 1u;
        const unsigned long long bal = __ballot(mine);
        const int pos = n + __popcll(bal & ((1ull << lane) - 1ull));
        if (mine) {
          candL[pos] = __longlong_as_double((long long)key[j]);
          candId[pos] = lane + kWave * j;
        }
        n += __popcll(bal);
      }
      for (int q = lane; q < 1024; q += kWave) chosen[q] = 0;
      wave_sync();
      if (lane < nc) {
        ck = (uint64_t)__double_as_longlong(candL[lane]);
        ci = candId[lane];
      }
      const uint64_t live = nc >= kWave ? ~0ull : (1ull << nc) - 1ull;
      const uint64_t tk = kth_largest_u64(ck, live, k);
      const uint64_t above = __ballot(lane < nc && ck > tk);
      const uint64_t tie = __ballot(lane < nc && ck == tk);
      const int room = k - __popcll(above);   // tied ones to take, lowest ids first
      const bool pick = ((above >> lane) & 1ull) ||
                        (((tie >> lane) & 1ull) && __popcll(tie & ((1ull << lane) - 1ull)) < room);
      if (pick) chosen[ci] = 1;
      wave_sync();
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j)
        if (j < nj && lane + kWave * j < E && chosen[lane + kWave * j]) taken |= 1u << j;
      wave_sync();
      k_rounds = 0;
    }
  }
  // Otherwise (more than 64 keys reach the bound: ties or near ties), k
  // rounds of the wave maximum.
  for (int r = 0; r < k_rounds; ++r) {
    const uint64_t m = wave_max_u64(kb);
    const unsigned long long tied = __ballot(jb >= 0 && kb == m);
    int wl, wj;
    if (__popcll(tied) == 1) {
      wl = __ffsll((long long)tied) - 1;
      wj = __builtin_amdgcn_readlane(jb, wl);
    } else {  // equal logits in several lanes: the lowest expert id wins
      int id = (jb >= 0 && kb == m) ? lane + kWave * jb : INT_MAX;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) id = min(id, __shfl_xor(id, o, kWave));
      wl = id & 63;
      wj = id >> 6;
    }
    if (lane == wl) {
      taken |= 1u << wj;
      lane_best(key, taken, kb, jb);
    }
  }

  // Certificate: every chosen expert's lower bound beats every other
  // expert's upper bound.  Otherwise the undecided ones are re-evaluated.
  double lo = INFINITY;
#pragma unroll
  for (int j = 0; j < kMaxJ; ++j)
    if ((taken >> j) & 1u) lo = fmin(lo, key_value(key[j]) - (double)b[j]);
  const double tau = wave_min(lo);
  uint32_t cand = 0;
#pragma unroll
  for (int j = 0; j < kMaxJ; ++j) {
    const int e = lane + kWave * j;
    if (j < nj && e < E && !((taken >> j) & 1u) && key_value(key[j]) + (double)b[j] >= tau)
      cand |= 1u << j;
  }
  const int nout = wave_sum((int)__popc(cand));
  if (nout > 0) {
    // Undecided: the chosen ones plus the challengers, evaluated exactly.
    const uint32_t all = cand | taken;
    int n = 0;
    for (int j = 0; j < nj; ++j) {
      const bool mine = (all >> j) & 1u;
      const unsigned long long bal = __ballot(mine);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (mine) candId[n + before] = lane + kWave * j;
      n += __popcll(bal);
    }
    for (int q = lane; q < 1024; q += kWave) chosen[q] = 0;
    wave_sync();
    for (int q = lane; q < n; q += kWave) {
      const double l = exact_logit<XF32>(x, wr, t, candId[q], d);
      candL[q] = sig ? sigmoid_score(l) + (double)(rm.bias ? rm.bias[candId[q]] : 0.0f) : l;
      candTaken[q] = 0;
    }
    wave_sync();
    for (int r = 0; r < k; ++r) {
      double bv = -INFINITY;
      int bi = INT_MAX, bq = -1;
      for (int q = lane; q < n; q += kWave)
        if (!candTaken[q] && better(candL[q], candId[q], bv, bi)) { bv = candL[q]; bi = candId[q]; bq = q; }
      int owner = bq;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const double ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        const int oq = __shfl_xor(owner, o, kWave);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; owner = oq; }
      }
      if (lane == 0) { candTaken[owner] = 1; chosen[bi] = 1; }
      wave_sync();
    }
    taken = 0;
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) {
      const int e = lane + kWave * j;
      if (j < nj && e < E && chosen[e]) taken |= 1u << j;
    }
    if (lane == 0 && diag) atomicAdd(&diag[K3MOE_DIAG_RECHECKED_TOKENS], 1);
    if (sig) {
      // with the logits exact, two different scores closer than the sides'
      // evaluation bound could still order differently on the two sides
      double lo_in = INFINITY, hi_out = -INFINITY, mag = 0.0;
      for (int q = lane; q < n; q += kWave) {
        mag = fmax(mag, fabs(candL[q]));
        if (chosen[candId[q]]) lo_in = fmin(lo_in, candL[q]);
        else hi_out = fmax(hi_out, candL[q]);
      }
      lo_in = wave_min(lo_in);
      hi_out = -wave_min(-hi_out);
      mag = -wave_min(-mag);
      const double gap = lo_in - hi_out;
      if (lane == 0 && diag && gap > 0.0 && gap <= 2.0 * kScoreEps * (2.0 + mag))
        atomicAdd(&diag[K3MOE_DIAG_SCORE_NEAR_TIES], 1);
    }
  }

  // Softmax over the chosen logits (or their sigmoid scores); outputs in
  // ascending expert id.  The chosen (id, logit) pairs are first compacted in
  // ascending id into chosen[] / candL[] (slot p = rank among the chosen), so
  // each slot's exponential is evaluated once, by lane p.
  uint64_t kmax = 0;
#pragma unroll
  for (int j = 0; j < kMaxJ; ++j)
    if (((taken >> j) & 1u) && key[j] > kmax) kmax = key[j];
  const double m = key_value(wave_max_u64(kmax));
  int base = 0;
#pragma unroll
  for (int j = 0; j < kMaxJ; ++j) {
    const bool mine = (taken >> j) & 1u;   // never set for j >= nj
    const unsigned long long bal = __ballot(mine);
    const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
    if (mine) {
      chosen[pos] = lane + kWave * j;
      // (sigmoid routing: the logit itself, read again rather than kept in
      // registers through the selection)
      candL[pos] = sig ? lrow[lane + kWave * j] : key_value(key[j]);
    }
    // one token: expert e = lane + 64 j has count 0/1 and offset = the
    // number of chosen experts below it (ids run j-major, then lane)
    const int e = lane + kWave * j;
    if (perm.counts && j < nj && e < E) {
      perm.counts[e] = mine ? 1 : 0;
      perm.offsets[e] = pos;
    }
    base += __popcll(bal);
  }
  if (perm.counts) {
    if (lane == 0) perm.offsets[E] = base;
    if (lane < k) {
      perm.sorted_pair[lane] = lane;
      perm.pair_pos[lane] = lane;
    }
  }
  wave_sync();
  // k <= 64: one slot per lane; z summed by the fixed butterfly
  const double ep = lane < k ? (sig ? sigmoid_score(candL[lane]) : exp(candL[lane] - m)) : 0.0;
  const double z = wave_sum(ep);
  if (lane < k) {
    idx_out[(size_t)t * k + lane] = chosen[lane];
    w_out[(size_t)t * k + lane] = (float)(rm.mode == K3MOE_ROUTER_SIGMOID ? ep : ep / z);
  }
}

template <bool XF32>
__global__ __launch_bounds__(64) void topk_softmax(const double* __restrict__ logits,
                                                   const float* __restrict__ lbound,
                                                   const void* __restrict__ x,
                                                   const uint16_t* __restrict__ wr,
                                                   int32_t* __restrict__ idx_out,
                                                   float* __restrict__ w_out,
                                                   float* __restrict__ logits_out,
                                                   int32_t* __restrict__ diag, int T, int d, int E,
                                                   int k, PermOut perm, RouterMode rm) {
  __shared__ TopkLds sm;
  if ((int)blockIdx.x >= T) return;
  topk_token<XF32>(blockIdx.x, threadIdx.x, sm, logits, lbound, x, wr, idx_out, w_out,
                   logits_out, diag, d, E, k, perm, rm);
}

// ------------------------------------------------- large batches: bf16 logits
// From kBf16RouterMinT tokens the fp64 logits above cost the layer more than
// this route does (52.6 GFLOP of fp64 matrix work at 4096 tokens: 0.97 against
// 0.63 ms for the whole route; below 512 tokens the fp64 route is the faster
// one).  The ids are the oracle's on both sides of the threshold; the weights
// come from fp64 logits of two arrangements (the fp64 matrix cores below it,
// the GEMV arrangement above), which can differ in the last bits.  The
// selection only needs
// fp64 values for the experts that can still reach the top k, so:
//   1. every logit on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32
//      accumulation), written as fp32: the shared experts' LDS-ring GEMM
//      (shared_gemm.hip) with x against the router rows;
//   2. route_refine (one wave per token, four tokens per workgroup): each fp32 logit gets a bound on
//      its distance to the oracle's value; the experts whose upper bound
//      reaches the k-th largest lower bound (k + a few) are recomputed in
//      fp64 with the GEMV router's arithmetic and bound, the others keep the
//      fp32 value and its bound;
//   3. topk_softmax as for the fp64 logits: its certificate and exact recheck
//      make the ids the oracle's whatever the bounds' widths, and the chosen
//      experts (all refined) give the weights.
// The fp32 bound: products of bf16 values are exact in fp32, and every
// addition of the matrix core's fp32 accumulation is taken to round once
// (to nearest or directed, relative error at most 2^-23), in any internal
// order: along any path of the sum a product meets at most d + d/32 + 8
// additions, so |l - exact| <= (d + d/32 + 8) 2^-23 S, with
// S = sum |x_i w_i| <= |x| |w| (Cauchy-Schwarz); the oracle's own distance to
// the exact sum, d 2^-53 S, is added, and d 2^-125 covers products that
// underflow fp32.

// |w_e| for every expert row (fp64 sum of exact bf16 squares, rounded up to
// fp32 with margin); one wave per row.
__global__ __launch_bounds__(256) void router_wnorm(const uint16_t* __restrict__ wr,
                                                    float* __restrict__ wnorm, int d, int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const uint16_t* row = wr + (size_t)e * d;
  double s = 0.0;
  for (int c = lane; c < d / 8; c += kWave) {
    const uint4 v = ldg16(row + (size_t)c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double a = (double)bf16_lo(w[q]), b = (double)bf16_hi(w[q]);
      s = __builtin_fma(a, a, s);
      s = __builtin_fma(b, b, s);
    }
  }
  s = wave_sum(s);
  if (lane == 0) wnorm[e] = (float)(sqrt(s) * (1.0 + 0x1p-20));
}

constexpr int kBf16RouterMinT = 512;

// A token's candidates are re-evaluated two rows at a time: fp64 products
// and sums in the GEMV router's arrangement.  (lbound holds the fp32 logits on
// entry; the token's workgroup reads them before it writes the row.)
__device__ __forceinline__ void refine_dot(const uint16_t* __restrict__ xr,
                                           const uint16_t* __restrict__ w0,
                                           const uint16_t* __restrict__ w1, int d, int lane,
                                           double (&acc)[2], float (&aabs)[2]) {
  constexpr int U = 8;
  const int nc = d / 8;
  double a4[2][4] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  float sa[2] = {0.0f, 0.0f};
  for (int c0 = 0; c0 < nc; c0 += kWave * U) {
    uint4 xv[U], wv0[U], wv1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + lane + kWave * u, nc - 1);
      xv[u] = ldg16(xr + (size_t)c * 8);
      wv0[u] = ldg16(w0 + (size_t)c * 8);
      wv1[u] = ldg16(w1 + (size_t)c * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = c0 + lane + kWave * u < nc;
      const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
      const uint32_t w[2][4] = {{wv0[u].x, wv0[u].y, wv0[u].z, wv0[u].w},
                                {wv1[u].x, wv1[u].y, wv1[u].z, wv1[u].w}};
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        double a = a4[p][u & 3];
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x0 = bf16_lo(xw[q]), x1 = bf16_hi(xw[q]);
          const float v0 = bf16_lo(w[p][q]), v1 = bf16_hi(w[p][q]);
          a = __builtin_fma((double)x0, (double)v0, a);      // exact products
          a = __builtin_fma((double)x1, (double)v1, a);
          s = s + fabsf(x0 * v0) + fabsf(x1 * v1);
        }
        a4[p][u & 3] = ok ? a : a4[p][u & 3];
        sa[p] = ok ? sa[p] + s : sa[p];
      }
    }
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    acc[p] = wave_sum((a4[p][0] + a4[p][1]) + (a4[p][2] + a4[p][3]));
    aabs[p] = wave_sum(sa[p]);
  }
}

// One workgroup of NW waves per NW tokens.  Wave w, for token NW b + w:
// bounds, the k-th largest lower end, the candidate list (LDS), and the
// non-candidates' values and bounds; then the waves share the fp64
// re-evaluation of all the workgroup's candidate pairs.
template <int NW>
__global__ __launch_bounds__(64 * NW) void route_refine(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ wr,
                                                        const float* __restrict__ wnorm,
                                                        double* __restrict__ logits,
                                                        float* __restrict__ lbound, int T, int d,
                                                        int E, int k, RouterMode rm) {
  __shared__ int s_cand_all[NW][1024];
  __shared__ int s_n_all[NW];
  __shared__ uint64_t s_key_all[NW][kWave];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * NW + wv;
  int* s_cand = s_cand_all[wv];
  uint64_t* s_key = s_key_all[wv];
  const uint16_t* xr = x + (size_t)t * d;
  if (lane == 0) s_n_all[wv] = 0;
  if (t < T) {
    const bool sig = rm.mode != K3MOE_ROUTER_SOFTMAX;
    const int nj = (E + kWave - 1) / kWave;
    // |x_t|, fp64 sum of exact squares
    double nx = 0.0;
    for (int c = lane; c < d / 8; c += kWave) {
      const uint4 v = ldg16(xr + (size_t)c * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double a = (double)bf16_lo(w[q]), b = (double)bf16_hi(w[q]);
        nx = __builtin_fma(a, a, nx);
        nx = __builtin_fma(b, b, nx);
      }
    }
    const double xn = sqrt(wave_sum(nx)) * (1.0 + 0x1p-40);
    const double c1 = ((double)d + d / 32 + 8.0) * 0x1p-23 + (double)d * 0x1p-53;
    const double c2 = (double)d * 0x1p-125;
    float l32[kMaxJ];
    double lo[kMaxJ], hi[kMaxJ], bnd[kMaxJ];
    int bad = 0;
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) {
      const int e = min(lane + kWave * j, E - 1);
      l32[j] = lbound[(size_t)t * E + e];
      const double wn = (double)wnorm[e];
      const double bias = rm.bias ? (double)rm.bias[e] : 0.0;
      bnd[j] = (c1 * xn * wn + c2) * 1.02;
      const double l = (double)l32[j];
      const bool ok = j < nj && lane + kWave * j < E;
      if (ok && !(isfinite(l) && isfinite(bnd[j]) && isfinite(bias))) bad = 1;
      if (sig) {   // the selection score's range, with the evaluation margins
        const double m = 4.0 * kScoreEps * (1.0 + fabs(bias));
        lo[j] = sigmoid_score(l - bnd[j]) + bias - m;
        hi[j] = sigmoid_score(l + bnd[j]) + bias + m;
      } else {
        lo[j] = l - bnd[j];
        hi[j] = l + bnd[j];
      }
      if (!ok) lo[j] = hi[j] = -INFINITY;
    }
    bad = wave_sum(bad);
    // the k-th largest lower end (with multiplicity, -inf for the lanes'
    // empty slots, NaN as -inf): the sample select of topk_token (the k-th
    // lane maximum bounds it from below; the entries at or above that bound,
    // when at most 64, give it exactly by a radix descent), else k rounds of
    // the wave maximum, each dropping one holder's entry
    double lk = -INFINITY;
    {
      uint64_t key[kMaxJ], kb = 0;
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) {
        key[j] = order_key(isnan(lo[j]) ? -INFINITY : lo[j]);
        kb = key[j] > kb ? key[j] : kb;
      }
      const uint64_t thr = kth_largest_u64(kb, ~0ull, k);
      uint32_t cm = 0;
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j)
        if (key[j] >= thr) cm |= 1u << j;
      const int nc = wave_sum((int)__popc(cm));
      if (nc <= kWave) {
        int n = 0;
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) {
          const bool mine = (cm >> j) & 1u;
          const unsigned long long bal = __ballot(mine);
          if (mine) s_key[n + __popcll(bal & ((1ull << lane) - 1ull))] = key[j];
          n += __popcll(bal);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint64_t ck = lane < nc ? s_key[lane] : 0;
        const uint64_t live = nc >= kWave ? ~0ull : (1ull << nc) - 1ull;
        lk = key_value(kth_largest_u64(ck, live, k));
      } else {
        double v[kMaxJ];
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) v[j] = lo[j];
        for (int r = 0; r < k; ++r) {
          double mv = -INFINITY;
          int mj = -1;
#pragma unroll
          for (int j = 0; j < kMaxJ; ++j)
            if (v[j] > mv) { mv = v[j]; mj = j; }
          lk = wave_max(mv);
          const unsigned long long h = __ballot(mj >= 0 && mv == lk);
          const int wl = h ? __ffsll((long long)h) - 1 : -1;
          if (lane == wl) {
#pragma unroll
            for (int j = 0; j < kMaxJ; ++j)
              if (j == mj) v[j] = -INFINITY;
          }
        }
      }
    }
    // candidates: every expert whose upper end reaches lk (all of them if a
    // value or bound is not finite), listed in (j, lane) order; the others
    // keep the fp32 value and its bound (rounded up to fp32)
    int n = 0;
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) {
      const int e = lane + kWave * j;
      const bool valid = j < nj && e < E;
      const bool mine = valid && (bad || hi[j] >= lk);
      const unsigned long long bal = __ballot(mine);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (mine) s_cand[n + before] = e;
      n += __popcll(bal);
      if (valid && !mine) {
        logits[(size_t)t * E + e] = (double)l32[j];
        lbound[(size_t)t * E + e] = (float)(bnd[j] * (1.0 + 0x1p-20));
      }
    }
    if (lane == 0) s_n_all[wv] = n;
  }
  __syncthreads();
  // the candidates' fp64 values and bounds (the GEMV router's arithmetic:
  // |acc - exact| <= (d/64 + 8) u S, |oracle - exact| <= d u S, u = 2^-53,
  // S <= 1.01 aabs), two rows of one token per pass; pass q of the
  // workgroup's list (token 0's passes, then token 1's, ...) goes to wave
  // q % NW
  int pe[NW + 1];
  pe[0] = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) pe[i + 1] = pe[i] + (s_n_all[i] + 1) / 2;
  for (int q = wv; q < pe[NW]; q += NW) {
    int ti = 0;
#pragma unroll
    for (int i = 1; i < NW; ++i) ti += q >= pe[i] ? 1 : 0;
    const int tt = blockIdx.x * NW + ti, n = s_n_all[ti];
    const int c = 2 * (q - pe[ti]);
    const int e0 = s_cand_all[ti][c], e1 = c + 1 < n ? s_cand_all[ti][c + 1] : e0;
    double acc[2];
    float aabs[2];
    refine_dot(x + (size_t)tt * d, wr + (size_t)e0 * d, wr + (size_t)e1 * d, d, lane, acc, aabs);
    if (lane == 0) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int e = p ? e1 : e0;
        logits[(size_t)tt * E + e] = acc[p];
        lbound[(size_t)tt * E + e] = (float)((2.0 * d + 64.0) * 0x1p-53 * (double)aabs[p] * 1.02);
      }
    }
  }
}

hipError_t launch_router_bf16(const uint16_t* x, const uint16_t* wr, const RouteWs& ws, int T,
                              int d, int E, int k, const RouterMode& rm, hipStream_t st) {
  router_wnorm<<<(E + 3) / 4, 256, 0, st>>>(wr, ws.wnorm, d, E);
  hipError_t err = launch_router_logits_lds(x, wr, ws.lbound, T, d, E, st);
  if (err != hipSuccess) return err;
  route_refine<4><<<(T + 3) / 4, 256, 0, st>>>(x, wr, ws.wnorm, ws.logits, ws.lbound, T, d, E, k,
                                              rm);
  return hipGetLastError();
}

// fp64 logits to the fp32 output
__global__ __launch_bounds__(256) void logits_to_f32(const double* __restrict__ l,
                                                     float* __restrict__ o, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) o[i] = (float)l[i];
}

// fp64 router tiles: 16 x 16 up to 64 tokens, 32 x 16 up to 256, else 32 x 32,
// so that small batches still spread the fp64 matrix work over the CUs
// (at 64 tokens and 896 experts: 224 workgroups instead of 56).
void launch_router_mfma(const uint16_t* x, const uint16_t* wr, double* logits, float* lbound,
                        int T, int d, int E, hipStream_t st) {
  if (T <= 64)
    router_mfma_f64<1, 1><<<dim3((T + 15) / 16, (E + 15) / 16), 256, 0, st>>>(x, wr, logits,
                                                                             lbound, T, d, E);
  else if (T <= 256)
    router_mfma_f64<2, 1><<<dim3((T + 31) / 32, (E + 15) / 16), 256, 0, st>>>(x, wr, logits,
                                                                             lbound, T, d, E);
  else
    router_mfma_f64<2, 2><<<dim3((T + 31) / 32, (E + 31) / 32), 256, 0, st>>>(x, wr, logits,
                                                                             lbound, T, d, E);
}

// One token: the selection (wave 0 of workgroup 0, the workgroup's only
// working wave) runs beside the shared experts' gate/up (every wave of the
// other workgroups takes one (expert, feature) item), which does not depend
// on the routing.  Workgroups of 4 waves; the streaming workgroups stage x in
// LDS, pass one barrier, and no barrier follows.
__global__ __launch_bounds__(256) void topk_shared_t1(
    const double* __restrict__ logits, const float* __restrict__ lbound,
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ diag, int d,
    int E, int k, PermOut perm, const uint16_t* __restrict__ w13s, float* __restrict__ hs, int fs,
    int S, RouterMode rm) {
  __shared__ TopkLds sm;
  __shared__ uint4 xs[kSgU * kWave];
  const int lane = threadIdx.x & 63;
  // workgroup 0: the selection alone (its wave 0), without the x staging and
  // barrier the streaming workgroups need (layer 105.6 -> 103.6 us)
  if (blockIdx.x == 0) {
    if (threadIdx.x < kWave)
      topk_token<false>(0, lane, sm, logits, lbound, x, wr, idx_out, w_out, nullptr, diag, d, E,
                        k, perm, rm);
    return;
  }
  stage_row(reinterpret_cast<const uint4*>(x), d / 8, xs);
  __syncthreads();
  const int gw = (blockIdx.x - 1) * 4 + (threadIdx.x >> 6);
  if (gw < S * fs) shared_gateup_item(gw, w13s, xs, hs, d, fs, lane);
}

}  // namespace

hipError_t launch_router_logits(const k3moe_shape& s, const void* x, const uint16_t* wr,
                                const RouteWs& ws, hipStream_t st) {
  const int T = (int)s.T;
  if (use_mfma(s))
    launch_router_mfma(static_cast<const uint16_t*>(x), wr, ws.logits, ws.lbound, T, s.d, s.E, st);
  else if (s.x_dtype == K3MOE_F32)
    router_gemv_f64<true><<<dim3((s.E + 3) / 4), 256, 0, st>>>(x, wr, ws.logits, ws.lbound, T, s.d,
                                                               s.E);
  else
    router_gemv_f64<false><<<dim3((s.E + 3) / 4), 256, 0, st>>>(x, wr, ws.logits, ws.lbound, T,
                                                                s.d, s.E);
  return hipGetLastError();
}

bool topk_shared_t1_ok(const k3moe_shape& s) {
  return s.T == 1 && s.x_dtype == K3MOE_BF16 && s.d == kSgU * 8 * kWave && s.n_shared > 0;
}

hipError_t launch_topk_shared_t1(const k3moe_shape& s, const void* x, const uint16_t* wr,
                                 const float* bias, int32_t* idx, float* w, int32_t* diag,
                                 const RouteWs& ws, const PermOut& perm,
                                 const k3moe_expert_bank& shared, float* hs, hipStream_t st) {
  if (!topk_shared_t1_ok(s)) return hipErrorInvalidValue;
  const int items = shared.n_experts * shared.f;
  RouterMode rm;
  rm.mode = s.router;
  rm.bias = bias;
  topk_shared_t1<<<1 + (items + 3) / 4, 256, 0, st>>>(
      ws.logits, ws.lbound, static_cast<const uint16_t*>(x), wr, idx, w, diag, s.d, s.E, s.k, perm,
      static_cast<const uint16_t*>(shared.w13), hs, shared.f, shared.n_experts, rm);
  return hipGetLastError();
}

hipError_t launch_route(const k3moe_shape& s, const void* x, const uint16_t* wr, const float* bias,
                        int32_t* idx, float* w, float* logits_out, int32_t* diag,
                        const RouteWs& ws, hipStream_t st, const PermOut& perm) {
  RouterMode rm;
  rm.mode = s.router;
  rm.bias = bias;
  if (perm.counts && s.T != 1) return hipErrorInvalidValue;
  const int T = (int)s.T;
  const bool xf32 = s.x_dtype == K3MOE_F32;
  const dim3 g1((s.E + 3) / 4);
  if (use_mfma(s) && T >= kBf16RouterMinT) {
    // bf16 logits, the candidates refined in fp64, the selection; the fp64
    // logits of every expert only when the caller asks for them
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    hipError_t err = launch_router_bf16(xb, wr, ws, T, s.d, s.E, s.k, rm, st);
    if (err != hipSuccess) return err;
    topk_softmax<false><<<T, 64, 0, st>>>(ws.logits, ws.lbound, x, wr, idx, w, nullptr, diag, T,
                                          s.d, s.E, s.k, perm, rm);
    err = hipGetLastError();
    if (err != hipSuccess || !logits_out) return err;
    launch_router_mfma(xb, wr, ws.logits, ws.lbound, T, s.d, s.E, st);
    const int64_t n = (int64_t)T * s.E;
    logits_to_f32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(ws.logits, logits_out, n);
    return hipGetLastError();
  }
  if (use_mfma(s))
    launch_router_mfma(static_cast<const uint16_t*>(x), wr, ws.logits, ws.lbound, T, s.d, s.E, st);
  else if (xf32)
    router_gemv_f64<true><<<g1, 256, 0, st>>>(x, wr, ws.logits, ws.lbound, T, s.d, s.E);
  else
    router_gemv_f64<false><<<g1, 256, 0, st>>>(x, wr, ws.logits, ws.lbound, T, s.d, s.E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (xf32)
    topk_softmax<true><<<T, 64, 0, st>>>(ws.logits, ws.lbound, x, wr, idx, w, logits_out, diag,
                                         T, s.d, s.E, s.k, perm, rm);
  else
    topk_softmax<false><<<T, 64, 0, st>>>(ws.logits, ws.lbound, x, wr, idx, w, logits_out, diag,
                                          T, s.d, s.E, s.k, perm, rm);
  return hipGetLastError();
}

}  // namespace k3
