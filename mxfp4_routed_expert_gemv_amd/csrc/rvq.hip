// Routed expert FFN on RVQ3 experts: residual vector quantisation at 3.00
// bits per weight, every 8-weight vector the sum of one entry from each of
// three 256-entry codebooks (WASTE article page, section "정확성 검증과
// 양자화").  The pages' engine never materialises the matrix: per token it
// builds a table of the dot products of every codebook entry with the
// token's activations and sums table entries (same section).  Kept here, with
// the table sized for LDS:
//   * a workgroup owns one pair (token, expert) and one slice of 128 columns
//     (16 groups of 8).  It builds T[s][g][j] = C_s[j] . v[8g .. 8g+7] for the
//     3 stages, 16 groups and 256 entries (48 KB of LDS; each entry an fp32
//     dot of 8 in element order; each codeword is read once), then every
//     row r of the matrix is
//       p[r] = sum over s = 0..2, then g = 0..15 of T[s][g][i_s[r][g]]
//     read from the row's 3 x 16 index bytes (one 16-byte load per stage);
//   * a second kernel adds the slices' partial sums of a row in slice order
//     (gate/up: then h = silu(g) * u; down: y).
// Index layout [3][cols/128][rows][16]: a stage's indices of one slice are
// contiguous over the rows, so consecutive threads (consecutive rows) read
// consecutive 16-byte chunks.  Every sum has a fixed order that depends only
// on the pair, so a token's outputs do not depend on the rest of the batch.
#include "internal.h"
#include "kern_common.h"

namespace k3 {
namespace {

constexpr int kRvqSlice = 128;           // columns per slice
constexpr int kRvqGroups = kRvqSlice / 8;
constexpr int kRvqEntries = 3 * kRvqGroups * 256;

// The expert whose sorted-position range holds q (offsets ascending, E + 1 entries).
__device__ __forceinline__ int rvq_expert_of(const int32_t* __restrict__ offsets, int E, int q) {
  int lo = 0, hi = E;   // offsets[lo] <= q < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= q) lo = mid; else hi = mid;
  }
  return lo;
}

// Partial sums of one (pair, slice): part[q][slice][r] for r < rows.
// GATEUP: v is the pair's token row of x (bf16 or fp32); else the pair's h
// row (fp32).
template <bool GATEUP, bool XF32>
__global__ __launch_bounds__(256) void rvq_partial(const void* __restrict__ v_src,
                                                   const uint8_t* __restrict__ idx,
                                                   const float* __restrict__ cb,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ sorted_pair,
                                                   float* __restrict__ part, int rows, int cols,
                                                   int E, int k) {
  __shared__ float tab[kRvqEntries];
  __shared__ float vs[kRvqSlice];
  __shared__ int s_e;
  const int q = blockIdx.x, slice = blockIdx.y, tid = threadIdx.x;
  const int nsl = cols / kRvqSlice;
  // pairs past offsets[E] were dropped by the permute: nothing to compute
  if (tid == 0) s_e = q < offsets[E] ? rvq_expert_of(offsets, E, q) : -1;
  __syncthreads();
  if (s_e < 0) return;
  if (tid < kRvqSlice) {
    const int c = slice * kRvqSlice + tid;
    float val;
    if (GATEUP) {
      const size_t t = (size_t)(sorted_pair[q] / k);
      val = XF32 ? static_cast<const float*>(v_src)[t * cols + c]
                 : __uint_as_float((uint32_t)static_cast<const uint16_t*>(v_src)[t * cols + c]
                                   << 16);
    } else {
      val = static_cast<const float*>(v_src)[(size_t)q * cols + c];
    }
    vs[tid] = val;
  }
  __syncthreads();
  const int e = s_e;
  const float* cbe = cb + (size_t)e * 3 * 256 * 8;
  const size_t mat = (size_t)e * 3 * nsl * rows;     // this expert's first index chunk
  const uint8_t* ib = idx + mat * 16;
  // rows r = tid + 256 i, their 3 x 16 index bytes DQ rows ahead of use; the
  // first DQ rows' are requested before the table is built
  constexpr int DQ = 4;
  auto load_row = [&](int r, uint4 (&iv)[3]) {
#pragma unroll
    for (int s = 0; s < 3; ++s)
      iv[s] = *reinterpret_cast<const uint4*>(ib + (((size_t)s * nsl + slice) * rows + r) * 16);
  };
  uint4 buf[DQ][3];
#pragma unroll
  for (int j = 0; j < DQ; ++j)
    if (tid + 256 * j < rows) load_row(tid + 256 * j, buf[j]);
  // table: entry (s * 16 + g) * 256 + j.  Thread t loads codeword (s, j) once
  // (3 of the 768 per thread) and writes its 16 dot products, one per group.
  for (int c = tid; c < 3 * 256; c += 256) {
    const int s = c >> 8, j = c & 255;
    const float4 c0 = *reinterpret_cast<const float4*>(cbe + (size_t)c * 8);
    const float4 c1 = *reinterpret_cast<const float4*>(cbe + (size_t)c * 8 + 4);
#pragma unroll 4
    for (int g = 0; g < kRvqGroups; ++g) {
      const float* vg = vs + g * 8;
      float a = c0.x * vg[0];
      a = __builtin_fmaf(c0.y, vg[1], a);
      a = __builtin_fmaf(c0.z, vg[2], a);
      a = __builtin_fmaf(c0.w, vg[3], a);
      a = __builtin_fmaf(c1.x, vg[4], a);
      a = __builtin_fmaf(c1.y, vg[5], a);
      a = __builtin_fmaf(c1.z, vg[6], a);
      a = __builtin_fmaf(c1.w, vg[7], a);
      tab[(s * kRvqGroups + g) * 256 + j] = a;
    }
  }
  __syncthreads();
  for (int r0 = tid; r0 < rows; r0 += 256 * DQ) {
#pragma unroll
    for (int jq = 0; jq < DQ; ++jq) {
      const int r = r0 + 256 * jq;
      if (r < rows) {
        const uint4 cur[3] = {buf[jq][0], buf[jq][1], buf[jq][2]};
        if (r + 256 * DQ < rows) load_row(r + 256 * DQ, buf[jq]);
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          const uint32_t w4[4] = {cur[s].x, cur[s].y, cur[s].z, cur[s].w};
#pragma unroll
          for (int g = 0; g < kRvqGroups; ++g) {
            const uint32_t i = (w4[g >> 2] >> (8 * (g & 3))) & 0xFFu;
            acc += tab[(s * kRvqGroups + g) * 256 + i];
          }
        }
        part[((size_t)q * nsl + slice) * rows + r] = acc;
      }
    }
  }
}

// The same partial sums with one stage's table in LDS at a time (16 KB, so
// that 4 workgroups fit a CU and a one-token batch's workgroups all run at
// once): the table of stage s is built, every row of the thread adds its 16
// entries of stage s to its running sum (registers, up to 16 rows a thread),
// then the next stage's table replaces it.  Each row's sum takes the same
// entries in the same order as rvq_partial, so the bits are the same.  Used
// for the gate/up (2f <= 4096 rows); the down keeps rvq_partial.
constexpr int kRvqRowsPerThread = 16;   // rows <= 256 * kRvqRowsPerThread
template <bool GATEUP, bool XF32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void rvq_partial_staged(const void* __restrict__ v_src,
                                                          const uint8_t* __restrict__ idx,
                                                          const float* __restrict__ cb,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted_pair,
                                                          float* __restrict__ part, int rows,
                                                          int cols, int E, int k) {
  constexpr int RB = 8;                     // rows whose indices are loaded together
  constexpr int RMAX = kRvqRowsPerThread;
  __shared__ float tab[kRvqGroups * 256];
  __shared__ float vs[kRvqSlice];
  __shared__ int s_e;
  const int q = blockIdx.x, slice = blockIdx.y, tid = threadIdx.x;
  const int nsl = cols / kRvqSlice;
  if (tid == 0) s_e = q < offsets[E] ? rvq_expert_of(offsets, E, q) : -1;
  __syncthreads();
  if (s_e < 0) return;
  if (tid < kRvqSlice) {
    const int c = slice * kRvqSlice + tid;
    float val;
    if (GATEUP) {
      const size_t t = (size_t)(sorted_pair[q] / k);
      val = XF32 ? static_cast<const float*>(v_src)[t * cols + c]
                 : __uint_as_float((uint32_t)static_cast<const uint16_t*>(v_src)[t * cols + c]
                                   << 16);
    } else {
      val = static_cast<const float*>(v_src)[(size_t)q * cols + c];
    }
    vs[tid] = val;
  }
  const int e = s_e;
  const float* cbe = cb + (size_t)e * 3 * 256 * 8;
  const uint8_t* ib = idx + (size_t)e * 3 * nsl * rows * 16;
  const int nr = (rows + 255) / 256;
  float acc[RMAX];
#pragma unroll
  for (int i = 0; i < RMAX; ++i) acc[i] = 0.0f;
  for (int s = 0; s < 3; ++s) {
    __syncthreads();   // vs written (s = 0); the previous stage's lookups done
    {
      // entry g * 256 + j of stage s: thread j's codeword against group g
      const float4 c0 = *reinterpret_cast<const float4*>(cbe + (size_t)(s * 256 + tid) * 8);
      const float4 c1 = *reinterpret_cast<const float4*>(cbe + (size_t)(s * 256 + tid) * 8 + 4);
#pragma unroll 4
      for (int g = 0; g < kRvqGroups; ++g) {
        const float* vg = vs + g * 8;
        float a = c0.x * vg[0];
        a = __builtin_fmaf(c0.y, vg[1], a);
        a = __builtin_fmaf(c0.z, vg[2], a);
        a = __builtin_fmaf(c0.w, vg[3], a);
        a = __builtin_fmaf(c1.x, vg[4], a);
        a = __builtin_fmaf(c1.y, vg[5], a);
        a = __builtin_fmaf(c1.z, vg[6], a);
        a = __builtin_fmaf(c1.w, vg[7], a);
        tab[g * 256 + tid] = a;
      }
    }
    __syncthreads();
    const uint8_t* is = ib + ((size_t)s * nsl + slice) * rows * 16;
#pragma unroll
    for (int i0 = 0; i0 < RMAX; i0 += RB) {
      if (i0 < nr) {
        uint4 iv[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const int r = min(tid + 256 * (i0 + j), rows - 1);
          iv[j] = *reinterpret_cast<const uint4*>(is + (size_t)r * 16);
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const uint32_t w4[4] = {iv[j].x, iv[j].y, iv[j].z, iv[j].w};
          float a = acc[i0 + j];
#pragma unroll
          for (int g = 0; g < kRvqGroups; ++g)
            a += tab[g * 256 + ((w4[g >> 2] >> (8 * (g & 3))) & 0xFFu)];
          acc[i0 + j] = a;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RMAX; ++i) {
    const int r = tid + 256 * i;
    if (i < nr && r < rows) part[((size_t)q * nsl + slice) * rows + r] = acc[i];
  }
}

// h[q][j] = silu(g) * u with g, u the slice sums (in slice order) of rows j
// and f + j; the loads of 8 slices are issued before they are added.
__global__ __launch_bounds__(64) void rvq_reduce_gateup(const float* __restrict__ part,
                                                        float* __restrict__ h, int64_t P, int f,
                                                        int nsl) {
  const int64_t n = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (n >= P * f) return;
  const int64_t q = n / f;
  const int j = (int)(n - q * f);
  const float* pq = part + (size_t)q * nsl * 2 * f + j;
  float g = 0.0f, u = 0.0f;
  for (int s0 = 0; s0 < nsl; s0 += 8) {
    float vg[8], vu[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = min(s0 + i, nsl - 1);
      vg[i] = pq[(size_t)s * 2 * f];
      vu[i] = pq[(size_t)s * 2 * f + f];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (s0 + i < nsl) {
        g += vg[i];
        u += vu[i];
      }
  }
  h[n] = silu_mul(g, u);
}

// y[q][o] = the slice sums (in slice order) of row o.
__global__ __launch_bounds__(64) void rvq_reduce_down(const float* __restrict__ part,
                                                      float* __restrict__ y, int64_t P, int d,
                                                      int nsl) {
  const int64_t n = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (n >= P * d) return;
  const int64_t q = n / d;
  const int o = (int)(n - q * d);
  const float* pq = part + (size_t)q * nsl * d + o;
  float acc = 0.0f;
  for (int s0 = 0; s0 < nsl; s0 += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = pq[(size_t)min(s0 + i, nsl - 1) * d];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (s0 + i < nsl) acc += v[i];
  }
  y[n] = acc;
}

}  // namespace

size_t rvq_part_floats(const k3moe_shape& s) {
  const size_t P = (size_t)s.T * s.k;
  const size_t gu = (size_t)2 * s.f * (s.d / kRvqSlice), dn = (size_t)s.d * (s.f / kRvqSlice);
  return P * (gu > dn ? gu : dn);
}

hipError_t launch_gateup_rvq(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                             const int32_t* offsets, const int32_t* sorted_pair, float* h,
                             float* part, hipStream_t st) {
  const int64_t P = s.T * s.k;
  const dim3 g((unsigned)P, s.d / kRvqSlice);
  const uint8_t* idx = static_cast<const uint8_t*>(b.w13);
  const float* cb = static_cast<const float*>(b.w13_scale);
  // one stage's table at a time where the rows fit the registers: 4
  // workgroups a CU instead of 3, so a one-token batch's 896 workgroups run
  // in one round (gate/up 0.366 -> 0.392 of the HBM peak at one token;
  // decode_b64 layer 3.56 -> 3.50 ms; same bits)
  const bool staged = 2 * s.f <= 256 * kRvqRowsPerThread;
  if (staged && s.x_dtype == K3MOE_F32)
    rvq_partial_staged<true, true><<<g, 256, 0, st>>>(x, idx, cb, offsets, sorted_pair, part,
                                                     2 * s.f, s.d, s.E, s.k);
  else if (staged)
    rvq_partial_staged<true, false><<<g, 256, 0, st>>>(x, idx, cb, offsets, sorted_pair, part,
                                                      2 * s.f, s.d, s.E, s.k);
  else if (s.x_dtype == K3MOE_F32)
    rvq_partial<true, true><<<g, 256, 0, st>>>(x, idx, cb, offsets, sorted_pair, part, 2 * s.f,
                                              s.d, s.E, s.k);
  else
    rvq_partial<true, false><<<g, 256, 0, st>>>(x, idx, cb, offsets, sorted_pair, part, 2 * s.f,
                                               s.d, s.E, s.k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n = P * s.f;
  rvq_reduce_gateup<<<(unsigned)((n + 63) / 64), 64, 0, st>>>(part, h, P, s.f, s.d / kRvqSlice);
  return hipGetLastError();
}

hipError_t launch_down_rvq(const k3moe_shape& s, const k3moe_expert_bank& b, const float* h,
                           const int32_t* offsets, float* y, float* part, hipStream_t st) {
  const int64_t P = s.T * s.k;
  const dim3 g((unsigned)P, s.f / kRvqSlice);
  rvq_partial<false, true><<<g, 256, 0, st>>>(h, static_cast<const uint8_t*>(b.w2),
                                               static_cast<const float*>(b.w2_scale), offsets,
                                               nullptr, part, s.d, s.f, s.E, s.k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n = P * s.d;
  rvq_reduce_down<<<(unsigned)((n + 63) / 64), 64, 0, st>>>(part, y, P, s.d, s.f / kRvqSlice);
  return hipGetLastError();
}

}  // namespace k3
