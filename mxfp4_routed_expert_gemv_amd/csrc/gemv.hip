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
// Routed kernels are persistent: each workgroup lists the experts that have
// pairs (in LDS, once), and each wave walks work items (expert, group of
// output rows) with a stride of the grid, issuing the next item's weight loads
// before computing the current one, so a wave always has a weight tile in
// flight.  A weight row is fetched from HBM once per call however many tokens
// chose the expert: the item loops over the expert's tokens with its rows held
// in registers.
#include "internal.h"
#include "kern_common.h"
#include "decode_t1.h"

namespace k3 {
namespace {

// ---------------------------------------------------------------- reductions
// Transposed butterfly over the wave for NV values per lane (NV a power of 2,
// <= 64).  At distance DIST a lane keeps half of its values and adds its
// partner's copy of them, so after log2(64) steps lane l holds the full sum
// of value index l >> (6 - log2 NV).  Every value is summed with the same
// pairing sequence (32, 16, 8, 4, 2, 1) as a plain butterfly, hence the same
// bits, whatever NV is.
template <int NV, int DIST>
struct XReduce {
  static __device__ __forceinline__ void run(float* v, int lane) {
    if constexpr (NV > 1) {
      constexpr int H = NV / 2;
      const bool up = (lane & DIST) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = up ? v[i] : v[H + i];
        const float keep = up ? v[H + i] : v[i];
        v[i] = keep + __shfl_xor(send, DIST, kWave);
      }
      if constexpr (DIST > 1) XReduce<H, DIST / 2>::run(v, lane);
    } else {
      v[0] = v[0] + __shfl_xor(v[0], DIST, kWave);
      if constexpr (DIST > 1) XReduce<1, DIST / 2>::run(v, lane);
    }
  }
};

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// ------------------------------------------------------- work-item metadata
// Loads here are never guarded: out-of-range lanes read a clamped, valid
// address and their value is discarded.  A guarded load gets a basic block of
// its own and is waited on before the next one is issued.

// Per workgroup, in LDS: the experts that have pairs (ascending), their
// sorted-pair ranges and the tokens of their first NTOK pairs.
template <int NTOK>
struct Meta {
  int n_act;
  int act[1024];
  int tok[NTOK > 0 ? NTOK : 1][1024];
};

// 256 threads.  offsets has E + 1 entries; E <= 1024.
template <int NTOK>
__device__ __forceinline__ void stage_meta(const int32_t* __restrict__ offsets,
                                           const int32_t* __restrict__ sorted_pair, int E, int k,
                                           Meta<NTOK>& m, int* sums) {
  const int tid = threadIdx.x;
  int o[5];
#pragma unroll
  for (int u = 0; u < 5; ++u) o[u] = offsets[min(tid * 4 + u, E)];
  int f[4], c = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    f[u] = (tid * 4 + u < E && o[u + 1] > o[u]) ? 1 : 0;
    c += f[u];
  }
  // exclusive position of this thread's first active expert: a scan within
  // each wave, then the totals of the lower waves
  const int lane = tid & 63, wv = tid >> 6;
  int incl = c;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) sums[wv] = incl;
  __syncthreads();
  int pos = incl - c;
  for (int w = 0; w < wv; ++w) pos += sums[w];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (f[u]) m.act[pos++] = tid * 4 + u;
  if (tid == 255) m.n_act = pos;
  __syncthreads();
  if constexpr (NTOK > 0) {
    const int n = m.n_act;
    if (n > 0) {
      int tk[4][NTOK];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = m.act[min(tid + 256 * u, n - 1)];
        const int q0 = offsets[e], q1 = offsets[e + 1] - 1;
#pragma unroll
        for (int mt = 0; mt < NTOK; ++mt) tk[u][mt] = sorted_pair[min(q0 + mt, q1)];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (tid + 256 * u < n)
#pragma unroll
          for (int mt = 0; mt < NTOK; ++mt) m.tok[mt][tid + 256 * u] = tk[u][mt] / k;
    }
    __syncthreads();
  }
}

// Copy n16 16-byte words of one activation row into LDS (256 threads).

// Persistent walk over work items: item it goes to wave it mod (#waves).
// Overlap of one wave's loads with another's decode comes from occupancy
// (several waves per SIMD), not from per-wave register double buffering:
// under register pressure the allocator reuses registers that are still the
// destinations of in-flight loads, and the wait that forces drains the
// prefetch.
template <class Op>
__device__ __forceinline__ void walk_items_single(const Op& op, int n_items) {
  typename Op::Regs A;
  const int GW = gridDim.x * (blockDim.x >> 6);
  for (int it = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); it < n_items; it += GW) {
    op.load(it, A);
    op.compute(it, A);
  }
}

// Double-buffered variant: the loads of a wave's next item are issued before
// its current item is computed.
template <class Op>
__device__ __forceinline__ void walk_items(const Op& op, int n_items) {
  typename Op::Regs A, B;
  const int GW = gridDim.x * (blockDim.x >> 6);
  int it = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (it >= n_items) return;
  op.load(it, A);
  while (true) {
    int nx = it + GW;
    if (nx < n_items) op.load(nx, B);
    op.compute(it, A);
    if (nx >= n_items) return;
    it = nx;
    nx = it + GW;
    if (nx < n_items) op.load(nx, A);
    op.compute(it, B);
    if (nx >= n_items) return;
    it = nx;
  }
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
  __device__ __forceinline__ void load_lds(const uint4* xs, int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = xs[b * 4 + i];
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
  __device__ __forceinline__ void load_lds(const uint4* xs, int b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = xs[b * 8 + i];
  }
  __device__ __forceinline__ float dot(const uint4& c) const { return block_dot_f32(c, v); }
};

// ------------------------------------------------------ routed gate/up (MXFP4)
// Item (j, rg): gate rows rg*R .. rg*R+R-1 of the j-th active expert and the
// matching up rows f + ...; for every sorted pair p of that expert,
// h[p][row] = silu(g) * u.  Lane l owns scale blocks l, l+64, ... (NU per
// pass).  XLDS: the batch is one token whose row sits in LDS.
template <int R, int MT, int NU, bool XF32, bool XLDS>
struct GateUpOp {
  static constexpr int NR = 2 * R;
  static constexpr int NV = NR * MT;
  const uint8_t* w13;
  const uint8_t* w13s;
  const void* x;
  const int32_t* sorted_pair;
  float* h;
  const Meta<XLDS ? 0 : MT>* meta;
  const uint4* xs;
  int d, f, k, rgroups;

  const int32_t* offsets;

  struct Regs {
    uint4 q[NU][NR];
    uint32_t s[NU][NR];
    int p0, p1;
  };

  __device__ __forceinline__ void load_blocks(int e, int rg, int b0, Regs& r) const {
    const int lane = threadIdx.x & 63, nb = d >> 5;
    const size_t rb = (size_t)(d >> 1), sb = (size_t)nb;
    const uint8_t* qe = w13 + (size_t)e * 2 * f * rb;
    const uint8_t* se = w13s + (size_t)e * 2 * f * sb;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int b = min(b0 + lane + kWave * u, nb - 1);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const size_t row = (size_t)(i < R ? rg * R + i : f + rg * R + i - R);
        r.q[u][i] = ldg16(qe + row * rb + (size_t)b * 16);
        r.s[u][i] = se[row * sb + b];
      }
    }
  }

  __device__ __forceinline__ void load(int it, Regs& r) const {
    const int j = it / rgroups, rg = it - j * rgroups, e = meta->act[j];
    r.p0 = offsets[e];   // issued before the weights: waiting for them keeps
    r.p1 = offsets[e + 1];  // the weight loads in flight
    load_blocks(e, rg, 0, r);
  }

  __device__ __forceinline__ void compute(int it, Regs& r) const {
    const int lane = threadIdx.x & 63, nb = d >> 5;
    const int j = it / rgroups, rg = it - j * rgroups, e = meta->act[j];
    const int p0 = r.p0, p1 = r.p1;
    for (int p = p0; p < p1; p += MT) {
      float v[NV];
      size_t xo[MT];
      bool tv[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        tv[mt] = p + mt < p1;
        int tok = 0;
        if (!XLDS) tok = (p == p0) ? meta->tok[mt][j] : sorted_pair[min(p + mt, p1 - 1)] / k;
        xo[mt] = (size_t)tok * d;
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = 0.0f;
      for (int b0 = 0; b0 < nb; b0 += kWave * NU) {
        if (b0 > 0) load_blocks(e, rg, b0, r);   // rows longer than one pass
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int bu = b0 + lane + kWave * u;
          const bool ok = bu < nb;
          const int b = min(bu, nb - 1);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if (!tv[mt]) continue;
            XBlock<XF32> xb;
            if (XLDS) xb.load_lds(xs, b);
            else xb.load(x, xo[mt] + (size_t)b * 32);
#pragma unroll
            for (int i = 0; i < NR; ++i) {
              const float t = __builtin_fmaf(xb.dot(r.q[u][i]), e8m0_to_f32(r.s[u][i]),
                                             v[i * MT + mt]);
              v[i * MT + mt] = ok ? t : v[i * MT + mt];
              // one row's 32 decoded weights live at a time
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      if (nb > kWave * NU && p + MT < p1) load_blocks(e, rg, 0, r);
      XReduce<NV, 32>::run(v, lane);
      // lane l now holds value index l >> (6 - log2 NV): gate rows in the
      // lower half of the lanes, the matching up rows 32 lanes higher.
      const float uval = __shfl_xor(v[0], 32, kWave);
      constexpr int SH = 6 - ilog2(NV);
      const int idx = lane >> SH;
      if (lane < 32 && (lane & ((1 << SH) - 1)) == 0) {
        const int i = idx / MT, mt = idx - i * MT;
        if (p + mt < p1) h[(size_t)(p + mt) * f + rg * R + i] = silu_mul(v[0], uval);
      }
    }
  }
};

template <int R, int MT, int NU, bool XF32, bool XLDS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void gateup_persistent(GateUpOp<R, MT, NU, XF32, XLDS> op, const int32_t* __restrict__ offsets,
                       int E) {
  __shared__ Meta<XLDS ? 0 : MT> meta;
  __shared__ int sums[256];
  extern __shared__ uint4 xs[];   // the token's row when XLDS (dynamic size)
  if (XLDS) stage_row(static_cast<const uint4*>(op.x), op.d * (XF32 ? 4 : 2) / 16, xs);
  stage_meta<XLDS ? 0 : MT>(offsets, op.sorted_pair, E, op.k, meta, sums);
  op.meta = &meta;
  op.xs = xs;
  walk_items_single(op, meta.n_act * op.rgroups);
}

// ----------------------------------------- routed gate/up, one token (MXFP4)
// The decode batch of one token: its row sits in LDS, and an item is one gate
// row with its up row.  The blocks of the two rows are walked in pairs with
// two register sets used in turn (the loads of the next block are issued
// before the current block is decoded), so only two blocks are live and the
// wave keeps a small register footprint: several waves per SIMD then overlap
// one wave's HBM wait with another's decode.  Per lane the blocks are summed
// in the same order (lane, lane+64, ...) as the batched kernel, with the same
// reduction tree, so a token's bits do not depend on the batch.
struct RowPair {
  uint4 qg, qu;
  uint32_t sg, su;
};

template <bool XF32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void gateup_t1(const uint8_t* __restrict__ w13, const uint8_t* __restrict__ w13s,
               const void* __restrict__ x, const int32_t* __restrict__ offsets,
               float* __restrict__ h, int d, int f, int E) {
  __shared__ Meta<0> meta;
  __shared__ int sums[256];
  extern __shared__ uint4 xs[];
  stage_row(static_cast<const uint4*>(x), d * (XF32 ? 4 : 2) / 16, xs);
  stage_meta<0>(offsets, nullptr, E, 1, meta, sums);
  const int lane = threadIdx.x & 63, nb = d >> 5;
  const size_t rb = (size_t)(d >> 1), sb = (size_t)nb;
  const int n_items = meta.n_act * f;
  const int GW = gridDim.x * 4;
  for (int it = blockIdx.x * 4 + (threadIdx.x >> 6); it < n_items; it += GW) {
    const int j = it / f, row = it - j * f, e = meta.act[j];
    const int p = offsets[e];
    const uint8_t* qg = w13 + ((size_t)e * 2 * f + row) * rb;
    const uint8_t* qu = qg + (size_t)f * rb;
    const uint8_t* sg = w13s + ((size_t)e * 2 * f + row) * sb;
    const uint8_t* su = sg + (size_t)f * sb;
    auto load = [&](int b, RowPair& r) {
      const int c = min(b, nb - 1);
      r.qg = ldg16(qg + (size_t)c * 16);
      r.qu = ldg16(qu + (size_t)c * 16);
      r.sg = sg[c];
      r.su = su[c];
    };
    float v[2] = {0.0f, 0.0f};
    auto step = [&](int b, const RowPair& r) {
      XBlock<XF32> xb;
      xb.load_lds(xs, min(b, nb - 1));
      const float tg = __builtin_fmaf(xb.dot(r.qg), e8m0_to_f32(r.sg), v[0]);
      const float tu = __builtin_fmaf(xb.dot(r.qu), e8m0_to_f32(r.su), v[1]);
      v[0] = b < nb ? tg : v[0];
      v[1] = b < nb ? tu : v[1];
    };
    RowPair A, B;
    load(lane, A);
#pragma unroll 1
    for (int b = lane; b - lane < nb; b += 2 * kWave) {
      load(b + kWave, B);
      step(b, A);
      load(b + 2 * kWave, A);
      step(b + kWave, B);
    }
    XReduce<2, 32>::run(v, lane);
    const float uval = __shfl_xor(v[0], 32, kWave);
    if (lane == 0) h[(size_t)p * f + row] = silu_mul(v[0], uval);
  }
}

// ------------------------------------------- routed down, one token (MXFP4)
// A workgroup takes a chunk of 128 output rows of one active expert, stages
// that expert's h row (the token's, f floats) in LDS once, and its waves walk
// items of 4 rows each.  Per lane the blocks are summed in the same order, and
// reduced with the same tree, as the batched kernel.
constexpr int kDownT1Rows = 4, kDownT1Chunk = 128;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void down_t1(const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2s,
             const float* __restrict__ h, const int32_t* __restrict__ offsets,
             float* __restrict__ y, int d, int f, int E) {
  constexpr int R = kDownT1Rows;
  __shared__ Meta<0> meta;
  __shared__ int sums[256];
  extern __shared__ uint4 hs[];   // f floats
  stage_meta<0>(offsets, nullptr, E, 1, meta, sums);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nb = f >> 5;
  const size_t rb = (size_t)(f >> 1), sb = (size_t)nb;
  const int chunks = d / kDownT1Chunk;
  const int n_chunks = meta.n_act * chunks;
  for (int c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const int j = c / chunks, e = meta.act[j];
    const int o0 = (c - j * chunks) * kDownT1Chunk;
    const int p = offsets[e];
    __syncthreads();   // the previous chunk's h is no longer read
    stage_row(reinterpret_cast<const uint4*>(h + (size_t)p * f), f / 4, hs);
    __syncthreads();
#pragma unroll 1
    for (int o = o0 + wave * R; o < o0 + kDownT1Chunk; o += 4 * R) {
      const uint8_t* qe = w2 + ((size_t)e * d + o) * rb;
      const uint8_t* se = w2s + ((size_t)e * d + o) * sb;
      float v[R];
#pragma unroll
      for (int i = 0; i < R; ++i) v[i] = 0.0f;
#pragma unroll 1
      for (int b0 = 0; b0 < nb; b0 += kWave) {
        const int bu = b0 + lane, b = min(bu, nb - 1);
        uint4 q[R];
        uint32_t sc[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          q[i] = ldg16(qe + (size_t)i * rb + (size_t)b * 16);
          sc[i] = se[(size_t)i * sb + b];
        }
        XBlock<true> hb;
        hb.load_lds(hs, b);
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const float t = __builtin_fmaf(hb.dot(q[i]), e8m0_to_f32(sc[i]), v[i]);
          v[i] = bu < nb ? t : v[i];
        }
      }
      XReduce<R, 32>::run(v, lane);
      constexpr int SH = 6 - ilog2(R);
      if ((lane & ((1 << SH) - 1)) == 0) y[(size_t)p * d + o + (lane >> SH)] = v[0];
    }
  }
}

// --------------------------------------------------------- routed down (MXFP4)
// Item (j, rg): rows o = rg*R .. rg*R+R-1 of the j-th active expert;
// y[p][o] = sum_j Wd[e][o][j] h[p][j] for every sorted pair p of the expert.
// The h blocks of the item's first MT pairs are fetched with its weights.
template <int R, int MT, int NU>
struct DownOp {
  static constexpr int NV = R * MT;
  const uint8_t* w2;
  const uint8_t* w2s;
  const float* h;
  float* y;
  const Meta<0>* meta;
  int d, f, rgroups;

  const int32_t* offsets;

  struct Regs {
    uint4 q[NU][R];
    uint32_t s[NU][R];
    uint4 hv[MT][NU][8];
    int p0, p1;
  };

  __device__ __forceinline__ void load_blocks(int e, int rg, int b0, Regs& r) const {
    const int lane = threadIdx.x & 63, nb = f >> 5;
    const size_t rb = (size_t)(f >> 1), sb = (size_t)nb;
    const uint8_t* qe = w2 + (size_t)e * d * rb;
    const uint8_t* se = w2s + (size_t)e * d * sb;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int b = min(b0 + lane + kWave * u, nb - 1);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const size_t row = (size_t)(rg * R + i);
        r.q[u][i] = ldg16(qe + row * rb + (size_t)b * 16);
        r.s[u][i] = se[row * sb + b];
      }
    }
  }

  __device__ __forceinline__ void load_h(int p, int p1, int b0, Regs& r) const {
    const int lane = threadIdx.x & 63, nb = f >> 5;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float* hp = h + (size_t)min(p + mt, p1 - 1) * f;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int b = min(b0 + lane + kWave * u, nb - 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) r.hv[mt][u][i] = ldg16(hp + (size_t)b * 32 + 4 * i);
      }
    }
  }

  __device__ __forceinline__ void load(int it, Regs& r) const {
    const int j = it / rgroups, rg = it - j * rgroups, e = meta->act[j];
    r.p0 = offsets[e];
    r.p1 = offsets[e + 1];
    load_blocks(e, rg, 0, r);
    load_h(r.p0, r.p1, 0, r);
  }

  __device__ __forceinline__ void compute(int it, Regs& r) const {
    const int lane = threadIdx.x & 63, nb = f >> 5;
    const int j = it / rgroups, rg = it - j * rgroups, e = meta->act[j];
    const int p0 = r.p0, p1 = r.p1;
    for (int p = p0; p < p1; p += MT) {
      float v[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = 0.0f;
      for (int b0 = 0; b0 < nb; b0 += kWave * NU) {
        if (b0 > 0) load_blocks(e, rg, b0, r);
        if (b0 > 0 || p > p0) load_h(p, p1, b0, r);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const bool ok = b0 + lane + kWave * u < nb;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if (p + mt >= p1) continue;
            XBlock<true> hb;
#pragma unroll
            for (int i = 0; i < 8; ++i) hb.v[i] = r.hv[mt][u][i];
#pragma unroll
            for (int i = 0; i < R; ++i) {
              const float t = __builtin_fmaf(hb.dot(r.q[u][i]), e8m0_to_f32(r.s[u][i]),
                                             v[i * MT + mt]);
              v[i * MT + mt] = ok ? t : v[i * MT + mt];
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      if (nb > kWave * NU && p + MT < p1) load_blocks(e, rg, 0, r);
      XReduce<NV, 32>::run(v, lane);
      constexpr int SH = 6 - ilog2(NV);
      const int idx = lane >> SH;
      if ((lane & ((1 << SH) - 1)) == 0) {
        const int i = idx / MT, mt = idx - i * MT;
        if (p + mt < p1) y[(size_t)(p + mt) * d + rg * R + i] = v[0];
      }
    }
  }
};

template <int R, int MT, int NU>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void down_persistent(DownOp<R, MT, NU> op, const int32_t* __restrict__ offsets, int E) {
  __shared__ Meta<0> meta;
  __shared__ int sums[256];
  stage_meta<0>(offsets, nullptr, E, 1, meta, sums);
  op.meta = &meta;
  walk_items_single(op, meta.n_act * op.rgroups);
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
  constexpr int NR = 2 * R, NV = NR * MT;
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int s = wid / rgroups, rg = wid - s * rgroups;
  if (s >= S) return;
  const int nc = d >> 3;
  const uint16_t* we = w13 + (size_t)s * 2 * fs * d;
  for (int t0 = 0; t0 < T; t0 += MT) {
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += kWave * NU) {
      uint4 wv[NU][NR];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int c = c0 + lane + kWave * u;
        if (c < nc)
#pragma unroll
          for (int i = 0; i < NR; ++i) {
            const size_t row = (size_t)(i < R ? rg * R + i : fs + rg * R + i - R);
            wv[u][i] = ldg16(we + row * d + (size_t)c * 8);
          }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int c = c0 + lane + kWave * u;
        if (c < nc)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (t0 + mt < T)
#pragma unroll
              for (int i = 0; i < NR; ++i)
                v[i * MT + mt] = chunk_dot<XF32>(wv[u][i], x, (size_t)(t0 + mt) * d + (size_t)c * 8,
                                                 v[i * MT + mt]);
      }
    }
    XReduce<NV, 32>::run(v, lane);
    const float uval = __shfl_xor(v[0], 32, kWave);
    constexpr int SH = 6 - ilog2(NV);
    const int idx = lane >> SH;
    if (lane < 32 && (lane & ((1 << SH) - 1)) == 0) {
      const int i = idx / MT, mt = idx - i * MT;
      if (t0 + mt < T) hs[((size_t)(t0 + mt) * S + s) * fs + rg * R + i] = silu_mul(v[0], uval);
    }
  }
}

// One token, shared experts' gate/up: one (expert, feature) item per wave.
__global__ __launch_bounds__(256) void shared_gateup_t1(const uint16_t* __restrict__ w13,
                                                        const uint16_t* __restrict__ x,
                                                        float* __restrict__ hs, int d, int fs,
                                                        int S) {
  __shared__ uint4 xs[kSgU * kWave];
  stage_row(reinterpret_cast<const uint4*>(x), d / 8, xs);
  __syncthreads();
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item < S * fs) shared_gateup_item(item, w13, xs, hs, d, fs, threadIdx.x & 63);
}

// One token, shared experts' down: each wave owns 2 output rows and, per lane,
// the 16-byte chunks c = lane + 64 u (u < 4) of every shared expert's rows,
// all loaded before any arithmetic.  Per (row, expert): fp32 fused
// multiply-adds over the lane's chunks in order, the fixed transposed
// butterfly over the wave, then the experts added in order.  Requires
// f_shared == 2048 (4 chunks of 8 per lane) and at most 2 shared experts.
// h (16 KB, the same for every wave) is staged once per workgroup in LDS:
// its loads go out first, then the weights', which stay in flight while h
// is written to LDS.  With the combine, lane s < k loads slot s's weight,
// position and routed outputs of the wave's rows beside the weights (not
// after the sums: two dependent round trips at the end of every wave), and
// the finishing lanes take them in slot order as combine_one does.
constexpr int kSdRows = 2, kSdU = 4, kSdMaxS = 2;
__global__ __launch_bounds__(256) void shared_down_t1(const uint16_t* __restrict__ w2,
                                                      const float* __restrict__ hs,
                                                      float* __restrict__ y, int d, int fs, int S,
                                                      CombineArgs comb) {
  constexpr int R = kSdRows, U = kSdU, MS = kSdMaxS;
  constexpr int HU = MS * U * kWave * 2 / 256;   // 16-byte units of h per thread
  static_assert(R == 2, "two rows per wave (lane groups 0 and 1 finish them)");
  __shared__ uint4 s_h[MS * U * kWave * 2];      // [expert][chunk c][2 halves]
  const int lane = threadIdx.x & 63;
  const int o0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  uint4 hv[HU];
#pragma unroll
  for (int q = 0; q < HU; ++q) {
    const int n = threadIdx.x + 256 * q, se = min(n / (U * kWave * 2), S - 1);
    hv[q] = ldg16(hs + (size_t)se * fs + (size_t)(n % (U * kWave * 2)) * 4);
  }
  const bool live = o0 < d;
  const int ob = live ? o0 : 0;
  float cw = 0.0f, cy[R];
  int cp = -1;
  const bool comb_lane = live && comb.y_perm && lane < comb.k;
  if (comb_lane) {
    cw = comb.topk_w[lane];
    cp = comb.pair_pos[lane];
  }
  uint4 wv[MS][R][U];
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const int sc = min(s, S - 1);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = lane + kWave * u;
#pragma unroll
      for (int i = 0; i < R; ++i)
        wv[s][i][u] = ldg16(w2 + ((size_t)sc * d + ob + i) * fs + (size_t)c * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
    cy[i] = comb_lane ? comb.y_perm[(size_t)(cp >= 0 ? cp : 0) * d + ob + i] : 0.0f;
#pragma unroll
  for (int q = 0; q < HU; ++q) s_h[threadIdx.x + 256 * q] = hv[q];
  __syncthreads();
  if (!live) return;
  float v[MS * R];
#pragma unroll
  for (int s = 0; s < MS; ++s)
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float a = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = lane + kWave * u;
        const uint4 ha = s_h[(s * U * kWave + c) * 2], hb = s_h[(s * U * kWave + c) * 2 + 1];
        const uint32_t ww[4] = {wv[s][i][u].x, wv[s][i][u].y, wv[s][i][u].z, wv[s][i][u].w};
        const float hh[8] = {__uint_as_float(ha.x), __uint_as_float(ha.y),
                             __uint_as_float(ha.z), __uint_as_float(ha.w),
                             __uint_as_float(hb.x), __uint_as_float(hb.y),
                             __uint_as_float(hb.z), __uint_as_float(hb.w)};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a = __builtin_fmaf(bf16_lo(ww[q]), hh[2 * q], a);
          a = __builtin_fmaf(bf16_hi(ww[q]), hh[2 * q + 1], a);
        }
      }
      v[s * R + i] = a;
    }
  XReduce<MS * R, 32>::run(v, lane);
  // lane group g = lane >> 4 holds total (s = g / R, row i = g % R)
  const int g = lane >> 4;
  float tot = v[0];
  // experts added in order: row i's total = t(s=0, i) + t(s=1, i)
  const float other = __shfl(tot, (lane + 16 * R) & 63, kWave);
  const float total = S > 1 ? tot + other : tot;
  if (comb.y_perm) {
    // the slots in order, as combine_one: skipped when the weight is 0 or
    // the pair was dropped
    float r[R];
#pragma unroll
    for (int i = 0; i < R; ++i) r[i] = total;
    for (int s = 0; s < comb.k; ++s) {
      const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cw), s));
      const int ps = __builtin_amdgcn_readlane(cp, s);
      if (ws != 0.0f && ps >= 0) {
#pragma unroll
        for (int i = 0; i < R; ++i)
          r[i] = __builtin_fmaf(ws, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cy[i]), s)),
                                r[i]);
      }
    }
    if ((lane & 15) == 0 && g < R) {
      const int o = o0 + g;
      const float rg = g == 0 ? r[0] : r[R - 1];
      if (comb.out_bf16) static_cast<uint16_t*>(comb.out)[o] = f32_to_bf16(rg);
      else static_cast<float*>(comb.out)[o] = rg;
    }
  } else if ((lane & 15) == 0 && g < R) {
    y[o0 + g] = total;
  }
}

// y[t][o] = sum over shared experts s in order of (sum_j W2[s][o][j] hs[t][s][j]).
template <int R, int MT, int NU>
__global__ __launch_bounds__(256) void gemv_down_bf16(const uint16_t* __restrict__ w2,
                                                      const float* __restrict__ hs,
                                                      float* __restrict__ y, int T, int d, int fs,
                                                      int S, int rgroups, CombineArgs comb) {
  constexpr int NV = R * MT;
  const int lane = threadIdx.x & 63;
  const int rg = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rg >= rgroups) return;
  const int nc = fs >> 3;
  const int o0 = rg * R;
  constexpr int SH = 6 - ilog2(NV);
  const int idx = lane >> SH;
  for (int t0 = 0; t0 < T; t0 += MT) {
    float tot = 0.0f;
    for (int s = 0; s < S; ++s) {
      const uint16_t* we = w2 + (size_t)s * d * fs;
      float v[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = 0.0f;
      for (int c0 = 0; c0 < nc; c0 += kWave * NU) {
        uint4 wv[NU][R];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int c = c0 + lane + kWave * u;
          if (c < nc)
#pragma unroll
            for (int i = 0; i < R; ++i) wv[u][i] = ldg16(we + (size_t)(o0 + i) * fs + (size_t)c * 8);
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int c = c0 + lane + kWave * u;
          if (c < nc)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              if (t0 + mt < T)
#pragma unroll
                for (int i = 0; i < R; ++i)
                  v[i * MT + mt] = chunk_dot<true>(wv[u][i], hs,
                                                   ((size_t)(t0 + mt) * S + s) * fs + (size_t)c * 8,
                                                   v[i * MT + mt]);
        }
      }
      XReduce<NV, 32>::run(v, lane);
      tot = (s == 0) ? v[0] : tot + v[0];   // lane keeps one (row, token) total
    }
    if ((lane & ((1 << SH) - 1)) == 0) {
      const int i = idx / MT, mt = idx - i * MT;
      if (t0 + mt < T) {
        const size_t oi = (size_t)(t0 + mt) * d + o0 + i;
        if (comb.y_perm) {
          const float v = combine_one(tot, comb.y_perm, comb.pair_pos, comb.topk_w, t0 + mt,
                                      comb.k, d, o0 + i);
          if (comb.out_bf16) static_cast<uint16_t*>(comb.out)[oi] = f32_to_bf16(v);
          else static_cast<float*>(comb.out)[oi] = v;
        } else {
          y[oi] = tot;
        }
      }
    }
  }
}

inline unsigned blocks_for_waves(int64_t waves) { return (unsigned)((waves + 3) / 4); }

inline int64_t max_active(const k3moe_shape& s) {
  const int64_t P = s.T * s.k;
  return P < s.E ? P : s.E;
}

// Persistent grid: enough workgroups for every item, at most `per_cu` per CU.
inline unsigned persistent_grid(int64_t items, int per_cu) {
  const int cus = cu_count();
  const int64_t cap = (int64_t)cus * per_cu;
  const int64_t need = (items + 3) / 4;
  return (unsigned)(need < cap ? (need > 0 ? need : 1) : cap);
}

template <int R, int MT, bool XF32, bool XLDS>
void gateup_launch(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                   const int32_t* offsets, const int32_t* sorted_pair, float* h, hipStream_t st) {
  constexpr int NU = 4;
  const int rg = s.f / R;
  const unsigned g = persistent_grid(max_active(s) * rg, 4);
  GateUpOp<R, MT, NU, XF32, XLDS> op{static_cast<const uint8_t*>(bank.w13),
                                     static_cast<const uint8_t*>(bank.w13_scale), x, sorted_pair,
                                     h, nullptr, nullptr, s.d, s.f, s.k, rg, offsets};
  const size_t lds = XLDS ? (size_t)s.d * (XF32 ? 4 : 2) : 0;
  gateup_persistent<<<g, 256, lds, st>>>(op, offsets, s.E);
}

template <int R, int MT>
void down_launch(const k3moe_shape& s, const k3moe_expert_bank& bank, const float* h,
                 const int32_t* offsets, float* y, hipStream_t st) {
  constexpr int NU = 1;
  const int rg = s.d / R;
  const unsigned g = persistent_grid(max_active(s) * rg, 4);
  DownOp<R, MT, NU> op{static_cast<const uint8_t*>(bank.w2),
                       static_cast<const uint8_t*>(bank.w2_scale), h, y, nullptr, s.d, s.f, rg,
                       offsets};
  down_persistent<<<g, 256, 0, st>>>(op, offsets, s.E);
}

}  // namespace

hipError_t launch_expert_gateup(const k3moe_shape& s, const k3moe_expert_bank& bank,
                                const void* x, const int32_t* offsets,
                                const int32_t* sorted_pair, float* h, const ExpertWs& ws,
                                hipStream_t st) {
  if (bank.format == K3MOE_FMT_RVQ3)
    return launch_gateup_rvq(s, bank, x, offsets, sorted_pair, h, ws.part, st);
  if (routed_scaled(s))
    return launch_gateup_scaled(s, bank, x, offsets, sorted_pair, h, ws.xq, st);
  // One token: its row is staged in LDS (up to 32 KB).  Items loop over their
  // expert's tokens one at a time with the weight rows held in registers.
  const bool f32 = s.x_dtype == K3MOE_F32;
  const size_t row_bytes = (size_t)s.d * (f32 ? 4 : 2);
  if (s.T == 1 && row_bytes <= 32768) {
    const unsigned g = persistent_grid((int64_t)s.k * s.f, 4);
    const uint8_t* w13 = static_cast<const uint8_t*>(bank.w13);
    const uint8_t* w13s = static_cast<const uint8_t*>(bank.w13_scale);
    if (f32) gateup_t1<true><<<g, 256, row_bytes, st>>>(w13, w13s, x, offsets, h, s.d, s.f, s.E);
    else gateup_t1<false><<<g, 256, row_bytes, st>>>(w13, w13s, x, offsets, h, s.d, s.f, s.E);
  } else if (f32) {
    gateup_launch<1, 1, true, false>(s, bank, x, offsets, sorted_pair, h, st);
  } else {
    gateup_launch<1, 1, false, false>(s, bank, x, offsets, sorted_pair, h, st);
  }
  return hipGetLastError();
}

hipError_t launch_expert_down(const k3moe_shape& s, const k3moe_expert_bank& bank, const float* h,
                              const int32_t* offsets, float* y, hipStream_t st) {
  if (routed_scaled(s)) return launch_down_scaled(s, bank, h, offsets, y, st);
  if (s.T == 1 && s.d % kDownT1Chunk == 0 && (size_t)s.f * 4 <= 32768) {
    const int chunks = s.d / kDownT1Chunk;
    const int cus = cu_count();
    const int64_t need = (int64_t)s.k * chunks, cap = (int64_t)cus * 8;
    const unsigned g = (unsigned)(need < cap ? need : cap);
    down_t1<<<g, 256, (size_t)s.f * 4, st>>>(static_cast<const uint8_t*>(bank.w2),
                                              static_cast<const uint8_t*>(bank.w2_scale), h,
                                              offsets, y, s.d, s.f, s.E);
  } else {
    down_launch<4, 1>(s, bank, h, offsets, y, st);
  }
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                             const int32_t* offsets, const int32_t* sorted_pair, float* y,
                             const ExpertWs& ws, hipStream_t st) {
  hipError_t err = launch_expert_gateup(s, bank, x, offsets, sorted_pair, ws.h, ws, st);
  if (err != hipSuccess) return err;
  if (bank.format == K3MOE_FMT_RVQ3) return launch_down_rvq(s, bank, ws.h, offsets, y, ws.part, st);
  return launch_expert_down(s, bank, ws.h, offsets, y, st);
}

hipError_t launch_shared_down_t1(const k3moe_shape& s, const k3moe_expert_bank& bank,
                                 const SharedWs& ws, float* y, hipStream_t st,
                                 const CombineArgs& comb) {
  const int S = bank.n_experts, fs = bank.f;
  if (s.T != 1 || fs != kSdU * 8 * kWave || S > kSdMaxS || s.d % (4 * kSdRows) != 0)
    return hipErrorInvalidValue;
  shared_down_t1<<<s.d / (4 * kSdRows), 256, 0, st>>>(static_cast<const uint16_t*>(bank.w2), ws.h,
                                                      y, s.d, fs, S, comb);
  return hipGetLastError();
}

bool shared_down_t1_ok(const k3moe_shape& s) {
  return s.T == 1 && s.f_shared == kSdU * 8 * kWave && s.n_shared <= kSdMaxS &&
         s.d % (4 * kSdRows) == 0;
}

hipError_t launch_shared_ffn(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                             float* y, const SharedWs& ws, hipStream_t st,
                             const CombineArgs& comb) {
  if (shared_mfma_ok(s)) return launch_shared_mfma(s, bank, x, ws.h, y, st, comb);
  constexpr int RG = 2, RD = 4;
  const int S = bank.n_experts, fs = bank.f, T = (int)s.T;
  const uint16_t* w13 = static_cast<const uint16_t*>(bank.w13);
  const uint16_t* w2 = static_cast<const uint16_t*>(bank.w2);
  const int rg_gu = fs / RG, rg_dn = s.d / RD;
  const unsigned g1 = blocks_for_waves((int64_t)S * rg_gu);
  const bool xf32 = s.x_dtype == K3MOE_F32;
  if (T == 1 && !xf32 && s.d == kSgU * 8 * kWave) {
    shared_gateup_t1<<<(S * fs + 3) / 4, 256, 0, st>>>(w13, static_cast<const uint16_t*>(x), ws.h,
                                                      s.d, fs, S);
  } else if (T == 1) {
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
  if (T == 1 && fs == kSdU * 8 * kWave && S <= kSdMaxS && s.d % (4 * kSdRows) == 0) {
    shared_down_t1<<<s.d / (4 * kSdRows), 256, 0, st>>>(w2, ws.h, y, s.d, fs, S, comb);
    return hipGetLastError();
  }
  const unsigned g2 = blocks_for_waves(rg_dn);
  if (T == 1)
    gemv_down_bf16<RD, 1, 2><<<g2, 256, 0, st>>>(w2, ws.h, y, T, s.d, fs, S, rg_dn, comb);
  else
    gemv_down_bf16<RD, 2, 2><<<g2, 256, 0, st>>>(w2, ws.h, y, T, s.d, fs, S, rg_dn, comb);
  return hipGetLastError();
}

}  // namespace k3
