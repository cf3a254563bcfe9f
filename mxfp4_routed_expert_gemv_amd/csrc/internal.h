// Host-side internal interface of libk3moe: kernel launchers (implemented in
// the .hip files) and the workspace layout shared by the entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/k3moe.h"

namespace k3 {

// Smallest token count that takes the matrix-core (MFMA) path class; the
// class also needs bf16 activations, d % 512 == 0 and f % 512 == 0.
constexpr int64_t kMfmaMinT = 32;
bool mfma_shape_ok(const k3moe_shape& s);
inline bool use_mfma(const k3moe_shape& s) { return s.T >= kMfmaMinT && mfma_shape_ok(s); }
// The routed experts run on the scaled-MXFP4 matrix-core instruction at any
// token count when the shape allows it (one token included: the instruction
// takes the stored E2M1 bytes as they are, which leaves the vector ALU free),
// so a token's routed outputs do not depend on the batch size at all there.
inline bool routed_scaled(const k3moe_shape& s) {
  return mfma_shape_ok(s) && s.routed_format == K3MOE_FMT_MXFP4;
}
// Tokens per chunk of the large-batch permute (one bit per token in LDS masks).
int permute_chunk_tokens(int k);

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Carves a workspace into 256-byte aligned pieces (or only sums their sizes
// when base is NULL).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align256(count * sizeof(T));
    return p;
  }
};

struct RouteWs {
  double* logits;   // [T][E] fp64
  float* lbound;    // [T][E] bound on |logit - exact fp64 sequential logit|
  float* wnorm;     // [E] |w_e| (matrix-core class: the bf16 logits' bounds); else nullptr
};
struct PermuteWs {
  int32_t* chunk_base;  // [nchunks][E]
};
struct ExpertWs {
  float* h;           // [P][f] 32-bit words (GEMV class: fp32 h; MFMA class: h in passes)
  uint8_t* xq;        // MFMA class: x in E4M3 passes, xq_bytes(s); else nullptr
  float* part;        // RVQ3 experts: slice partial sums, rvq_part_floats(s); else nullptr
};
// Floats of the RVQ3 experts' slice partial sums (the larger of gate/up and down).
size_t rvq_part_floats(const k3moe_shape& s);
// Bytes of the quantised activations of the MFMA class (0 in the GEMV class).
size_t xq_bytes(const k3moe_shape& s);
ExpertWs carve_gateup(const k3moe_shape& s, void* ws, size_t* bytes);
struct SharedWs {
  float* h;           // [T][n_shared][f_shared]
};
struct LayerWs {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_pos;
  float* y_perm;
  float* shared_y;
  float* shared_h;    // [T][n_shared][f_shared], live from the shared gate/up to its down
  void* scratch;      // route, permute and routed-expert workspaces (stages run in order)
  size_t scratch_bytes;
};

RouteWs carve_route(const k3moe_shape& s, void* ws, size_t* bytes);
PermuteWs carve_permute(const k3moe_shape& s, void* ws, size_t* bytes);
ExpertWs carve_expert(const k3moe_shape& s, void* ws, size_t* bytes);
SharedWs carve_shared(const k3moe_shape& s, void* ws, size_t* bytes);
LayerWs carve_layer(const k3moe_shape& s, void* ws, size_t* bytes);

// Outputs of k3moe_permute, written by the top-k kernel itself when the
// batch is one token (its ids, already in ascending order, are the sorted
// order); counts == nullptr means "not requested".
struct PermOut {
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* sorted_pair = nullptr;
  int32_t* pair_pos = nullptr;
};
// The combine folded into the shared experts' down kernel: its fp32 result
// for (t, o) takes the place of shared_y[t][o] and the routed terms follow in
// the same order as in the combine kernel (same bits).  y_perm == nullptr
// means "not requested".
struct CombineArgs {
  const float* y_perm = nullptr;
  const int32_t* pair_pos = nullptr;
  const float* topk_w = nullptr;
  void* out = nullptr;
  int k = 0;
  bool out_bf16 = false;
};

// Launchers: enqueue on `st`, return hipSuccess or the launch error.
hipError_t launch_route(const k3moe_shape& s, const void* x, const uint16_t* wr, const float* bias,
                        int32_t* idx, float* w, float* logits_out, int32_t* diag,
                        const RouteWs& ws, hipStream_t st, const PermOut& perm = PermOut());
// The two halves of launch_route, and the one-token selection fused with the
// shared experts' gate/up (which writes SharedWs::h).
hipError_t launch_router_logits(const k3moe_shape& s, const void* x, const uint16_t* wr,
                                const RouteWs& ws, hipStream_t st);
bool topk_shared_t1_ok(const k3moe_shape& s);
hipError_t launch_topk_shared_t1(const k3moe_shape& s, const void* x, const uint16_t* wr,
                                 const float* bias, int32_t* idx, float* w, int32_t* diag,
                                 const RouteWs& ws, const PermOut& perm,
                                 const k3moe_expert_bank& shared, float* hs, hipStream_t st);
bool shared_down_t1_ok(const k3moe_shape& s);
hipError_t launch_shared_down_t1(const k3moe_shape& s, const k3moe_expert_bank& bank,
                                 const SharedWs& ws, float* y, hipStream_t st,
                                 const CombineArgs& comb);
hipError_t launch_permute(const k3moe_shape& s, const int32_t* idx, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                          int32_t* diag, const PermuteWs& ws, hipStream_t st);
hipError_t launch_expert_gateup(const k3moe_shape& s, const k3moe_expert_bank& bank,
                                const void* x, const int32_t* offsets,
                                const int32_t* sorted_pair, float* h, const ExpertWs& ws,
                                hipStream_t st);
// RVQ3 experts: table-based gate/up (+ SiLU-GLU, h fp32) and down.
hipError_t launch_gateup_rvq(const k3moe_shape& s, const k3moe_expert_bank& b, const void* x,
                             const int32_t* offsets, const int32_t* sorted_pair, float* h,
                             float* part, hipStream_t st);
hipError_t launch_down_rvq(const k3moe_shape& s, const k3moe_expert_bank& b, const float* h,
                           const int32_t* offsets, float* y, float* part, hipStream_t st);
hipError_t launch_expert_down(const k3moe_shape& s, const k3moe_expert_bank& bank, const float* h,
                              const int32_t* offsets, float* y, hipStream_t st);
// Scaled-MXFP4 matrix-core path (MFMA class): x quantisation + gate/up, down.
hipError_t launch_gateup_scaled(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                                const int32_t* offsets, const int32_t* sorted_pair, float* h,
                                uint8_t* xq, hipStream_t st);
hipError_t launch_down_scaled(const k3moe_shape& s, const k3moe_expert_bank& bank, const float* h,
                              const int32_t* offsets, float* y, hipStream_t st);
// Compute units of the current device (queried once per device and cached;
// safe to call from several threads at once).
int cu_count();
// Persistent grid of one workgroup per CU, rounded up to a multiple of the 8
// XCDs (the item split of the grouped kernels gives each XCD one contiguous
// range): the routed grouped GEMMs and the shared experts' LDS-ring GEMMs.
int grouped_grid();
// The m-tile height (in 16-row blocks) of the routed grouped GEMMs for a batch.
int pick_mf(const k3moe_shape& s, int max_mf);
bool shared_mfma_ok(const k3moe_shape& s);
// The shared experts' GEMMs with both operands staged through LDS rings
// (shared_gemm.hip), for the matrix-core class beyond the small-batch
// kernels; h then holds two bf16 planes (hi, lo) in the same bytes.
bool shared_lds_ok(const k3moe_shape& s);
hipError_t launch_shared_lds(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                             float* h, float* y, hipStream_t st);
// The router's fp32 logits [T][E] on the same LDS-ring GEMM (d % 64 == 0).
hipError_t launch_router_logits_lds(const uint16_t* x, const uint16_t* wr, float* l, int T, int d,
                                    int E, hipStream_t st);
hipError_t launch_shared_mfma(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                              float* h, float* y, hipStream_t st, const CombineArgs& comb);
hipError_t launch_expert_ffn(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                             const int32_t* offsets, const int32_t* sorted_pair, float* y,
                             const ExpertWs& ws, hipStream_t st);
hipError_t launch_shared_ffn(const k3moe_shape& s, const k3moe_expert_bank& bank, const void* x,
                             float* y, const SharedWs& ws, hipStream_t st,
                             const CombineArgs& comb = CombineArgs());
hipError_t launch_combine(const k3moe_shape& s, const float* y_perm, const int32_t* pair_pos,
                          const float* topk_w, const float* shared_y, void* out, hipStream_t st);

// Whole-layer entry points: the host-side validation (nothing enqueued; *need
// = workspace bytes, 0 for an empty batch), the status of a workspace that is
// too small, and the stages of a validated call on a workspace of at least
// *need bytes.
k3moe_status layer_validate(const k3moe_shape* shape, const k3moe_layer_weights* weights,
                            const void* x, const void* out, const int32_t* diag, size_t* need);
k3moe_status workspace_too_small(size_t have, size_t need);
// K3MOE_EHIP with the HIP error's text as the last error.
k3moe_status hip_failure(hipError_t e, const char* what);
// The shape checks of every entry point; a status with `msg` as the last error.
k3moe_status shape_status(const k3moe_shape* shape);
k3moe_status fail_status(k3moe_status st, const char* msg);
k3moe_status layer_run(const k3moe_shape& s, const k3moe_layer_weights& weights, const void* x,
                       void* out, int32_t* diag, void* workspace, hipStream_t st);

}  // namespace k3
