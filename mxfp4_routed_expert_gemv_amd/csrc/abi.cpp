// C-ABI entry points of libk3moe: argument validation (host only, before any
// launch), workspace carving and dispatch to the kernel launchers.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>

#include "internal.h"

namespace k3 {

// One cache slot per device id; a slot is written with the same value by
// whichever thread gets there first, so concurrent first calls agree.
int cu_count() {
  constexpr int kSlots = 64;
  static std::atomic<int> cache[kSlots];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const int slot = dev < kSlots ? dev : kSlots - 1;
  int cus = dev < kSlots ? cache[slot].load(std::memory_order_relaxed) : 0;
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < kSlots) cache[slot].store(cus, std::memory_order_relaxed);
  return cus;
}

namespace {

thread_local std::string g_last_error;

k3moe_status fail(k3moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
k3moe_status fail(k3moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

k3moe_status ok() {
  g_last_error.clear();
  return K3MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define K3_CHECK(expr)                         \
  do {                                         \
    k3moe_status st_ = (expr);                 \
    if (st_ != K3MOE_OK) return st_;           \
  } while (0)

k3moe_status check_shape(const k3moe_shape* s) {
  if (!s) return fail(K3MOE_EINVAL, "shape is NULL");
  if (s->T < 0 || s->d < 0 || s->f < 0 || s->E < 0 || s->k < 0 || s->n_shared < 0 ||
      s->f_shared < 0)
    return fail(K3MOE_EINVAL, "negative size in shape");
  if (s->x_dtype != K3MOE_F32 && s->x_dtype != K3MOE_BF16)
    return fail(K3MOE_EUNSUPPORTED, "x_dtype %d is not F32 or BF16", s->x_dtype);
  if (s->out_dtype != K3MOE_F32 && s->out_dtype != K3MOE_BF16)
    return fail(K3MOE_EUNSUPPORTED, "out_dtype %d is not F32 or BF16", s->out_dtype);
  if (s->router != K3MOE_ROUTER_SOFTMAX && s->router != K3MOE_ROUTER_SIGMOID &&
      s->router != K3MOE_ROUTER_SIGMOID_NORM)
    return fail(K3MOE_EUNSUPPORTED, "router %d is not one of K3MOE_ROUTER_*", s->router);
  if (s->act != K3MOE_ACT_EXACT && s->act != K3MOE_ACT_MXFP4)
    return fail(K3MOE_EUNSUPPORTED, "act %d is not one of K3MOE_ACT_*", s->act);
  if (s->act == K3MOE_ACT_MXFP4 && !(s->x_dtype == K3MOE_BF16 && s->d % 512 == 0 &&
                                     s->f % 512 == 0))
    return fail(K3MOE_EUNSUPPORTED,
                "MXFP4 activations need bf16 x, d %% 512 == 0 and f %% 512 == 0");
  if (s->routed_format != K3MOE_FMT_MXFP4 && s->routed_format != K3MOE_FMT_RVQ3)
    return fail(K3MOE_EUNSUPPORTED, "routed_format %d is not MXFP4 or RVQ3", s->routed_format);
  if (s->routed_format == K3MOE_FMT_RVQ3 && (s->d % 128 || s->f % 128))
    return fail(K3MOE_ESHAPE, "RVQ3 experts need d %% 128 == 0 and f %% 128 == 0");
  if (s->routed_format == K3MOE_FMT_RVQ3 && s->act != K3MOE_ACT_EXACT)
    return fail(K3MOE_EUNSUPPORTED, "MXFP4 activations are for MXFP4 experts");
  if (s->d < 32 || s->d > 16384 || s->d % 32)
    return fail(K3MOE_ESHAPE, "d = %d: need 32 <= d <= 16384, d %% 32 == 0", s->d);
  if (s->f < 32 || s->f > 16384 || s->f % 32)
    return fail(K3MOE_ESHAPE, "f = %d: need 32 <= f <= 16384, f %% 32 == 0", s->f);
  if (s->E < 1 || s->E > 1024) return fail(K3MOE_ESHAPE, "E = %d: need 1 <= E <= 1024", s->E);
  if (s->k < 1 || s->k > 64 || s->k > s->E)
    return fail(K3MOE_ESHAPE, "k = %d: need 1 <= k <= min(E, 64)", s->k);
  if (s->n_shared > 8) return fail(K3MOE_ESHAPE, "n_shared = %d: need <= 8", s->n_shared);
  if (s->n_shared > 0 && (s->f_shared < 32 || s->f_shared > 16384 || s->f_shared % 32))
    return fail(K3MOE_ESHAPE, "f_shared = %d: need 32 <= f_shared <= 16384, %% 32 == 0",
                s->f_shared);
  if (s->T * (int64_t)s->k >= (int64_t(1) << 31))
    return fail(K3MOE_ESHAPE, "T * k = %lld: need < 2^31", (long long)(s->T * s->k));
  return K3MOE_OK;
}

k3moe_status need_ptr(const void* p, const char* name) {
  if (!p) return fail(K3MOE_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(K3MOE_EALIGN, "%s is not 16-byte aligned", name);
  return K3MOE_OK;
}

k3moe_status opt_ptr(const void* p, const char* name) {
  if (p && !aligned16(p)) return fail(K3MOE_EALIGN, "%s is not 16-byte aligned", name);
  return K3MOE_OK;
}

k3moe_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return K3MOE_OK;
  if (!ws) return fail(K3MOE_EWORKSPACE, "workspace is NULL; %zu bytes needed", need);
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(K3MOE_EALIGN, "workspace is not 256-byte aligned");
  if (have < need) return fail(K3MOE_EWORKSPACE, "workspace has %zu bytes; %zu needed", have, need);
  return K3MOE_OK;
}

k3moe_status check_routed_bank(const k3moe_shape& s, const k3moe_expert_bank* b) {
  if (!b) return fail(K3MOE_EINVAL, "expert bank is NULL");
  if (b->format != K3MOE_FMT_MXFP4 && b->format != K3MOE_FMT_RVQ3)
    return fail(K3MOE_EUNSUPPORTED, "routed experts must be MXFP4 or RVQ3 (format %d)",
                b->format);
  if (b->format != s.routed_format)
    return fail(K3MOE_EINVAL, "routed bank format %d differs from shape routed_format %d",
                b->format, s.routed_format);
  if (b->n_experts != s.E || b->d != s.d || b->f != s.f)
    return fail(K3MOE_EINVAL, "routed bank (n=%d, d=%d, f=%d) does not match shape (E=%d, d=%d, f=%d)",
                b->n_experts, b->d, b->f, s.E, s.d, s.f);
  K3_CHECK(need_ptr(b->w13, "routed.w13"));
  K3_CHECK(need_ptr(b->w13_scale, "routed.w13_scale"));
  K3_CHECK(need_ptr(b->w2, "routed.w2"));
  K3_CHECK(need_ptr(b->w2_scale, "routed.w2_scale"));
  return K3MOE_OK;
}

k3moe_status check_shared_bank(const k3moe_shape& s, const k3moe_expert_bank* b) {
  if (!b) return fail(K3MOE_EINVAL, "shared bank is NULL");
  if (b->format != K3MOE_FMT_BF16)
    return fail(K3MOE_EUNSUPPORTED, "shared experts must be BF16 (format %d)", b->format);
  if (b->n_experts != s.n_shared || b->d != s.d || b->f != s.f_shared)
    return fail(K3MOE_EINVAL, "shared bank (n=%d, d=%d, f=%d) does not match shape (n_shared=%d, d=%d, f_shared=%d)",
                b->n_experts, b->d, b->f, s.n_shared, s.d, s.f_shared);
  if (s.n_shared == 0) return K3MOE_OK;
  K3_CHECK(need_ptr(b->w13, "shared.w13"));
  K3_CHECK(need_ptr(b->w2, "shared.w2"));
  return K3MOE_OK;
}

k3moe_status check_bias(const k3moe_shape& s, const float* bias) {
  if (bias && s.router == K3MOE_ROUTER_SOFTMAX)
    return fail(K3MOE_EINVAL, "router_bias is given but the softmax router takes none");
  return opt_ptr(bias, "router_bias");
}

k3moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(K3MOE_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

}  // namespace

// ----------------------------------------------------------------- workspace
RouteWs carve_route(const k3moe_shape& s, void* ws, size_t* bytes) {
  Carver c(ws);
  RouteWs r;
  r.logits = c.take<double>((size_t)s.T * s.E);
  r.lbound = c.take<float>((size_t)s.T * s.E);
  r.wnorm = use_mfma(s) ? c.take<float>((size_t)s.E) : nullptr;
  if (bytes) *bytes = c.off;
  return r;
}

PermuteWs carve_permute(const k3moe_shape& s, void* ws, size_t* bytes) {
  Carver c(ws);
  PermuteWs r;
  const int ch = permute_chunk_tokens(s.k);
  const size_t nchunks = (size_t)((s.T + ch - 1) / ch);
  r.chunk_base = c.take<int32_t>(nchunks * s.E);
  if (bytes) *bytes = c.off;
  return r;
}

ExpertWs carve_gateup(const k3moe_shape& s, void* ws, size_t* bytes) {
  Carver c(ws);
  ExpertWs r;
  r.h = nullptr;
  r.xq = routed_scaled(s) ? c.take<uint8_t>(xq_bytes(s)) : nullptr;
  r.part = s.routed_format == K3MOE_FMT_RVQ3 ? c.take<float>(rvq_part_floats(s)) : nullptr;
  if (bytes) *bytes = c.off;
  return r;
}

ExpertWs carve_expert(const k3moe_shape& s, void* ws, size_t* bytes) {
  Carver c(ws);
  ExpertWs r;
  r.h = c.take<float>((size_t)s.T * s.k * s.f);
  r.xq = routed_scaled(s) ? c.take<uint8_t>(xq_bytes(s)) : nullptr;
  r.part = s.routed_format == K3MOE_FMT_RVQ3 ? c.take<float>(rvq_part_floats(s)) : nullptr;
  if (bytes) *bytes = c.off;
  return r;
}

SharedWs carve_shared(const k3moe_shape& s, void* ws, size_t* bytes) {
  Carver c(ws);
  SharedWs r;
  r.h = c.take<float>((size_t)s.T * s.n_shared * s.f_shared);
  if (bytes) *bytes = c.off;
  return r;
}

LayerWs carve_layer(const k3moe_shape& s, void* ws, size_t* bytes) {
  Carver c(ws);
  LayerWs r;
  const size_t P = (size_t)s.T * s.k;
  r.topk_idx = c.take<int32_t>(P);
  r.topk_w = c.take<float>(P);
  r.counts = c.take<int32_t>(s.E);
  r.offsets = c.take<int32_t>((size_t)s.E + 1);
  r.sorted_pair = c.take<int32_t>(P);
  r.pair_pos = c.take<int32_t>(P);
  r.y_perm = c.take<float>(P * s.d);
  r.shared_y = s.n_shared > 0 ? c.take<float>((size_t)s.T * s.d) : nullptr;
  r.shared_h = s.n_shared > 0 ? carve_shared(s, c.base ? c.base + c.off : nullptr, nullptr).h
                              : nullptr;
  if (s.n_shared > 0) {
    size_t sh = 0;
    carve_shared(s, nullptr, &sh);
    c.off += sh;
  }
  size_t a = 0, b = 0, e = 0;
  carve_route(s, nullptr, &a);
  carve_permute(s, nullptr, &b);
  carve_expert(s, nullptr, &e);
  size_t m = a;
  if (b > m) m = b;
  if (e > m) m = e;
  r.scratch_bytes = m;
  r.scratch = c.take<char>(m);
  if (bytes) *bytes = c.off;
  return r;
}

// Validation of a whole-layer call, before anything is enqueued; *need
// receives the workspace bytes (0 for an empty batch).
k3moe_status layer_validate(const k3moe_shape* shape, const k3moe_layer_weights* weights,
                            const void* x, const void* out, const int32_t* diag, size_t* need) {
  *need = 0;
  K3_CHECK(check_shape(shape));
  const k3moe_shape& s = *shape;
  if (!weights) return fail(K3MOE_EINVAL, "weights is NULL");
  K3_CHECK(check_routed_bank(s, &weights->routed));
  K3_CHECK(check_shared_bank(s, &weights->shared));
  if (s.T == 0) return ok();
  K3_CHECK(need_ptr(weights->w_router, "w_router"));
  K3_CHECK(check_bias(s, weights->router_bias));
  K3_CHECK(need_ptr(x, "x"));
  K3_CHECK(need_ptr(out, "out"));
  K3_CHECK(opt_ptr(diag, "diag"));
  carve_layer(s, nullptr, need);
  return K3MOE_OK;
}

k3moe_status hip_failure(hipError_t e, const char* what) { return hip_status(e, what); }
k3moe_status shape_status(const k3moe_shape* shape) { return check_shape(shape); }
k3moe_status fail_status(k3moe_status st, const char* msg) { return fail(st, "%s", msg); }

k3moe_status workspace_too_small(size_t have, size_t need) {
  return fail(K3MOE_EWORKSPACE, "the call needs %zu bytes of workspace; %zu are available", need,
              have);
}

// The layer's stages on a validated call, with a workspace of at least
// k3moe_workspace_bytes(shape, K3MOE_OP_LAYER) bytes.
k3moe_status layer_run(const k3moe_shape& s, const k3moe_layer_weights& wts, const void* x,
                       void* out, int32_t* diag, void* workspace, hipStream_t st) {
  const k3moe_layer_weights* weights = &wts;
  const LayerWs L = carve_layer(s, workspace, nullptr);
  if (topk_shared_t1_ok(s) && shared_down_t1_ok(s)) {
    // One token: router logits; then the selection (which also writes the
    // permutation) beside the shared experts' gate/up; the routed experts;
    // the shared experts' down finishing each output with the combine.
    const RouteWs rws = carve_route(s, L.scratch, nullptr);
    PermOut perm;
    perm.counts = L.counts;
    perm.offsets = L.offsets;
    perm.sorted_pair = L.sorted_pair;
    perm.pair_pos = L.pair_pos;
    SharedWs sws;
    sws.h = L.shared_h;
    hipError_t e = launch_router_logits(s, x, static_cast<const uint16_t*>(weights->w_router),
                                        rws, st);
    if (e != hipSuccess) return hip_status(e, "k3moe_layer router");
    e = launch_topk_shared_t1(s, x, static_cast<const uint16_t*>(weights->w_router),
                              weights->router_bias, L.topk_idx, L.topk_w, diag, rws, perm,
                              weights->shared, sws.h, st);
    if (e != hipSuccess) return hip_status(e, "k3moe_layer top-k + shared gate/up");
    e = launch_expert_ffn(s, weights->routed, x, L.offsets, L.sorted_pair, L.y_perm,
                          carve_expert(s, L.scratch, nullptr), st);
    if (e != hipSuccess) return hip_status(e, "k3moe_layer routed experts");
    CombineArgs comb;
    comb.y_perm = L.y_perm;
    comb.pair_pos = L.pair_pos;
    comb.topk_w = L.topk_w;
    comb.out = out;
    comb.k = s.k;
    comb.out_bf16 = s.out_dtype == K3MOE_BF16;
    e = launch_shared_down_t1(s, weights->shared, sws, L.shared_y, st, comb);
    return hip_status(e, "k3moe_layer shared down + combine");
  }
  // One token: the top-k kernel also writes the (trivial) permutation.
  PermOut perm;
  if (s.T == 1) {
    perm.counts = L.counts;
    perm.offsets = L.offsets;
    perm.sorted_pair = L.sorted_pair;
    perm.pair_pos = L.pair_pos;
  }
  hipError_t e = launch_route(s, x, static_cast<const uint16_t*>(weights->w_router),
                              weights->router_bias, L.topk_idx, L.topk_w, nullptr, diag,
                              carve_route(s, L.scratch, nullptr), st, perm);
  if (e != hipSuccess) return hip_status(e, "k3moe_layer route");
  if (s.T != 1) {
    e = launch_permute(s, L.topk_idx, L.counts, L.offsets, L.sorted_pair, L.pair_pos, diag,
                       carve_permute(s, L.scratch, nullptr), st);
    if (e != hipSuccess) return hip_status(e, "k3moe_layer permute");
  }
  e = launch_expert_ffn(s, weights->routed, x, L.offsets, L.sorted_pair, L.y_perm,
                        carve_expert(s, L.scratch, nullptr), st);
  if (e != hipSuccess) return hip_status(e, "k3moe_layer routed experts");
  if (s.n_shared > 0 && !shared_mfma_ok(s)) {
    // the shared experts' down GEMV finishes each output with the combine
    CombineArgs comb;
    comb.y_perm = L.y_perm;
    comb.pair_pos = L.pair_pos;
    comb.topk_w = L.topk_w;
    comb.out = out;
    comb.k = s.k;
    comb.out_bf16 = s.out_dtype == K3MOE_BF16;
    SharedWs sws;
    sws.h = L.shared_h;
    e = launch_shared_ffn(s, weights->shared, x, L.shared_y, sws, st, comb);
    return hip_status(e, "k3moe_layer shared experts + combine");
  }
  if (s.n_shared > 0) {
    SharedWs sws;
    sws.h = L.shared_h;
    e = launch_shared_ffn(s, weights->shared, x, L.shared_y, sws, st);
    if (e != hipSuccess) return hip_status(e, "k3moe_layer shared experts");
  }
  e = launch_combine(s, L.y_perm, L.pair_pos, L.topk_w, s.n_shared > 0 ? L.shared_y : nullptr,
                     out, st);
  return hip_status(e, "k3moe_layer combine");
}

}  // namespace k3

using namespace k3;

extern "C" {

size_t k3moe_workspace_bytes(const k3moe_shape* shape, int op) {
  if (check_shape(shape) != K3MOE_OK) return 0;
  if (shape->T == 0) return 0;
  size_t n = 0;
  switch (op) {
    case K3MOE_OP_ROUTE: carve_route(*shape, nullptr, &n); break;
    case K3MOE_OP_PERMUTE: carve_permute(*shape, nullptr, &n); break;
    case K3MOE_OP_EXPERT_FFN: carve_expert(*shape, nullptr, &n); break;
    case K3MOE_OP_EXPERT_GATEUP: carve_gateup(*shape, nullptr, &n); break;
    case K3MOE_OP_SHARED_FFN: carve_shared(*shape, nullptr, &n); break;
    case K3MOE_OP_COMBINE: n = 0; break;
    case K3MOE_OP_LAYER: carve_layer(*shape, nullptr, &n); break;
    default: return 0;
  }
  return n;
}

uint64_t k3moe_mxfp4_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return (uint64_t)rows * (uint64_t)cols * 17u / 32u;
}

int k3moe_path_class(const k3moe_shape* shape) {
  if (check_shape(shape) != K3MOE_OK) return K3MOE_PATH_GEMV;
  return use_mfma(*shape) ? K3MOE_PATH_MFMA : K3MOE_PATH_GEMV;
}

k3moe_status k3moe_route(const k3moe_shape* shape, const void* x, const void* w_router,
                         const float* router_bias, int32_t* topk_idx, float* topk_w,
                         float* logits, int32_t* diag, void* workspace, size_t workspace_bytes,
                         void* stream) {
  K3_CHECK(check_shape(shape));
  const k3moe_shape& s = *shape;
  if (s.T == 0) return ok();
  K3_CHECK(need_ptr(x, "x"));
  K3_CHECK(need_ptr(w_router, "w_router"));
  K3_CHECK(check_bias(s, router_bias));
  K3_CHECK(need_ptr(topk_idx, "topk_idx"));
  K3_CHECK(need_ptr(topk_w, "topk_w"));
  K3_CHECK(opt_ptr(logits, "logits"));
  K3_CHECK(opt_ptr(diag, "diag"));
  size_t need = 0;
  carve_route(s, nullptr, &need);
  K3_CHECK(check_ws(workspace, workspace_bytes, need));
  const RouteWs ws = carve_route(s, workspace, nullptr);
  return hip_status(launch_route(s, x, static_cast<const uint16_t*>(w_router), router_bias,
                                 topk_idx, topk_w,
                                 logits, diag, ws, static_cast<hipStream_t>(stream)),
                    "k3moe_route launch");
}

k3moe_status k3moe_permute(const k3moe_shape* shape, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                           int32_t* diag, void* workspace, size_t workspace_bytes, void* stream) {
  K3_CHECK(check_shape(shape));
  const k3moe_shape& s = *shape;
  if (s.T == 0) return ok();
  K3_CHECK(need_ptr(topk_idx, "topk_idx"));
  K3_CHECK(need_ptr(counts, "counts"));
  K3_CHECK(need_ptr(offsets, "offsets"));
  K3_CHECK(need_ptr(sorted_pair, "sorted_pair"));
  K3_CHECK(need_ptr(pair_pos, "pair_pos"));
  K3_CHECK(opt_ptr(diag, "diag"));
  size_t need = 0;
  carve_permute(s, nullptr, &need);
  K3_CHECK(check_ws(workspace, workspace_bytes, need));
  const PermuteWs ws = carve_permute(s, workspace, nullptr);
  return hip_status(launch_permute(s, topk_idx, counts, offsets, sorted_pair, pair_pos, diag, ws,
                                   static_cast<hipStream_t>(stream)),
                    "k3moe_permute launch");
}

k3moe_status k3moe_expert_ffn(const k3moe_shape* shape, const k3moe_expert_bank* bank,
                              const void* x, const int32_t* offsets, const int32_t* sorted_pair,
                              float* y, void* workspace, size_t workspace_bytes, void* stream) {
  K3_CHECK(check_shape(shape));
  const k3moe_shape& s = *shape;
  if (!bank) return fail(K3MOE_EINVAL, "expert bank is NULL");
  if (bank->format == K3MOE_FMT_BF16) {
    // shared mode: every token through every expert of the bank, summed in order
    if (sorted_pair)
      return fail(K3MOE_EUNSUPPORTED, "a BF16 bank takes no sorted_pair (shared mode)");
    return k3moe_shared_ffn(shape, bank, x, y, workspace, workspace_bytes, stream);
  }
  K3_CHECK(check_routed_bank(s, bank));
  if (!sorted_pair)
    return fail(K3MOE_EUNSUPPORTED, "an MXFP4 bank needs sorted_pair (routed mode)");
  if (s.T == 0) return ok();
  K3_CHECK(need_ptr(x, "x"));
  K3_CHECK(need_ptr(offsets, "offsets"));
  K3_CHECK(need_ptr(sorted_pair, "sorted_pair"));
  K3_CHECK(need_ptr(y, "y"));
  size_t need = 0;
  carve_expert(s, nullptr, &need);
  K3_CHECK(check_ws(workspace, workspace_bytes, need));
  const ExpertWs ws = carve_expert(s, workspace, nullptr);
  return hip_status(launch_expert_ffn(s, *bank, x, offsets, sorted_pair, y, ws,
                                      static_cast<hipStream_t>(stream)),
                    "k3moe_expert_ffn launch");
}

k3moe_status k3moe_expert_gateup(const k3moe_shape* shape, const k3moe_expert_bank* bank,
                                 const void* x, const int32_t* offsets,
                                 const int32_t* sorted_pair, float* h, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  K3_CHECK(check_shape(shape));
  const k3moe_shape& s = *shape;
  K3_CHECK(check_routed_bank(s, bank));
  if (s.T == 0) return ok();
  K3_CHECK(need_ptr(x, "x"));
  K3_CHECK(need_ptr(offsets, "offsets"));
  K3_CHECK(need_ptr(sorted_pair, "sorted_pair"));
  K3_CHECK(need_ptr(h, "h"));
  size_t need = 0;
  carve_gateup(s, nullptr, &need);
  K3_CHECK(check_ws(workspace, workspace_bytes, need));
  const ExpertWs ws = carve_gateup(s, workspace, nullptr);
  return hip_status(launch_expert_gateup(s, *bank, x, offsets, sorted_pair, h, ws,
                                         static_cast<hipStream_t>(stream)),
                    "k3moe_expert_gateup launch");
}

k3moe_status k3moe_expert_down(const k3moe_shape* shape, const k3moe_expert_bank* bank,
                               const float* h, const int32_t* offsets, float* y, void* stream) {
  K3_CHECK(check_shape(shape));
  const k3moe_shape& s = *shape;
  K3_CHECK(check_routed_bank(s, bank));
  if (bank->format == K3MOE_FMT_RVQ3)
    return fail(K3MOE_EUNSUPPORTED,
                "the RVQ3 down product needs a workspace: use k3moe_expert_ffn");
  if (s.T == 0) return ok();
  K3_CHECK(need_ptr(h, "h"));
  K3_CHECK(need_ptr(offsets, "offsets"));
  K3_CHECK(need_ptr(y, "y"));
  return hip_status(launch_expert_down(s, *bank, h, offsets, y, static_cast<hipStream_t>(stream)),
                    "k3moe_expert_down launch");
}

k3moe_status k3moe_shared_ffn(const k3moe_shape* shape, const k3moe_expert_bank* bank,
                              const void* x, float* y, void* workspace, size_t workspace_bytes,
                              void* stream) {
  K3_CHECK(check_shape(shape));
  const k3moe_shape& s = *shape;
  K3_CHECK(check_shared_bank(s, bank));
  if (s.n_shared == 0) return fail(K3MOE_EINVAL, "shape has no shared experts");
  if (s.T == 0) return ok();
  K3_CHECK(need_ptr(x, "x"));
  K3_CHECK(need_ptr(y, "y"));
  size_t need = 0;
  carve_shared(s, nullptr, &need);
  K3_CHECK(check_ws(workspace, workspace_bytes, need));
  const SharedWs ws = carve_shared(s, workspace, nullptr);
  return hip_status(launch_shared_ffn(s, *bank, x, y, ws, static_cast<hipStream_t>(stream)),
                    "k3moe_shared_ffn launch");
}

k3moe_status k3moe_combine(const k3moe_shape* shape, const float* y_perm, const int32_t* pair_pos,
                           const float* topk_w, const float* shared_y, void* out, void* stream) {
  K3_CHECK(check_shape(shape));
  const k3moe_shape& s = *shape;
  if (s.T == 0) return ok();
  K3_CHECK(need_ptr(y_perm, "y_perm"));
  K3_CHECK(need_ptr(pair_pos, "pair_pos"));
  K3_CHECK(need_ptr(topk_w, "topk_w"));
  K3_CHECK(opt_ptr(shared_y, "shared_y"));
  K3_CHECK(need_ptr(out, "out"));
  return hip_status(launch_combine(s, y_perm, pair_pos, topk_w, shared_y, out,
                                   static_cast<hipStream_t>(stream)),
                    "k3moe_combine launch");
}

k3moe_status k3moe_layer(const k3moe_shape* shape, const k3moe_layer_weights* weights,
                         const void* x, void* out, int32_t* diag, void* workspace,
                         size_t workspace_bytes, void* stream) {
  size_t need = 0;
  K3_CHECK(layer_validate(shape, weights, x, out, diag, &need));
  if (shape->T == 0) return ok();
  K3_CHECK(check_ws(workspace, workspace_bytes, need));
  return layer_run(*shape, *weights, x, out, diag, workspace, static_cast<hipStream_t>(stream));
}

const char* k3moe_status_str(k3moe_status status) {
  switch (status) {
    case K3MOE_OK: return "ok";
    case K3MOE_EINVAL: return "invalid argument";
    case K3MOE_ESHAPE: return "unsupported shape";
    case K3MOE_EALIGN: return "misaligned pointer";
    case K3MOE_EWORKSPACE: return "workspace missing or too small";
    case K3MOE_EUNSUPPORTED: return "unsupported dtype or weight format";
    case K3MOE_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* k3moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
