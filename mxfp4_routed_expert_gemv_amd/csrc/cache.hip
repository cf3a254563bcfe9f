// Host-resident routed experts streamed into an HBM expert cache.
//
// The pages' engines keep the routed experts on disk and the hot ones in an
// LRU cache in RAM whose size is a dial: the same weights, the same top-16
// and the same outputs at every budget (kimi-k3-in-c review page, "at a
// glance" list and the memory-ladder discussion; explainer page, "le cache
// LRU").  WASTE issues an expert's read as soon as the router names it and
// computes on experts as they arrive, and runs the next layer's router one
// residual early to prefetch (WASTE article page, section "속도는 어디서
// 나왔나").  Retargeted to one MI355X: the experts live in pinned host
// memory, the cache is a bank of `slots` expert slots in HBM, and a call
//   1. routes the batch on the GPU and brings the expert ids to the host
//      (one synchronisation of the compute stream);
//   2. plans on the host: every distinct id is a hit (its slot is touched)
//      or a miss (the least recently used slot that this batch does not use
//      is evicted and refilled by four host-to-device copies on the copy
//      stream);
//   3. runs the shared experts on the compute stream while the copies fly,
//      then waits for them (an event), maps ids to slot ids, and runs the
//      permute, routed experts and combine of the resident layer on the slot
//      bank.  Every kernel and every order is the resident layer's, so the
//      outputs are the same bits at every cache size.
// Prefetch inserts experts (copied on the copy stream) without using them;
// a later call that routes to one counts a prefetch hit.
#include <mutex>
#include <string.h>
#include <vector>

#include "internal.h"

namespace k3 {
namespace {

// ids [n] -> slot ids [n] through map [E]: every id of a routed batch in
// [0, E) maps to a resident slot; an id outside stays outside (-1), to be
// dropped by the permute as the layer drops it.
__global__ __launch_bounds__(256) void remap_ids(const int32_t* __restrict__ ids,
                                                 const int32_t* __restrict__ map,
                                                 int32_t* __restrict__ out, int64_t n, int E) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int id = ids[i];
  out[i] = (id >= 0 && id < E) ? map[id] : -1;
}

}  // namespace
}  // namespace k3

struct k3moe_expert_cache {
  k3moe_shape shape;               // the layer shape the cache serves (T ignored)
  k3moe_expert_bank host;          // pinned host bank, n_experts = E
  k3moe_expert_bank slots;         // device bank, n_experts = number of slots
  std::vector<int32_t> slot_of;    // [E]: slot of a resident expert, or -1
  std::vector<int32_t> expert_in;  // [slots]: expert held, or -1
  std::vector<int64_t> last_use;   // [slots]: tick of the last use (0 = never)
  std::vector<uint8_t> prefetched; // [slots]: filled by a prefetch and not used since
  std::vector<int32_t> pinned;     // [slots]: tick of the batch that needs it now
  int64_t tick = 0;
  k3moe_cache_stats stats{};
  hipEvent_t copies_done = nullptr;  // the last expert copies enqueued (layer or prefetch)
  hipEvent_t reads_done = nullptr;   // the last layer call's kernels
  bool copies_recorded = false;
  bool reads_recorded = false;
  std::vector<int32_t> ids_host;   // routed ids of the current batch
  std::vector<int32_t> map_host;   // expert -> slot for the current batch
  std::mutex lock;                 // one call at a time per cache
};

namespace k3 {
namespace {

size_t bank_bytes_per_expert(const k3moe_shape& s, int which) {
  // which: 0 w13 codes, 1 w13 scales, 2 w2 codes, 3 w2 scales
  switch (which) {
    case 0: return (size_t)2 * s.f * s.d / 2;
    case 1: return (size_t)2 * s.f * s.d / 32;
    case 2: return (size_t)s.d * s.f / 2;
    default: return (size_t)s.d * s.f / 32;
  }
}

const void* bank_ptr(const k3moe_expert_bank& b, int which) {
  return which == 0 ? b.w13 : which == 1 ? b.w13_scale : which == 2 ? b.w2 : b.w2_scale;
}

// Makes expert e resident for the batch of tick `now` (use = true) or as a
// prefetch (use = false); enqueues its copies on `cs` when it was not
// resident.  Returns the slot, or -1 when every slot is needed by this batch.
int plan_one(k3moe_expert_cache& c, int e, bool use, int64_t now, hipStream_t cs, bool copy,
             hipError_t* err) {
  // the counters of lookups, hits and misses are a batch's; a prefetch of a
  // resident expert only refreshes it
  if (use) ++c.stats.lookups;
  int sl = c.slot_of[e];
  if (sl >= 0) {
    if (use) {
      ++c.stats.hits;
      if (c.prefetched[sl]) ++c.stats.prefetch_hits;
      c.prefetched[sl] = 0;
    }
    c.last_use[sl] = now;
    c.pinned[sl] = (int32_t)now;
    return sl;
  }
  if (use) ++c.stats.misses;
  // victim: a free slot, else the least recently used one not needed now
  int victim = -1;
  const int ns = (int)c.expert_in.size();
  for (int i = 0; i < ns; ++i) {
    if (c.pinned[i] == (int32_t)now) continue;
    if (c.expert_in[i] < 0) { victim = i; break; }
    if (victim < 0 || c.last_use[i] < c.last_use[victim]) victim = i;
  }
  if (victim < 0) return -1;
  if (c.expert_in[victim] >= 0) {
    c.slot_of[c.expert_in[victim]] = -1;
    ++c.stats.evictions;
  }
  c.expert_in[victim] = e;
  c.slot_of[e] = victim;
  c.last_use[victim] = now;
  c.pinned[victim] = (int32_t)now;
  c.prefetched[victim] = use ? 0 : 1;
  if (!use) ++c.stats.prefetched;
  for (int w = 0; w < 4; ++w) {
    const size_t n = bank_bytes_per_expert(c.shape, w);
    c.stats.bytes_copied += (int64_t)n;
    if (!copy) continue;
    const hipError_t r = hipMemcpyAsync(
        static_cast<char*>(const_cast<void*>(bank_ptr(c.slots, w))) + (size_t)victim * n,
        static_cast<const char*>(bank_ptr(c.host, w)) + (size_t)e * n, n,
        hipMemcpyHostToDevice, cs);
    if (r != hipSuccess && *err == hipSuccess) *err = r;
  }
  return victim;
}

// One batch: the distinct experts `ids` (n of them, each in [0, E)) become
// resident, their slots in slot_out.  Hits are refreshed and pinned first, so
// no miss of the batch can evict an expert the batch uses; then every miss
// takes a free slot or the least recently used unpinned one.  Returns false
// when the slots run out.
bool plan_batch(k3moe_expert_cache& c, const int32_t* ids, int n, int64_t now, hipStream_t cs,
                bool copy, int32_t* slot_out, hipError_t* err) {
  for (int i = 0; i < n; ++i) {
    const int sl = c.slot_of[ids[i]];
    slot_out[i] = -1;
    if (sl >= 0) slot_out[i] = plan_one(c, ids[i], true, now, cs, copy, err);
  }
  for (int i = 0; i < n; ++i) {
    if (slot_out[i] >= 0) continue;
    slot_out[i] = plan_one(c, ids[i], true, now, cs, copy, err);
    if (slot_out[i] < 0) return false;
  }
  return true;
}

}  // namespace
}  // namespace k3

namespace k3 {
namespace {

struct CacheWs {
  LayerWs inner;     // the resident layer's buffers, on slot ids
  RouteWs route;     // the router's scratch (all E experts)
  int32_t* slot_ids; // [P]
  int32_t* map;      // [E]
};

CacheWs carve_cache(const k3moe_shape& s, int slots, void* ws, size_t* bytes) {
  k3moe_shape si = s;
  si.E = slots;
  Carver c(ws);
  CacheWs r;
  size_t n = 0;
  carve_layer(si, nullptr, &n);
  r.inner = carve_layer(si, c.base, nullptr);
  c.off += n;
  size_t m = 0;
  carve_route(s, nullptr, &m);
  r.route = carve_route(s, c.base ? c.base + c.off : nullptr, nullptr);
  c.off += m;
  r.slot_ids = c.take<int32_t>((size_t)s.T * s.k);
  r.map = c.take<int32_t>((size_t)s.E);
  if (bytes) *bytes = c.off;
  return r;
}

k3moe_status check_cache_banks(const k3moe_shape& s, const k3moe_expert_bank* host,
                               const k3moe_expert_bank* slots) {
  if (!host || !slots) return fail_status(K3MOE_EINVAL, "host bank or slot bank is NULL");
  if (host->format != K3MOE_FMT_MXFP4 || slots->format != K3MOE_FMT_MXFP4)
    return fail_status(K3MOE_EUNSUPPORTED, "the expert cache holds MXFP4 banks");
  if (s.routed_format != K3MOE_FMT_MXFP4 || s.act != K3MOE_ACT_EXACT)
    return fail_status(K3MOE_EUNSUPPORTED, "the expert cache serves MXFP4 experts, exact mode");
  if (host->n_experts != s.E || host->d != s.d || host->f != s.f || slots->d != s.d ||
      slots->f != s.f)
    return fail_status(K3MOE_EINVAL, "bank sizes do not match the shape");
  if (slots->n_experts < s.k || slots->n_experts > 1024)
    return fail_status(K3MOE_ESHAPE, "the cache needs k <= slots <= 1024");
  const void* p[8] = {host->w13, host->w13_scale, host->w2, host->w2_scale,
                      slots->w13, slots->w13_scale, slots->w2, slots->w2_scale};
  for (const void* q : p) {
    if (!q) return fail_status(K3MOE_EINVAL, "a bank pointer is NULL");
    if (reinterpret_cast<uintptr_t>(q) & 15u)
      return fail_status(K3MOE_EALIGN, "a bank pointer is not 16-byte aligned");
  }
  return K3MOE_OK;
}

hipError_t ensure_events(k3moe_expert_cache& c) {
  hipError_t e = hipSuccess;
  if (!c.copies_done) e = hipEventCreateWithFlags(&c.copies_done, hipEventDisableTiming);
  if (e == hipSuccess && !c.reads_done)
    e = hipEventCreateWithFlags(&c.reads_done, hipEventDisableTiming);
  return e;
}

// Orders new copies on `ps` after the reads of the slots by the last layer
// call and after earlier copies on any stream (a slot is only refilled once
// nothing enqueued before reads it or writes it).
hipError_t order_copies(k3moe_expert_cache& c, hipStream_t ps) {
  hipError_t e = hipSuccess;
  if (c.reads_recorded) e = hipStreamWaitEvent(ps, c.reads_done, 0);
  if (e == hipSuccess && c.copies_recorded) e = hipStreamWaitEvent(ps, c.copies_done, 0);
  return e;
}

}  // namespace
}  // namespace k3

using namespace k3;

extern "C" {

k3moe_status k3moe_cache_create(const k3moe_shape* shape, const k3moe_expert_bank* host_bank,
                                const k3moe_expert_bank* slot_bank, k3moe_expert_cache** cache) {
  if (!cache) return fail_status(K3MOE_EINVAL, "cache is NULL");
  *cache = nullptr;
  const k3moe_status st = shape_status(shape);
  if (st != K3MOE_OK) return st;
  const k3moe_status sb = check_cache_banks(*shape, host_bank, slot_bank);
  if (sb != K3MOE_OK) return sb;
  k3moe_expert_cache* c = new (std::nothrow) k3moe_expert_cache();
  if (!c) return fail_status(K3MOE_EINVAL, "out of host memory");
  c->shape = *shape;
  c->host = *host_bank;
  c->slots = *slot_bank;
  const int ns = slot_bank->n_experts;
  c->slot_of.assign(shape->E, -1);
  c->expert_in.assign(ns, -1);
  c->last_use.assign(ns, 0);
  c->prefetched.assign(ns, 0);
  c->pinned.assign(ns, -1);
  c->map_host.assign(shape->E, -1);
  *cache = c;
  return K3MOE_OK;
}

void k3moe_cache_destroy(k3moe_expert_cache* cache) {
  if (!cache) return;
  if (cache->copies_done) (void)hipEventDestroy(cache->copies_done);
  if (cache->reads_done) (void)hipEventDestroy(cache->reads_done);
  delete cache;
}

k3moe_status k3moe_cache_stats_get(const k3moe_expert_cache* cache, k3moe_cache_stats* stats) {
  if (!cache || !stats) return fail_status(K3MOE_EINVAL, "cache or stats is NULL");
  *stats = cache->stats;
  return K3MOE_OK;
}

k3moe_status k3moe_cache_plan(k3moe_expert_cache* cache, const int32_t* ids, int32_t n,
                              int32_t* slot_of) {
  if (!cache || (n > 0 && (!ids || !slot_of)) || n < 0)
    return fail_status(K3MOE_EINVAL, "cache, ids or slot_of is NULL, or n < 0");
  std::lock_guard<std::mutex> g(cache->lock);
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= cache->shape.E)
      return fail_status(K3MOE_EINVAL, "an expert id is outside [0, E)");
    for (int j = 0; j < i; ++j)
      if (ids[j] == ids[i]) return fail_status(K3MOE_EINVAL, "ids repeat");
  }
  const int64_t now = ++cache->tick;
  hipError_t err = hipSuccess;
  if (!plan_batch(*cache, ids, n, now, nullptr, false, slot_of, &err))
    return fail_status(K3MOE_ESHAPE, "more distinct experts than cache slots");
  return K3MOE_OK;
}

k3moe_status k3moe_cache_prefetch(k3moe_expert_cache* cache, const int32_t* ids, int32_t n,
                                  void* copy_stream) {
  if (!cache || (n > 0 && !ids) || n < 0) return fail_status(K3MOE_EINVAL, "bad arguments");
  std::lock_guard<std::mutex> g(cache->lock);
  const int64_t now = ++cache->tick;
  hipError_t err = hipSuccess;
  const hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= cache->shape.E)
      return fail_status(K3MOE_EINVAL, "an expert id is outside [0, E)");
  err = ensure_events(*cache);
  if (err == hipSuccess) err = order_copies(*cache, cs);
  if (err != hipSuccess) return hip_failure(err, "k3moe_cache_prefetch ordering");
  // a prefetch never evicts what the same prefetch brought in, and gives up
  // quietly when every slot is taken by it
  for (int i = 0; i < n; ++i)
    if (plan_one(*cache, ids[i], false, now, cs, true, &err) < 0) break;
  if (err == hipSuccess) err = hipEventRecord(cache->copies_done, cs);
  if (err != hipSuccess) return hip_failure(err, "k3moe_cache_prefetch copies");
  cache->copies_recorded = true;
  return K3MOE_OK;
}

size_t k3moe_cache_workspace_bytes(const k3moe_shape* shape, int32_t slots) {
  if (shape_status(shape) != K3MOE_OK || slots < shape->k || slots > 1024 || shape->T == 0)
    return 0;
  size_t n = 0;
  carve_cache(*shape, slots, nullptr, &n);
  return n;
}

k3moe_status k3moe_cache_layer(k3moe_expert_cache* cache, const k3moe_shape* shape,
                               const k3moe_layer_weights* weights, const void* x, void* out,
                               int32_t* diag, void* workspace, size_t workspace_bytes,
                               void* stream, void* copy_stream) {
  if (!cache) return fail_status(K3MOE_EINVAL, "cache is NULL");
  k3moe_status st = shape_status(shape);
  if (st != K3MOE_OK) return st;
  const k3moe_shape& s = *shape;
  if (s.E != cache->shape.E || s.d != cache->shape.d || s.f != cache->shape.f ||
      s.routed_format != K3MOE_FMT_MXFP4 || s.act != K3MOE_ACT_EXACT)
    return fail_status(K3MOE_EINVAL, "the shape differs from the cache's");
  if (!weights) return fail_status(K3MOE_EINVAL, "weights is NULL");
  // the resident layer's checks, with the slot bank standing in for the routed one
  k3moe_layer_weights wv = *weights;
  wv.routed = cache->slots;
  wv.routed.n_experts = s.E;
  size_t need_layer = 0;
  st = layer_validate(shape, &wv, x, out, diag, &need_layer);
  if (st != K3MOE_OK) return st;
  if (s.T == 0) return K3MOE_OK;
  const int ns = cache->slots.n_experts;
  const size_t need = k3moe_cache_workspace_bytes(shape, ns);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail_status(K3MOE_EWORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (workspace_bytes < need) return workspace_too_small(workspace_bytes, need);

  std::lock_guard<std::mutex> g(cache->lock);
  const hipStream_t cs = static_cast<hipStream_t>(stream);
  const hipStream_t ps = copy_stream ? static_cast<hipStream_t>(copy_stream) : cs;
  const CacheWs W = carve_cache(s, ns, workspace, nullptr);
  const LayerWs& L = W.inner;
  const int64_t P = s.T * s.k;
  // 1. route on the GPU, ids to the host
  hipError_t e = launch_route(s, x, static_cast<const uint16_t*>(weights->w_router),
                              weights->router_bias, L.topk_idx, L.topk_w, nullptr, diag, W.route,
                              cs);
  if (e != hipSuccess) return hip_failure(e, "k3moe_cache_layer route");
  cache->ids_host.resize((size_t)P);
  e = hipMemcpyAsync(cache->ids_host.data(), L.topk_idx, (size_t)P * 4, hipMemcpyDeviceToHost,
                     cs);
  if (e == hipSuccess) e = hipStreamSynchronize(cs);
  if (e != hipSuccess) return hip_failure(e, "k3moe_cache_layer ids to host");
  // the last call's kernels (on whatever stream) are done with the slots and
  // the slot map before any of them is rewritten
  e = ensure_events(*cache);
  if (e == hipSuccess && cache->reads_recorded) e = hipEventSynchronize(cache->reads_done);
  if (e == hipSuccess) e = order_copies(*cache, ps);
  if (e != hipSuccess) return hip_failure(e, "k3moe_cache_layer ordering");
  // 2. plan: the batch's distinct experts (ids outside [0, E) are dropped by
  // the permute, as in the layer); hits are refreshed, misses replace the
  // least recently used slots the batch does not need
  const int64_t now = ++cache->tick;
  std::fill(cache->map_host.begin(), cache->map_host.end(), -1);
  std::vector<int32_t> distinct;
  for (int64_t i = 0; i < P; ++i) {
    const int id = cache->ids_host[i];
    if (id < 0 || id >= s.E || cache->map_host[id] == -2) continue;
    cache->map_host[id] = -2;
    distinct.push_back(id);
  }
  std::vector<int32_t> slot(distinct.size());
  hipError_t cerr = hipSuccess;
  if (!plan_batch(*cache, distinct.data(), (int)distinct.size(), now, ps, true, slot.data(),
                  &cerr))
    return fail_status(K3MOE_ESHAPE,
                       "the batch routes to more distinct experts than the cache has slots");
  for (size_t i = 0; i < distinct.size(); ++i) cache->map_host[distinct[i]] = slot[i];
  if (cerr != hipSuccess) return hip_failure(cerr, "k3moe_cache_layer expert copies");
  e = hipEventRecord(cache->copies_done, ps);
  if (e == hipSuccess) cache->copies_recorded = true;
  if (e == hipSuccess)
    e = hipMemcpyAsync(W.map, cache->map_host.data(), (size_t)s.E * 4, hipMemcpyHostToDevice, cs);
  if (e != hipSuccess) return hip_failure(e, "k3moe_cache_layer slot map");
  // 3. the shared experts while the copies fly, then the routed experts on slots
  k3moe_shape si = s;
  si.E = ns;
  if (s.n_shared > 0) {
    SharedWs sws;
    sws.h = L.shared_h;
    e = launch_shared_ffn(s, weights->shared, x, L.shared_y, sws, cs);
    if (e != hipSuccess) return hip_failure(e, "k3moe_cache_layer shared experts");
  }
  e = hipStreamWaitEvent(cs, cache->copies_done, 0);
  if (e != hipSuccess) return hip_failure(e, "k3moe_cache_layer wait for copies");
  remap_ids<<<(unsigned)((P + 255) / 256), 256, 0, cs>>>(L.topk_idx, W.map, W.slot_ids, P, s.E);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_failure(e, "k3moe_cache_layer remap");
  e = launch_permute(si, W.slot_ids, L.counts, L.offsets, L.sorted_pair, L.pair_pos, diag,
                     carve_permute(si, L.scratch, nullptr), cs);
  if (e != hipSuccess) return hip_failure(e, "k3moe_cache_layer permute");
  e = launch_expert_ffn(si, cache->slots, x, L.offsets, L.sorted_pair, L.y_perm,
                        carve_expert(si, L.scratch, nullptr), cs);
  if (e != hipSuccess) return hip_failure(e, "k3moe_cache_layer routed experts");
  e = launch_combine(s, L.y_perm, L.pair_pos, L.topk_w, s.n_shared > 0 ? L.shared_y : nullptr,
                     out, cs);
  if (e == hipSuccess) e = hipEventRecord(cache->reads_done, cs);
  if (e != hipSuccess) return hip_failure(e, "k3moe_cache_layer combine");
  cache->reads_recorded = true;
  return K3MOE_OK;
}

}  // extern "C"
