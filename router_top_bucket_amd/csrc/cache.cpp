// Expert streaming from a pinned host pool into a device expert cache ("Run
// Kimi 3.1 locally on one GPU", sections "One GPU, three storage tiers" and
// "Read the experts the router needs").  Experts found in the device cache
// run immediately; the rest are copied up from the host pool over several
// streams, and each group of copies is computed as soon as it lands.  The
// disk tier of the pages has no counterpart here: the host pool holds every
// expert.
//
// A call: route and bucket on the caller's stream, wait for the bucketing on
// the host (the experts to fetch are known only then), plan slots
// (CachePolicy), then
//   - the FFN over the experts already in the device cache (and the shared
//     experts, resident for good) on the caller's stream;
//   - the misses cut into `upload_groups` groups in the active order; each
//     group's records are copied host -> device on the upload streams (round
//     robin), and the caller's stream waits for that group's copies and runs
//     the FFN over it while the next groups are still uploading;
//   - the combine.
// Every expert's arithmetic is the resident path's (the FFN kernels only look
// its record up through a slot map), so every output is bit-identical to
// moe_layer_mxfp4 on the same layer held in device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "../../include/moe.h"
#include "cache_policy.h"
#include "checks.h"
#include "launch.h"

namespace {

constexpr int kMaxUploadStreams = 8;
constexpr int kMaxUploadGroups = 16;

}  // namespace

struct moe_expert_cache {
  moe_cache_config cfg;
  moe::CachePolicy policy;
  int shared_base;  // first slot of the shared experts (layer l, shared s: shared_base + l*S + s)
  int policy_base;  // first slot of the transient and cached slots
  hipStream_t up[kMaxUploadStreams] = {};
  hipEvent_t ev[kMaxUploadGroups][kMaxUploadStreams] = {};
  int32_t *h_route = nullptr;  // pinned: offsets [NE+1], active [NE], n_active [1]
  int32_t *h_plan = nullptr;   // pinned: map [NE], lists [NE], counts [kMaxUploadGroups+1]
  int32_t *d_plan = nullptr;   // device copy of h_plan
  moe_cache_stats stats = {};
  std::vector<int32_t> ex, rows, slot, hit, adm;

  moe_expert_cache(const moe_cache_config &c, int n_cache)
      : cfg(c), policy(c.n_layers, c.n_routed, n_cache, c.n_transient, c.admit_min_rows) {}
  int NE() const { return cfg.n_routed + cfg.n_shared; }
  size_t plan_ints() const { return (size_t)2 * NE() + kMaxUploadGroups + 1; }
};

namespace {

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

void release(moe_expert_cache *c) {
  for (auto &s : c->up)
    if (s) (void)hipStreamDestroy(s);
  for (auto &row : c->ev)
    for (auto &e : row)
      if (e) (void)hipEventDestroy(e);
  if (c->h_route) (void)hipHostFree(c->h_route);
  if (c->h_plan) (void)hipHostFree(c->h_plan);
  if (c->d_plan) (void)hipFree(c->d_plan);
  delete c;
}

bool is_pinned_host(const void *p) {
  hipPointerAttribute_t a;
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // leave no error behind for the caller's next call
    return false;
  }
  return a.type == hipMemoryTypeHost;
}

}  // namespace

extern "C" {

int moe_cache_create(const moe_cache_config *cfg, moe_expert_cache **out) {
  if (!cfg || !out) return MOE_EINVAL;
  *out = nullptr;
  const moe_cache_config &c = *cfg;
  if (!c.device_pool || !c.host_pool || c.n_layers < 1 || c.n_routed < 1 || c.n_shared < 0) return MOE_EINVAL;
  if (c.d <= 0 || c.f <= 0 || c.d % 32 || c.f % 32) return MOE_EINVAL;
  const int64_t rec = (int64_t)3 * c.d * c.f * 17 / 32;
  if (c.stride < rec || c.stride % 16) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(c.device_pool) % 16 || reinterpret_cast<uintptr_t>(c.host_pool) % 16)
    return MOE_EINVAL;
  if (c.n_upload_streams < 1 || c.n_upload_streams > kMaxUploadStreams) return MOE_EINVAL;
  if (c.upload_groups < 1 || c.upload_groups > kMaxUploadGroups) return MOE_EINVAL;
  if (c.admit_min_rows < 0 || c.n_transient < 0) return MOE_EINVAL;
  if (c.layout != MOE_LAYOUT_ROWS && c.layout != MOE_LAYOUT_TILES) return MOE_EINVAL;
  const int64_t shared = (int64_t)c.n_layers * c.n_shared;
  const int64_t n_cache = (int64_t)c.n_slots - shared - c.n_transient;
  if (n_cache < 1) return MOE_EINVAL;
  if (c.n_routed + c.n_shared > 4096 || (int64_t)c.n_layers * c.n_routed > (1 << 30)) return MOE_EUNSUPPORTED;
  if (!is_pinned_host(c.host_pool)) return MOE_EINVAL;

  moe_expert_cache *m = new moe_expert_cache(c, (int)n_cache);
  m->shared_base = 0;
  m->policy_base = (int)shared;
  bool ok = true;
  for (int i = 0; i < c.n_upload_streams && ok; ++i)
    ok = hipStreamCreateWithFlags(&m->up[i], hipStreamNonBlocking) == hipSuccess;
  for (int g = 0; g < c.upload_groups && ok; ++g)
    for (int i = 0; i < c.n_upload_streams && ok; ++i)
      ok = hipEventCreateWithFlags(&m->ev[g][i], hipEventDisableTiming) == hipSuccess;
  const int NE = m->NE();
  ok = ok && hipHostMalloc((void **)&m->h_route, sizeof(int32_t) * (2 * NE + 2)) == hipSuccess;
  ok = ok && hipHostMalloc((void **)&m->h_plan, sizeof(int32_t) * m->plan_ints()) == hipSuccess;
  ok = ok && hipMalloc((void **)&m->d_plan, sizeof(int32_t) * m->plan_ints()) == hipSuccess;
  // the shared experts of every layer, uploaded once
  for (int l = 0; l < c.n_layers && ok; ++l)
    for (int s = 0; s < c.n_shared && ok; ++s) {
      uint8_t *dst = (uint8_t *)c.device_pool + (int64_t)(m->shared_base + l * c.n_shared + s) * c.stride;
      const uint8_t *src = (const uint8_t *)c.host_pool + ((int64_t)l * NE + c.n_routed + s) * c.stride;
      ok = hipMemcpy(dst, src, (size_t)c.stride, hipMemcpyHostToDevice) == hipSuccess;
    }
  if (!ok) {
    (void)hipGetLastError();
    release(m);
    return MOE_EHIP;
  }
  const size_t nmax = (size_t)NE;
  m->ex.resize(nmax);
  m->rows.resize(nmax);
  m->slot.resize(nmax);
  m->hit.resize(nmax);
  m->adm.resize(nmax);
  *out = m;
  return MOE_OK;
}

int moe_cache_destroy(moe_expert_cache *cache) {
  if (!cache) return MOE_EINVAL;
  // kernels of earlier calls may still read the plan buffers
  (void)hipDeviceSynchronize();
  release(cache);
  return MOE_OK;
}

int moe_cache_get_stats(const moe_expert_cache *cache, moe_cache_stats *stats) {
  if (!cache || !stats) return MOE_EINVAL;
  *stats = cache->stats;
  return MOE_OK;
}

int moe_layer_streamed(moe_expert_cache *cache, int32_t layer, const void *x, moe_dtype x_dtype,
                       const float *w_router, float *logits, int32_t M, int32_t k, int32_t *topk_ids, float *topk_w,
                       int32_t *offsets, int32_t *perm, int32_t *active, int32_t *n_active, int32_t *dev_error,
                       float *y_slots, float *out, void *workspace, size_t workspace_bytes, void *stream) {
  if (!cache) return MOE_EINVAL;
  moe_expert_cache &c = *cache;
  const moe_cache_config &cf = c.cfg;
  if (layer < 0 || layer >= cf.n_layers) return MOE_EINVAL;
  const int E = cf.n_routed, S = cf.n_shared, NE = c.NE();
  // the argument checks of moe_layer_mxfp4, on a descriptor of this layer's
  // device-pool view (its records are never addressed through it)
  moe_experts W{(const uint8_t *)cf.device_pool, cf.stride, cf.d, cf.f, E, S, cf.layout};
  const int rc = moe_layer_check(x, x_dtype, w_router, logits, M, k, &W, topk_ids, topk_w, offsets, perm, active,
                                 n_active, dev_error, y_slots, out, workspace, workspace_bytes);
  if (rc != MOE_OK || M == 0) return rc;
  // the worst case of a call must fit the pool: every routed expert it can
  // touch needs a transient or a cached slot
  const int64_t worst = std::min<int64_t>(E, (int64_t)M * k);
  if (worst > (int64_t)c.policy.n_cache() + c.policy.n_transient()) return MOE_EUNSUPPORTED;

  const hipStream_t st = as_stream(stream);
  const int bf = x_dtype == MOE_BF16;
  if (moe::route_bucket_launch(x, bf, w_router, logits, M, cf.d, E, k, S, topk_ids, topk_w, offsets, perm, active,
                                n_active, dev_error, st))
    return MOE_EHIP;
  int32_t *h_off = c.h_route, *h_act = c.h_route + NE + 1, *h_na = c.h_route + 2 * NE + 1;
  if (hipMemcpyAsync(h_off, offsets, sizeof(int32_t) * (NE + 1), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(h_act, active, sizeof(int32_t) * NE, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(h_na, n_active, sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return MOE_EHIP;

  // routed experts of the call, ascending (the active list), with their rows
  const int na = std::max(0, std::min(*h_na, NE));
  int n = 0;
  for (int i = 0; i < na; ++i) {
    const int e = h_act[i];
    if (e >= 0 && e < E) {
      c.ex[n] = e;
      c.rows[n] = h_off[e + 1] - h_off[e];
      ++n;
    }
  }
  const int misses = c.policy.plan(layer, c.ex.data(), c.rows.data(), n, c.slot.data(), c.hit.data(), c.adm.data());
  if (misses < 0) return MOE_EUNSUPPORTED;

  // slot map, hit list (with the shared experts), miss groups, counts
  int32_t *map = c.h_plan, *lists = c.h_plan + NE, *counts = c.h_plan + 2 * NE;
  std::fill(map, map + NE, -1);
  for (int i = 0; i < n; ++i) map[c.ex[i]] = c.policy_base + c.slot[i];
  for (int s = 0; s < S; ++s) map[E + s] = c.shared_base + layer * S + s;
  int pos = 0;
  for (int i = 0; i < n; ++i)
    if (c.hit[i]) lists[pos++] = c.ex[i];
  for (int i = 0; i < na; ++i)
    if (h_act[i] >= E && h_act[i] < NE) lists[pos++] = h_act[i];
  counts[0] = pos;
  const int groups = std::min(cf.upload_groups, std::max(misses, 1));
  std::vector<int> miss_idx;
  miss_idx.reserve(misses);
  for (int i = 0; i < n; ++i)
    if (!c.hit[i]) miss_idx.push_back(i);
  for (int g = 0; g < groups; ++g) {
    const int a = (int)((int64_t)misses * g / groups), b = (int)((int64_t)misses * (g + 1) / groups);
    for (int j = a; j < b; ++j) lists[pos++] = c.ex[miss_idx[j]];
    counts[1 + g] = b - a;
  }
  // from here on a failure leaves this call's admitted misses unfilled: they
  // leave the cache, so no later call takes a never-uploaded slot for a hit
  auto fail = [&]() {
    for (int i = 0; i < n; ++i)
      if (c.adm[i]) c.policy.forget(layer, c.ex[i]);
    return MOE_EHIP;
  };
  if (hipMemcpyAsync(c.d_plan, c.h_plan, sizeof(int32_t) * c.plan_ints(), hipMemcpyHostToDevice, st) != hipSuccess)
    return fail();
  const int32_t *d_map = c.d_plan, *d_lists = c.d_plan + NE, *d_counts = c.d_plan + 2 * NE;

  auto ffn = [&](int list_start, int count_idx, int count) -> int {
    if (count == 0) return 0;
    return moe::ffn_launch(x, bf, M, k, (const uint8_t *)cf.device_pool, cf.stride, cf.d, cf.f, E, S, offsets, perm,
                           d_lists + list_start, d_counts + count_idx, y_slots, workspace,
                           moe::kStageGateUp | moe::kStageDown, d_map, cf.n_slots, count,
                           cf.layout == MOE_LAYOUT_TILES, st);
  };
  if (ffn(0, 0, counts[0])) return fail();
  int lstart = counts[0], up_i = 0;
  for (int g = 0; g < groups && misses > 0; ++g) {
    bool used[kMaxUploadStreams] = {};
    const int a = (int)((int64_t)misses * g / groups), b = (int)((int64_t)misses * (g + 1) / groups);
    for (int j = a; j < b; ++j) {
      const int i = miss_idx[j];
      const int s = up_i++ % cf.n_upload_streams;
      uint8_t *dst = (uint8_t *)cf.device_pool + (int64_t)(c.policy_base + c.slot[i]) * cf.stride;
      const uint8_t *src = (const uint8_t *)cf.host_pool + ((int64_t)layer * NE + c.ex[i]) * cf.stride;
      if (hipMemcpyAsync(dst, src, (size_t)cf.stride, hipMemcpyHostToDevice, c.up[s]) != hipSuccess) return fail();
      used[s] = true;
    }
    for (int s = 0; s < cf.n_upload_streams; ++s)
      if (used[s] && (hipEventRecord(c.ev[g][s], c.up[s]) != hipSuccess ||
                      hipStreamWaitEvent(st, c.ev[g][s], 0) != hipSuccess))
        return fail();
    if (ffn(lstart, 1 + g, b - a)) return fail();
    lstart += b - a;
  }
  if (moe::combine_launch(y_slots, topk_w, M, k, S, cf.d, out, st)) return fail();

  c.stats.calls += 1;
  c.stats.hits += n - misses;
  c.stats.misses += misses;
  for (int i = 0; i < n; ++i) c.stats.admitted += c.adm[i];
  c.stats.bytes_uploaded += (int64_t)misses * cf.stride;
  return MOE_OK;
}

int moe_cache_simulate(int32_t n_layers, int32_t n_routed, int32_t n_cache, int32_t n_transient,
                       int32_t admit_min_rows, int32_t n_calls, const int32_t *call_layer, const int32_t *call_n,
                       const int32_t *experts, const int32_t *rows, int32_t *slot, int32_t *hit, int32_t *admitted) {
  if (n_layers < 1 || n_routed < 1 || n_cache < 1 || n_transient < 0 || admit_min_rows < 0 || n_calls < 0)
    return MOE_EINVAL;
  if (n_calls > 0 && (!call_layer || !call_n || !experts || !rows || !slot || !hit || !admitted)) return MOE_EINVAL;
  moe::CachePolicy p(n_layers, n_routed, n_cache, n_transient, admit_min_rows);
  int64_t at = 0;
  for (int i = 0; i < n_calls; ++i) {
    if (call_n[i] < 0) return MOE_EINVAL;
    if (p.plan(call_layer[i], experts + at, rows + at, call_n[i], slot + at, hit + at, admitted + at) < 0)
      return MOE_EUNSUPPORTED;
    at += call_n[i];
  }
  return MOE_OK;
}

}  // extern "C"
