// Host-side core of the HeadKV C ABI (no HIP calls).
#include "hkv_host.h"

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

namespace hkv {
namespace {
thread_local char g_last_error[512] = "";

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
}  // namespace

hkv_status fail(hkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error[0] = '\0'; }

const char* last_error() { return g_last_error; }

hkv_status derive(const hkv_config* c, Derived* d) {
  if (!c) return fail(HKV_E_INVAL, "config is NULL");
  if (c->layers <= 0 || c->batch <= 0 || c->heads <= 0)
    return fail(HKV_E_INVAL, "layers, batch and heads must be positive");
  if (c->heads > kMaxHeads) return fail(HKV_E_UNSUPPORTED, "heads > %d", kMaxHeads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(HKV_E_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", c->head_dim);
  if (c->dtype != HKV_DT_BF16 && c->dtype != HKV_DT_F32)
    return fail(HKV_E_INVAL, "dtype %d unknown", c->dtype);
  if (c->w_obs < 1 || c->w_obs > kMaxWobs)
    return fail(HKV_E_INVAL, "w_obs must be in [1, %d]", kMaxWobs);
  if (c->prefill_len < c->w_obs)
    return fail(HKV_E_INVAL, "prefill_len (%d) < w_obs (%d)", c->prefill_len, c->w_obs);
  if (c->final_len <= c->prefill_len)
    return fail(HKV_E_INVAL, "final_len must exceed prefill_len");
  if (c->full_cache != 0 && c->full_cache != 1)
    return fail(HKV_E_INVAL, "full_cache must be 0 or 1");
  if (c->variant & ~(HKV_VARIANT_UNSTRATIFIED | HKV_VARIANT_UNIFORM_BUDGET))
    return fail(HKV_E_INVAL, "variant has unknown bits 0x%x", c->variant);
  const int64_t S = int64_t(c->layers) * c->batch * c->heads;
  if (S > (int64_t(1) << 31) - 1) return fail(HKV_E_INVAL, "too many streams");
  d->S = S;
  if (c->full_cache) {
    d->A = 0;
    d->group_slots = int64_t(c->heads) * c->final_len;
  } else {
    if (c->prefill_len > kMaxPrefill)
      return fail(HKV_E_UNSUPPORTED, "prefill_len > %d", kMaxPrefill);
    if (c->local_window < 1) return fail(HKV_E_INVAL, "local_window must be >= 1");
    if (!(c->tau > 0.0f && c->tau <= 1.0f)) return fail(HKV_E_INVAL, "tau must be in (0, 1]");
    if (c->rho_num < 1 || c->rho_den < 1 || c->rho_num > c->rho_den)
      return fail(HKV_E_INVAL, "rho must be a fraction in (0, 1]");
    if (c->evict_m < 2 || (c->evict_m & 1) || c->evict_m > kMaxEvict)
      return fail(HKV_E_INVAL, "evict_m must be even and in [2, %d]", kMaxEvict);
    if (c->evict_m != c->w_obs)
      return fail(HKV_E_UNSUPPORTED, "evict_m must equal w_obs (scores span W queries)");
    if (c->split_dist < c->w_obs)
      return fail(HKV_E_INVAL, "split_dist must be >= w_obs");
    const int64_t A = int64_t(c->final_len) * c->rho_num / c->rho_den;
    if (A < c->local_window || A < c->evict_m)
      return fail(HKV_E_INVAL, "floor(rho*N) = %lld must be >= local_window and evict_m",
                  (long long)A);
    d->A = int32_t(A);
    d->group_slots = int64_t(c->heads) * (A + c->evict_m);
    // without the near/far split every candidate is near: with an empty far
    // subset the quotas hand all evictions to the near one
    d->split = (c->variant & HKV_VARIANT_UNSTRATIFIED) ? INT32_MAX : c->split_dist;
  }
  d->pool_slots = d->group_slots * c->layers * c->batch;
  size_t off = 0;
  d->ws_init_scores = off;
  off = align256(off + size_t(S) * size_t(c->prefill_len) * sizeof(float));
  d->ws_tile = off;
  off = align256(off + size_t(d->pool_slots) * size_t(c->w_obs) * sizeof(float));
  d->ws_pos = off;
  off = align256(off + size_t(d->pool_slots) * sizeof(int32_t));
  d->ws_keys = off;
  off = align256(off + size_t(d->pool_slots) * sizeof(uint64_t));
  d->ws_part = off;
  off = align256(off + size_t(S) * kMaxSplit * size_t(c->head_dim + 4) * sizeof(float));
  d->ws_bytes = off;
  return HKV_OK;
}

hkv_status check_state_buffers(const hkv_config* c, const hkv_state* st, bool need_workspace) {
  if (!st) return fail(HKV_E_INVAL, "state is NULL");
  if (!st->k_pool || !st->v_pool || !st->pos || !st->score || !st->base || !st->cap ||
      !st->count || !st->budget || !st->n_tokens || !st->label || !st->err ||
      !st->free_slots || !st->n_free || !st->qstat)
    return fail(HKV_E_INVAL, "state has a NULL buffer");
  if (!aligned16(st->k_pool) || !aligned16(st->v_pool) || !aligned16(st->qstat))
    return fail(HKV_E_INVAL, "k_pool, v_pool and qstat must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(st->base) & 7u) || (reinterpret_cast<uintptr_t>(st->pos) & 3u) ||
      (reinterpret_cast<uintptr_t>(st->score) & 3u) || (reinterpret_cast<uintptr_t>(st->label) & 3u) ||
      (reinterpret_cast<uintptr_t>(st->count) & 3u) || (reinterpret_cast<uintptr_t>(st->cap) & 3u) ||
      (reinterpret_cast<uintptr_t>(st->budget) & 3u) || (reinterpret_cast<uintptr_t>(st->n_tokens) & 3u) ||
      (reinterpret_cast<uintptr_t>(st->free_slots) & 3u) || (reinterpret_cast<uintptr_t>(st->n_free) & 3u))
    return fail(HKV_E_INVAL, "state index buffers misaligned");
  Derived d;
  hkv_status s = derive(c, &d);
  if (s != HKV_OK) return s;
  // one pool buffer: slot j's K row, then its V row ([pool_slots, 2, head_dim])
  const size_t row = size_t(c->head_dim) * (c->dtype == HKV_DT_BF16 ? 2 : 4);
  if (static_cast<const char*>(st->v_pool) != static_cast<const char*>(st->k_pool) + row)
    return fail(HKV_E_INVAL, "v_pool must be k_pool + head_dim elements (one [pool_slots, 2, "
                "head_dim] buffer)");
  if (!need_workspace) return HKV_OK;
  if (!st->workspace || (reinterpret_cast<uintptr_t>(st->workspace) & 255u))
    return fail(HKV_E_INVAL, "workspace must be non-NULL and 256-byte aligned");
  if (st->workspace_bytes < d.ws_bytes)
    return fail(HKV_E_INVAL, "workspace_bytes %zu < required %zu", st->workspace_bytes,
                d.ws_bytes);
  return HKV_OK;
}

hkv_status check_range(const Derived& d, int32_t s_begin, int32_t s_count) {
  if (s_begin < 0 || s_count < 0 || int64_t(s_begin) + s_count > d.S)
    return fail(HKV_E_INVAL, "stream range [%d, %d+%d) outside [0, %lld)", s_begin, s_begin,
                s_count, (long long)d.S);
  return HKV_OK;
}

hkv_status check_step(const hkv_config* c, int32_t t) {
  if (t < c->prefill_len || t >= c->final_len)
    return fail(HKV_E_INVAL, "step t=%d outside [prefill_len, final_len)", t);
  return HKV_OK;
}

hkv_status check_data_ptr(const void* p, int64_t ld, int eb, const char* what) {
  if (!p) return fail(HKV_E_INVAL, "%s is NULL", what);
  if (!aligned16(p)) return fail(HKV_E_INVAL, "%s must be 16-byte aligned", what);
  if (ld < 0 || ((ld * eb) & 15)) return fail(HKV_E_INVAL, "%s stride must be a multiple of 16 bytes", what);
  return HKV_OK;
}

}  // namespace hkv

extern "C" {

size_t hkv_pool_slots(const hkv_config* cfg) {
  hkv::Derived d;
  return hkv::derive(cfg, &d) == HKV_OK ? size_t(d.pool_slots) : 0;
}

size_t hkv_workspace_bytes(const hkv_config* cfg) {
  hkv::Derived d;
  return hkv::derive(cfg, &d) == HKV_OK ? d.ws_bytes : 0;
}

hkv_status hkv_validate(const hkv_config* cfg) {
  hkv::Derived d;
  hkv::clear_error();
  return hkv::derive(cfg, &d);
}

const char* hkv_status_string(int32_t s) {
  switch (s) {
    case HKV_OK: return "ok";
    case HKV_E_INVAL: return "invalid argument";
    case HKV_E_STATE: return "call out of order";
    case HKV_E_CAPACITY: return "stream capacity exceeded on the device";
    case HKV_E_HIP: return "HIP runtime error";
    case HKV_E_UNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
  }
}

const char* hkv_last_error(void) { return hkv::last_error(); }

}  // extern "C"
