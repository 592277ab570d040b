// Host-side core of the HeadKV C ABI: configuration checks, derived sizes and
// argument checks.  Pure C++ (no HIP), so it also builds with g++ alone for
// host-only tests and sanitizer runs.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/hkv.h"

namespace hkv {

// Limits of this implementation (checked by hkv_validate).
constexpr int kMaxPrefill = 1024;   // classification keeps W x P logits on chip
constexpr int kMaxWobs = 8;         // observation / scoring window queries
constexpr int kMaxEvict = 8;        // evictions per decode event (M = W)
constexpr int kMaxHeads = 1024;
constexpr int kMaxSplit = 8;        // workgroups per stream in the split decode step

struct Derived {
  int64_t S = 0;            // streams
  int32_t A = 0;            // floor(N * rho) per head (compressed only)
  int32_t split = 0;        // near/far split distance in effect (variants)
  int64_t group_slots = 0;  // pool slots per (layer, sequence) group
  int64_t pool_slots = 0;
  // workspace layout (bytes from the workspace start, 256-B aligned)
  size_t ws_init_scores = 0;   // float [S * P]
  size_t ws_tile = 0;          // float [pool_slots * w_obs]
  size_t ws_pos = 0;           // int32 [pool_slots]
  size_t ws_keys = 0;          // uint64 [pool_slots]
  size_t ws_part = 0;          // float [S, kMaxSplit, head_dim + 4]: split partial states
  size_t ws_bytes = 0;
};

// Fills `d` for a valid config; returns the validation status.
hkv_status derive(const hkv_config* cfg, Derived* d);

// Records the detail text returned by hkv_last_error on this thread.
hkv_status fail(hkv_status st, const char* fmt, ...);
void clear_error();
const char* last_error();

// need_workspace = false skips the workspace checks (the entry point that keeps
// its scratch in the library's own static buffer).
hkv_status check_state_buffers(const hkv_config* cfg, const hkv_state* st,
                               bool need_workspace = true);
hkv_status check_range(const Derived& d, int32_t s_begin, int32_t s_count);
hkv_status check_step(const hkv_config* cfg, int32_t t);
hkv_status check_data_ptr(const void* p, int64_t ld, int elem_bytes, const char* what);

inline int elem_bytes(const hkv_config* c) { return c->dtype == HKV_DT_BF16 ? 2 : 4; }

}  // namespace hkv
