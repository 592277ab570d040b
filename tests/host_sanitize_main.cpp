// Host-only driver of the library's host core (configuration checks, derived
// sizes, argument checks, error text), built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitize.py.  No HIP call: the
// state pointers below are aligned integers that the checks never dereference.
#include <climits>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../kv_cache_compression_hkv_amd/csrc/hkv_host.h"

namespace {
int g_fail = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAIL line %d: %s (last error: %s)\n", line, what, hkv_last_error());
    ++g_fail;
  }
}
#define EXPECT(x) expect((x), #x, __LINE__)

hkv_config base_cfg() {
  hkv_config c{};
  c.layers = 2;
  c.batch = 2;
  c.heads = 4;
  c.head_dim = 64;
  c.dtype = HKV_DT_BF16;
  c.final_len = 200;
  c.prefill_len = 40;
  c.local_window = 16;
  c.tau = 0.9f;
  c.rho_num = 1;
  c.rho_den = 4;
  c.split_dist = 24;
  c.w_obs = 8;
  c.evict_m = 8;
  c.full_cache = 0;
  c.variant = 0;
  return c;
}

hkv_state fake_state(const hkv_config& c, int phase) {
  hkv_state st{};
  void* a = reinterpret_cast<void*>(uintptr_t(1) << 20);
  st.k_pool = a;   // one [pool_slots, 2, head_dim] buffer: V rows one K row later
  st.v_pool = static_cast<char*>(a) + size_t(c.head_dim) * (c.dtype == HKV_DT_BF16 ? 2 : 4);
  st.pos = st.count = st.cap = st.budget = st.n_tokens = st.free_slots = st.n_free = st.err =
      static_cast<int32_t*>(a);
  st.score = st.qstat = static_cast<float*>(a);
  st.base = static_cast<int64_t*>(a);
  st.label = static_cast<uint8_t*>(a);
  st.workspace = a;
  st.workspace_bytes = hkv_workspace_bytes(&c);
  st.phase = phase;
  return st;
}
}  // namespace

int main() {
  using namespace hkv;
  // the five workload shapes, compressed and uncompressed
  struct Shape { int L, B, H, d, dt, N, P, w, rn, rd, D; };
  const Shape shapes[] = {
      {1, 1, 4, 64, HKV_DT_F32, 256, 64, 16, 1, 4, 32},
      {36, 16, 20, 64, HKV_DT_BF16, 696, 184, 32, 1, 6, 48},
      {24, 32, 16, 128, HKV_DT_BF16, 640, 128, 32, 1, 4, 48},
      {30, 32, 32, 128, HKV_DT_BF16, 640, 128, 32, 1, 6, 48},
      {30, 32, 32, 128, HKV_DT_BF16, 640, 128, 32, 1, 8, 48},
      {32, 8, 32, 128, HKV_DT_BF16, 2416, 192, 98, 1, 8, 196},
  };
  for (const Shape& s : shapes) {
    hkv_config c = base_cfg();
    c.layers = s.L; c.batch = s.B; c.heads = s.H; c.head_dim = s.d; c.dtype = s.dt;
    c.final_len = s.N; c.prefill_len = s.P; c.local_window = s.w;
    c.rho_num = s.rn; c.rho_den = s.rd; c.split_dist = s.D;
    EXPECT(hkv_validate(&c) == HKV_OK);
    const size_t S = size_t(s.L) * s.B * s.H;
    const size_t A = size_t(s.N) * s.rn / s.rd;
    EXPECT(hkv_pool_slots(&c) == S * (A + 8));
    EXPECT(hkv_workspace_bytes(&c) >= S * s.P * 4 + hkv_pool_slots(&c) * 12);
    c.full_cache = 1;
    EXPECT(hkv_pool_slots(&c) == S * size_t(s.N));
  }

  // every rejected configuration, with its status and a non-empty reason
  constexpr int kAny = 1;            // must not overflow; any status
  struct Bad { void (*edit)(hkv_config&); int want; };
  const Bad bad[] = {
      {[](hkv_config& c) { c.head_dim = 96; }, HKV_E_UNSUPPORTED},
      {[](hkv_config& c) { c.layers = 0; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.heads = 5000; }, HKV_E_UNSUPPORTED},
      {[](hkv_config& c) { c.dtype = 7; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.prefill_len = 4; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.final_len = 40; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.tau = 0.0f; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.tau = 1.5f; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.rho_num = 5; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.rho_den = 100; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.evict_m = c.w_obs = 7; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.evict_m = c.w_obs = 10; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.evict_m = 6; }, HKV_E_UNSUPPORTED},
      {[](hkv_config& c) { c.split_dist = 4; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.prefill_len = 2000; c.final_len = 3000; }, HKV_E_UNSUPPORTED},
      {[](hkv_config& c) { c.local_window = 0; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.variant = 4; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.variant = -1; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.full_cache = 2; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.layers = c.batch = 2048; c.heads = 1024; }, HKV_E_INVAL},
      {[](hkv_config& c) { c.final_len = INT_MAX; c.rho_num = c.rho_den = 1; }, kAny},
  };
  for (const Bad& b : bad) {
    hkv_config c = base_cfg();
    b.edit(c);
    const hkv_status got = hkv_validate(&c);
    if (b.want == kAny) continue;
    EXPECT(got == b.want);
    EXPECT(hkv_pool_slots(&c) == 0);
    EXPECT(std::strlen(hkv_last_error()) > 0);
  }
  EXPECT(hkv_validate(nullptr) == HKV_E_INVAL);
  EXPECT(hkv_pool_slots(nullptr) == 0);

  // argument checks of the entry points (host side only)
  hkv_config c = base_cfg();
  Derived d;
  EXPECT(derive(&c, &d) == HKV_OK);
  hkv_state st = fake_state(c, 1);
  EXPECT(check_state_buffers(&c, &st) == HKV_OK);
  hkv_state small = st;
  small.workspace_bytes = 16;
  EXPECT(check_state_buffers(&c, &small) == HKV_E_INVAL);
  hkv_state mis = st;
  mis.pos = reinterpret_cast<int32_t*>(uintptr_t(1) << 20 | 2);
  EXPECT(check_state_buffers(&c, &mis) == HKV_E_INVAL);
  hkv_state apart = st;   // V rows not one K row after the K rows
  apart.v_pool = st.k_pool;
  EXPECT(check_state_buffers(&c, &apart) == HKV_E_INVAL);
  hkv_state nul{};
  EXPECT(check_state_buffers(&c, &nul) == HKV_E_INVAL);
  EXPECT(check_state_buffers(&c, nullptr) == HKV_E_INVAL);
  EXPECT(check_range(d, 0, int32_t(d.S)) == HKV_OK);
  EXPECT(check_range(d, 1, int32_t(d.S)) == HKV_E_INVAL);
  EXPECT(check_range(d, -1, 1) == HKV_E_INVAL);
  EXPECT(check_range(d, INT32_MAX, INT32_MAX) == HKV_E_INVAL);
  EXPECT(check_step(&c, 39) == HKV_E_INVAL);
  EXPECT(check_step(&c, 40) == HKV_OK);
  EXPECT(check_step(&c, 200) == HKV_E_INVAL);
  const void* p16 = reinterpret_cast<const void*>(uintptr_t(1) << 21);
  EXPECT(check_data_ptr(p16, 64, 2, "x") == HKV_OK);
  EXPECT(check_data_ptr(nullptr, 64, 2, "x") == HKV_E_INVAL);
  EXPECT(check_data_ptr(reinterpret_cast<const char*>(p16) + 2, 64, 2, "x") == HKV_E_INVAL);
  EXPECT(check_data_ptr(p16, 63, 2, "x") == HKV_E_INVAL);
  EXPECT(check_data_ptr(p16, -8, 2, "x") == HKV_E_INVAL);

  // error text: truncated, never overrun; per thread
  std::string longname(4000, 'n');
  EXPECT(check_data_ptr(nullptr, 0, 2, longname.c_str()) == HKV_E_INVAL);
  EXPECT(std::strlen(hkv_last_error()) < 512);
  std::vector<std::thread> th;
  std::vector<int> ok(8, 0);
  for (int i = 0; i < 8; ++i)
    th.emplace_back([i, &ok] {
      hkv_config cc = base_cfg();
      cc.layers = -i;
      for (int k = 0; k < 200; ++k) {
        clear_error();
        if (hkv_validate(&cc) != HKV_E_INVAL) return;
        if (std::strstr(hkv_last_error(), "positive") == nullptr) return;
      }
      ok[i] = 1;
    });
  for (auto& t : th) t.join();
  for (int i = 0; i < 8; ++i) EXPECT(ok[i] == 1);
  for (int s : {0, -1, -2, -3, -4, -5, -99, INT_MIN}) EXPECT(hkv_status_string(s) != nullptr);

  if (g_fail) {
    std::fprintf(stderr, "%d host checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed under the sanitizers\n");
  return 0;
}
