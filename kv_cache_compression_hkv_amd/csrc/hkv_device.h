// Device building blocks for the HeadKV kernels on CDNA4 (gfx950, wave64):
// 16-byte row fragments, DPP reductions inside a row group, and the bottom-k
// radix select used by Stratified Token Eviction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hkv {
namespace dev {

constexpr int kWave = 64;
constexpr float kNeg = -3.0e38f;       // finite "minus infinity" for masked logits

// ---------------------------------------------------------------- element types
// A lane moves one 16-byte fragment of a row: 8 bf16 or 4 fp32 values.
template <class T>
struct Frag;

template <>
struct Frag<uint16_t> {                 // bf16 bit patterns
  static constexpr int N = 8;
  __device__ static inline void to_f32(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
    f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xffff0000u);
    f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xffff0000u);
  }
  // fp32 -> bf16, round to nearest even (finite inputs)
  __device__ static inline uint16_t from_f32(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
  }
};

template <>
struct Frag<float> {
  static constexpr int N = 4;
  __device__ static inline void to_f32(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
  __device__ static inline float from_f32(float x) { return x; }
};

__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming load of a 16-byte fragment that is read once per launch (cached K/V
// rows): non-temporal, so it does not displace the small per-stream data that
// every launch reads again.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
#ifndef HKV_NT_LOADS
#define HKV_NT_LOADS 1
#endif
__device__ inline uint4 ld16_stream(const void* p) {
#if HKV_NT_LOADS
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return ld16(p);
#endif
}
// The same for the other data read once per launch (queries, the appended
// row's source); a separate switch so that each can be measured alone.
#ifndef HKV_NT_ONCE
#define HKV_NT_ONCE 1
#endif
__device__ inline uint4 ld16_once(const void* p) {
#if HKV_NT_ONCE
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return ld16(p);
#endif
}
__device__ inline void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
// Non-temporal store of a 16-byte fragment: the appended rows, scattered over
// the pool one row per stream, are written past the caches' retention.
__device__ inline void st16_stream(void* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

// ---------------------------------------------------------------- reductions
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of G lanes (G = 8, 16 or 32); every lane of the
// group receives the total.  xor-1 and xor-2 by quad permutes, then the half-row
// and row mirrors, then a swizzle across 16-lane rows.
template <int G>
__device__ inline float group_sum(float x) {
  x += dpp<0xB1>(x);                       // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);                       // quad_perm [2,3,0,1]
  if constexpr (G >= 8) x += dpp<0x141>(x);    // row_half_mirror
  if constexpr (G >= 16) x += dpp<0x140>(x);   // row_mirror
  if constexpr (G >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Reductions across the groups of a wave (lanes with the same offset in their group).
template <int G>
__device__ inline float cross_group_max(float x) {
#pragma unroll
  for (int off = G; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
template <int G>
__device__ inline float cross_group_sum(float x) {
#pragma unroll
  for (int off = G; off < kWave; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ inline float wave_max(float x) { return cross_group_max<1>(x); }

__device__ inline int wave_sum_int(int x) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off);
  return x;
}
__device__ inline float wave_sum(float x) { return cross_group_sum<1>(x); }

// Inclusive prefix sum over the wave (Hillis-Steele).
template <class V>
__device__ inline V wave_inclusive_scan(V x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    V y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ inline uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---------------------------------------------------------------- eviction keys
// key = (score bits << 32) | position.  Scores are non-negative, so the fp32
// bit pattern orders like the value; positions break ties (older first).  Keys
// are unique because positions are.
__device__ inline uint64_t make_key(float score, int pos) {
  return (uint64_t(__float_as_uint(score)) << 32) | uint32_t(pos);
}
__device__ inline int key_pos(uint64_t k) { return int(uint32_t(k)); }
__device__ inline float key_score(uint64_t k) { return __uint_as_float(uint32_t(k >> 32)); }

// Subset of a slot at step t: 0 near (W <= t-pos < D), 1 far (t-pos >= D),
// 2 protected (t-pos < W, not a candidate).
__device__ inline int subset_of(uint64_t k, int t, int W, int D) {
  const int dist = t - key_pos(k);
  return dist < W ? 2 : (dist < D ? 0 : 1);
}

struct SelectShared {
  uint32_t hist[2][256];
  uint64_t prefix[2];
  uint64_t thr[2];
  int krem[2];
  int done[2];
  int cnt[2];
  int quota[2];
  int ok;
};

// Counts the near/far candidates among keys[0..n) and sets the quotas for E
// evictions: floor(E/2) near and the rest far; a short subset gives all it has
// and the other makes up the difference.  Result in sh.quota / sh.ok.
template <int NT>
__device__ void ste_quotas(const uint64_t* keys, int n, int t, int W, int D, int E,
                           SelectShared& sh) {
  const int tid = threadIdx.x;
  if (tid < 2) sh.cnt[tid] = 0;
  __syncthreads();
  int nn = 0, nf = 0;
  for (int j = tid; j < n; j += NT) {
    const int sb = subset_of(keys[j], t, W, D);
    nn += sb == 0;
    nf += sb == 1;
  }
  if (nn) atomicAdd(&sh.cnt[0], nn);
  if (nf) atomicAdd(&sh.cnt[1], nf);
  __syncthreads();
  if (tid == 0) {
    int qn = E / 2, qf = E - qn;
    if (sh.cnt[0] < qn) {
      qn = sh.cnt[0];
      qf = E - qn;
    } else if (sh.cnt[1] < qf) {
      qf = sh.cnt[1];
      qn = E - qf;
    }
    sh.ok = (qn <= sh.cnt[0] && qf <= sh.cnt[1]) ? 1 : 0;
    sh.quota[0] = qn;
    sh.quota[1] = qf;
  }
  __syncthreads();
}

// MSD radix select, 8-bit digits: for each subset b with quota q_b > 0 finds
// the q_b-th smallest key, thr[b].  A slot is evicted iff its key <= thr of its
// subset.  Both subsets share the passes; a subset finishes as soon as the
// bucket holding its threshold contains exactly the keys still needed.
template <int NT>
__device__ void ste_radix_select(const uint64_t* keys, int n, int t, int W, int D,
                                 SelectShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    for (int b = 0; b < 2; ++b) {
      sh.prefix[b] = 0;
      sh.thr[b] = 0;
      sh.krem[b] = sh.quota[b];
      sh.done[b] = sh.quota[b] == 0;
    }
  }
  for (int shift = 56; shift >= 0; shift -= 8) {
    __syncthreads();
    if (sh.done[0] && sh.done[1]) break;
    for (int i = tid; i < 512; i += NT) (&sh.hist[0][0])[i] = 0;
    __syncthreads();
    const uint64_t hi = shift == 56 ? 0ull : (~0ull << (shift + 8));
    for (int j = tid; j < n; j += NT) {
      const uint64_t k = keys[j];
      const int sb = subset_of(k, t, W, D);
      if (sb < 2 && !sh.done[sb] && ((k ^ sh.prefix[sb]) & hi) == 0)
        atomicAdd(&sh.hist[sb][(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    for (int sb = wave; sb < 2; sb += NT / 64) {
      if (sh.done[sb]) continue;
      const uint32_t* h = sh.hist[sb];
      const uint32_t c0 = h[4 * lane], c1 = h[4 * lane + 1], c2 = h[4 * lane + 2],
                     c3 = h[4 * lane + 3];
      const uint32_t tot = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_inclusive_scan(tot, lane);
      const uint32_t ex = incl - tot;
      const uint32_t k = uint32_t(sh.krem[sb]);
      if (ex < k && k <= incl) {
        uint32_t before = ex, bin = 4 * lane, cb = c0;
        if (k > before + c0) { before += c0; bin += 1; cb = c1;
          if (k > before + c1) { before += c1; bin += 1; cb = c2;
            if (k > before + c2) { before += c2; bin += 1; cb = c3; } } }
        const uint64_t pre = sh.prefix[sb] | (uint64_t(bin) << shift);
        const uint32_t rem = k - before;
        sh.prefix[sb] = pre;
        sh.krem[sb] = int(rem);
        if (rem == cb || shift == 0) {
          sh.thr[sb] = pre | ((shift ? (1ull << shift) : 1ull) - 1ull);
          sh.done[sb] = 1;
        }
      }
    }
  }
  __syncthreads();
}

__device__ inline bool is_evicted(uint64_t k, int t, int W, int D, const SelectShared& sh) {
  const int sb = subset_of(k, t, W, D);
  return sb < 2 && sh.quota[sb] > 0 && k <= sh.thr[sb];
}

}  // namespace dev
}  // namespace hkv
