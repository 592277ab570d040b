// HeadKV decode-time kernels for MI355X (gfx950) and the C-ABI entry points
// that launch them.
//
// Method (pages "Head-Aware Key-Value Compression for Efficient Autoregressive
// Image Generation", technical summary, section "Methodology"): step 2 classifies
// each head once by accumulating attention backward from the current position
// to tau; step 3 keeps a sliding window for Local heads and applies Stratified
// Token Eviction to Global heads.  The readings of the open points are listed in
// include/hkv.h.
//
// Kernels (one workgroup of 4 waves per (layer, sequence, head) stream):
//   k_classify  W x P logit tile of the observation queries, causal softmax per
//               row, reverse prefix scan of the last row -> count and label;
//               column sums -> initial scores.
//   k_layout    per-group budget from the Local count, stream offsets, pool
//               build: ring copy, plain copy, or initial STE with compaction.
//   k_step      decode step: append (optional), ragged flash-decode over the
//               stream's slots with the STE score side-output, and eviction of
//               due Global streams (optional) — fused in one launch.
#include <hip/hip_runtime.h>

#include <cmath>

#include "hkv_device.h"
#include "hkv_host.h"

namespace hkv {
namespace dev {

// Tuning knobs (compile-time): waves per workgroup, row fragments in flight per
// lane, prefetched score slots per thread, minimum waves per SIMD.
#ifndef HKV_NW
#define HKV_NW 4
#endif
#ifndef HKV_U
#define HKV_U 2
#endif
#ifndef HKV_KPT
#define HKV_KPT 1
#endif
#ifndef HKV_WPE
#define HKV_WPE 1
#endif
constexpr int kNW = HKV_NW;            // waves per workgroup
constexpr int kNT = kNW * kWave;

struct StepArgs {
  const char* k_new; const char* v_new; long long ld_kv;   // ld in elements
  const char* q; long long ld_q;
  char* out; long long ld_o;
  int* log;
  char* k_pool; char* v_pool;
  int* pos; float* score;
  const long long* base; int* count; const int* budget; const int* cap;
  const unsigned char* label;
  int* err;
  float* ws_logits; uint64_t* ws_keys;
  int s_begin, t, w, W, M, D;
  int S;                               // streams in the state (label array length)
  float scale_log2;                    // log2(e) / sqrt(head_dim)
};

struct CombineShared {
  float m[kNW];
  float l[kNW];
  float o[kNW][128];
};

struct EvictShared {
  int cnt[2];
  int nh, nm, ne;
  int holes[kMaxEvict], movers[kMaxEvict];
  int mover_rank[kMaxEvict];           // tail slot B + r -> mover index, or -1
};

// Eviction key with the subset in the top bits: (subset << 62) | (score bits <<
// 31) | position.  Scores are non-negative (sign bit clear) and positions are
// below 2**31, so inside one subset keys order by (score, position) and the
// subsets occupy disjoint key ranges.  Subset 2 = protected (not a candidate).
__device__ inline uint64_t make_skey(int sub, float score, int pos) {
  return (uint64_t(sub) << 62) | (uint64_t(__float_as_uint(score)) << 31) | uint32_t(pos);
}
__device__ inline int skey_sub(uint64_t k) { return int(k >> 62); }
__device__ inline int skey_pos(uint64_t k) { return int(uint32_t(k) & 0x7fffffffu); }
__device__ inline float skey_score(uint64_t k) { return __uint_as_float(uint32_t(k >> 31) & 0x7fffffffu); }

// Source of fragment idx of the tail rows [B, B + M): row B + idx / (2G), K
// (first G fragments of the row) or V, 16-byte piece idx % G; the token appended
// in this launch is read from its source row.
template <class T, int D, bool AP>
__device__ inline const char* tail_src_impl(const StepArgs& a, int s, long long base,
                                            int slot_new, int B, int idx) {
  constexpr int VE = Frag<T>::N, G = D / VE, ES = sizeof(T);
  const int row = B + idx / (2 * G);
  const bool isv = (idx % (2 * G)) >= G;
  const int sb = idx % G;
  if (AP && row == slot_new)
    return (isv ? a.v_new : a.k_new) + ((long long)s * a.ld_kv + sb * VE) * ES;
  return (isv ? a.v_pool : a.k_pool) + ((base + row) * D + sb * VE) * ES;
}

// Body of a decode step for one stream after its metadata is known.  `lg`,
// `keys` and `evf` are per-slot scratch: on chip (LDS) for streams of at most
// kLdsSlots slots, else in the workspace; instantiating both cases lets the
// compiler address the on-chip case with LDS instructions.
struct StepCtx {
  long long base;
  int s, lab, c, B, slot_new;
  bool glob, write_mode, due;
};

template <class T, int D, bool AP, bool AT, bool EV>
__device__ __forceinline__ void step_body(const StepArgs& a, const StepCtx& x, uint4 q_raw,
                                          float* lg, uint64_t* keys, uint8_t* evf,
                                          CombineShared& cs, EvictShared& es) {
  using F = Frag<T>;
  constexpr int VE = F::N;           // elements per 16-byte fragment
  constexpr int G = D / VE;          // lanes per row
  constexpr int R = kWave / G;       // rows per wave instruction
  constexpr int U = HKV_U;           // row fragments in flight per lane
  constexpr int ES = sizeof(T);
  constexpr int KPT = HKV_KPT;       // prefetched score slots per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane / G, sub = lane % G;
  const long long base = x.base;
  const int s = x.s, c = x.c, B = x.B, slot_new = x.slot_new;
  const bool glob = x.glob, write_mode = x.write_mode, due = x.due;
  auto tail_src = [](const StepArgs& aa, int ss, long long bb, int sn, int BB, int idx) {
    return tail_src_impl<T, D, AP>(aa, ss, bb, sn, BB, idx);
  };

  // prefetch the score window and, on an eviction step, the positions
  float sc_old[KPT > 0 ? KPT : 1];
  int pos_old[KPT > 0 ? KPT : 1];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int j = tid + k * kNT;
    const bool fresh = AP && j == slot_new;
    sc_old[k] = 0.f;
    pos_old[k] = 0;
    if (j < c && glob && !fresh && (due || (AT && !write_mode))) sc_old[k] = a.score[base + j];
    if (j < c && due) pos_old[k] = fresh ? a.t : a.pos[base + j];
  }

  // ---------------- append token t
  if (AP) {
    if (tid < 2 * G) {
      const bool isv = tid >= G;
      const int sb = tid % G;
      const char* src = (isv ? a.v_new : a.k_new) + ((long long)s * a.ld_kv + sb * VE) * ES;
      char* dst = (isv ? a.v_pool : a.k_pool) + ((base + slot_new) * D + sb * VE) * ES;
      st16(dst, ld16(src));
    }
    if (tid == 0) {
      a.pos[base + slot_new] = a.t;
      if (glob && !AT) a.score[base + slot_new] = 0.0f;
    }
  }

  // ---------------- attention over slots [0, c)
  float Mx = 0.f, inv_l = 0.f;
  if (AT) {
    float qv[VE];
    {
      float qf[VE];
      F::to_f32(q_raw, qf);
#pragma unroll
      for (int i = 0; i < VE; ++i) qv[i] = qf[i] * a.scale_log2;
    }
    const char* kbase = a.k_pool + (base * D + sub * VE) * ES;
    const char* vbase = a.v_pool + (base * D + sub * VE) * ES;
    const char* knew = a.k_new + ((long long)s * a.ld_kv + sub * VE) * ES;
    const char* vnew = a.v_new + ((long long)s * a.ld_kv + sub * VE) * ES;

    const int ntiles = (c + R - 1) / R;
    const int per = (ntiles + kNW - 1) / kNW;
    const int t0 = wave * per;
    const int t1 = min(ntiles, t0 + per);

    float m_run = kNeg, l_run = 0.f;
    float acc[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = 0.f;

    for (int tt = t0; tt < t1; tt += U) {
      uint4 kr[U], vr[U];
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = (tt + u) * R + g;
        valid[u] = (tt + u < t1) && row < c;
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
        if (valid[u]) {
          const bool fresh = AP && row == slot_new;
          kr[u] = ld16(fresh ? knew : kbase + (long long)row * D * ES);
          vr[u] = ld16(fresh ? vnew : vbase + (long long)row * D * ES);
        }
      }
      float sc[U];
      float m_tile = kNeg;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float kf[VE];
        F::to_f32(kr[u], kf);
        float d0 = 0.f;
#pragma unroll
        for (int i = 0; i < VE; ++i) d0 = fmaf(qv[i], kf[i], d0);
        d0 = group_sum<G>(d0);
        sc[u] = valid[u] ? d0 : kNeg;
        m_tile = fmaxf(m_tile, sc[u]);
        if (glob && sub == 0 && valid[u]) lg[(tt + u) * R + g] = d0;
      }
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[i] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = valid[u] ? exp2f(sc[u] - m_new) : 0.f;
        l_run += p;
        float vf[VE];
        F::to_f32(vr[u], vf);
#pragma unroll
        for (int i = 0; i < VE; ++i) acc[i] = fmaf(p, vf[i], acc[i]);
      }
      m_run = m_new;
    }
    // combine the R groups of the wave
    const float m_w = cross_group_max<G>(m_run);
    const float f = exp2f(m_run - m_w);
    l_run = cross_group_sum<G>(l_run * f);
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = cross_group_sum<G>(acc[i] * f);
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < VE; ++i) cs.o[wave][sub * VE + i] = acc[i];
      if (sub == 0) {
        cs.m[wave] = m_w;
        cs.l[wave] = l_run;
      }
    }
    __syncthreads();
    // combine the waves
    Mx = cs.m[0];
#pragma unroll
    for (int w2 = 1; w2 < kNW; ++w2) Mx = fmaxf(Mx, cs.m[w2]);
    float L = 0.f, fw[kNW];
#pragma unroll
    for (int w2 = 0; w2 < kNW; ++w2) {
      fw[w2] = exp2f(cs.m[w2] - Mx);
      L += cs.l[w2] * fw[w2];
    }
    inv_l = 1.0f / L;
    if (tid < D) {
      float o = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kNW; ++w2) o = fmaf(cs.o[w2][tid], fw[w2], o);
      T* op = reinterpret_cast<T*>(a.out + ((long long)s * a.ld_o) * ES);
      op[tid] = F::from_f32(o * inv_l);
    }
  }

  // ---------------- score side-output (Global streams) / eviction keys
  if (!AT && due) __syncthreads();                     // counters zeroed
  if (glob && (AT || due)) {
    const int t = a.t, W = a.W, Dd = a.D;
    int nn = 0, nf = 0;
    auto handle = [&](int j, float old, int pos_j) {
      const bool fresh = AP && j == slot_new;
      float ns = old;
      if (AT) {
        const float p = exp2f(lg[j] - Mx) * inv_l;
        ns = (fresh || write_mode) ? p : old + p;
      } else if (fresh) {
        ns = 0.0f;
      }
      if (due) {
        const int dist = t - pos_j;
        const int sb = dist < W ? 2 : (dist < Dd ? 0 : 1);
        nn += sb == 0;
        nf += sb == 1;
        keys[j] = make_skey(sb, ns, pos_j);
      } else {
        a.score[base + j] = ns;
      }
    };
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int j = tid + k * kNT;
      if (j < c) handle(j, sc_old[k], pos_old[k]);
    }
    for (int j = tid + KPT * kNT; j < c; j += kNT) {
      const bool fresh = AP && j == slot_new;
      const float old = (!fresh && (due || !write_mode)) ? a.score[base + j] : 0.f;
      handle(j, old, due ? (fresh ? a.t : a.pos[base + j]) : 0);
    }
    if (due) {
      nn = wave_sum_int(nn);
      nf = wave_sum_int(nf);
      if (lane == 0) {
        if (nn) atomicAdd(&es.cnt[0], nn);
        if (nf) atomicAdd(&es.cnt[1], nf);
      }
    }
  }

  // ---------------- Stratified Token Eviction (due Global streams)
  int c_final = c;
  if (EV && due) {
    // Every mover lies in the tail [B, c) (c - B = M on an eviction step): fetch
    // those rows now so the loads overlap the selection.  Fragment idx of the
    // tail: row B + idx / (2G), K or V, 16-byte piece idx % G.
    constexpr int MVF = 2;                             // fragments fetched per thread
    const int n_frag = 2 * G * (c - B);
    uint4 mv_frag[MVF];
#pragma unroll
    for (int f = 0; f < MVF; ++f) {
      const int idx = tid + f * kNT;
      mv_frag[f] = make_uint4(0, 0, 0, 0);
      if (idx < n_frag) mv_frag[f] = ld16(tail_src(a, s, base, slot_new, B, idx));
    }
    __syncthreads();                                   // keys and subset sizes complete
    // Quotas: floor(M/2) near, the rest far; a short subset gives all it has.
    const int E = a.M;
    const int nn = es.cnt[0], nf = es.cnt[1];
    int qn = E / 2, qf = E - qn;
    if (nn < qn) {
      qn = nn;
      qf = E - qn;
    } else if (nf < qf) {
      qf = nf;
      qn = E - qf;
    }
    const bool sel_ok = qn <= nn && qf <= nf;
    // Rank of each candidate inside its subset (keys of one subset form one
    // key range); evicted iff rank < quota.
    if (sel_ok) {
      for (int j = tid; j < c; j += kNT) {
        const uint64_t kj = keys[j];
        const int sb = skey_sub(kj);
        const uint64_t lo = uint64_t(sb & 1) << 62;
        int r = 0;
        int i = 0;
        for (; i + 8 <= c; i += 8) {
          uint64_t kk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) kk[u] = keys[i + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) r += (kk[u] >= lo) & (kk[u] < kj);
        }
        for (; i < c; ++i) {
          const uint64_t ki = keys[i];
          r += (ki >= lo) & (ki < kj);
        }
        evf[j] = (sb < 2 && r < (sb == 0 ? qn : qf)) ? 1 : 0;
      }
    }
    if (!sel_ok) {
      if (tid == 0) atomicOr(a.err, HKV_ERRBIT_SELECT);
      if (a.log && tid < a.M) a.log[(long long)s * a.M + tid] = -1;
    } else {
      __syncthreads();
      if (wave == 0) {
        int nh = 0, nm = 0, ne = 0;
        const uint64_t lt = lanemask_lt(lane);
        for (int j0 = 0; j0 < c; j0 += kWave) {
          const int j = j0 + lane;
          const bool in = j < c;
          const bool ev = in && evf[j];
          const bool hole = ev && j < B;
          const bool mover = in && !ev && j >= B;
          const uint64_t mh = __ballot(hole), mm = __ballot(mover), me = __ballot(ev);
          if (hole) {
            const int r = nh + __popcll(mh & lt);
            if (r < kMaxEvict) es.holes[r] = j;
          }
          if (mover) {
            const int r = nm + __popcll(mm & lt);
            if (r < kMaxEvict) es.movers[r] = j;
          }
          if (j >= B && j < B + a.M) es.mover_rank[j - B] = mover ? nm + __popcll(mm & lt) : -1;
          if (ev && a.log) {
            const int r = ne + __popcll(me & lt);
            if (r < a.M) a.log[(long long)s * a.M + r] = skey_pos(keys[j]);
          }
          nh += __popcll(mh);
          nm += __popcll(mm);
          ne += __popcll(me);
        }
        if (lane == 0) {
          es.nh = nh;
          es.nm = nm;
          es.ne = ne;
        }
        if (a.log && lane < a.M && lane >= ne) a.log[(long long)s * a.M + lane] = -1;
      }
      __syncthreads();
      const int nmv = es.nh;
      if (es.nh != es.nm || es.ne != a.M || es.nh > kMaxEvict) {
        if (tid == 0) atomicOr(a.err, HKV_ERRBIT_LAYOUT);
      } else {
        // K/V rows of the movers into the holes (tail fill), mostly from the
        // fragments fetched before the selection
        for (int idx = tid, f = 0; idx < n_frag; idx += kNT, ++f) {
          const int k = es.mover_rank[idx / (2 * G)];
          if (k < 0) continue;
          uint4 v;
          if (f < MVF) {
#pragma unroll
            for (int ff = 0; ff < MVF; ++ff)
              if (ff == f) v = mv_frag[ff];
          } else {
            v = ld16(tail_src(a, s, base, slot_new, B, idx));
          }
          const bool isv = (idx % (2 * G)) >= G;
          st16((isv ? a.v_pool : a.k_pool) + ((base + es.holes[k]) * D + (idx % G) * VE) * ES, v);
        }
        if (tid < nmv) {
          const uint64_t mk = keys[es.movers[tid]];
          a.pos[base + es.holes[tid]] = skey_pos(mk);
          a.score[base + es.holes[tid]] = skey_score(mk);
        }
        if (AT) {   // deferred score writes of the kept slots below the budget
          for (int j = tid; j < B; j += kNT)
            if (!evf[j]) a.score[base + j] = skey_score(keys[j]);
        }
        c_final = B;
      }
    }
  } else if (EV && a.log && tid < a.M) {
    a.log[(long long)s * a.M + tid] = -1;
  }

  if (tid == 0 && (AP || c_final != c)) a.count[s] = c_final;
}

// ------------------------------------------------------------------ k_step
// One workgroup per stream.  Every thread reads the stream's metadata itself
// (uniform loads, no barrier); the query, the score window and the positions
// needed by an eviction are requested together with the first K/V rows.
template <class T, int D, bool AP, bool AT, bool EV>
__global__ __launch_bounds__(kNT, HKV_WPE) void k_step(StepArgs a) {
  using F = Frag<T>;
  constexpr int VE = F::N;           // elements per 16-byte fragment
  constexpr int G = D / VE;          // lanes per row
  constexpr int R = kWave / G;       // rows per wave instruction
  constexpr int U = HKV_U;           // row fragments in flight per lane
  constexpr int ES = sizeof(T);
  constexpr int KPT = HKV_KPT;       // prefetched score slots per thread

  __shared__ CombineShared cs;
  __shared__ EvictShared es;
  __shared__ float lds_lg[AT ? kLdsSlots : 1];
  __shared__ uint64_t lds_key[EV ? kLdsSlots : 1];
  __shared__ uint8_t lds_evf[EV ? kLdsSlots : 1];
  (void)R; (void)U; (void)KPT;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = a.s_begin + blockIdx.x;
  const int g = lane / G, sub = lane % G;
  if (EV && tid < 2) es.cnt[tid] = 0;

  // query fragment first: its address does not depend on the stream metadata
  uint4 q_raw = make_uint4(0, 0, 0, 0);
  if (AT) q_raw = ld16(a.q + ((long long)s * a.ld_q + sub * VE) * ES);

  // the label byte through the scalar path (aligned 32-bit word), except in a
  // last partial word
  int lab;
  if (4LL * ((s >> 2) + 1) <= a.S)
    lab = int((reinterpret_cast<const uint32_t*>(a.label)[s >> 2] >> ((s & 3) * 8)) & 0xffu);
  else
    lab = a.label[s];
  const int c0 = a.count[s];
  const int capv = a.cap[s];
  const int B = a.budget[s];
  const long long base = a.base[s];
  const bool glob = lab == HKV_GLOBAL;
  int c = c0, slot_new = -1;
  bool ok = true;
  if (AP) {
    if (lab == HKV_LOCAL) {
      slot_new = a.t % a.w;
      c = c0 + 1 < a.w ? c0 + 1 : a.w;
    } else {
      slot_new = c0;
      c = c0 + 1;
      if (c0 >= capv) {
        ok = false;
        if (tid == 0) atomicOr(a.err, HKV_ERRBIT_CAPACITY);
      }
    }
  }
  if (ok && (c < 1 || c > capv || lab > HKV_FULL)) {
    ok = false;
    if (tid == 0) atomicOr(a.err, HKV_ERRBIT_LAYOUT);
  }
  if (!ok) {
    if (EV && a.log && tid < a.M) a.log[(long long)s * a.M + tid] = -1;
    return;
  }
  const bool write_mode = glob && (c == B + a.M - a.W + 1);
  const bool due = EV && glob && (c == B + a.M);

  StepCtx x;
  x.base = base;
  x.s = s;
  x.lab = lab;
  x.c = c;
  x.B = B;
  x.slot_new = slot_new;
  x.glob = glob;
  x.write_mode = write_mode;
  x.due = due;
  (void)lane; (void)wave; (void)g;
  if (c <= kLdsSlots)
    step_body<T, D, AP, AT, EV>(a, x, q_raw, lds_lg, lds_key, lds_evf, cs, es);
  else
    step_body<T, D, AP, AT, EV>(a, x, q_raw, a.ws_logits + base, a.ws_keys + base,
                                reinterpret_cast<uint8_t*>(a.ws_logits + base), cs, es);
}

// ------------------------------------------------------------------ k_classify
struct ClassifyArgs {
  const char* k_stage; long long ld_stage;
  const char* q_obs; long long ld_qobs;
  float* init_scores;          // [S, P]
  int* n_tokens; unsigned char* label;
  int P, W, w;
  float tau, scale_log2;
};

template <class T, int D>
__global__ __launch_bounds__(kNT) void k_classify(ClassifyArgs a) {
  using F = Frag<T>;
  constexpr int VE = F::N, G = D / VE, R = kWave / G, ES = sizeof(T);
  constexpr int WM = 8;                     // observation queries held per lane
  extern __shared__ float lg[];             // [W][P]
  __shared__ float mrow[WM], lrow[WM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x;
  const int P = a.P, W = a.W;
  const int g = lane / G, sub = lane % G;

  float qv[WM][VE];
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    float qf[VE];
    if (i < W) {
      F::to_f32(ld16(a.q_obs + ((long long)s * a.ld_qobs + (long long)i * D + sub * VE) * ES), qf);
    } else {
#pragma unroll
      for (int e = 0; e < VE; ++e) qf[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < VE; ++e) qv[i][e] = qf[e] * a.scale_log2;
  }

  const char* kb = a.k_stage + ((long long)s * a.ld_stage + sub * VE) * ES;
  for (int j0 = wave * R; j0 < P; j0 += kNW * R) {
    const int j = j0 + g;
    float kf[VE];
    if (j < P) {
      F::to_f32(ld16(kb + (long long)j * D * ES), kf);
    } else {
#pragma unroll
      for (int e = 0; e < VE; ++e) kf[e] = 0.f;
    }
    float mine = 0.f;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      float d0 = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) d0 = fmaf(qv[i][e], kf[e], d0);
      d0 = group_sum<G>(d0);
      if (i == sub) mine = d0;
    }
    if (j < P && sub < W) lg[sub * P + j] = mine;
  }
  __syncthreads();

  // softmax statistics of each observation query over its causal span
  for (int i = wave; i < W; i += kNW) {
    const int lim = P - W + i;              // query position; keys 0..lim
    float m = kNeg;
    for (int j = lane; j <= lim; j += kWave) m = fmaxf(m, lg[i * P + j]);
    m = wave_max(m);
    float l = 0.f;
    for (int j = lane; j <= lim; j += kWave) l += exp2f(lg[i * P + j] - m);
    l = wave_sum(l);
    if (lane == 0) {
      mrow[i] = m;
      lrow[i] = l;
    }
  }
  __syncthreads();

  // count: attention of the last query accumulated backward from position P-1
  if (wave == 0) {
    const int i = W - 1;
    const float m = mrow[i], inv = 1.0f / lrow[i];
    float carry = 0.f;
    int n = P;
    for (int d0 = 0; d0 < P; d0 += kWave) {
      const int dist = d0 + lane;
      const float p = dist < P ? exp2f(lg[i * P + (P - 1 - dist)] - m) * inv : 0.f;
      const float x = wave_inclusive_scan(p, lane) + carry;
      const uint64_t hit = __ballot(dist < P && x >= a.tau);
      if (hit) {
        n = d0 + __ffsll((unsigned long long)hit);   // 1-based lane index = count
        break;
      }
      carry = __shfl(x, 63);
    }
    if (lane == 0) {
      a.n_tokens[s] = n;
      a.label[s] = n < a.w ? HKV_LOCAL : HKV_GLOBAL;
    }
  }
  // initial scores: column sums of the causal W x P probability tile
  for (int j = tid; j < P; j += kNT) {
    float sc = 0.f;
    for (int i = 0; i < W; ++i)
      if (j <= P - W + i) sc += exp2f(lg[i * P + j] - mrow[i]) * (1.0f / lrow[i]);
    a.init_scores[(long long)s * P + j] = sc;
  }
}

// ------------------------------------------------------------------ k_layout
struct LayoutArgs {
  const char* k_stage; const char* v_stage; long long ld_stage;
  const float* init_scores;
  char* k_pool; char* v_pool;
  int* pos; float* score;
  long long* base; int* cap; int* count; int* budget; int* n_tokens; unsigned char* label;
  int* err;
  int H, N, P, w, W, M, D, A, full;
  long long group_slots;
};

template <class T, int D>
__global__ __launch_bounds__(kNT) void k_layout(LayoutArgs a) {
  constexpr int VE = Frag<T>::N, G = D / VE, ES = sizeof(T);
  __shared__ long long s_base;
  __shared__ int s_lab, s_B, s_count, s_mode;   // mode: 0 copy P, 1 ring, 2 STE
  __shared__ SelectShared ss;
  __shared__ uint64_t keys[kMaxPrefill];
  __shared__ int dest[kMaxPrefill];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x;
  const int P = a.P;

  if (tid == 0) {
    if (a.full) {
      s_base = (long long)s * a.N;
      s_lab = HKV_FULL;
      s_B = a.N;
      s_count = P;
      s_mode = 0;
      a.cap[s] = a.N;
      a.n_tokens[s] = 0;
      a.label[s] = HKV_FULL;
    } else {
      const int grp = s / a.H, h = s % a.H;
      const unsigned char* lab = a.label + (long long)grp * a.H;
      int n_l = 0;
      for (int x = 0; x < a.H; ++x) n_l += lab[x] == HKV_LOCAL;
      const int n_g = a.H - n_l;
      const int Bg = n_g ? (a.H * a.A - n_l * a.w) / n_g : 0;
      long long off = (long long)grp * a.group_slots;
      for (int x = 0; x < h; ++x) off += lab[x] == HKV_LOCAL ? a.w : Bg + a.M;
      s_base = off;
      s_lab = lab[h];
      if (lab[h] == HKV_LOCAL) {
        s_B = a.w;
        s_count = P < a.w ? P : a.w;
        s_mode = 1;
        a.cap[s] = a.w;
      } else {
        s_B = Bg;
        s_count = P <= Bg ? P : Bg;
        s_mode = P <= Bg ? 0 : 2;
        a.cap[s] = Bg + a.M;
      }
    }
    a.base[s] = s_base;
    a.budget[s] = s_B;
    a.count[s] = s_count;
  }
  __syncthreads();
  const long long base = s_base;
  const int mode = s_mode;
  const char* ks = a.k_stage + (long long)s * a.ld_stage * ES;
  const char* vs = a.v_stage + (long long)s * a.ld_stage * ES;

  if (mode == 2) {
    // initial STE at t = P-1 over the prefill with the window scores
    for (int j = tid; j < P; j += kNT) keys[j] = make_key(a.init_scores[(long long)s * P + j], j);
    const int E = P - s_B;
    ste_quotas<kNT>(keys, P, P - 1, a.W, a.D, E, ss);
    if (!ss.ok) {
      if (tid == 0) atomicOr(a.err, HKV_ERRBIT_SELECT);
      return;
    }
    ste_radix_select<kNT>(keys, P, P - 1, a.W, a.D, ss);
    if (wave == 0) {
      int kept = 0;
      const uint64_t lt = lanemask_lt(lane);
      for (int j0 = 0; j0 < P; j0 += kWave) {
        const int j = j0 + lane;
        const bool keep = j < P && !is_evicted(keys[j], P - 1, a.W, a.D, ss);
        const uint64_t mk = __ballot(keep);
        const int rank = kept + __popcll(mk & lt);
        if (j < P) dest[j] = (keep && rank < s_B) ? rank : -1;
        kept += __popcll(mk);
      }
      if (lane == 0 && kept != s_B) atomicOr(a.err, HKV_ERRBIT_LAYOUT);
    }
    __syncthreads();
  } else {
    for (int j = tid; j < P; j += kNT) {
      if (mode == 1) dest[j] = (j >= P - a.w) ? j % a.w : -1;
      else dest[j] = j;
    }
    __syncthreads();
  }
  for (int idx = tid; idx < P * 2 * G; idx += kNT) {
    const int j = idx / (2 * G), r = idx % (2 * G);
    const int to = dest[j];
    if (to < 0) continue;
    const bool isv = r >= G;
    const int sub = r % G;
    const char* src = (isv ? vs : ks) + ((long long)j * D + sub * VE) * ES;
    st16((isv ? a.v_pool : a.k_pool) + ((base + to) * D + sub * VE) * ES, ld16(src));
  }
  for (int j = tid; j < P; j += kNT) {
    const int to = dest[j];
    if (to < 0) continue;
    a.pos[base + to] = j;
    a.score[base + to] = (s_lab == HKV_GLOBAL) ? a.init_scores[(long long)s * P + j] : 0.0f;
  }
}

__global__ void k_reset_err(int* err) { *err = 0; }

}  // namespace dev

// ------------------------------------------------------------------ host glue
namespace {

hkv_status hip_fail(hipError_t e, const char* what) {
  return fail(HKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

hkv_status after_launch(const char* what) {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? HKV_OK : hip_fail(e, what);
}

template <class T, int D, bool AP, bool AT, bool EV>
void launch_step_t(const dev::StepArgs& a, int n, hipStream_t st) {
  hipLaunchKernelGGL((dev::k_step<T, D, AP, AT, EV>), dim3(n), dim3(dev::kNT), 0, st, a);
}

template <bool AP, bool AT, bool EV>
void launch_step(const hkv_config* c, const dev::StepArgs& a, int n, hipStream_t st) {
  if (c->dtype == HKV_DT_BF16) {
    if (c->head_dim == 64) launch_step_t<uint16_t, 64, AP, AT, EV>(a, n, st);
    else launch_step_t<uint16_t, 128, AP, AT, EV>(a, n, st);
  } else {
    if (c->head_dim == 64) launch_step_t<float, 64, AP, AT, EV>(a, n, st);
    else launch_step_t<float, 128, AP, AT, EV>(a, n, st);
  }
}

float scale_log2_of(int d) { return float(1.4426950408889634 / std::sqrt(double(d))); }

dev::StepArgs step_args(const hkv_config* c, hkv_state* st, const Derived& d, int t) {
  dev::StepArgs a{};
  a.k_pool = static_cast<char*>(st->k_pool);
  a.v_pool = static_cast<char*>(st->v_pool);
  a.pos = st->pos;
  a.score = st->score;
  a.base = reinterpret_cast<const long long*>(st->base);
  a.count = st->count;
  a.budget = st->budget;
  a.cap = st->cap;
  a.label = st->label;
  a.err = st->err;
  a.ws_logits = reinterpret_cast<float*>(static_cast<char*>(st->workspace) + d.ws_logits);
  a.ws_keys = reinterpret_cast<uint64_t*>(static_cast<char*>(st->workspace) + d.ws_keys);
  a.t = t;
  a.w = c->local_window;
  a.W = c->w_obs;
  a.M = c->evict_m;
  a.D = c->split_dist;
  a.scale_log2 = scale_log2_of(c->head_dim);
  a.S = int(d.S);
  return a;
}

hkv_status common_checks(const hkv_config* c, hkv_state* st, int32_t t, int32_t s_begin,
                         int32_t s_count, Derived* d) {
  clear_error();
  hkv_status r = derive(c, d);
  if (r != HKV_OK) return r;
  if ((r = check_state_buffers(c, st)) != HKV_OK) return r;
  if (st->phase != 1) return fail(HKV_E_STATE, "state not classified (call hkv_classify first)");
  if ((r = check_step(c, t)) != HKV_OK) return r;
  return check_range(*d, s_begin, s_count);
}

}  // namespace
}  // namespace hkv

using namespace hkv;

extern "C" {

hkv_status hkv_classify(const hkv_config* c, hkv_state* st, const void* k_stage,
                        const void* v_stage, int64_t ld_stage, const void* q_obs,
                        int64_t ld_qobs, void* stream) {
  clear_error();
  Derived d;
  hkv_status r = derive(c, &d);
  if (r != HKV_OK) return r;
  if ((r = check_state_buffers(c, st)) != HKV_OK) return r;
  const int eb = elem_bytes(c);
  if ((r = check_data_ptr(k_stage, ld_stage, eb, "k_stage")) != HKV_OK) return r;
  if ((r = check_data_ptr(v_stage, ld_stage, eb, "v_stage")) != HKV_OK) return r;
  if (ld_stage < int64_t(c->prefill_len) * c->head_dim)
    return fail(HKV_E_INVAL, "ld_stage smaller than prefill_len * head_dim");
  if (!c->full_cache) {
    if ((r = check_data_ptr(q_obs, ld_qobs, eb, "q_obs")) != HKV_OK) return r;
    if (ld_qobs < int64_t(c->w_obs) * c->head_dim)
      return fail(HKV_E_INVAL, "ld_qobs smaller than w_obs * head_dim");
    if (c->w_obs > 8) return fail(HKV_E_UNSUPPORTED, "classification holds at most 8 queries");
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(st->workspace);
  float* init_scores = reinterpret_cast<float*>(ws + d.ws_init_scores);

  hipLaunchKernelGGL(dev::k_reset_err, dim3(1), dim3(1), 0, hs, st->err);
  if ((r = after_launch("reset")) != HKV_OK) return r;

  if (!c->full_cache) {
    dev::ClassifyArgs a{};
    a.k_stage = static_cast<const char*>(k_stage);
    a.ld_stage = ld_stage;
    a.q_obs = static_cast<const char*>(q_obs);
    a.ld_qobs = ld_qobs;
    a.init_scores = init_scores;
    a.n_tokens = st->n_tokens;
    a.label = st->label;
    a.P = c->prefill_len;
    a.W = c->w_obs;
    a.w = c->local_window;
    a.tau = c->tau;
    a.scale_log2 = scale_log2_of(c->head_dim);
    const size_t lds = size_t(c->w_obs) * c->prefill_len * sizeof(float);
    const int n = int(d.S);
    if (c->dtype == HKV_DT_BF16) {
      if (c->head_dim == 64)
        hipLaunchKernelGGL((dev::k_classify<uint16_t, 64>), dim3(n), dim3(dev::kNT), lds, hs, a);
      else
        hipLaunchKernelGGL((dev::k_classify<uint16_t, 128>), dim3(n), dim3(dev::kNT), lds, hs, a);
    } else {
      if (c->head_dim == 64)
        hipLaunchKernelGGL((dev::k_classify<float, 64>), dim3(n), dim3(dev::kNT), lds, hs, a);
      else
        hipLaunchKernelGGL((dev::k_classify<float, 128>), dim3(n), dim3(dev::kNT), lds, hs, a);
    }
    if ((r = after_launch("k_classify")) != HKV_OK) return r;
  }

  dev::LayoutArgs b{};
  b.k_stage = static_cast<const char*>(k_stage);
  b.v_stage = static_cast<const char*>(v_stage);
  b.ld_stage = ld_stage;
  b.init_scores = init_scores;
  b.k_pool = static_cast<char*>(st->k_pool);
  b.v_pool = static_cast<char*>(st->v_pool);
  b.pos = st->pos;
  b.score = st->score;
  b.base = reinterpret_cast<long long*>(st->base);
  b.cap = st->cap;
  b.count = st->count;
  b.budget = st->budget;
  b.n_tokens = st->n_tokens;
  b.label = st->label;
  b.err = st->err;
  b.H = c->heads;
  b.N = c->final_len;
  b.P = c->prefill_len;
  b.w = c->local_window;
  b.W = c->w_obs;
  b.M = c->evict_m;
  b.D = c->split_dist;
  b.A = d.A;
  b.full = c->full_cache;
  b.group_slots = d.group_slots;
  const int n = int(d.S);
  if (c->dtype == HKV_DT_BF16) {
    if (c->head_dim == 64)
      hipLaunchKernelGGL((dev::k_layout<uint16_t, 64>), dim3(n), dim3(dev::kNT), 0, hs, b);
    else
      hipLaunchKernelGGL((dev::k_layout<uint16_t, 128>), dim3(n), dim3(dev::kNT), 0, hs, b);
  } else {
    if (c->head_dim == 64)
      hipLaunchKernelGGL((dev::k_layout<float, 64>), dim3(n), dim3(dev::kNT), 0, hs, b);
    else
      hipLaunchKernelGGL((dev::k_layout<float, 128>), dim3(n), dim3(dev::kNT), 0, hs, b);
  }
  if ((r = after_launch("k_layout")) != HKV_OK) return r;
  st->phase = 1;
  return HKV_OK;
}

hkv_status hkv_append(const hkv_config* c, hkv_state* st, int32_t t, const void* k_new,
                      const void* v_new, int64_t ld_kv, int32_t s_begin, int32_t s_count,
                      void* stream) {
  Derived d;
  hkv_status r = common_checks(c, st, t, s_begin, s_count, &d);
  if (r != HKV_OK) return r;
  const int eb = elem_bytes(c);
  if ((r = check_data_ptr(k_new, ld_kv, eb, "k_new")) != HKV_OK) return r;
  if ((r = check_data_ptr(v_new, ld_kv, eb, "v_new")) != HKV_OK) return r;
  if (s_count == 0) return HKV_OK;
  dev::StepArgs a = step_args(c, st, d, t);
  a.k_new = static_cast<const char*>(k_new);
  a.v_new = static_cast<const char*>(v_new);
  a.ld_kv = ld_kv;
  a.s_begin = s_begin;
  launch_step<true, false, false>(c, a, s_count, static_cast<hipStream_t>(stream));
  return after_launch("k_step(append)");
}

hkv_status hkv_decode_attn(const hkv_config* c, hkv_state* st, int32_t t, const void* q,
                           int64_t ld_q, void* out, int64_t ld_o, int32_t s_begin,
                           int32_t s_count, void* stream) {
  Derived d;
  hkv_status r = common_checks(c, st, t, s_begin, s_count, &d);
  if (r != HKV_OK) return r;
  const int eb = elem_bytes(c);
  if ((r = check_data_ptr(q, ld_q, eb, "q")) != HKV_OK) return r;
  if (!out) return fail(HKV_E_INVAL, "out is NULL");
  if ((reinterpret_cast<uintptr_t>(out) & 3u) || ld_o < c->head_dim)
    return fail(HKV_E_INVAL, "out misaligned or ld_o < head_dim");
  if (s_count == 0) return HKV_OK;
  dev::StepArgs a = step_args(c, st, d, t);
  a.q = static_cast<const char*>(q);
  a.ld_q = ld_q;
  a.out = static_cast<char*>(out);
  a.ld_o = ld_o;
  a.s_begin = s_begin;
  launch_step<false, true, false>(c, a, s_count, static_cast<hipStream_t>(stream));
  return after_launch("k_step(attn)");
}

hkv_status hkv_ste_evict(const hkv_config* c, hkv_state* st, int32_t t, int32_t* log,
                         int32_t s_begin, int32_t s_count, void* stream) {
  Derived d;
  hkv_status r = common_checks(c, st, t, s_begin, s_count, &d);
  if (r != HKV_OK) return r;
  if (log && (reinterpret_cast<uintptr_t>(log) & 3u))
    return fail(HKV_E_INVAL, "evicted_pos_log misaligned");
  if (s_count == 0) return HKV_OK;
  dev::StepArgs a = step_args(c, st, d, t);
  a.log = log;
  a.s_begin = s_begin;
  launch_step<false, false, true>(c, a, s_count, static_cast<hipStream_t>(stream));
  return after_launch("k_step(evict)");
}

hkv_status hkv_decode_step(const hkv_config* c, hkv_state* st, int32_t t, const void* k_new,
                           const void* v_new, int64_t ld_kv, const void* q, int64_t ld_q,
                           void* out, int64_t ld_o, int32_t* log, int32_t s_begin,
                           int32_t s_count, void* stream) {
  Derived d;
  hkv_status r = common_checks(c, st, t, s_begin, s_count, &d);
  if (r != HKV_OK) return r;
  const int eb = elem_bytes(c);
  if ((r = check_data_ptr(k_new, ld_kv, eb, "k_new")) != HKV_OK) return r;
  if ((r = check_data_ptr(v_new, ld_kv, eb, "v_new")) != HKV_OK) return r;
  if ((r = check_data_ptr(q, ld_q, eb, "q")) != HKV_OK) return r;
  if (!out) return fail(HKV_E_INVAL, "out is NULL");
  if ((reinterpret_cast<uintptr_t>(out) & 3u) || ld_o < c->head_dim)
    return fail(HKV_E_INVAL, "out misaligned or ld_o < head_dim");
  if (log && (reinterpret_cast<uintptr_t>(log) & 3u))
    return fail(HKV_E_INVAL, "evicted_pos_log misaligned");
  if (s_count == 0) return HKV_OK;
  dev::StepArgs a = step_args(c, st, d, t);
  a.k_new = static_cast<const char*>(k_new);
  a.v_new = static_cast<const char*>(v_new);
  a.ld_kv = ld_kv;
  a.q = static_cast<const char*>(q);
  a.ld_q = ld_q;
  a.out = static_cast<char*>(out);
  a.ld_o = ld_o;
  a.log = log;
  a.s_begin = s_begin;
  launch_step<true, true, true>(c, a, s_count, static_cast<hipStream_t>(stream));
  return after_launch("k_step(fused)");
}

hkv_status hkv_check(const hkv_config* c, const hkv_state* st, void* stream) {
  clear_error();
  Derived d;
  hkv_status r = derive(c, &d);
  if (r != HKV_OK) return r;
  if (!st || !st->err) return fail(HKV_E_INVAL, "state or err is NULL");
  int host = 0;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&host, st->err, sizeof(int), hipMemcpyDeviceToHost, hs);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(err)");
  e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  if (host & HKV_ERRBIT_CAPACITY) return fail(HKV_E_CAPACITY, "device error bits 0x%x", host);
  if (host) return fail(HKV_E_STATE, "device error bits 0x%x", host);
  return HKV_OK;
}

}  // extern "C"
