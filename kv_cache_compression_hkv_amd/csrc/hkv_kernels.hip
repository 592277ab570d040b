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
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "hkv_device.h"
#include "hkv_host.h"

namespace hkv {
namespace dev {

// Tuning knobs (compile-time): waves per workgroup, row fragments in flight per
// lane (per element type and head size), key tiles in flight per wave on the
// matrix-core path.
#ifndef HKV_NW
#define HKV_NW 4
#endif
#ifndef HKV_U_B64
#define HKV_U_B64 4
#endif
#ifndef HKV_U_B128S            // bf16 d128, short streams
#define HKV_U_B128S 3
#endif
#ifndef HKV_U_B128L            // bf16 d128, long streams
#define HKV_U_B128L 3
#endif
#ifndef HKV_U_F32
#define HKV_U_F32 2
#endif
#ifndef HKV_UT
#define HKV_UT 1
#endif
// Occupancy the compiler schedules the decode step for (waves per SIMD): it
// bounds the registers and so decides how many loads the hot loop keeps in
// flight per wave versus how many waves overlap.  Measured on MI355X.
#ifndef HKV_WPE_B64
#define HKV_WPE_B64 6
#endif
#ifndef HKV_WPE_B128S
#define HKV_WPE_B128S 7
#endif
#ifndef HKV_WPE_B128L
#define HKV_WPE_B128L 5
#endif
#ifndef HKV_WPE_F32
#define HKV_WPE_F32 4
#endif
constexpr int kNW = HKV_NW;            // waves per workgroup
constexpr int kNT = kNW * kWave;

// Key tiles in flight per wave in the eviction's matrix-core passes (bf16 d128,
// short / long streams).
#ifndef HKV_UE_S
#define HKV_UE_S 1
#endif
#ifndef HKV_UE_L
#define HKV_UE_L 2
#endif
// ... when that pass is the only one (window statistics from the ring)
#ifndef HKV_UER_S
#define HKV_UER_S 1
#endif
#ifndef HKV_UER_L
#define HKV_UER_L 2
#endif
// The split decode step's attention kernel: row fragments in flight per lane
// and occupancy (0: those of the fused step), key tiles in flight in its
// scoring pass.  Its grids hold a few workgroups per compute unit.
#ifndef HKV_U_SPLIT
#define HKV_U_SPLIT 0
#endif
#ifndef HKV_WPE_SPLIT
#define HKV_WPE_SPLIT 0
#endif
#ifndef HKV_UE_SPLIT
#define HKV_UE_SPLIT 1
#endif
// Pool rows: each slot holds its K row and its V row side by side ([slot][2][D]
// elements; v_pool = k_pool + D elements), so a slot's rows lie in one
// 2*D-element span; kPoolRow<D> is the pool's row stride in elements.  (The
// appended rows of a step, one slot per stream scattered over the pool, are
// then written to one place per stream instead of two: 1-2% faster per launch
// on the d128 workloads, the same on LlamaGen-XL; measured on MI355X.)
template <int D>
constexpr int kPoolRow = 2 * D;
template <int V>
struct Int {
  static constexpr int value = V;
};
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2):
// block b runs on XCD b % 8.  Both mappings below keep the streams that share a
// cache line of per-stream data (16 per 64 B) on one L2; each is a bijection of
// [0, n).
//   CH = 0: each XCD takes one contiguous run of n/8 streams.
//   CH > 0: chunks of CH consecutive streams are dealt to the XCDs in turn (a
//   ragged tail of fewer than 8*CH blocks maps to itself), so that every XCD
//   gets a like share of every layer.  Where labels, budgets or eviction steps
//   differ between layers, a contiguous run per XCD leaves some XCDs with more
//   work than others, and the launch lasts as long as the busiest.
#ifndef HKV_XCD_REMAP
#define HKV_XCD_REMAP 1
#endif
constexpr int kXcds = 8;
template <int CH = 0>
__device__ __forceinline__ int xcd_block(int b, int n) {
#if HKV_XCD_REMAP
  const int x = b % kXcds, i = b / kXcds;
  if constexpr (CH > 0) {
    const int n_full = n / (kXcds * CH) * (kXcds * CH);
    if (b >= n_full) return b;
    return ((i / CH) * kXcds + x) * CH + i % CH;
  } else {
    const int q = n / kXcds, r = n % kXcds;
    return x * q + (x < r ? x : r) + i;
  }
#else
  (void)n;
  return b;
#endif
}

struct StepArgs {
  const char* k_new; const char* v_new; long long ld_kv;   // ld in elements
  const char* q; long long ld_q;                            // current query
  const char* q_win; long long ld_qw;                       // last W queries, oldest first
  char* out; long long ld_o;
  int* log;
  char* k_pool; char* v_pool;
  int* pos; float* score;
  const long long* base; int* count; const int* budget; const int* cap;
  const unsigned char* label;
  int* free_slots; int* n_free;
  float4* qstat;                       // [S, W] ring of query statistics (max, 1/sum, step)
  int* err;
  float* ws_tile; int* ws_pos; uint64_t* ws_keys;   // per-slot spill
  int s_begin, t, w, W, M, D;
  int S;                               // streams in the state (label array length)
  float scale_log2;                    // log2(e) / sqrt(head_dim)
  int res64;                           // streams with s % 64 < res64 are resident
};

struct CombineShared {
  float m[kNW];
  float l[kNW];
  float o[kNW][128];
};

struct EvictShared {
  float4 ring[kMaxWobs];               // the stream's query-statistics ring, staged (bf16 d64)
  int cnt[2];
  float qm[kMaxWobs], ql[kMaxWobs];    // softmax max / 1/sum of each window query
  float pm[kNW][kMaxWobs], pl[kNW][kMaxWobs];   // per-wave partials of the tile pass
  uint64_t cand_key[2][kNW][kMaxEvict];  // per subset and wave: its bottom-q keys
  int cand_slot[2][kNW][kMaxEvict];
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

// Minimum of a 64-bit value over the wave (uniform result): DPP inside each
// 16-lane row (quad xor 1, quad xor 2, half-row mirror, row mirror), then the
// four row minima read out to scalars.
template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_mov_dpp(int(uint32_t(x)), CTRL, 0xF, 0xF, true));
  const uint32_t hi = uint32_t(__builtin_amdgcn_mov_dpp(int(uint32_t(x >> 32)), CTRL, 0xF, 0xF, true));
  return (uint64_t(hi) << 32) | lo;
}
__device__ inline uint64_t readlane_u64(uint64_t x, int l) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(x)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(x >> 32)), l));
  return (uint64_t(hi) << 32) | lo;
}
__device__ inline uint64_t wave_min_u64(uint64_t x) {
  uint64_t y;
  y = dpp_u64<0xB1>(x);  x = y < x ? y : x;
  y = dpp_u64<0x4E>(x);  x = y < x ? y : x;
  y = dpp_u64<0x141>(x); x = y < x ? y : x;
  y = dpp_u64<0x140>(x); x = y < x ? y : x;
  uint64_t m = readlane_u64(x, 0);
#pragma unroll
  for (int r = 16; r < kWave; r += 16) {
    const uint64_t v = readlane_u64(x, r);
    m = v < m ? v : m;
  }
  return m;
}

struct StepCtx {
  long long base;
  int s, lab, c, B, slot_new;          // c: slots holding a token (no free slot when due)
  bool glob, due;
  bool resident;                       // rows loaded with caching (kept across launches)
};

// Per-slot scratch of an eviction: the W x c logit tile and the positions, or
// (when the eviction forms the keys itself) the keys.  On chip (LDS) for
// streams up to the kernel's on-chip size, else in the workspace, which then
// also holds the keys of the slots beyond the registers' share; instantiating
// both cases lets the compiler address the on-chip case with LDS instructions.
struct Scratch {
  float* tile;
  int* pos;
  uint64_t* keys;
};

// ------------------------------------------------------------------ eviction
// Stratified Token Eviction of one due Global stream (c == B + M slots):
//   1. scores: with a query window, the causal W x c probability tile of the
//      last W queries (query i at position t-W+1+i sees slots with pos <= its
//      position), summed over the queries; without one, the state's scores;
//   2. keys (subset, score, position); near/far sizes and quotas;
//   3. the quota's lowest keys of each subset: each wave's own bottom-q, then
//      the exact rank inside the union of the waves' candidates;
//   4. the evicted slots are freed (position -1, listed ascending in the free
//      list for the next appends); no row moves.  Returns n_free = M.
// Attention of a bf16 Global stream at its eviction point on the matrix cores
// (one pass yields the output and the W x c scoring tile), or on the vector
// ALUs like every other stream, the eviction then forming the tile in a second
// matrix-core pass over K (loaded with caching in the first).  The first keeps
// the d64 kernel at 6 waves/SIMD; for d128 its registers would cap the whole
// kernel at 4 waves, the second runs at 8 (short streams) or 5 (long).
// Measured on MI355X.
#ifndef HKV_MFMA_ATTN_B64
#define HKV_MFMA_ATTN_B64 1
#endif
#ifndef HKV_MFMA_ATTN_B128
#define HKV_MFMA_ATTN_B128 0
#endif
template <class T, int D>
struct StepMfmaAttn {
  static constexpr bool value =
      sizeof(T) == 2 && (D == 64 ? HKV_MFMA_ATTN_B64 != 0 : HKV_MFMA_ATTN_B128 != 0);
};

// Shape of the decode step per element type, head size and stream class C.
// bf16 d128 has two: short streams (C = 0) run 7 waves/SIMD, long streams
// (C = 1) 5 waves, both with 3 rows in flight per lane; the host picks the class
// from the configured budget.  C = 2 is the bf16 d64 eviction of the split
// decode step, which has no matrix-core attention pass to take its tile from
// and scores its slots from K like d128.
//
// How an eviction scores its slots, and how many its scratch holds on chip.
// bf16 with the attention on the vector ALUs (kKeys): on the matrix cores, either
// in one pass that keeps the W x c logit tile on chip (short streams up to
// kOnePass slots) or in two passes over K, the first for each window query's
// softmax statistics and the second writing each slot's key directly (8 bytes
// per slot, in the same on-chip buffer).  Otherwise the tile and the positions
// (36 bytes per slot) come from the attention (bf16 d64) or a vector-ALU pass
// (fp32).  Sizes measured on MI355X: the d128 short-stream kernel's LDS stays
// small enough for its 7 workgroups per CU (8 would fit too).
#ifndef HKV_ONCHIP_KEYS
#define HKV_ONCHIP_KEYS 1280
#endif
#ifndef HKV_ONEPASS_S
#define HKV_ONEPASS_S 320
#endif
#ifndef HKV_ONCHIP_TILE_B16
#define HKV_ONCHIP_TILE_B16 512
#endif
#ifndef HKV_ONCHIP_TILE_F32
#define HKV_ONCHIP_TILE_F32 512
#endif
template <class T, int D, int C>
struct StepCfg {
  static constexpr bool kB16 = sizeof(T) == 2;
  static constexpr int kWaves =
      !kB16 ? HKV_WPE_F32 : (D == 64 ? HKV_WPE_B64 : (C ? HKV_WPE_B128L : HKV_WPE_B128S));
  static constexpr int kRows =
      !kB16 ? HKV_U_F32 : (D == 64 ? HKV_U_B64 : (C ? HKV_U_B128L : HKV_U_B128S));
  static constexpr int kTilesInFlight = C ? HKV_UE_L : HKV_UE_S;
  static constexpr int kTilesInFlightRing = C ? HKV_UER_L : HKV_UER_S;
  static constexpr bool kKeys = kB16 && (C == 2 || !StepMfmaAttn<T, D>::value);
  // a share of the streams reads its rows with caching (decided per stream)
  static constexpr bool kResident = kB16 && D == 128;
  // streams per chunk of the XCD mapping (xcd_block): bf16 d128 workloads mix
  // Local and Global streams unevenly over the layers; bf16 d64 ran 1.5%
  // faster on contiguous runs (measured on MI355X)
  static constexpr int kXcdChunk = kB16 && D == 128 ? 64 : 0;
  static constexpr int kOnePass = kKeys && !C ? HKV_ONEPASS_S : 0;
  static constexpr int kSlots =
      kKeys ? HKV_ONCHIP_KEYS : (kB16 ? HKV_ONCHIP_TILE_B16 : HKV_ONCHIP_TILE_F32);
  static_assert(!kKeys || kMaxWobs * kOnePass * 4 <= kSlots * 8, "tile fits the keys buffer");
};

// Window queries of a bf16 stream staged on chip for the eviction's score tile:
// W rows of D elements, 16 bytes of padding per row so that the 16-byte reads of
// consecutive rows fall in distinct banks.
template <int D>
struct QStage {
  static constexpr int kPitch = D / 4 + 2;   // row pitch in 8-byte units
  // 8-byte units per thread: one, or two (16 bytes) when the workgroup has
  // fewer threads than the W rows have 8-byte pieces
  static constexpr int kPer = (kMaxWobs * D / 4 + kNT - 1) / kNT;
  static_assert(kPer == 1 || kPer == 2, "one or two 8-byte pieces per thread");
  using Piece = typename std::conditional<kPer == 1, uint2, uint4>::type;
  // query row and 8-byte column of thread tid's piece
  __device__ static int row(int tid) { return tid / (D / 4 / kPer); }
  __device__ static int col(int tid) { return (tid % (D / 4 / kPer)) * kPer; }
  // thread tid's piece of stream s's window queries (rows beyond W: not read)
  __device__ static Piece load(const char* q_win, long long row0, int tid) {
    return *reinterpret_cast<const Piece*>(q_win + (row0 + (long long)row(tid) * D + col(tid) * 4) * 2);
  }
  __device__ static void store(uint2* qs, int tid, Piece v) {
    *reinterpret_cast<Piece*>(qs + row(tid) * kPitch + col(tid)) = v;
  }
};

// Window statistics of an eviction taken from the query-statistics ring when
// its entries are current (1), or always formed by the eviction itself (0).
#ifndef HKV_RING
#define HKV_RING 1
#endif

// Softmax max and 1/sum of window queries 0 .. nq-1 over the slots each sees
// (query i: position <= t - W + 1 + i), from the W x c logit tile; one wave per
// query.  Kept out of line: it is the eviction's fallback when the ring of
// query statistics is stale, and inlined it would cost the decode step
// registers on every launch.
__device__ __noinline__ void window_stats(const int* pos, const float* tile, int c, int t, int W,
                                          int nq, float* qm, float* ql) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = wave; i < nq; i += kNW) {
    const int lim = t - W + 1 + i;
    float m = kNeg;
    for (int j = lane; j < c; j += kWave)
      if (pos[j] <= lim) m = fmaxf(m, tile[i * c + j]);
    m = wave_max(m);
    float l = 0.f;
    for (int j = lane; j < c; j += kWave)
      if (pos[j] <= lim) l += exp2f(tile[i * c + j] - m);
    l = wave_sum(l);
    if (lane == 0) {
      qm[i] = m;
      ql[i] = 1.0f / l;
    }
  }
}

template <class T, int D, int C, bool AP>
__device__ __forceinline__ int evict_stream(const StepArgs& a, const StepCtx& x, Scratch sc,
                                            EvictShared& es, uint64_t* skeys, bool tile_ready,
                                            uint2* qs, bool q_staged, bool cur_known,
                                            float cur_m, float cur_il, const float4* ring_lds,
                                            bool split_scores = false) {
  // (returns the number of freed slots: M, or 0 if nothing was evicted; skeys:
  // on-chip room for kNT keys, free once the eviction starts; es.cnt zeroed
  // by the caller before a barrier; cur_known: this launch's attention gave
  // the current query's softmax max cur_m and 1/sum cur_il; ring_lds: the
  // stream's ring row staged on chip before a barrier, or null; split_scores
  // (bf16): the split decode step's workgroups left each slot's partial score
  // and current-query logit in the workspace, see k_split_attn)
  using F = Frag<T>;
  constexpr int VE = F::N, G = D / VE, R = kWave / G, ES = sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane / G, sub = lane % G;
  const long long base = x.base;
  const int s = x.s, c = x.c, slot_new = x.slot_new;
  const int t = a.t, W = a.W, Dd = a.D;

  const bool window = a.q_win != nullptr;
  constexpr uint64_t kNone = ~0ull;    // no slot (subset field 3)
  // slots tid + k*kNT, k < SPT, have their keys in registers for the selection;
  // any further ones are read from the scratch keys
  constexpr int SPT = 2;
  uint64_t kv[SPT];
  // streams of at most kNT slots are selected by wave 0 alone, over every key:
  // from the scratch keys when the keys were formed there, else from skeys
  const bool small = c <= kNT;
  bool keys_in_scratch = false;
  auto sub_of = [&](int pj) {
    const int dist = t - pj;
    return dist < W ? 2 : (dist < Dd ? 0 : 1);
  };

  using OC = StepCfg<T, D, C>;
  if constexpr (OC::kKeys) {
    // bf16 with the attention on the vector ALUs.  With a query window the
    // matrix cores form the logits: in one pass that also keeps the W x c tile
    // and the positions on chip (streams up to kOnePass slots), or in two, the
    // second writing the keys directly to the scratch.  Without one the keys
    // come from the state's scores.
    int nn = 0, nf = 0;                // subset sizes seen by this wave
    // statistics of the W window queries from the ring: the attention of each
    // of the last W decode steps left its query's max and 1/sum there (the
    // current one's also come from this launch's attention).  No eviction
    // happens inside the window (M = W), so the slots a window query saw are
    // exactly those whose position does not exceed its own, and its
    // probabilities follow from its logits and these two numbers.  Lane i < W
    // holds query i's; a stale entry (a step whose attention did not run)
    // sends the stream down the path that forms the statistics itself.
    float rm = 0.f, ril = 0.f;
    bool rok = true;
    if (window && lane < W) {
      const int step = t - W + 1 + lane;
      if (lane == W - 1 && cur_known) {
        rm = cur_m;
        ril = cur_il;
      } else {
        const float4 e = a.qstat[(long long)s * W + step % W];
        rm = e.x;
        ril = e.y;
        rok = __float_as_int(e.z) == step;
      }
    }
    const bool ring = HKV_RING && window && __ballot(!rok) == 0;   // (the same in every wave)
    const bool one_pass = window && !split_scores && !ring && c <= OC::kOnePass;
    keys_in_scratch = !one_pass;
    if (window && !split_scores) {
      // v_mfma_f32_16x16x32_bf16: A = the W queries (rows W..15 zero), B = 16
      // keys per tile, K = 32 head elements per instruction; lane l holds A row
      // l%16 and B column l%16 at elements (l/16)*8 .. +7, and receives D rows
      // (l/16)*4 .. +3, column l%16.
      typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      constexpr int KC = D / 32;
      const int li = lane % 16, lk = lane / 16;
      constexpr int QP = QStage<D>::kPitch;
      if (!q_staged) {
        // (a standalone eviction stages the window queries here)
        using QS = QStage<D>;
        if (QS::row(tid) < W) QS::store(qs, tid, QS::load(a.q_win, (long long)s * a.ld_qw, tid));
        __syncthreads();
      }
      // A operand chunk kc of this lane: query row li, elements lk*8 + kc*32 .. +7,
      // read from the staged rows at each use (rows W..15 are zero)
      auto qa_of = [&](int kc) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (li < W) u = *reinterpret_cast<const uint4*>(qs + li * QP + lk * 2 + kc * 8);
        return __builtin_bit_cast(bf16x8, u);
      };
      const char* knew = a.k_new + ((long long)s * a.ld_kv) * ES;
      const int ntile = (c + 15) / 16;
      // one pass over the slots' key tiles: UE tiles in flight per wave (absent
      // tiles skipped, ragged columns zeroed); body(j, valid, position, logits)
      auto tiles = [&](auto ue, auto&& body) {
        constexpr int UE = decltype(ue)::value;
        for (int kt0 = wave; kt0 < ntile; kt0 += kNW * UE) {
          uint4 kb[UE][KC];
          int pj[UE];
          bool vj[UE];
#pragma unroll
          for (int u = 0; u < UE; ++u) {
            const int j = (kt0 + u * kNW) * 16 + li;
            const bool tile_in = kt0 + u * kNW < ntile;     // uniform across the wave
            vj[u] = tile_in && j < c;
            if (tile_in) {
              const int jj = vj[u] ? j : 0;
              const bool fresh = AP && jj == slot_new;
              const char* row = fresh ? knew : a.k_pool + ((base + jj) * kPoolRow<D>) * ES;
#pragma unroll
              for (int kc = 0; kc < KC; ++kc) kb[u][kc] = ld16(row + (lk * 8 + kc * 32) * ES);
              pj[u] = fresh ? t : a.pos[base + jj];
            } else {
#pragma unroll
              for (int kc = 0; kc < KC; ++kc) kb[u][kc] = make_uint4(0, 0, 0, 0);
              pj[u] = 0;
            }
          }
#pragma unroll
          for (int u = 0; u < UE; ++u) {
            if (kt0 + u * kNW >= ntile) break;                // uniform
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa_of(kc), __builtin_bit_cast(bf16x8, kb[u][kc]),
                                                            acc, 0, 0, 0);
            body((kt0 + u * kNW) * 16 + li, vj[u], pj[u], acc);
          }
        }
      };

      // pass 1 (without the ring's statistics): each lane's online softmax
      // statistics of its 4 query rows over the slots each query sees; reduced
      // over the 16 key columns, then waves (one pass: also the tile and the
      // positions)
      if (!ring) {
      float wm[4], wl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wm[r] = kNeg;
        wl[r] = 0.f;
      }
      tiles(Int<OC::kTilesInFlight>{}, [&](int j, bool vj, int pj, const f32x4& acc) {
        if (one_pass && lk == 0 && vj) sc.pos[j] = pj;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = lk * 4 + r;
          const float v = acc[r] * a.scale_log2;
          if (one_pass && vj && i < W) sc.tile[i * c + j] = v;
          const bool vis = vj && i < W && pj <= t - W + 1 + i;
          const float vv = vis ? v : kNeg;
          const float mn = fmaxf(wm[r], vv);
          wl[r] = wl[r] * exp2f(wm[r] - mn) + (vis ? exp2f(vv - mn) : 0.f);
          wm[r] = mn;
        }
      });
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mm = wm[r];
        mm = fmaxf(mm, dpp<0xB1>(mm));
        mm = fmaxf(mm, dpp<0x4E>(mm));
        mm = fmaxf(mm, dpp<0x141>(mm));
        mm = fmaxf(mm, dpp<0x140>(mm));
        const float ll = group_sum<16>(wl[r] * exp2f(wm[r] - mm));
        const int i = lk * 4 + r;
        if (li == 0 && i < W) {
          es.pm[wave][i] = mm;
          es.pl[wave][i] = ll;
        }
      }
      __syncthreads();
      if (tid < W) {                   // combine the waves' statistics of query tid
        float M = kNeg;
#pragma unroll
        for (int w2 = 0; w2 < kNW; ++w2) M = fmaxf(M, es.pm[w2][tid]);
        float L = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kNW; ++w2) L += es.pl[w2][tid] * exp2f(es.pm[w2][tid] - M);
        es.qm[tid] = M;
        es.ql[tid] = 1.0f / L;
      }
      __syncthreads();                 // window statistics (and tile) complete
      }

      if (one_pass) {
        // scores from the tile: thread tid owns slots tid + k*kNT
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
          const int j = tid + k * kNT;
          kv[k] = kNone;
          if (j < c) {
            const int pj = sc.pos[j];
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < kMaxWobs; ++i)
              if (i < W && pj <= t - W + 1 + i) v += exp2f(sc.tile[i * c + j] - es.qm[i]) * es.ql[i];
            kv[k] = make_skey(sub_of(pj), v, pj);
          }
          const int sb = int(kv[k] >> 62);
          nn += __popcll(__ballot(sb == 0));
          nf += __popcll(__ballot(sb == 1));
        }
        if (small && tid < c) skeys[tid] = kv[0];
      } else {
        // pass 2: the same logits, now as probabilities summed over each slot's
        // visible queries (rows 0-3 in lanes 0-15, rows 4-7 in lanes 16-31);
        // lanes 0-15 write the keys
        // (probability = 2^(logit - max) / sum = 2^(logit - (max + log2 sum)))
        float qm_r[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = lk * 4 + r;
          const float m_ring = __shfl(rm, i & 15), il_ring = __shfl(ril, i & 15);
          const float m = ring ? m_ring : es.qm[i & 7], il = ring ? il_ring : es.ql[i & 7];
          qm_r[r] = i < W ? m - __log2f(il) : 0.f;
        }
        auto key_of = [&](int j, bool vj, int pj, const f32x4& acc) {
          float pr = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = lk * 4 + r;
            if (vj && i < W && pj <= t - W + 1 + i) pr += exp2f(acc[r] * a.scale_log2 - qm_r[r]);
          }
          pr += __shfl_xor(pr, 16);
          const bool own = lk == 0 && vj;
          const int sb = sub_of(pj);
          if (own) sc.keys[j] = make_skey(sb, pr, pj);
          nn += __popcll(__ballot(own && sb == 0));
          nf += __popcll(__ballot(own && sb == 1));
        };
        // with the ring's statistics this is the only pass over K: more of its
        // tiles in flight
        if (ring)
          tiles(Int<OC::kTilesInFlightRing>{}, key_of);
        else
          tiles(Int<OC::kTilesInFlight>{}, key_of);
      }
    } else {
      // keys from the split workgroups' scores (the current query's share
      // added here, with its merged max and sum), or from the state's scores
      __syncthreads();                 // subset counters zeroed before any wave adds
      for (int j0 = wave * kWave; j0 < c; j0 += kNT) {
        const int j = j0 + lane;
        const bool own = j < c;
        int pj = 0;
        float sv = 0.f;
        if (own) {
          if (split_scores) {
            const float2 v = reinterpret_cast<const float2*>(a.ws_tile + base * W)[j];
            pj = a.ws_pos[base + j];
            sv = v.x + exp2f(v.y - (cur_m - __log2f(cur_il)));   // (log2 of 2^max * sum)
          } else {
            const bool fresh = AP && j == slot_new;
            pj = fresh ? t : a.pos[base + j];
            sv = fresh ? 0.0f : a.score[base + j];
          }
        }
        const int sb = sub_of(pj);
        if (own) sc.keys[j] = make_skey(sb, sv, pj);
        nn += __popcll(__ballot(own && sb == 0));
        nf += __popcll(__ballot(own && sb == 1));
      }
    }
    if (lane == 0) {
      if (nn) atomicAdd(&es.cnt[0], nn);
      if (nf) atomicAdd(&es.cnt[1], nf);
    }
    if (tid < 2 * kNW * kMaxEvict) (&es.cand_key[0][0][0])[tid] = kNone;   // unused entries
    __syncthreads();                   // keys and subset sizes
    if (!one_pass && !small) {
#pragma unroll
      for (int k = 0; k < SPT; ++k) {
        const int j = tid + k * kNT;
        kv[k] = j < c ? sc.keys[j] : kNone;
      }
    }
  } else {
    // the W x c tile of logits, then the scores.  Positions of all slots
    // (already staged by the attention when tile_ready).
    if (!tile_ready)
      for (int j = tid; j < c; j += kNT) sc.pos[j] = (AP && j == slot_new) ? t : a.pos[base + j];
    if (window && !tile_ready) {
      if constexpr (StepMfmaAttn<T, D>::value) {
        // the attention's matrix-core pass always delivers this tile
        if (tid == 0) atomicOr(a.err, HKV_ERRBIT_LAYOUT);
        if (a.log && tid < a.M) a.log[(long long)s * a.M + tid] = -1;
        return 0;
      } else {
        // fp32: each lane keeps its fragment of every window query in registers
        float qf[kMaxWobs][VE];
#pragma unroll
        for (int i = 0; i < kMaxWobs; ++i) {
          float tmp[VE];
          if (i < W) {
            F::to_f32(ld16(a.q_win + ((long long)s * a.ld_qw + (long long)i * D + sub * VE) * ES), tmp);
          } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) tmp[e] = 0.f;
          }
#pragma unroll
          for (int e = 0; e < VE; ++e) qf[i][e] = tmp[e] * a.scale_log2;
        }
        const char* kbase = a.k_pool + (base * kPoolRow<D> + sub * VE) * ES;
        const char* knew = a.k_new + ((long long)s * a.ld_kv + sub * VE) * ES;
        for (int j0 = wave * R; j0 < c; j0 += kNW * R) {
          const int j = j0 + g;
          if (j < c) {
            float kf[VE];
            F::to_f32(ld16((AP && j == slot_new) ? knew : kbase + (long long)j * kPoolRow<D> * ES), kf);
            float mine = 0.f;
#pragma unroll
            for (int i = 0; i < kMaxWobs; ++i) {
              float d0 = 0.f;
#pragma unroll
              for (int e = 0; e < VE; ++e) d0 = fmaf(qf[i][e], kf[e], d0);
              d0 = group_sum<G>(d0);
              if (i == sub) mine = d0;
            }
            if (sub < W) sc.tile[sub * c + j] = mine;
          }
        }
      }
      __syncthreads();
    }
    // softmax statistics of each window query over the slots it sees.  With a
    // tile from the attention the current query's came with it, and the
    // earlier ones come from the ring when it is current (lanes i < W-1 of
    // every wave read entry i, so every wave takes the same branch).
    if (window) {
      bool ring = false;
      if (tile_ready && HKV_RING) {
        bool ok = true;
        float4 e = make_float4(0.f, 0.f, 0.f, 0.f);
        if (lane < W - 1) {
          const int step = t - W + 1 + lane;
          e = ring_lds ? ring_lds[step % W] : a.qstat[(long long)s * W + step % W];
          ok = __float_as_int(e.z) == step;
        }
        ring = __ballot(!ok) == 0;
        if (ring && wave == 0 && lane < W - 1) {
          es.qm[lane] = e.x;
          es.ql[lane] = e.y;
        }
      }
      if (!ring) window_stats(sc.pos, sc.tile, c, t, W, tile_ready ? W - 1 : W, es.qm, es.ql);
    }
    __syncthreads();            // tile, positions and window statistics complete

    // scores and keys of the slots.  Thread tid owns slots tid + k*kNT: the
    // first SPT in registers, any further ones (streams beyond the on-chip
    // size) as keys in the workspace, each read back only by the thread that
    // wrote it.
    int nn = 0, nf = 0;
    auto score_of = [&](int j, int pj) {
      float v = 0.f;
      if (window) {
#pragma unroll
        for (int i = 0; i < kMaxWobs; ++i)
          if (i < W && pj <= t - W + 1 + i) v += exp2f(sc.tile[i * c + j] - es.qm[i]) * es.ql[i];
      } else {
        v = (AP && j == slot_new) ? 0.0f : a.score[base + j];
      }
      return v;
    };
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int j = tid + k * kNT;
      kv[k] = kNone;
      if (j < c) {
        const int pj = sc.pos[j];
        kv[k] = make_skey(sub_of(pj), score_of(j, pj), pj);
      }
      const int sb = int(kv[k] >> 62);
      const uint64_t m0 = __ballot(sb == 0), m1 = __ballot(sb == 1);
      if (lane == 0) {
        nn += __popcll(m0);
        nf += __popcll(m1);
      }
    }
    for (int j = tid + SPT * kNT; j < c; j += kNT) {
      const int pj = sc.pos[j];
      const int sb = sub_of(pj);
      nn += sb == 0;
      nf += sb == 1;
      sc.keys[j] = make_skey(sb, score_of(j, pj), pj);
    }
    if (c > SPT * kNT) {
      nn = wave_sum_int(nn);
      nf = wave_sum_int(nf);
    }
    if (small && tid < c) skeys[tid] = kv[0];
    if (lane == 0) {
      if (nn) atomicAdd(&es.cnt[0], nn);
      if (nf) atomicAdd(&es.cnt[1], nf);
    }
    if (tid < 2 * kNW * kMaxEvict) (&es.cand_key[0][0][0])[tid] = kNone;   // unused entries
    __syncthreads();            // subset sizes
  }

  // quotas: floor(M/2) near, the rest far; a short subset gives all it has
  const int E = a.M;
  const int n_near = es.cnt[0], n_far = es.cnt[1];
  int qn = E / 2, qf = E - qn;
  if (n_near < qn) {
    qn = n_near;
    qf = E - qn;
  } else if (n_far < qf) {
    qf = n_far;
    qn = E - qf;
  }
  if (qn > n_near || qf > n_far) {
    if (tid == 0) atomicOr(a.err, HKV_ERRBIT_SELECT);
    if (a.log && tid < a.M) a.log[(long long)s * a.M + tid] = -1;
    return 0;
  }

  if (small) {
    // wave 0 alone, keys of slots lane + 64*i (i < 4).  Subset 0 keys lie in
    // [0, 2^62), subset 1 in [2^62, 2^63): each round takes the smallest key of
    // each subset at or above its lower bound, and the bound moves past it, so
    // after q rounds a subset's evicted keys are exactly those below its bound.
    if (wave != 0) return 0;
    constexpr uint64_t kSub1 = 1ull << 62, kSub2 = 2ull << 62;
    const uint64_t* src = keys_in_scratch ? sc.keys : skeys;
    uint64_t k4[kNT / kWave];
#pragma unroll
    for (int i = 0; i < kNT / kWave; ++i) {
      const int j = lane + i * kWave;
      k4[i] = j < c ? src[j] : kNone;
    }
    uint64_t lo0 = 0, lo1 = kSub1;
    const int qmax = qn > qf ? qn : qf;
    for (int r = 0; r < qmax; ++r) {
      uint64_t my0 = kSub1, my1 = kSub2;     // (no key)
#pragma unroll
      for (int i = 0; i < kNT / kWave; ++i) {
        const uint64_t kk = k4[i];
        if (kk >= lo0 && kk < my0) my0 = kk;
        if (kk >= lo1 && kk < my1) my1 = kk;
      }
      const uint64_t m0 = wave_min_u64(r < qn ? my0 : kSub1);
      const uint64_t m1 = wave_min_u64(r < qf ? my1 : kSub2);
      if (m0 < kSub1) lo0 = m0 + 1;
      if (m1 < kSub2) lo1 = m1 + 1;
    }
    // the evicted slots, listed in ascending slot order
    int ne = 0;
#pragma unroll
    for (int i = 0; i < kNT / kWave; ++i) {
      const uint64_t kk = k4[i];
      const bool ev = kk < lo0 || (kk >= kSub1 && kk < lo1);
      const uint64_t bal = __ballot(ev);
      const int rs = ne + __popcll(bal & ((1ull << lane) - 1));
      const int j = lane + i * kWave;
      if (ev && rs < a.M) {
        a.free_slots[(long long)s * a.M + rs] = j;
        if (a.log) a.log[(long long)s * a.M + rs] = skey_pos(kk);
        a.pos[base + j] = -1;
      }
      if (a.log && j < c) a.score[base + j] = skey_score(kk);
      ne += __popcll(bal);
    }
    if (a.log && lane < a.M && lane >= ne) a.log[(long long)s * a.M + lane] = -1;
    if (ne != a.M) {
      if (lane == 0) atomicOr(a.err, HKV_ERRBIT_LAYOUT);
      return 0;
    }
    return a.M;
  }

  // bottom-q of each subset in two levels.  Every wave takes its own q smallest
  // keys, one per round: the wave-wide minimum over the keys above the previous
  // round's minimum (keys are unique).  The union over the waves holds the
  // subset's q smallest; wave 0 ranks the union.
  {
    uint64_t prev0 = 0, prev1 = 0;
    int n0 = 0, n1 = 0;
    const int qmax = qn > qf ? qn : qf;
    for (int r = 0; r < qmax; ++r) {
      uint64_t my0 = kNone, my1 = kNone;
      int j0 = 0, j1 = 0;
#pragma unroll
      for (int k = 0; k < SPT; ++k) {
        const uint64_t kk = kv[k];
        const int sb = int(kk >> 62);
        if (sb == 0 && (n0 == 0 || kk > prev0) && kk < my0) { my0 = kk; j0 = tid + k * kNT; }
        if (sb == 1 && (n1 == 0 || kk > prev1) && kk < my1) { my1 = kk; j1 = tid + k * kNT; }
      }
      for (int j = tid + SPT * kNT; j < c; j += kNT) {
        const uint64_t kk = sc.keys[j];
        const int sb = int(kk >> 62);
        if (sb == 0 && (n0 == 0 || kk > prev0) && kk < my0) { my0 = kk; j0 = j; }
        if (sb == 1 && (n1 == 0 || kk > prev1) && kk < my1) { my1 = kk; j1 = j; }
      }
      const uint64_t m0 = wave_min_u64(r < qn ? my0 : kNone);
      const uint64_t m1 = wave_min_u64(r < qf ? my1 : kNone);
      if (m0 != kNone) {
        if (my0 == m0) {
          es.cand_key[0][wave][n0] = m0;
          es.cand_slot[0][wave][n0] = j0;
        }
        prev0 = m0;
        ++n0;
      }
      if (m1 != kNone) {
        if (my1 == m1) {
          es.cand_key[1][wave][n1] = m1;
          es.cand_slot[1][wave][n1] = j1;
        }
        prev1 = m1;
        ++n1;
      }
    }
  }
  __syncthreads();              // candidates of every wave

  // wave 0: lanes 0-31 rank the near candidates, lanes 32-63 the far ones
  // (entry e of the union; unused entries hold kNone); the evicted slots are
  // listed in ascending slot order (free list, log) and freed
  static_assert(kNW * kMaxEvict <= 32, "candidate union must fit half a wave");
  int ne_all = a.M;
  if (wave == 0) {
    constexpr int NC = kNW * kMaxEvict;
    const int sub = lane >> 5, e = lane & 31;
    const uint64_t* ck = &es.cand_key[sub][0][0];
    const uint64_t mine = e < NC ? ck[e] : kNone;
    int rank = 0;
#pragma unroll
    for (int e2 = 0; e2 < NC; ++e2) rank += ck[e2] < mine;
    const bool ev = mine != kNone && rank < (sub == 0 ? qn : qf);
    const uint64_t evm = __ballot(ev);
    const int ne = __popcll(evm);
    const int j = ev ? (&es.cand_slot[sub][0][0])[e] : 0;
    int rs = 0;                                // rank of the slot among the evicted
    for (uint64_t mm = evm; mm; mm &= mm - 1) {
      const int l = __ffsll((unsigned long long)mm) - 1;
      rs += __builtin_amdgcn_readlane(j, l) < j;
    }
    if (ev && rs < a.M) {
      a.free_slots[(long long)s * a.M + rs] = j;
      if (a.log) a.log[(long long)s * a.M + rs] = skey_pos(mine);
      a.pos[base + j] = -1;
    }
    if (a.log && lane < a.M && lane >= ne) a.log[(long long)s * a.M + lane] = -1;
    ne_all = ne;
  }
  // with a log, the scores the event ranked (every slot, the evicted ones
  // included; the append that refills a freed slot resets its score)
  if (a.log) {
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int j = tid + k * kNT;
      if (j < c) a.score[base + j] = skey_score(kv[k]);
    }
    for (int j = tid + SPT * kNT; j < c; j += kNT) a.score[base + j] = skey_score(sc.keys[j]);
  }
  // (only wave 0's value is used: the epilogue runs on thread 0)
  if (ne_all != a.M) {
    if (tid == 0) atomicOr(a.err, HKV_ERRBIT_LAYOUT);
    return 0;
  }
  return a.M;
}

// ------------------------------------------------------------------ attention (bf16)
// Flash-decode over the slots [0, c) of one stream with the logits on the matrix
// cores.  v_mfma_f32_16x16x32_bf16 with A = queries (16 rows), B = 16 keys: rows
// 3, 7, 11 and 15 of A hold the current query, so every lane receives the
// current logit of its key column in D[.][3]; on an eviction step the other
// rows hold the W-1 earlier window queries (row (i/3)*4 + i%3 for query i) and
// the W x c scoring tile comes out of the same instructions.  Lane l holds key
// column l%16 and head elements (l/16)*8 + 32*kc .. +7 of K and V; softmax and
// P.V run per lane on its column and are reduced over the 16 columns at the end.
template <int D, bool AP, bool KC_>
__device__ __forceinline__ void attend_mfma(const StepArgs& a, const StepCtx& x, bool due,
                                            Scratch sc, CombineShared& cs) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  using F = Frag<uint16_t>;
  constexpr int KC = D / 32, ES = 2;
  constexpr int UT = HKV_UT;                    // key tiles in flight per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const long long base = x.base;
  const int s = x.s, c = x.c, slot_new = x.slot_new, W = a.W;

  // A operand: the query of row li
  const char* qsrc = nullptr;
  if ((li & 3) == 3) {
    qsrc = a.q + (long long)s * a.ld_q * ES;
  } else if (due) {
    const int i = (li >> 2) * 3 + (li & 3);
    if (i < W - 1) qsrc = a.q_win + ((long long)s * a.ld_qw + (long long)i * D) * ES;
  }
  bf16x8 qa[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qa[kc] = __builtin_bit_cast(bf16x8, qsrc ? ld16_once(qsrc + (lk * 8 + kc * 32) * ES)
                                             : make_uint4(0, 0, 0, 0));

  const char* knew = a.k_new + (long long)s * a.ld_kv * ES;
  const char* vnew = a.v_new + (long long)s * a.ld_kv * ES;
  const int ntile = (c + 15) >> 4;
  const int per = (ntile + kNW - 1) / kNW;
  const int t0 = wave * per;
  const int t1 = min(ntile, t0 + per);

  float m_run = kNeg, l_run = 0.f;
  float acc[KC][8];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[kc][e] = 0.f;

  for (int tt = t0; tt < t1; tt += UT) {
    uint4 kb[UT][KC], vb[UT][KC];
    int pv[UT];
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int j = (tt + u) * 16 + li;
      const bool valid = (tt + u < t1) && j < c;
      const int jj = valid ? j : 0;              // branch-free: clamp, then zero
      const bool fresh = AP && jj == slot_new;
      const char* kr = fresh ? knew : a.k_pool + (base + jj) * kPoolRow<D> * ES;
      const char* vr = fresh ? vnew : a.v_pool + (base + jj) * kPoolRow<D> * ES;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        kb[u][kc] = KC_ ? ld16(kr + (lk * 8 + kc * 32) * ES) : ld16_stream(kr + (lk * 8 + kc * 32) * ES);
        vb[u][kc] = ld16_stream(vr + (lk * 8 + kc * 32) * ES);
      }
      pv[u] = 0;
      if (due) pv[u] = fresh ? a.t : a.pos[base + jj];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (!valid) {
          kb[u][kc] = make_uint4(0, 0, 0, 0);
          vb[u][kc] = make_uint4(0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int j = (tt + u) * 16 + li;
      const bool valid = (tt + u < t1) && j < c;
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kc], __builtin_bit_cast(bf16x8, kb[u][kc]),
                                                    S, 0, 0, 0);
      const float cur = S[3] * a.scale_log2;
      if (due && valid) {
        if (lk == 0) {
          sc.tile[(W - 1) * c + j] = cur;
          sc.pos[j] = pv[u];
        }
#pragma unroll
        for (int r = 0; r < 3; ++r) {
          const int i = lk * 3 + r;
          if (i < W - 1) sc.tile[i * c + j] = S[r] * a.scale_log2;
        }
      }
      const float sv = valid ? cur : kNeg;
      const float m_new = fmaxf(m_run, sv);
      const float alpha = exp2f(m_run - m_new);
      const float p = valid ? exp2f(sv - m_new) : 0.f;
      l_run = fmaf(l_run, alpha, p);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        float vf[8];
        F::to_f32(vb[u][kc], vf);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[kc][e] = fmaf(p, vf[e], acc[kc][e] * alpha);
      }
      m_run = m_new;
    }
  }
  // reduce over the 16 key columns of each 16-lane row
  float m_w = m_run;
  m_w = fmaxf(m_w, dpp<0xB1>(m_w));
  m_w = fmaxf(m_w, dpp<0x4E>(m_w));
  m_w = fmaxf(m_w, dpp<0x141>(m_w));
  m_w = fmaxf(m_w, dpp<0x140>(m_w));
  const float f = exp2f(m_run - m_w);
  const float l_w = group_sum<16>(l_run * f);
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[kc][e] = group_sum<16>(acc[kc][e] * f);
  if (li == 0) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) cs.o[wave][lk * 8 + kc * 32 + e] = acc[kc][e];
    if (lk == 0) {
      cs.m[wave] = m_w;
      cs.l[wave] = l_w;
    }
  }
}

// The vector-ALU flash-decode loop over a stream's rows [t0, t1) of row tiles,
// with its load policy fixed at compile time: a cache hint is part of the
// load instruction, so a per-stream policy takes one copy of the loop each.
// Invalid rows (ragged tail, freed slots) read row 0 and are zeroed, so all
// fragments of a tile are in flight.  The same loop is written out inline in
// k_step for the kernels with a launch-wide policy: called from there, the
// bf16 d64 kernel spills (80 B, measured).
template <class T, int D, int U, bool AP, bool cache_k, bool cache_v>
__device__ __forceinline__ void rows_attend(int t0, int t1, int g, int ext, int nf, const int (&fr)[kMaxEvict],
    int slot_new, const char* kbase, const char* vbase, const char* knew, const char* vnew,
    const float (&qv)[Frag<T>::N], float& m_run, float& l_run, float (&acc)[Frag<T>::N]) {
  using F = Frag<T>;
  constexpr int VE = F::N, G = D / VE, R = kWave / G, ES = sizeof(T);
  auto is_free = [&](int row) {
    bool f = false;
#pragma unroll
    for (int k = 0; k < kMaxEvict; ++k) f |= (row == fr[k]);
    return f;
  };
    for (int tt = t0; tt < t1; tt += U) {
    uint4 kr[U], vr[U];
    bool valid[U];
    // branch-free: an invalid row (ragged tail, freed slot) reads row 0 of
    // the stream and is zeroed, so all fragments of the tile are in flight
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int row = (tt + u) * R + g;
      asm("" : "+v"(row));                  // (opaque: as in k_step's loop)
      valid[u] = (tt + u < t1) && row < ext && !(nf && is_free(row));
      const int rr = valid[u] ? row : 0;
      const bool fresh = AP && rr == slot_new;
      const char* kp = fresh ? knew : kbase + (long long)rr * kPoolRow<D> * ES;
      const char* vp = fresh ? vnew : vbase + (long long)rr * kPoolRow<D> * ES;
      kr[u] = cache_k ? ld16(kp) : ld16_stream(kp);
      vr[u] = cache_v ? ld16(vp) : ld16_stream(vp);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!valid[u]) {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float scr[U];
    float m_tile = kNeg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VE];
      F::to_f32(kr[u], kf);
      float d0 = 0.f;
#pragma unroll
      for (int i = 0; i < VE; ++i) d0 = fmaf(qv[i], kf[i], d0);
      d0 = group_sum<G>(d0);
      scr[u] = valid[u] ? d0 : kNeg;
      m_tile = fmaxf(m_tile, scr[u]);
    }
    const float m_new = fmaxf(m_run, m_tile);
    const float alpha = exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = valid[u] ? exp2f(scr[u] - m_new) : 0.f;
      l_run += p;
      float vf[VE];
      F::to_f32(vr[u], vf);
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[i] = fmaf(p, vf[i], acc[i]);
    }
    m_run = m_new;
  }
}

// ------------------------------------------------------------------ k_step
// One workgroup per stream: append token t (optional), attend over the slots
// present (optional) and, if the stream is a Global stream at B + M slots, evict
// (optional) — one launch.  Every thread reads the stream's metadata itself
// (uniform scalar loads, no barrier); the query is requested first.
template <class T, int D, int C, bool AP, bool AT, bool EV, int KP>
__global__ __launch_bounds__(kNT)
__attribute__((amdgpu_waves_per_eu(StepCfg<T, D, C>::kWaves, StepCfg<T, D, C>::kWaves)))
void k_step(StepArgs a) {
  using F = Frag<T>;
  constexpr int VE = F::N;           // elements per 16-byte fragment
  constexpr int G = D / VE;          // lanes per row
  constexpr int R = kWave / G;       // rows per wave instruction
  constexpr int U = StepCfg<T, D, C>::kRows;  // row fragments in flight per lane
  constexpr int ES = sizeof(T);

  __shared__ CombineShared cs;
  __shared__ EvictShared es;
  using OC = StepCfg<T, D, C>;
  // eviction scratch: the W x c tile and positions, or the keys (which also
  // hold a one-pass tile); positions of a one-pass tile
  __shared__ float lds_tile[EV && !OC::kKeys ? kMaxWobs * OC::kSlots : 1];
  __shared__ int lds_pos[EV ? (OC::kKeys ? (OC::kOnePass ? OC::kOnePass : 1) : OC::kSlots) : 1];
  __shared__ uint64_t lds_keys[EV && OC::kKeys ? OC::kSlots : 1];
  // window queries of a due bf16 stream whose score tile the eviction computes
  constexpr bool kQs = EV && sizeof(T) == 2 && !StepMfmaAttn<T, D>::value;
  __shared__ __align__(16) uint2 lds_qw[kQs ? kMaxWobs * QStage<D>::kPitch : 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = a.s_begin + xcd_block<StepCfg<T, D, C>::kXcdChunk>(blockIdx.x, gridDim.x);
  const int g = lane / G, sub = lane % G;

  constexpr bool kMfma = StepMfmaAttn<T, D>::value;  // eviction-point attention on the matrix cores
  // query fragment first: its address does not depend on the stream metadata
  uint4 q_raw = make_uint4(0, 0, 0, 0);
  if (AT) q_raw = ld16_once(a.q + ((long long)s * a.ld_q + sub * VE) * ES);
  // so is the new token's row (the append's source): threads 0..G-1 take K,
  // G..2G-1 take V
  uint4 app = make_uint4(0, 0, 0, 0);
  if (AP && tid < 2 * G)
    app = ld16_once((tid >= G ? a.v_new : a.k_new) + ((long long)s * a.ld_kv + (tid % G) * VE) * ES);

  // Stream metadata.  Every load is issued before the first wait (scalar loads
  // return out of order, so a wait is for all of them): none depends on
  // another, and a stream that needs fewer discards the rest.  The free-list
  // row is read whole (entries past M repeat the last one); the label byte
  // through the vector path (no scalar byte load), so no branch separates it
  // from the others.
  const int ext0 = a.count[s];               // table extent (slots in use incl. freed)
  const int capv = a.cap[s];
  const int B = a.budget[s];
  const long long base = a.base[s];
  const int nf_raw = a.n_free[s];
  int fl[kMaxEvict];
  {
    const int last = (a.M > 0 ? a.M : 1) - 1;
    const int* row = a.free_slots + (long long)s * a.M;
#pragma unroll
    for (int k = 0; k < kMaxEvict; ++k) fl[k] = row[k < last ? k : last];
  }
  const int lab = a.label[s];
  // bf16 d64: the stream's ring of window-query statistics (what its eviction
  // scores with) comes with the metadata and is staged on chip below, so the
  // eviction does not wait on a load of its own.  (At d128 the registers it
  // holds meanwhile cost more than the wait: measured on MI355X.)
  constexpr bool kRingStaged = EV && AT && kMfma;
  float4 ring_raw = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (kRingStaged) ring_raw = a.qstat[(long long)s * a.W + min(lane & 7, a.W - 1)];
  const bool glob = lab == HKV_GLOBAL;
  const int nf0 = glob ? nf_raw : 0;         // freed slots not yet refilled
  int ext = ext0, nf = nf0, slot_new = -1;
  bool ok = nf0 >= 0 && nf0 <= a.M;
  if (ok && AP) {
    if (lab == HKV_LOCAL) {                   // ring of B slots (B = w, or A)
      slot_new = a.t % B;
      ext = ext0 + 1 < B ? ext0 + 1 : B;
    } else if (nf0 > 0) {                     // lowest freed slot: entry M - nf0
#pragma unroll
      for (int k = 0; k < kMaxEvict; ++k)
        if (k == a.M - nf0) slot_new = fl[k];
      nf = nf0 - 1;
      ok = slot_new >= 0 && slot_new < ext0;
    } else {
      slot_new = ext0;
      ext = ext0 + 1;
      if (ext0 >= capv) {
        ok = false;
        if (tid == 0) atomicOr(a.err, HKV_ERRBIT_CAPACITY);
      }
    }
  }
  const int c = ext - nf;                     // slots holding a token
  if (ok && (c < 1 || ext > capv || lab > HKV_FULL)) ok = false;
  if (!ok) {
    if (tid == 0) atomicOr(a.err, HKV_ERRBIT_LAYOUT);
    if (EV && a.log && tid < a.M) a.log[(long long)s * a.M + tid] = -1;
    return;
  }
  const bool due = EV && glob && (c == B + a.M);
  if constexpr (kRingStaged)                  // (read after the combine's barrier)
    if (wave == 0 && lane < a.W) es.ring[lane] = ring_raw;
  // freed slots still empty: entries M - nf .. M - 1 of the free list
  int fr[kMaxEvict];
#pragma unroll
  for (int k = 0; k < kMaxEvict; ++k) fr[k] = (k >= a.M - nf && k < a.M) ? fl[k] : -1;
  auto is_free = [&](int row) {
    bool f = false;
#pragma unroll
    for (int k = 0; k < kMaxEvict; ++k) f |= (row == fr[k]);
    return f;
  };

  // ---------------- append token t
  // (The rows are written non-temporally: 0.8% faster per launch on Janus-Pro-7B's
  // shape; measured on MI355X.)
  if (AP) {
    if (tid < 2 * G) {
      const bool isv = tid >= G;
      const int sb = tid % G;
      char* dst = (isv ? a.v_pool : a.k_pool) + ((base + slot_new) * kPoolRow<D> + sb * VE) * ES;
      st16_stream(dst, app);
    }
    if (tid == 0) {
      a.pos[base + slot_new] = a.t;
      if (glob) a.score[base + slot_new] = 0.0f;
    }
  }

  // eviction scratch of a due stream: on chip up to the kernel's on-chip size
  const bool onchip = c <= OC::kSlots;
  Scratch scr_l{OC::kKeys ? reinterpret_cast<float*>(lds_keys) : lds_tile, lds_pos,
                OC::kKeys ? lds_keys : nullptr};
  Scratch scr_g{a.ws_tile + base * a.W, a.ws_pos + base, a.ws_keys + base};
  StepCtx x;
  x.base = base;
  x.s = s;
  x.lab = lab;
  x.c = c;
  x.B = B;
  x.slot_new = slot_new;
  x.glob = glob;
  x.due = due;
  // a fixed share of the streams reads its rows with caching, the rest
  // streams them past the caches: the resident share stays in the memory-side
  // cache from one launch to the next, the streamed rows do not displace it
  // KP: this launch keeps a share of its reads resident (per stream where
  // OC::kResident, else all K rows)
  constexpr bool kResShare = OC::kResident && KP != 0;
  const bool resident = kResShare && (s & 63) < a.res64;
  x.resident = resident;

  // ---------------- attention over slots [0, c)
  // With kMfma a bf16 Global stream at its eviction point (c == B + M) attends
  // on the matrix cores — in the fused step this also yields its W x c scoring
  // tile; every other stream attends on the vector ALUs.  The choice depends on
  // the stream state only, so standalone and fused attention give identical
  // bits.  Without kMfma a due stream keeps its K rows in the caches for the
  // eviction's own tile pass.
  const bool at_point = kMfma && glob && c == B + a.M;
  const bool tile_here = at_point && EV && due && a.q_win != nullptr;
  const bool mfma_pass = at_point && (AT || tile_here);
  if (mfma_pass) {
    // (a standalone eviction runs the same pass and discards its output, so the
    // scores equal the fused step's bit for bit)
    if (onchip)
      attend_mfma<D, AP, KP != 0>(a, x, tile_here, scr_l, cs);
    else
      attend_mfma<D, AP, KP != 0>(a, x, tile_here, scr_g, cs);
  }
  if (AT && !mfma_pass) {
    float qv[VE];
    {
      float qf[VE];
      F::to_f32(q_raw, qf);
#pragma unroll
      for (int i = 0; i < VE; ++i) qv[i] = qf[i] * a.scale_log2;
    }
    const char* kbase = a.k_pool + (base * kPoolRow<D> + sub * VE) * ES;
    const char* vbase = a.v_pool + (base * kPoolRow<D> + sub * VE) * ES;
    const char* knew = a.k_new + ((long long)s * a.ld_kv + sub * VE) * ES;
    const char* vnew = a.v_new + ((long long)s * a.ld_kv + sub * VE) * ES;

    const int ntiles = (ext + R - 1) / R;
    const int per = (ntiles + kNW - 1) / kNW;
    const int t0 = wave * per;
    const int t1 = min(ntiles, t0 + per);
    const bool keep_k = !kMfma && EV && due && a.q_win != nullptr;
    // the window queries of such a stream are fetched alongside its keys and
    // staged on chip after the loop
    const bool stage_q = kQs && keep_k;
    using QS = QStage<D>;
    typename QS::Piece qw_raw{};
    if (stage_q && QS::row(tid) < a.W) qw_raw = QS::load(a.q_win, (long long)s * a.ld_qw, tid);

    float m_run = kNeg, l_run = 0.f;
    float acc[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = 0.f;

    // load policy: K is cached for a resident stream, for a launch that keeps
    // all K rows resident, and for an eviction that reads K again; V only for a
    // resident stream; everything else is streamed
    if constexpr (kResShare) {
      // resident streams, eviction-point streams (K read again) and the rest
      if (resident)
        rows_attend<T, D, U, AP, true, true>(t0, t1, g, ext, nf, fr, slot_new, kbase, vbase, knew,
                                             vnew, qv, m_run, l_run, acc);
      else if (keep_k)
        rows_attend<T, D, U, AP, true, false>(t0, t1, g, ext, nf, fr, slot_new, kbase, vbase, knew,
                                              vnew, qv, m_run, l_run, acc);
      else
        rows_attend<T, D, U, AP, false, false>(t0, t1, g, ext, nf, fr, slot_new, kbase, vbase,
                                               knew, vnew, qv, m_run, l_run, acc);
    } else {
      // one policy for the launch: K cached when the launch keeps all K rows
      // resident (or, fp32, for an eviction that reads K again), V streamed
      const bool cache_k = (KP && !OC::kResident) || (!kMfma && keep_k);
      for (int tt = t0; tt < t1; tt += U) {
        uint4 kr[U], vr[U];
        bool valid[U];
        // branch-free: an invalid row (ragged tail, freed slot) reads row 0 of
        // the stream and is zeroed, so all fragments of the tile are in flight
#pragma unroll
        for (int u = 0; u < U; ++u) {
          int row = (tt + u) * R + g;
          // (opaque to the compiler: otherwise it folds u * R into eight
          // per-tile copies of the freed slots, which crowd the scalar
          // registers of the d64 kernel: 57.3 -> 56.3 us per launch on
          // LlamaGen-XL, measured)
          asm("" : "+v"(row));
          valid[u] = (tt + u < t1) && row < ext && !(nf && is_free(row));
          const int rr = valid[u] ? row : 0;
          const bool fresh = AP && rr == slot_new;
          const char* kp = fresh ? knew : kbase + (long long)rr * kPoolRow<D> * ES;
          const char* vp = fresh ? vnew : vbase + (long long)rr * kPoolRow<D> * ES;
          kr[u] = cache_k ? ld16(kp) : ld16_stream(kp);
          vr[u] = ld16_stream(vp);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (!valid[u]) {
            kr[u] = make_uint4(0, 0, 0, 0);
            vr[u] = make_uint4(0, 0, 0, 0);
          }
        }
        float scr[U];
        float m_tile = kNeg;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float kf[VE];
          F::to_f32(kr[u], kf);
          float d0 = 0.f;
#pragma unroll
          for (int i = 0; i < VE; ++i) d0 = fmaf(qv[i], kf[i], d0);
          d0 = group_sum<G>(d0);
          scr[u] = valid[u] ? d0 : kNeg;
          m_tile = fmaxf(m_tile, scr[u]);
        }
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < VE; ++i) acc[i] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float p = valid[u] ? exp2f(scr[u] - m_new) : 0.f;
          l_run += p;
          float vf[VE];
          F::to_f32(vr[u], vf);
#pragma unroll
          for (int i = 0; i < VE; ++i) acc[i] = fmaf(p, vf[i], acc[i]);
        }
        m_run = m_new;
      }
    }
    if (stage_q && QS::row(tid) < a.W) QS::store(lds_qw, tid, qw_raw);
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
  }
  if (EV && due && tid < 2) es.cnt[tid] = 0;   // subset sizes (before a barrier)
  float cur_m = 0.f, cur_il = 0.f;              // current query: softmax max, 1/sum
  if (AT || tile_here) {
    // combine the waves
    __syncthreads();
    float Mx = cs.m[0];
#pragma unroll
    for (int w2 = 1; w2 < kNW; ++w2) Mx = fmaxf(Mx, cs.m[w2]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kNW; ++w2) {
      const float fw = exp2f(cs.m[w2] - Mx);
      L = fmaf(cs.l[w2], fw, L);
      if (AT && tid < D) o = fmaf(cs.o[w2][tid], fw, o);
    }
    cur_m = Mx;
    cur_il = 1.0f / L;
    if (tile_here && tid == 0) {         // statistics of the current query
      es.qm[a.W - 1] = Mx;
      es.ql[a.W - 1] = cur_il;
    }
    if (AT && tid < D) {
      T* op = reinterpret_cast<T*>(a.out + ((long long)s * a.ld_o) * ES);
      op[tid] = F::from_f32(o / L);
    }
    // the ring entry of this step: what a later eviction scores this query with
    if (AT && glob && tid == 0)
      a.qstat[(long long)s * a.W + a.t % a.W] = make_float4(Mx, cur_il, __int_as_float(a.t), 0.f);
  }

  // ---------------- Stratified Token Eviction (due Global streams)
  int nf_final = nf;
  if (EV) {
    if (due) {
      const bool ready = tile_here;
      const bool q_staged = AT && !kMfma && a.q_win != nullptr;   // staged by the attention
      // the attention's combine buffer is free by now: room for kNT keys
      static_assert(sizeof(cs.o) >= kNT * sizeof(uint64_t), "combine buffer holds kNT keys");
      uint64_t* skeys = reinterpret_cast<uint64_t*>(&cs.o[0][0]);
      if (onchip)
        nf_final = evict_stream<T, D, C, AP>(a, x, scr_l, es, skeys, ready, lds_qw, q_staged, AT,
                                             cur_m, cur_il, kRingStaged ? es.ring : nullptr);
      else
        nf_final = evict_stream<T, D, C, AP>(a, x, scr_g, es, skeys, ready, lds_qw, q_staged, AT,
                                             cur_m, cur_il, kRingStaged ? es.ring : nullptr);
    } else if (a.log && tid < a.M) {
      a.log[(long long)s * a.M + tid] = -1;
    }
  }

  if (tid == 0) {
    if (AP) a.count[s] = ext;
    if (glob && nf_final != nf0) a.n_free[s] = nf_final;
  }
}


// ------------------------------------------------------------------ split decode step
// The decode step of hkv_decode_step_split, for launches with few streams (one
// layer of a model): k_split_attn spreads each stream's slots over n_split
// workgroups that each leave a partial softmax state (max, sum, unnormalised
// output) in the workspace, and k_combine_evict, launched after it on the same
// stream, merges them into the output and runs the eviction of due streams.
// The kernel boundary orders the two, so no device-scope fence is needed.
// Split 0 also appends token t; the stream metadata (extent, free count) is
// written back by the second kernel only, so every split reads the same values.
struct StreamMeta {
  long long base;
  int lab, ext0, cap, B, nf0;
  int ext, nf, slot_new, c;   // after the append of token t
  bool glob, ok, full;        // full: append into a stream at capacity
  int fl[kMaxEvict];          // the free-list row (entries past M repeat the last)
};

// Metadata of stream s and the slot token t goes to (the rules of k_step).
__device__ __forceinline__ StreamMeta stream_meta(const StepArgs& a, int s) {
  // every load issued before the first wait, as in k_step
  StreamMeta m;
  m.ext0 = a.count[s];
  m.cap = a.cap[s];
  m.B = a.budget[s];
  m.base = a.base[s];
  const int nf_raw = a.n_free[s];
  {
    const int last = (a.M > 0 ? a.M : 1) - 1;
    const int* row = a.free_slots + (long long)s * a.M;
#pragma unroll
    for (int k = 0; k < kMaxEvict; ++k) m.fl[k] = row[k < last ? k : last];
  }
  m.lab = a.label[s];
  m.glob = m.lab == HKV_GLOBAL;
  m.nf0 = m.glob ? nf_raw : 0;
  m.ext = m.ext0;
  m.nf = m.nf0;
  m.slot_new = -1;
  m.full = false;
  m.ok = m.nf0 >= 0 && m.nf0 <= a.M;
  if (m.ok) {
    if (m.lab == HKV_LOCAL) {
      m.slot_new = a.t % m.B;
      m.ext = m.ext0 + 1 < m.B ? m.ext0 + 1 : m.B;
    } else if (m.nf0 > 0) {
#pragma unroll
      for (int k = 0; k < kMaxEvict; ++k)
        if (k == a.M - m.nf0) m.slot_new = m.fl[k];
      m.nf = m.nf0 - 1;
      m.ok = m.slot_new >= 0 && m.slot_new < m.ext0;
    } else {
      m.slot_new = m.ext0;
      m.ext = m.ext0 + 1;
      if (m.ext0 >= m.cap) {
        m.ok = false;
        m.full = true;
      }
    }
  }
  m.c = m.ext - m.nf;
  if (m.ok && (m.c < 1 || m.ext > m.cap || m.lab > HKV_FULL)) m.ok = false;
  return m;
}

template <class T, int D, int C>
struct SplitCfg {
  static constexpr int kWaves = HKV_WPE_SPLIT ? HKV_WPE_SPLIT : StepCfg<T, D, C>::kWaves;
  static constexpr int kRows = HKV_U_SPLIT ? HKV_U_SPLIT : StepCfg<T, D, C>::kRows;
};

template <class T, int D, int C>
__global__ __launch_bounds__(kNT)
__attribute__((amdgpu_waves_per_eu(SplitCfg<T, D, C>::kWaves, SplitCfg<T, D, C>::kWaves)))
void k_split_attn(StepArgs a, int n_split, float* part) {
  using F = Frag<T>;
  constexpr int VE = F::N, G = D / VE, R = kWave / G, ES = sizeof(T);
  constexpr int U = SplitCfg<T, D, C>::kRows;
  constexpr int PS = D + 4;                        // floats per partial state
  __shared__ CombineShared cs;
  constexpr bool kScores = sizeof(T) == 2;         // bf16: the splits score their slots
  __shared__ __align__(16) uint2 lds_qw[kScores ? kMaxWobs * QStage<D>::kPitch : 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = xcd_block(blockIdx.x, gridDim.x);
  const int s = a.s_begin + blk / n_split, p = blk % n_split;
  const int g = lane / G, sub = lane % G;

  const uint4 q_raw = ld16_once(a.q + ((long long)s * a.ld_q + sub * VE) * ES);
  uint4 app = make_uint4(0, 0, 0, 0);
  if (p == 0 && tid < 2 * G)
    app = ld16_once((tid >= G ? a.v_new : a.k_new) + ((long long)s * a.ld_kv + (tid % G) * VE) * ES);
  const StreamMeta m = stream_meta(a, s);
  if (!m.ok) return;                               // (reported by k_combine_evict)
  const long long base = m.base;
  const int ext = m.ext, nf = m.nf, slot_new = m.slot_new;
  int fr[kMaxEvict];
#pragma unroll
  for (int k = 0; k < kMaxEvict; ++k) fr[k] = (k >= a.M - nf && k < a.M) ? m.fl[k] : -1;
  auto is_free = [&](int row) {
    bool f = false;
#pragma unroll
    for (int k = 0; k < kMaxEvict; ++k) f |= (row == fr[k]);
    return f;
  };
  if (p == 0) {                                    // append token t
    if (tid < 2 * G) {
      const bool isv = tid >= G;
      char* dst = (isv ? a.v_pool : a.k_pool) + ((base + slot_new) * kPoolRow<D> + (tid % G) * VE) * ES;
      st16_stream(dst, app);
    }
    if (tid == 0) {
      a.pos[base + slot_new] = a.t;
      if (m.glob) a.score[base + slot_new] = 0.0f;
    }
  }
  // this split's share of the row tiles of [0, ext), then each wave's share
  const int ntiles = (ext + R - 1) / R;
  const int per_split = (ntiles + n_split - 1) / n_split;
  const int s0 = min(ntiles, p * per_split), s1 = min(ntiles, s0 + per_split);
  const int per = (s1 - s0 + kNW - 1) / kNW;
  const int t0 = s0 + wave * per, t1 = min(s1, t0 + per);
  // a stream that evicts at this step keeps its K rows in the caches for the
  // eviction's pass over them
  const bool keep_k = m.glob && m.c == m.B + a.M && a.q_win != nullptr;

  float qv[VE];
  {
    float qf[VE];
    F::to_f32(q_raw, qf);
#pragma unroll
    for (int i = 0; i < VE; ++i) qv[i] = qf[i] * a.scale_log2;
  }
  const char* kbase = a.k_pool + (base * kPoolRow<D> + sub * VE) * ES;
  const char* vbase = a.v_pool + (base * kPoolRow<D> + sub * VE) * ES;
  const char* knew = a.k_new + ((long long)s * a.ld_kv + sub * VE) * ES;
  const char* vnew = a.v_new + ((long long)s * a.ld_kv + sub * VE) * ES;
  float m_run = kNeg, l_run = 0.f;
  float acc[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) acc[i] = 0.f;
  for (int tt = t0; tt < t1; tt += U) {
    uint4 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int row = (tt + u) * R + g;
      asm("" : "+v"(row));                  // (opaque: as in k_step's loop)
      valid[u] = (tt + u < t1) && row < ext && !(nf && is_free(row));
      const int rr = valid[u] ? row : 0;
      const bool fresh = rr == slot_new;
      kr[u] = keep_k ? ld16(fresh ? knew : kbase + (long long)rr * kPoolRow<D> * ES)
                     : ld16_stream(fresh ? knew : kbase + (long long)rr * kPoolRow<D> * ES);
      vr[u] = ld16_stream(fresh ? vnew : vbase + (long long)rr * kPoolRow<D> * ES);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!valid[u]) {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float scr[U];
    float m_tile = kNeg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VE];
      F::to_f32(kr[u], kf);
      float d0 = 0.f;
#pragma unroll
      for (int i = 0; i < VE; ++i) d0 = fmaf(qv[i], kf[i], d0);
      d0 = group_sum<G>(d0);
      scr[u] = valid[u] ? d0 : kNeg;
      m_tile = fmaxf(m_tile, scr[u]);
    }
    const float m_new = fmaxf(m_run, m_tile);
    const float alpha = exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = valid[u] ? exp2f(scr[u] - m_new) : 0.f;
      l_run += pu;
      float vf[VE];
      F::to_f32(vr[u], vf);
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[i] = fmaf(pu, vf[i], acc[i]);
    }
    m_run = m_new;
  }
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
  float Mx = cs.m[0];
#pragma unroll
  for (int w2 = 1; w2 < kNW; ++w2) Mx = fmaxf(Mx, cs.m[w2]);
  float L = 0.f, o = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < kNW; ++w2) {
    const float fw = exp2f(cs.m[w2] - Mx);
    L = fmaf(cs.l[w2], fw, L);
    if (tid < D) o = fmaf(cs.o[w2][tid], fw, o);
  }
  float* ps = part + ((long long)s * kMaxSplit + p) * PS;
  if (tid < D) ps[tid] = o;
  if (tid == 0) {
    ps[D] = Mx;
    ps[D + 1] = L;
  }

  // A Global stream at its eviction point (bf16): this split scores its own
  // slots for the eviction, so that k_combine_evict needs no pass over K.  The
  // matrix cores form the window queries' logits over the split's rows; each
  // slot keeps the probability mass of queries 0..W-2 (their softmax max and
  // sum from the ring, each query over the slots whose position does not
  // exceed its own) and the current query's logit, whose share needs the
  // statistics merged over all splits.  Stale ring entries leave the scoring
  // to k_combine_evict (it makes the same check).
  if constexpr (kScores) {
    const int W = a.W, t = a.t;
    const bool due = m.glob && m.c == m.B + a.M && a.q_win != nullptr;
    float qo_l = 0.f;                              // lane i < W-1: query i's log2(2^max * sum)
    bool rok = true;
    if (due && lane < W - 1) {
      const int step = t - W + 1 + lane;
      const float4 e = a.qstat[(long long)s * W + step % W];
      rok = __float_as_int(e.z) == step;
      qo_l = e.x - __log2f(e.y);
    }
    if (due && __ballot(!rok) == 0) {              // (the same in every wave)
      typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      using QS = QStage<D>;
      constexpr int KC = D / 32, QP = QS::kPitch;
      if (QS::row(tid) < W) QS::store(lds_qw, tid, QS::load(a.q_win, (long long)s * a.ld_qw, tid));
      __syncthreads();
      // v_mfma_f32_16x16x32_bf16: lane l holds A row (query) l%16 and B column
      // (slot) l%16 at elements (l/16)*8 .. +7 of each 32-element chunk, and
      // receives D rows (l/16)*4 .. +3 of slot column l%16
      const int li = lane & 15, lk = lane >> 4;
      float qo_r[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) qo_r[r] = __shfl(qo_l, lk * 4 + r);
      const int r0 = s0 * R, r1 = min(s1 * R, m.c);
      const int nt = r1 > r0 ? (r1 - r0 + 15) / 16 : 0;
      const char* krow_new = a.k_new + ((long long)s * a.ld_kv) * ES;
      float* wsp = a.ws_tile + m.base * W;         // per slot: (partial score, current logit)
      constexpr int UE = HKV_UE_SPLIT;
      for (int kt0 = wave; kt0 < nt; kt0 += kNW * UE) {
        uint4 kb[UE][KC];
        int pj[UE];
#pragma unroll
        for (int u = 0; u < UE; ++u) {
          const int j = r0 + (kt0 + u * kNW) * 16 + li;
          const bool tile_in = kt0 + u * kNW < nt;   // uniform across the wave
          const int jj = tile_in && j < r1 ? j : r0;
          const bool fresh = jj == m.slot_new;       // (split 0 may not have stored it yet)
          const char* row = fresh ? krow_new : a.k_pool + ((m.base + jj) * kPoolRow<D>) * ES;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc)
            kb[u][kc] = tile_in ? ld16(row + (lk * 8 + kc * 32) * ES) : make_uint4(0, 0, 0, 0);
          pj[u] = tile_in ? (fresh ? t : a.pos[m.base + jj]) : 0;
        }
#pragma unroll
        for (int u = 0; u < UE; ++u) {
          if (kt0 + u * kNW >= nt) break;                // uniform
          const int j = r0 + (kt0 + u * kNW) * 16 + li;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            uint4 q = make_uint4(0, 0, 0, 0);
            if (li < W) q = *reinterpret_cast<const uint4*>(lds_qw + li * QP + lk * 2 + kc * 8);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, q),
                                                          __builtin_bit_cast(bf16x8, kb[u][kc]), acc, 0, 0, 0);
          }
          float pr = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = lk * 4 + r;
            if (i < W - 1 && pj[u] <= t - W + 1 + i) pr += exp2f(acc[r] * a.scale_log2 - qo_r[r]);
          }
          pr += __shfl_xor(pr, 16);                 // rows 0-3 and 4-7
          const int rc = (W - 1) & 3;
          const float cv = rc == 0 ? acc[0] : rc == 1 ? acc[1] : rc == 2 ? acc[2] : acc[3];
          const float cl = __shfl(cv * a.scale_log2, li + 16 * ((W - 1) >> 2));
          if (lk == 0 && j < r1) {
            wsp[2 * j] = pr;
            wsp[2 * j + 1] = cl;
            a.ws_pos[m.base + j] = pj[u];
          }
        }
      }
    }
  }
}

template <class T, int D, int C>
__global__ __launch_bounds__(kNT) void k_combine_evict(StepArgs a, int n_split, const float* part) {
  using F = Frag<T>;
  constexpr int ES = sizeof(T);
  constexpr int CE = (sizeof(T) == 2 && D == 64) ? 2 : C;   // eviction shape
  using OC = StepCfg<T, D, CE>;
  constexpr int PS = D + 4;
  __shared__ EvictShared es;
  __shared__ uint64_t skeys[kNT];
  __shared__ float lds_tile[!OC::kKeys ? kMaxWobs * OC::kSlots : 1];
  __shared__ int lds_pos[OC::kKeys ? (OC::kOnePass ? OC::kOnePass : 1) : OC::kSlots];
  __shared__ uint64_t lds_keys[OC::kKeys ? OC::kSlots : 1];
  constexpr bool kQs = OC::kKeys;
  __shared__ __align__(16) uint2 lds_qw[kQs ? kMaxWobs * QStage<D>::kPitch : 2];
  const int tid = threadIdx.x;
  const int s = a.s_begin + xcd_block(blockIdx.x, gridDim.x);

  const StreamMeta m = stream_meta(a, s);
  if (!m.ok) {
    if (tid == 0) atomicOr(a.err, m.full ? (HKV_ERRBIT_CAPACITY | HKV_ERRBIT_LAYOUT) : HKV_ERRBIT_LAYOUT);
    if (a.log && tid < a.M) a.log[(long long)s * a.M + tid] = -1;
    return;
  }
  const bool due = m.glob && m.c == m.B + a.M;
  if (due && tid < 2) es.cnt[tid] = 0;
  // did the splits score the slots (bf16, window given, ring of queries
  // 0..W-2 current: the check k_split_attn made)?
  bool split_scores = false;
  if (sizeof(T) == 2 && due && a.q_win != nullptr) {
    bool rok = true;
    const int lane = tid & 63;
    if (lane < a.W - 1) {
      const int step = a.t - a.W + 1 + lane;
      rok = __float_as_int(a.qstat[(long long)s * a.W + step % a.W].z) == step;
    }
    split_scores = __ballot(!rok) == 0;
  }
  // merge the partial states
  const float* ps = part + (long long)s * kMaxSplit * PS;
  float Mx = kNeg;
  for (int q = 0; q < n_split; ++q) Mx = fmaxf(Mx, ps[q * PS + D]);
  float L = 0.f, o = 0.f;
  for (int q = 0; q < n_split; ++q) {
    const float fw = exp2f(ps[q * PS + D] - Mx);
    L = fmaf(ps[q * PS + D + 1], fw, L);
    if (tid < D) o = fmaf(ps[q * PS + tid], fw, o);
  }
  const float cur_il = 1.0f / L;
  if (tid < D) {
    T* op = reinterpret_cast<T*>(a.out + ((long long)s * a.ld_o) * ES);
    op[tid] = F::from_f32(o / L);
  }
  if (m.glob && tid == 0)
    a.qstat[(long long)s * a.W + a.t % a.W] = make_float4(Mx, cur_il, __int_as_float(a.t), 0.f);
  __syncthreads();                                 // subset counters zeroed
  int nf_final = m.nf;
  if (due) {
    StepCtx x;
    x.base = m.base;
    x.s = s;
    x.lab = m.lab;
    x.c = m.c;
    x.B = m.B;
    x.slot_new = m.slot_new;
    x.glob = m.glob;
    x.due = due;
    if (m.c <= OC::kSlots) {
      Scratch sc{OC::kKeys ? reinterpret_cast<float*>(lds_keys) : lds_tile, lds_pos,
                 OC::kKeys ? lds_keys : nullptr};
      nf_final = evict_stream<T, D, CE, false>(a, x, sc, es, skeys, false, lds_qw, false, true,
                                               Mx, cur_il, nullptr, split_scores);
    } else {
      Scratch sc{a.ws_tile + m.base * a.W, a.ws_pos + m.base, a.ws_keys + m.base};
      nf_final = evict_stream<T, D, CE, false>(a, x, sc, es, skeys, false, lds_qw, false, true,
                                               Mx, cur_il, nullptr, split_scores);
    }
  } else if (a.log && tid < a.M) {
    a.log[(long long)s * a.M + tid] = -1;
  }
  if (tid == 0) {
    a.count[s] = m.ext;
    if (m.glob && nf_final != m.nf0) a.n_free[s] = nf_final;
  }
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

// bf16 classification logits on the matrix cores (1) or the vector ALUs (0).
#ifndef HKV_CLASSIFY_MFMA
#define HKV_CLASSIFY_MFMA 1
#endif

template <class T, int D>
__global__ __launch_bounds__(kNT) void k_classify(ClassifyArgs a) {
  using F = Frag<T>;
  constexpr int VE = F::N, G = D / VE, R = kWave / G, ES = sizeof(T);
  constexpr int WM = 8;                     // observation queries held per lane
  extern __shared__ float lg[];             // [W][P]
  __shared__ float mrow[WM], lrow[WM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = xcd_block(blockIdx.x, gridDim.x);
  const int P = a.P, W = a.W;

  if constexpr (sizeof(T) == 2 && HKV_CLASSIFY_MFMA) {
    // bf16: the W x P logit tile on the matrix cores, v_mfma_f32_16x16x32_bf16
    // with A = the W queries (rows W..15 zero) and B = 16 keys per tile; lane l
    // holds A row l%16 and B column (key) l%16 at head elements (l/16)*8 + 32*kc
    // .. +7 and receives D rows (queries) (l/16)*4 .. +3 of key column l%16.
    // Each wave takes every fourth 16-key tile, UT tiles of loads in flight.
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int KC = D / 32;
    constexpr int UT = D == 64 ? 4 : 3;
    const int li = lane & 15, lk = lane >> 4;
    bf16x8 qa[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (li < W) u = ld16_once(a.q_obs + ((long long)s * a.ld_qobs + (long long)li * D + lk * 8 + kc * 32) * ES);
      qa[kc] = __builtin_bit_cast(bf16x8, u);
    }
    const char* kbase = a.k_stage + ((long long)s * a.ld_stage + lk * 8) * ES;
    const int ntile = (P + 15) / 16;
    for (int t0 = wave; t0 < ntile; t0 += kNW * UT) {
      uint4 kb[UT][KC];
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        const int j = min((t0 + u * kNW) * 16 + li, P - 1);    // ragged tail: clamp
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          kb[u][kc] = (t0 + u * kNW < ntile) ? ld16_stream(kbase + ((long long)j * D + kc * 32) * ES)
                                             : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        if (t0 + u * kNW >= ntile) break;                     // uniform
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kc], __builtin_bit_cast(bf16x8, kb[u][kc]),
                                                        acc, 0, 0, 0);
        const int j = (t0 + u * kNW) * 16 + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = lk * 4 + r;
          if (i < W && j < P) lg[i * P + j] = acc[r] * a.scale_log2;
        }
      }
    }
  } else {
    // vector ALU, G lanes per key row, every observation query in registers
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

// ------------------------------------------------------------------ k_prefill
// Causal attention over the P prefill positions of every stream (bf16), with
// the classification of the compressed layouts as its by-product: the logits of
// the W observation queries (the last W positions) against every key they see
// stay on chip, and after the pass the count, label and initial scores follow
// exactly as in k_classify.  K is read once for both.
//
// One workgroup per (stream, block of 64 queries), blocks counted from the end
// so block 0 holds the observation queries; wave w takes 16 of the block's
// queries.  The logits are formed transposed on the matrix cores,
// S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16 keys, B = 16 queries):
// lane l then holds keys (l/16)*4 .. +3 of a 16-key tile for query l%16.  Two
// such tiles give each lane 8 keys of its query, which is the B operand of
// O^T += V^T P^T (A = 16 head elements x 32 keys, the same key order), so the
// probabilities never leave the registers.  Each 64-key block of K and V is
// staged in LDS once for the four waves (coalesced 16-byte loads; V transposed
// in registers, 4 keys x 8 elements per thread, and written as 8-byte rows).
struct PrefillArgs {
  const char* q_stage; long long ld_q;
  const char* k_stage; const char* v_stage; long long ld_stage;
  char* out; long long ld_out;
  float* init_scores;          // [S, P]
  int* n_tokens; unsigned char* label;
  int P, W, w, nqb, classify;
  float tau, scale_log2;
};

// Probabilities of the prefill's P.V product as two bf16 parts (1) or one (0).
#ifndef HKV_PV_SPLIT
#define HKV_PV_SPLIT 1
#endif

template <int D, int NWQ>
__global__ __launch_bounds__(64 * NWQ) __attribute__((amdgpu_waves_per_eu(4, 8)))
void k_prefill(PrefillArgs a) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int KC = D / 32;                // matrix-core steps over the head elements
  constexpr int DT = D / 16;                // 16-element output tiles
  constexpr int BK = 64;                    // keys per block
  constexpr int VP = BK + 8;                // padded row of the transposed V block
  constexpr int ES = 2;
  constexpr int KP = D + 8;                 // padded row of the K block
  constexpr int NT = 64 * NWQ;              // threads; wave w takes queries 16w .. 16w+15
  constexpr int QB = 16 * NWQ;              // of the workgroup's block of QB queries
  __shared__ __align__(16) uint16_t ks[BK * KP];  // K block, [key][head element]
  __shared__ __align__(16) uint16_t vt[D * VP];   // V block, [head element][key]
  __shared__ float mrow[kMaxWobs], lrow[kMaxWobs];
  extern __shared__ float lg[];             // [W][P] observation logits (block 0)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int blk = xcd_block(blockIdx.x, gridDim.x);
  const int s = blk / a.nqb, qb = blk - (blk / a.nqb) * a.nqb;
  const int P = a.P, W = a.W;
  const int q_hi = P - QB * qb;             // the block's queries: [max(0, q_hi - QB), q_hi)
  const int q_w = q_hi - QB + 16 * wave;    // this wave's first query
  const int myq = q_w + li;
  const bool qvalid = myq >= 0 && myq < q_hi;
  const bool obs = a.classify && qb == 0;
  const long long sb = (long long)s * a.ld_stage;

  // B operand of the logits: query myq, head elements lk*8 + kc*32 .. +7
  bf16x8 qf[KC];
  {
    const int qr = qvalid ? myq : 0;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      uint4 u = ld16(a.q_stage + ((long long)s * a.ld_q + (long long)qr * D + lk * 8 + kc * 32) * ES);
      if (!qvalid) u = make_uint4(0, 0, 0, 0);
      qf[kc] = __builtin_bit_cast(bf16x8, u);
    }
  }
  f32x4 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNeg, l = 0.f;                  // running statistics of query myq

  const int nkb = (q_hi - 1) / BK + 1;      // key blocks the block's queries see
  // K block: chunk c = 8 elements (e0) of key c / (D/8); rows past P clamp
  // (their probabilities are zero).  V block, transposed: patch p = keys
  // 4*(p / (D/8)) .. +3, elements 8*(p % (D/8)) .. +7, one 8-byte row per
  // element.  fetch() loads a block into registers, stage() writes it to LDS.
  // At d64 the next block is fetched before the current one is used, so its
  // loads overlap the arithmetic (at d128 the registers would cost a wave).
  constexpr bool kPF = D == 64;
  constexpr int KN = (BK * D / 8 + NT - 1) / NT;
  uint4 kq[kPF ? KN : 1], vq[kPF ? 4 : 1];   // the fetched block (d64)
  // keys 4*kg .. +3 (rows v[0..3]), elements e0 .. +7 of V, written transposed
  auto put_v = [&](const uint4* v, int kg, int e0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = e < 2 ? v[i].x : e < 4 ? v[i].y : e < 6 ? v[i].z : v[i].w;
        h[i] = (e & 1) ? (w >> 16) : (w & 0xffffu);
      }
      *reinterpret_cast<uint2*>(vt + (e0 + e) * VP + 4 * kg) =
          make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
  };
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const int c = tid + i * NT;
      if (c < BK * D / 8) {
        const int key = c / (D / 8), e0 = (c % (D / 8)) * 8;
        kq[i] = ld16(a.k_stage + (sb + (long long)min(k0 + key, P - 1) * D + e0) * ES);
      }
    }
    if (tid < BK * D / 32) {
      const int kg = tid / (D / 8), e0 = (tid % (D / 8)) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vq[i] = ld16(a.v_stage + (sb + (long long)min(k0 + 4 * kg + i, P - 1) * D + e0) * ES);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const int c = tid + i * NT;
      if (c < BK * D / 8) {
        const int key = c / (D / 8), e0 = (c % (D / 8)) * 8;
        *reinterpret_cast<uint4*>(ks + key * KP + e0) = kq[i];
      }
    }
    if (tid < BK * D / 32) put_v(vq, tid / (D / 8), (tid % (D / 8)) * 8);
  };
  if constexpr (kPF) fetch(0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * BK;
    __syncthreads();                        // the previous block's K and V reads are done
    if constexpr (kPF) {
      stage();
    } else {
      // (each piece stored as it arrives: fewer registers than fetch + stage)
#pragma unroll
      for (int c = tid; c < BK * D / 8; c += NT) {
        const int key = c / (D / 8), e0 = (c % (D / 8)) * 8;
        const int kr = min(k0 + key, P - 1);
        *reinterpret_cast<uint4*>(ks + key * KP + e0) =
            ld16(a.k_stage + (sb + (long long)kr * D + e0) * ES);
      }
      if (tid < BK * D / 32) {
        const int kg = tid / (D / 8), e0 = (tid % (D / 8)) * 8;
        uint4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = ld16(a.v_stage + (sb + (long long)min(k0 + 4 * kg + i, P - 1) * D + e0) * ES);
        put_v(v, kg, e0);
      }
    }
    __syncthreads();                        // K and V blocks staged
    if constexpr (kPF) {
      if (kb + 1 < nkb) fetch(k0 + BK);
    }
    if (q_w + 15 < k0) continue;            // (uniform) no query of the wave sees the block
    // logits of the 4 key tiles: lane holds keys k0 + t*16 + lk*4 + r, query myq
    float sv[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint4 kf[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        kf[kc] = *reinterpret_cast<const uint4*>(ks + (t * 16 + li) * KP + lk * 8 + kc * 32);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kc]), qf[kc],
                                                      acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + t * 16 + lk * 4 + r;
        const bool vis = qvalid && key <= myq;
        sv[t][r] = vis ? acc[r] * a.scale_log2 : kNeg;
        if (obs && vis && myq >= P - W) lg[(myq - (P - W)) * P + key] = sv[t][r];
      }
    }
    // online softmax of query myq (its 64 keys sit in the 4 lanes li, li+16, ...)
    float mb = kNeg;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) mb = fmaxf(mb, sv[t][r]);
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float mn = fmaxf(m, mb);
    const float alpha = exp2f(m - mn);
    float pr[4][4], ps = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[t][r] = sv[t][r] > kNeg ? exp2f(sv[t][r] - mn) : 0.f;
        ps += pr[t][r];
      }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = l * alpha + ps;
    m = mn;
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] *= alpha;
    // O^T += V^T P^T over 32 keys at a time: keys {2c*16 + lk*4 + e, (2c+1)*16 + lk*4 + e}.
    // The probabilities enter the matrix cores as bf16; with HKV_PV_SPLIT each is
    // split into a bf16 high part and the bf16 rounding of the rest, two
    // products, so that P carries about 16 bits instead of 8 (the output's error
    // budget then goes to the bf16 rounding of the output alone)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 pb, pl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[e] = __bf16(pr[2 * c][e]);
        pb[4 + e] = __bf16(pr[2 * c + 1][e]);
        pl[e] = __bf16(pr[2 * c][e] - float(pb[e]));
        pl[4 + e] = __bf16(pr[2 * c + 1][e] - float(pb[4 + e]));
      }
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const uint16_t* row = vt + (t * 16 + li) * VP;
        const uint2 lo = *reinterpret_cast<const uint2*>(row + 2 * c * 16 + lk * 4);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + (2 * c + 1) * 16 + lk * 4);
        const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pb, o[t],
                                                       0, 0, 0);
        if (HKV_PV_SPLIT)
          o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pl, o[t],
                                                         0, 0, 0);
      }
    }
  }
  // output row myq: head elements t*16 + lk*4 .. +3
  if (qvalid) {
    const float inv = 1.0f / l;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out + ((long long)s * a.ld_out + (long long)myq * D) * ES);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      uint2 pk;
      pk.x = uint32_t(Frag<uint16_t>::from_f32(o[t][0] * inv)) |
             (uint32_t(Frag<uint16_t>::from_f32(o[t][1] * inv)) << 16);
      pk.y = uint32_t(Frag<uint16_t>::from_f32(o[t][2] * inv)) |
             (uint32_t(Frag<uint16_t>::from_f32(o[t][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(orow + t * 16 + lk * 4) = pk;
    }
  }
  if (!obs) return;
  // ---- classification of the stream, from the observation queries' logits
  if (qvalid && myq >= P - W && lk == 0) {
    mrow[myq - (P - W)] = m;
    lrow[myq - (P - W)] = l;
  }
  __syncthreads();
  // count: attention of the last query accumulated backward from position P-1
  if (wave == 0) {
    const int i = W - 1;
    const float mm = mrow[i], inv = 1.0f / lrow[i];
    float carry = 0.f;
    int n = P;
    for (int d0 = 0; d0 < P; d0 += kWave) {
      const int dist = d0 + lane;
      const float p = dist < P ? exp2f(lg[i * P + (P - 1 - dist)] - mm) * inv : 0.f;
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
  for (int j = tid; j < P; j += NT) {
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
  int* n_free;
  float4* qstat;
  int* err;
  int H, N, P, w, W, M, D, A, full, uniform;
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
      // Local heads: ring of wl slots; Global heads: budget Bg (uniform
      // variant: both floor(rho*N))
      const int wl = a.uniform ? a.A : a.w;
      const int Bg = a.uniform ? a.A : (n_g ? (a.H * a.A - n_l * a.w) / n_g : 0);
      long long off = (long long)grp * a.group_slots;
      for (int x = 0; x < h; ++x) off += lab[x] == HKV_LOCAL ? wl : Bg + a.M;
      s_base = off;
      s_lab = lab[h];
      if (lab[h] == HKV_LOCAL) {
        s_B = wl;
        s_count = P < wl ? P : wl;
        s_mode = 1;
        a.cap[s] = wl;
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
    a.n_free[s] = 0;
  }
  // no decode query yet: every ring entry stale
  if (tid < a.W) a.qstat[(long long)s * a.W + tid] = make_float4(0.f, 0.f, __int_as_float(-1), 0.f);
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
  } else if (!a.full) {
    for (int j = tid; j < P; j += kNT) {
      if (mode == 1) dest[j] = (j >= P - s_B) ? j % s_B : -1;
      else dest[j] = j;
    }
    __syncthreads();
  }
  // (the full layout maps position j to slot j; its prefill may exceed the
  // on-chip table)
  const bool full = a.full;
  for (int idx = tid; idx < P * 2 * G; idx += kNT) {
    const int j = idx / (2 * G), r = idx % (2 * G);
    const int to = full ? j : dest[j];
    if (to < 0) continue;
    const bool isv = r >= G;
    const int sub = r % G;
    const char* src = (isv ? vs : ks) + ((long long)j * D + sub * VE) * ES;
    st16((isv ? a.v_pool : a.k_pool) + ((base + to) * kPoolRow<D> + sub * VE) * ES, ld16(src));
  }
  for (int j = tid; j < P; j += kNT) {
    const int to = full ? j : dest[j];
    if (to < 0) continue;
    a.pos[base + to] = j;
    a.score[base + to] = (s_lab == HKV_GLOBAL) ? a.init_scores[(long long)s * P + j] : 0.0f;
  }
}

__global__ void k_reset_err(int* err) { *err = 0; }

// Classification scores [S, P] of hkv_classify_noalloc: a file-scope buffer that
// each device holds once for the life of the process, so that the call needs no
// caller workspace and allocates nothing.  Host code never passes `scratch`
// itself to a kernel: it uses the device address hipGetSymbolAddress returns.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

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


// Residency of the decode step's reads in the memory-side cache (the 256 MB
// Infinity Cache in front of HBM).  Each step reads every cached row once, in
// the same order, and the pool is larger than that cache: loaded with default
// caching, the rows would evict each other before the next step comes back to
// them.  So rows are streamed past the caches (non-temporal loads), except for
// a fixed share of about 140 MiB that is loaded with caching every step and so
// is found in the cache by the next one.  bf16 d128 takes the share per
// stream (streams with s % 64 < res64); bf16 d64 all K rows or none, whichever
// is nearer the target (a per-stream choice costs that kernel registers it
// does not have).  The byte target was measured on MI355X: about 140-210 MB
// helped every workload, more thrashes.  HKV_RESIDENT_MB overrides it (0:
// stream everything).
struct Residency {
  int res64 = 0;        // bf16 d128: resident share of the streams, in 64ths
  bool cache_k = false; // bf16 d64: K rows loaded with caching
};

Residency residency(const hkv_config* c, const Derived& d) {
  static const double target = [] {
    const char* e = getenv("HKV_RESIDENT_MB");
    return (e ? atof(e) : 140.0) * double(1 << 20);
  }();
  Residency r;
  if (c->dtype != HKV_DT_BF16 || target <= 0.0) return r;
  const double kv_bytes = double(d.pool_slots) * 2.0 * c->head_dim * 2.0;   // K and V rows
  if (c->head_dim == 128) {
    const double share = std::floor(64.0 * target / kv_bytes + 0.5);
    r.res64 = share > 64.0 ? 64 : int(share);
  } else {
    r.cache_k = kv_bytes / 2.0 < 2.0 * target;
  }
  return r;
}

template <class T, int D, int C, bool AP, bool AT, bool EV, int KP = 0>
void launch_step_t(const dev::StepArgs& a, int n, hipStream_t st) {
  hipLaunchKernelGGL((dev::k_step<T, D, C, AP, AT, EV, KP>), dim3(n), dim3(dev::kNT), 0, st, a);
}

template <class T, int D, int C>
void launch_split_t(const dev::StepArgs& a, int n, int n_split, float* part, hipStream_t st) {
  hipLaunchKernelGGL((dev::k_split_attn<T, D, C>), dim3(n * n_split), dim3(dev::kNT), 0, st, a,
                     n_split, part);
  hipLaunchKernelGGL((dev::k_combine_evict<T, D, C>), dim3(n), dim3(dev::kNT), 0, st, a, n_split,
                     static_cast<const float*>(part));
}

// Stream class of the bf16 d128 decode step: long streams (the uncompressed
// layout, or a per-head budget above this many slots) keep more rows in flight
// per wave; short ones run more waves.  Measured on MI355X.
#ifndef HKV_LONG_BUDGET
#define HKV_LONG_BUDGET 192
#endif
bool long_streams(const hkv_config* c) {
  if (c->full_cache) return true;
  return int64_t(c->rho_num) * c->final_len / c->rho_den > HKV_LONG_BUDGET;
}

template <bool AP, bool AT, bool EV>
void launch_step(const hkv_config* c, const dev::StepArgs& a0, int n, hipStream_t st) {
  // the resident share pays off in a launch over every stream; a launch over a
  // part of them (one layer of a model run layer by layer) is bound by its
  // workgroups' latency and measured slower with it
  Derived d;
  derive(c, &d);
  const Residency r = n == d.S ? residency(c, d) : Residency{};
  dev::StepArgs a = a0;
  a.res64 = r.res64;
  if (c->dtype == HKV_DT_BF16) {
    if (c->head_dim == 64) {
      if (r.cache_k) launch_step_t<uint16_t, 64, 0, AP, AT, EV, 1>(a, n, st);
      else launch_step_t<uint16_t, 64, 0, AP, AT, EV, 0>(a, n, st);
    }
    else if (long_streams(c)) {
      if (r.res64) launch_step_t<uint16_t, 128, 1, AP, AT, EV, 1>(a, n, st);
      else launch_step_t<uint16_t, 128, 1, AP, AT, EV, 0>(a, n, st);
    } else {
      if (r.res64) launch_step_t<uint16_t, 128, 0, AP, AT, EV, 1>(a, n, st);
      else launch_step_t<uint16_t, 128, 0, AP, AT, EV, 0>(a, n, st);
    }
  } else {
    if (c->head_dim == 64) launch_step_t<float, 64, 0, AP, AT, EV>(a, n, st);
    else launch_step_t<float, 128, 0, AP, AT, EV>(a, n, st);
  }
}

void launch_split(const hkv_config* c, const dev::StepArgs& a, int n, int n_split, float* part,
                  hipStream_t st) {
  if (c->dtype == HKV_DT_BF16) {
    if (c->head_dim == 64) launch_split_t<uint16_t, 64, 0>(a, n, n_split, part, st);
    else if (long_streams(c)) launch_split_t<uint16_t, 128, 1>(a, n, n_split, part, st);
    else launch_split_t<uint16_t, 128, 0>(a, n, n_split, part, st);
  } else {
    if (c->head_dim == 64) launch_split_t<float, 64, 0>(a, n, n_split, part, st);
    else launch_split_t<float, 128, 0>(a, n, n_split, part, st);
  }
}

float scale_log2_of(int d) { return float(1.4426950408889634 / std::sqrt(double(d))); }

dev::StepArgs step_args(const hkv_config* c, hkv_state* st, const Derived& d, int t) {
  dev::StepArgs a{};
  char* ws = static_cast<char*>(st->workspace);
  a.k_pool = static_cast<char*>(st->k_pool);
  a.v_pool = static_cast<char*>(st->v_pool);
  a.pos = st->pos;
  a.score = st->score;
  a.base = reinterpret_cast<const long long*>(st->base);
  a.count = st->count;
  a.budget = st->budget;
  a.cap = st->cap;
  a.label = st->label;
  a.free_slots = st->free_slots;
  a.n_free = st->n_free;
  a.qstat = reinterpret_cast<float4*>(st->qstat);
  a.err = st->err;
  a.ws_tile = reinterpret_cast<float*>(ws + d.ws_tile);
  a.ws_pos = reinterpret_cast<int*>(ws + d.ws_pos);
  a.ws_keys = reinterpret_cast<uint64_t*>(ws + d.ws_keys);
  a.t = t;
  a.w = c->local_window;
  a.W = c->w_obs;
  a.M = c->evict_m;
  a.D = d.split;
  a.scale_log2 = scale_log2_of(c->head_dim);
  a.S = int(d.S);
  a.res64 = 0;                         // set per launch (launch_step)
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

// Classification (k_classify, or k_prefill when q_stage is given, which also
// writes the prefill attention to `pout`) and initial layout (k_layout).
// Device address of dev::scratch on the current device, looked up once per
// device (each device holds its own copy of the buffer).
static hkv_status noalloc_scratch(float** out) {
  static std::mutex mu;
  static float* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(HKV_E_UNSUPPORTED, "device index %d beyond 63", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(dev::scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(HKV_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return HKV_OK;
}

// init_scores_override: where the classification scores go instead of the
// state's workspace (NULL: the workspace).
static hkv_status classify_impl(const hkv_config* c, hkv_state* st, const void* k_stage,
                                const void* v_stage, int64_t ld_stage, const void* q_obs,
                                int64_t ld_qobs, const void* q_stage, int64_t ld_q, void* pout,
                                int64_t ld_out, void* stream,
                                float* init_scores_override = nullptr) {
  clear_error();
  Derived d;
  hkv_status r = derive(c, &d);
  if (r != HKV_OK) return r;
  if ((r = check_state_buffers(c, st, init_scores_override == nullptr)) != HKV_OK) return r;
  const int eb = elem_bytes(c);
  if ((r = check_data_ptr(k_stage, ld_stage, eb, "k_stage")) != HKV_OK) return r;
  if ((r = check_data_ptr(v_stage, ld_stage, eb, "v_stage")) != HKV_OK) return r;
  if (ld_stage < int64_t(c->prefill_len) * c->head_dim)
    return fail(HKV_E_INVAL, "ld_stage smaller than prefill_len * head_dim");
  if (q_stage) {
    if (c->dtype != HKV_DT_BF16)
      return fail(HKV_E_UNSUPPORTED, "the fused prefill is built for bf16 only");
    if ((r = check_data_ptr(q_stage, ld_q, eb, "q_stage")) != HKV_OK) return r;
    if (ld_q < int64_t(c->prefill_len) * c->head_dim)
      return fail(HKV_E_INVAL, "ld_q smaller than prefill_len * head_dim");
    if ((r = check_data_ptr(pout, ld_out, eb, "out")) != HKV_OK) return r;
    if (ld_out < int64_t(c->prefill_len) * c->head_dim)
      return fail(HKV_E_INVAL, "ld_out smaller than prefill_len * head_dim");
    if (c->w_obs > 8) return fail(HKV_E_UNSUPPORTED, "classification holds at most 8 queries");
  } else if (!c->full_cache) {
    if ((r = check_data_ptr(q_obs, ld_qobs, eb, "q_obs")) != HKV_OK) return r;
    if (ld_qobs < int64_t(c->w_obs) * c->head_dim)
      return fail(HKV_E_INVAL, "ld_qobs smaller than w_obs * head_dim");
    if (c->w_obs > 8) return fail(HKV_E_UNSUPPORTED, "classification holds at most 8 queries");
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  float* init_scores = init_scores_override
                           ? init_scores_override
                           : reinterpret_cast<float*>(static_cast<char*>(st->workspace) +
                                                      d.ws_init_scores);

  hipLaunchKernelGGL(dev::k_reset_err, dim3(1), dim3(1), 0, hs, st->err);
  if ((r = after_launch("reset")) != HKV_OK) return r;

  if (q_stage) {
    dev::PrefillArgs a{};
    a.q_stage = static_cast<const char*>(q_stage);
    a.ld_q = ld_q;
    a.k_stage = static_cast<const char*>(k_stage);
    a.v_stage = static_cast<const char*>(v_stage);
    a.ld_stage = ld_stage;
    a.out = static_cast<char*>(pout);
    a.ld_out = ld_out;
    a.init_scores = init_scores;
    a.n_tokens = st->n_tokens;
    a.label = st->label;
    a.P = c->prefill_len;
    a.W = c->w_obs;
    a.w = c->local_window;
    // 8 waves (128 queries) per workgroup when one workgroup then covers the
    // whole prefill: each K and V block is staged once per stream.  Longer
    // prefills keep 64-query workgroups, which run their key blocks side by
    // side instead of one after another (measured on MI355X)
    const int nwq = c->prefill_len > 64 && c->prefill_len <= 128 ? 8 : 4;
    a.nqb = (c->prefill_len + 16 * nwq - 1) / (16 * nwq);
    a.classify = c->full_cache ? 0 : 1;
    a.tau = c->tau;
    a.scale_log2 = scale_log2_of(c->head_dim);
    const size_t lds = a.classify ? size_t(c->w_obs) * c->prefill_len * sizeof(float) : 0;
    const int n = int(d.S) * a.nqb;
    if (c->head_dim == 64)
      if (nwq == 8)
        hipLaunchKernelGGL((dev::k_prefill<64, 8>), dim3(n), dim3(512), lds, hs, a);
      else
        hipLaunchKernelGGL((dev::k_prefill<64, 4>), dim3(n), dim3(256), lds, hs, a);
    else
      if (nwq == 8)
        hipLaunchKernelGGL((dev::k_prefill<128, 8>), dim3(n), dim3(512), lds, hs, a);
      else
        hipLaunchKernelGGL((dev::k_prefill<128, 4>), dim3(n), dim3(256), lds, hs, a);
    if ((r = after_launch("k_prefill")) != HKV_OK) return r;
  } else if (!c->full_cache) {
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
  b.n_free = st->n_free;
  b.qstat = reinterpret_cast<float4*>(st->qstat);
  b.err = st->err;
  b.H = c->heads;
  b.N = c->final_len;
  b.P = c->prefill_len;
  b.w = c->local_window;
  b.W = c->w_obs;
  b.M = c->evict_m;
  b.D = d.split;
  b.A = d.A;
  b.full = c->full_cache;
  b.uniform = (c->variant & HKV_VARIANT_UNIFORM_BUDGET) ? 1 : 0;
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

hkv_status hkv_classify(const hkv_config* c, hkv_state* st, const void* k_stage,
                        const void* v_stage, int64_t ld_stage, const void* q_obs,
                        int64_t ld_qobs, void* stream) {
  return classify_impl(c, st, k_stage, v_stage, ld_stage, q_obs, ld_qobs, nullptr, 0, nullptr, 0,
                       stream);
}

hkv_status hkv_classify_noalloc(const hkv_config* c, hkv_state* st, const void* k_stage,
                                const void* v_stage, int64_t ld_stage, const void* q_obs,
                                int64_t ld_qobs, void* stream) {
  clear_error();
  Derived d;
  hkv_status r = derive(c, &d);
  if (r != HKV_OK) return r;
  const size_t need = size_t(d.S) * size_t(c->prefill_len) * sizeof(float);
  if (need > dev::kNoAllocScratchBytes)
    return fail(HKV_E_UNSUPPORTED,
                "hkv_classify_noalloc: streams * prefill_len * 4 = %zu bytes exceeds its "
                "%zu-byte scratch; use hkv_classify with a workspace",
                need, dev::kNoAllocScratchBytes);
  float* scr = nullptr;
  if ((r = noalloc_scratch(&scr)) != HKV_OK) return r;
  return classify_impl(c, st, k_stage, v_stage, ld_stage, q_obs, ld_qobs, nullptr, 0, nullptr, 0,
                       stream, scr);
}

hkv_status hkv_prefill(const hkv_config* c, hkv_state* st, const void* q_stage, int64_t ld_q,
                       const void* k_stage, const void* v_stage, int64_t ld_stage, void* out,
                       int64_t ld_out, void* stream) {
  if (!q_stage) {
    clear_error();
    return fail(HKV_E_INVAL, "q_stage is NULL");
  }
  return classify_impl(c, st, k_stage, v_stage, ld_stage, nullptr, 0, q_stage, ld_q, out, ld_out,
                       stream);
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

hkv_status hkv_ste_evict(const hkv_config* c, hkv_state* st, int32_t t, const void* q_win,
                         int64_t ld_qw, int32_t* log, int32_t s_begin, int32_t s_count,
                         void* stream) {
  Derived d;
  hkv_status r = common_checks(c, st, t, s_begin, s_count, &d);
  if (r != HKV_OK) return r;
  if (q_win) {
    if ((r = check_data_ptr(q_win, ld_qw, elem_bytes(c), "q_win")) != HKV_OK) return r;
    if (ld_qw < int64_t(c->w_obs) * c->head_dim)
      return fail(HKV_E_INVAL, "ld_qw smaller than w_obs * head_dim");
  }
  if (log && (reinterpret_cast<uintptr_t>(log) & 3u))
    return fail(HKV_E_INVAL, "evicted_pos_log misaligned");
  if (s_count == 0) return HKV_OK;
  dev::StepArgs a = step_args(c, st, d, t);
  a.q_win = static_cast<const char*>(q_win);
  a.ld_qw = ld_qw;
  if (q_win) {                      // newest query of the window
    a.q = a.q_win + (long long)(c->w_obs - 1) * c->head_dim * elem_bytes(c);
    a.ld_q = ld_qw;
  }
  a.log = log;
  a.s_begin = s_begin;
  launch_step<false, false, true>(c, a, s_count, static_cast<hipStream_t>(stream));
  return after_launch("k_step(evict)");
}

hkv_status hkv_decode_step(const hkv_config* c, hkv_state* st, int32_t t, const void* k_new,
                           const void* v_new, int64_t ld_kv, const void* q_win, int64_t ld_qw,
                           void* out, int64_t ld_o, int32_t* log, int32_t s_begin,
                           int32_t s_count, void* stream) {
  Derived d;
  hkv_status r = common_checks(c, st, t, s_begin, s_count, &d);
  if (r != HKV_OK) return r;
  const int eb = elem_bytes(c);
  if ((r = check_data_ptr(k_new, ld_kv, eb, "k_new")) != HKV_OK) return r;
  if ((r = check_data_ptr(v_new, ld_kv, eb, "v_new")) != HKV_OK) return r;
  if ((r = check_data_ptr(q_win, ld_qw, eb, "q_win")) != HKV_OK) return r;
  if (ld_qw < int64_t(c->w_obs) * c->head_dim)
    return fail(HKV_E_INVAL, "ld_qw smaller than w_obs * head_dim");
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
  a.q_win = static_cast<const char*>(q_win);
  a.ld_qw = ld_qw;
  a.q = a.q_win + (long long)(c->w_obs - 1) * c->head_dim * eb;   // newest query of the window
  a.ld_q = ld_qw;
  a.out = static_cast<char*>(out);
  a.ld_o = ld_o;
  a.log = log;
  a.s_begin = s_begin;
  launch_step<true, true, true>(c, a, s_count, static_cast<hipStream_t>(stream));
  return after_launch("k_step(fused)");
}

hkv_status hkv_decode_step_split(const hkv_config* c, hkv_state* st, int32_t t, const void* k_new,
                                 const void* v_new, int64_t ld_kv, const void* q_win,
                                 int64_t ld_qw, void* out, int64_t ld_o, int32_t* log,
                                 int32_t s_begin, int32_t s_count, int32_t n_split, void* stream) {
  Derived d;
  hkv_status r = common_checks(c, st, t, s_begin, s_count, &d);
  if (r != HKV_OK) return r;
  if (n_split < 1 || n_split > kMaxSplit)
    return fail(HKV_E_INVAL, "n_split %d outside [1, %d]", n_split, kMaxSplit);
  const int eb = elem_bytes(c);
  if ((r = check_data_ptr(k_new, ld_kv, eb, "k_new")) != HKV_OK) return r;
  if ((r = check_data_ptr(v_new, ld_kv, eb, "v_new")) != HKV_OK) return r;
  if ((r = check_data_ptr(q_win, ld_qw, eb, "q_win")) != HKV_OK) return r;
  if (ld_qw < int64_t(c->w_obs) * c->head_dim)
    return fail(HKV_E_INVAL, "ld_qw smaller than w_obs * head_dim");
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
  a.q_win = static_cast<const char*>(q_win);
  a.ld_qw = ld_qw;
  a.q = a.q_win + (long long)(c->w_obs - 1) * c->head_dim * eb;   // newest query of the window
  a.ld_q = ld_qw;
  a.out = static_cast<char*>(out);
  a.ld_o = ld_o;
  a.log = log;
  a.s_begin = s_begin;
  float* part = reinterpret_cast<float*>(static_cast<char*>(st->workspace) + d.ws_part);
  launch_split(c, a, s_count, n_split, part, static_cast<hipStream_t>(stream));
  return after_launch("k_split_attn/k_combine_evict");
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
