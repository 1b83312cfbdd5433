// Device code of the two-level HGA router, shared by the router kernel and
// the fused route-then-attend kernel ("Long-Context Fine-Tuning with Limited
// VRAM", section 2.1, "Chunk selection" and "Group selection").
//
// One 512-thread workgroup routes one (query block, KV head) item. Every
// phase is a chain of dependent memory round trips, so each issues all of
// its loads before using any:
//   1. block query: mean of the block's queries over its 64 positions and the
//      G query heads of the KV head, accumulated in float64 (exact for
//      bfloat16 inputs, so independent of the summation order);
//   2. chunk stage: the candidates are the closed chunks before the block
//      that are neither sink nor local, a range [lo, hi); eight lanes score a
//      summary row (four rows per lane group in flight), each score the
//      float64 dot of the block query with the float32 chunk summary, stored
//      as a 64-bit order key (ascending key = descending score);
//   3. exact top-k by one wave with no block barrier, keys in registers: an
//      8-pass radix select (8 bits per pass, MSB first, stopping as soon as
//      the boundary bucket is taken whole) finds the k-th key T; the kept set
//      is every key below T plus the first keys equal to T in candidate order,
//      which is the lower-index tie rule because candidates are laid out in
//      ascending index order; ranks from ballots compact the kept positions,
//      so the output is ascending;
//   4. group stage: the groups of the kept chunks (ascending) are
//      scored the same way against the group summaries (device or pinned host
//      memory) and selected the same way; when the budget covers every group
//      of the kept chunks, all are kept and their summaries are never read.
// Outputs are ascending and -1 padded.
#pragma once

#include "hga_internal.h"

namespace hga {
namespace route {

constexpr int kThreads = 512;   // threads of a routing workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kLanesPerCand = 8;
constexpr int kRowsInFlight = 4;   // summary rows per lane group per round
constexpr int kGroupRowsWindow = 2;   // the same for the group stage with a window
constexpr int kQuadsPerLane = 128 / 4 / kLanesPerCand;   // float4s per lane and row (d <= 128)

template <typename T>
struct Slice;  // one 16-byte slice of a query row

template <>
struct Slice<float> {
  static constexpr int E = 4;
  __device__ static void add(const uint4& v, double* acc) {
    acc[0] += __uint_as_float(v.x); acc[1] += __uint_as_float(v.y);
    acc[2] += __uint_as_float(v.z); acc[3] += __uint_as_float(v.w);
  }
};

template <>
struct Slice<uint16_t> {
  static constexpr int E = 8;
  __device__ static void add(const uint4& v, double* acc) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// Order key: ascending key == descending score. -0 and +0 map to the same key.
__device__ inline unsigned long long order_key(double sc) {
  unsigned long long u = (unsigned long long)__double_as_longlong(sc);
  if (sc == 0.0) u = 0ull;
  u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
  return ~u;
}

struct RouteSmem {
  unsigned long long key[kMaxCand];      // order keys; also stages block-query partial sums
  int chunks[kMaxKeptChunks];            // kept chunks, ascending
  int hist[256];                         // radix histogram of the selecting wave
  double qbar[128];
};

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: a
// Hillis-Steele scan inside each row of 16 lanes, then the row totals
// (lane 15 of a row to the next row, lane 31 to the upper two rows).
__device__ inline int wave_inclusive_sum(int x) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr | 1, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr | 2, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr | 4, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr | 8, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowBcast15, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowBcast31, 0xc, 0xf, false);
  return x;
}

// One wave keeps the k smallest of key[0..n) in (key, position) order
// (0 < k < n <= 64 KPL) and calls emit(rank, position) for each kept
// position, ranks ascending with the position. Lane l holds the keys at
// positions l + 64 j in registers; hist is a 256-bin array private to the wave.
template <int KPL, typename EmitFn>
__device__ void wave_select_kpl(const unsigned long long* key, int n, int k, int* hist, EmitFn emit) {
  const int lane = threadIdx.x & 63;
  const unsigned long long lt = (1ull << lane) - 1ull;   // lanes below this one
  unsigned long long x[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) x[j] = lane + 64 * j < n ? key[lane + 64 * j] : ~0ull;
  auto valid = [&](int j) { return lane + 64 * j < n; };
  unsigned long long prefix = 0ull, mask = 0ull;
  int kk = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    *reinterpret_cast<int4*>(&hist[4 * lane]) = int4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const bool act = valid(j) && (x[j] & mask) == prefix;
      const int dg = (int)((x[j] >> shift) & 255);
      const unsigned long long am = __ballot(act);
      if (am) {
        // a wave whose matching keys share one digit adds them in one atomic
        const int first = __ffsll(am) - 1;
        const int d0 = __builtin_amdgcn_readlane(dg, first);
        if (__ballot(act && dg == d0) == am) {
          if (lane == first) atomicAdd(&hist[d0], __popcll(am));
        } else if (act) {
          atomicAdd(&hist[dg], 1);
        }
      }
    }
    // the bucket holding the kk-th smallest matching key
    const int4 hv = *reinterpret_cast<const int4*>(&hist[4 * lane]);
    const int sum = hv.x + hv.y + hv.z + hv.w;
    const int incl = wave_inclusive_sum(sum);
    const int excl = incl - sum;
    const bool mine = excl < kk && kk <= incl;
    int r = kk - excl, dg = 4 * lane, cnt = hv.x;
    if (r > hv.x) { r -= hv.x; ++dg; cnt = hv.y; if (r > hv.y) { r -= hv.y; ++dg; cnt = hv.z; if (r > hv.z) { r -= hv.z; ++dg; cnt = hv.w; } } }
    const int owner = __ffsll(__ballot(mine)) - 1;
    dg = __builtin_amdgcn_readlane(dg, owner);
    r = __builtin_amdgcn_readlane(r, owner);
    cnt = __builtin_amdgcn_readlane(cnt, owner);
    prefix |= (unsigned long long)dg << shift;
    mask |= 255ull << shift;
    kk = r;
    if (kk == cnt) break;   // the whole bucket is kept: no finer digit is needed
  }
  // kept: masked key below the prefix, or equal to it among the first kk in
  // position order; ranks in position order from ballots (row j before row
  // j + 1, lanes ascending within a row)
  int eq_seen = 0, kept_seen = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const unsigned long long xm = x[j] & mask;
    const bool eq = valid(j) && xm == prefix;
    const unsigned long long em = __ballot(eq);
    const bool keep = valid(j) && (xm < prefix || (eq && eq_seen + __popcll(em & lt) < kk));
    const unsigned long long km = __ballot(keep);
    if (keep) emit(kept_seen + __popcll(km & lt), lane + 64 * j);
    eq_seen += __popcll(em);
    kept_seen += __popcll(km);
  }
}

// The same for at most kMax keys (512 or 1024), with every variant inlined:
// the caller then makes no function call and holds no stack frame (a call
// from the fused route-and-attend kernel kept 232 bytes per lane in scratch
// memory).
template <int kMax, typename EmitFn>
__device__ __attribute__((always_inline)) void wave_select_inline(const unsigned long long* key, int n, int k,
                                                                  int* hist, EmitFn emit) {
  static_assert(kMax == 512 || kMax == 1024, "inlined selections");
  if (n <= 64) wave_select_kpl<1>(key, n, k, hist, emit);
  else if (n <= 128) wave_select_kpl<2>(key, n, k, hist, emit);
  else if (n <= 256) wave_select_kpl<4>(key, n, k, hist, emit);
  else if (kMax == 512 || n <= 512) wave_select_kpl<8>(key, n, k, hist, emit);
  else wave_select_kpl<16>(key, n, k, hist, emit);
}

template <typename EmitFn>
__device__ void wave_select(const unsigned long long* key, int n, int k, int* hist, EmitFn emit) {
  if (n <= 64) wave_select_kpl<1>(key, n, k, hist, emit);
  else if (n <= 128) wave_select_kpl<2>(key, n, k, hist, emit);
  else if (n <= 256) wave_select_kpl<4>(key, n, k, hist, emit);
  else if (n <= 512) wave_select_kpl<8>(key, n, k, hist, emit);
  else if (n <= 1024) wave_select_kpl<16>(key, n, k, hist, emit);
  else if (n <= 2048) wave_select_kpl<32>(key, n, k, hist, emit);
  else wave_select_kpl<64>(key, n, k, hist, emit);
}

// Score summary rows c in [0, n) against the block query: row(c) points at d
// float32 values; the order key goes to key[c]. Eight lanes per row,
// kRowsInFlight rows per lane group per round; a round's loads are all
// issued before any is used, and the first round's may be issued early
// (before the block query exists) by load_round.
template <int R = kRowsInFlight>
struct ScoreRound {
  int c[R];
  float4 v[kQuadsPerLane][R];
};
template <int R>
constexpr int round_rows() { return R * kWaves * (64 / kLanesPerCand); }

// kFlat (the single-round scoring of the fused route-and-attend kernel): no
// load depends on a per-lane condition (slots past the last row read the
// last row, or row 0 of the candidates when there are none; quads past d
// read the row's first quad; finish_round uses neither; only a slot group
// with no row for the whole wave skips its loads), and finish_round takes
// the data through an empty asm. Otherwise the compiler converted each loaded value to float64
// inside the load's condition, right after the load, so every load waited on
// its own (one round trip each) and the first round waited before the block
// query's loads could issue. The router kernel, two rounds in flight, keeps
// the conditional loads (the flat form slowed it down).
template <bool kFlat, bool kSkipEmpty = true, typename RowFn, int R>
__device__ __attribute__((always_inline)) void load_round(int base, int d, int n, RowFn row, ScoreRound<R>& rd) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / kLanesPerCand, lic = lane % kLanesPerCand;
  constexpr int per_wave = 64 / kLanesPerCand;
  constexpr int per_round = kWaves * per_wave;
  const float* r[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    rd.c[u] = base + u * per_round + wave * per_wave + sub;
    if (kFlat)
      r[u] = row(rd.c[u] < n ? rd.c[u] : (n > 0 ? n - 1 : 0));
    else
      r[u] = rd.c[u] < n ? row(rd.c[u]) : nullptr;
  }
#pragma unroll
  for (int i = 0; i < kQuadsPerLane; ++i)
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int q4 = lic + i * kLanesPerCand;
      if (kFlat) {
        // a slot group with no row of the round for this wave skips its loads
        // (a wave-uniform branch)
        const int first_row = base + u * per_round + __builtin_amdgcn_readfirstlane(wave) * per_wave;
        if (!kSkipEmpty || first_row < n)
          rd.v[i][u] = *reinterpret_cast<const float4*>(r[u] + 4 * (q4 < d / 4 ? q4 : 0));
      } else {
        rd.v[i][u] = float4{0.f, 0.f, 0.f, 0.f};
        if (r[u] && q4 < d / 4) rd.v[i][u] = *reinterpret_cast<const float4*>(r[u] + 4 * q4);
      }
    }
}

template <bool kFlat, int R>
__device__ inline void finish_round(const ScoreRound<R>& rd_in, const double* qbar, int d, int n,
                                    unsigned long long* key) {
  const int lic = (threadIdx.x & 63) % kLanesPerCand;
  ScoreRound<R> rd = rd_in;
  if (kFlat) {
#pragma unroll
    for (int i = 0; i < kQuadsPerLane; ++i)
#pragma unroll
      for (int u = 0; u < R; ++u)
        asm volatile("" : "+v"(rd.v[i][u].x), "+v"(rd.v[i][u].y), "+v"(rd.v[i][u].z), "+v"(rd.v[i][u].w));
  }
  double acc[R];
#pragma unroll
  for (int u = 0; u < R; ++u) acc[u] = 0.0;
#pragma unroll
  for (int i = 0; i < kQuadsPerLane; ++i) {
    const int q4 = lic + i * kLanesPerCand;
    if (q4 >= d / 4) break;
    const double q0 = qbar[4 * q4], q1 = qbar[4 * q4 + 1], q2 = qbar[4 * q4 + 2], q3 = qbar[4 * q4 + 3];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      acc[u] += q0 * (double)rd.v[i][u].x; acc[u] += q1 * (double)rd.v[i][u].y;
      acc[u] += q2 * (double)rd.v[i][u].z; acc[u] += q3 * (double)rd.v[i][u].w;
    }
  }
#pragma unroll
  for (int u = 0; u < R; ++u) {
#pragma unroll
    for (int off = kLanesPerCand / 2; off > 0; off >>= 1) acc[u] += __shfl_xor(acc[u], off, kLanesPerCand);
    if (lic == 0 && rd.c[u] < n) key[rd.c[u]] = order_key(acc[u]);
  }
}

constexpr int kRoundRows = round_rows<kRowsInFlight>();   // rows per round

// Whether every item of the call selects among at most m candidates at both
// stages (the chunk candidates of the last block, the most any block has;
// the groups of the kept chunks), so that route_item may inline its
// selections (kSelectMax = m).
inline bool select_fits(const Shape& s, int m) {
  const int64_t last_chunk = (s.q0 + s.nq - 1) / kChunk;   // the last block's chunk
  return last_chunk - s.sink_chunks - s.local_chunks <= m && (int64_t)s.kc * (kChunk / s.g) <= m;
}
inline bool select512_fits(const Shape& s) { return select_fits(s, 512); }

// Rounds from row `from` on (a multiple of kRoundRows), the loads of round
// `from` already issued into cur. With kPipelined the next round's loads are
// issued before a round is scored, so two rounds are in flight (their
// registers are left to the router kernel: inside the fused kernel they
// would push the attention's state out to scratch memory).
template <bool kPipelined, typename RowFn, int R>
__device__ __attribute__((always_inline)) void score_rows(const double* qbar, int d, int n, RowFn row,
                                                          unsigned long long* key, ScoreRound<R>& cur, int from) {
  constexpr int RR = round_rows<R>();
  if (!kPipelined) {
    finish_round<true>(cur, qbar, d, n, key);
    for (int base = from + RR; base < n; base += RR) {
      load_round<true>(base, d, n, row, cur);
      finish_round<true>(cur, qbar, d, n, key);
    }
    return;
  }
  ScoreRound<R> nxt;
  for (int base = from; base < n; base += 2 * RR) {
    const bool more = base + RR < n;
    if (more) load_round<false>(base + RR, d, n, row, nxt);
    finish_round<false>(cur, qbar, d, n, key);
    if (!more) break;
    if (base + 2 * RR < n) load_round<false>(base + 2 * RR, d, n, row, cur);
    finish_round<false>(nxt, qbar, d, n, key);
  }
}

struct RouteArgs {
  const void* q;
  const float* cs;
  const float* gs_host;
  const float* gs_dev;
  int64_t split;         // group summaries of tokens [0, split) are in gs_host
  int32_t* chunk_idx;
  int32_t* group_idx;
  int32_t* n_sel;
  Shape s;
  double* qbar_out;      // if set, each item's block query is stored ([nb][Hkv][d])
  bool chunks_only;      // stop after the chunk stage (the group stage runs later)
  // Marks of the persistent host-tier cache (unused when null): the history
  // (tokens below need_split) an item needs, OR-ed into [Hkv][need_split / 64]
  // words, and the requests counted in counters.
  uint64_t* kv_need;     // with the group stage: bit u of chunk m = group u of m is attended
  uint64_t* gs_need;     // with chunks_only: bit 0 of chunk m = its group summaries are scored
  long long* counters;
  int64_t need_split;
};

template <bool kPipelined, typename GroupEmit, typename RowFn>
__device__ __attribute__((always_inline)) int group_stage(const RouteArgs& a, int b, int h, RouteSmem& sm, int nsc,
                                                          bool write_out, GroupEmit emit, RowFn gs_row);

}  // namespace route

// The router kernel over every item with the given arguments (with
// chunks_only, the chunk stage only; with qbar_out, the block queries kept).
hipError_t launch_route_args(const route::RouteArgs& a, hipStream_t st);

namespace route {

// Route item (query block b, KV head h) with all kThreads threads of the
// workgroup. emit(rank, group) is called once per kept group (ranks 0..n-1,
// ascending groups), by wave 0 or spread over the workgroup; the caller
// synchronises before reading what it stored. With write_out the item's rows
// of chunk_idx, group_idx (-1 padding; the kept entries are left to emit) and
// n_sel are written. Returns the number of kept groups. kCache enables the
// persistent cache's options of the arguments (qbar_out, chunks_only: then
// the number of kept chunks is returned, the chunks in sm.chunks); without
// it they are ignored and cost nothing. after_query() is
// called by every thread once the block query is formed (the fused kernel
// starts its first key/value tile loads there, behind the router's first
// loads). kSelectMax (512 or 1024; 0: any number): both selections take at
// most that many candidates (the caller checks), so they are inlined and the
// item is routed with no function call.
struct NoHook {
  __device__ void operator()() const {}
};
// Hooks for work that needs no routing (the fused kernel's query operands
// and first attention tiles): queries_issued() runs once the block query's
// first rows and the first round of chunk summaries are requested;
// chunks_kept() runs after the barrier that follows the chunk
// selection; scored() before the barrier after the group scores, and
// selected() once the wave selecting the groups is done (every other wave
// reaches it right after that barrier). With no group selection the window
// still has that barrier. NoWindow has no hooks and adds no barrier.
struct NoWindow {
  static constexpr bool kActive = false;
  __device__ void queries_issued() const {}
  __device__ void chunks_selected() const {}
  __device__ void chunks_kept() const {}
  __device__ void groups_issued() const {}
  __device__ void scored() const {}
  __device__ void selected() const {}
};
template <typename F0, typename F1, typename F2, typename F3, typename F4, typename F5>
struct EarlyWindow {
  static constexpr bool kActive = true;
  F0 f0;
  F1 f1;
  F2 f2;
  F3 f3;
  F4 f4;
  F5 f5;
  __device__ __attribute__((always_inline)) void queries_issued() const { f0(); }
  __device__ __attribute__((always_inline)) void chunks_selected() const { f4(); }
  __device__ __attribute__((always_inline)) void chunks_kept() const { f1(); }
  __device__ __attribute__((always_inline)) void groups_issued() const { f5(); }
  __device__ __attribute__((always_inline)) void scored() const { f2(); }
  __device__ __attribute__((always_inline)) void selected() const { f3(); }
};
template <typename T, bool kPipelined, bool kCache = false, typename GroupEmit, typename AfterQuery = NoHook,
          int kSelectMax = 0, typename Window = NoWindow>
__device__ __attribute__((always_inline)) int route_item(const RouteArgs& a, int b, int h, RouteSmem& sm,
                                                         bool write_out, GroupEmit emit, AfterQuery after_query = {},
                                                         Window window = {}) {
  constexpr int E = Slice<T>::E;
  constexpr int kRowsPerThread = 8;   // block-query rows loaded per thread per round
  const Shape& S = a.s;
  const int d = S.d;
  const int64_t s = S.q0 + (int64_t)b * S.B;
  const int64_t ms = s / S.c;
  const int tid = threadIdx.x, wave = tid >> 6;

  // chunk-stage candidates [lo, hi); the first round of their summaries is
  // requested now, so its latency overlaps the block query's
  int64_t lo, hi;
  fixed_windows(ms, S.sink_chunks, S.local_chunks, &lo, &hi);
  const int ncand = (int)(hi - lo);
  const int nsc = ncand < S.kc ? ncand : S.kc;
  const bool chunk_select = nsc > 0 && nsc < ncand;
  const float* csh = a.cs + (int64_t)h * (S.kvs / S.c) * d;
  auto chunk_row = [&](int c) { return csh + (lo + c) * d; };
  // block-query rows: thread (p, ph) sums 16-byte slice p of rows ph,
  // ph + phases, ...; with a window the first kRowsPerThread of them load
  // before the first round of chunk summaries, unconditionally (rows past
  // the item read its last row and count as zero), so the block query waits
  // for its own rows only
  const int P = d / E;                       // 16-byte slices per row
  const int phases = kThreads / P;
  const int p = tid % P, ph = tid / P;
  const int nrows = S.G * S.B;
  const T* qbase = static_cast<const T*>(a.q);
  auto q_slice = [&](int rr) {
    const int64_t row = (int64_t)(h * S.G + rr / S.B) * S.qs + (s - S.q0) + rr % S.B;
    return reinterpret_cast<const uint4*>(qbase + row * d + p * E);
  };
  uint4 v0[kRowsPerThread];
  if constexpr (Window::kActive) {
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
      const int rr = ph + u * phases;
      v0[u] = *q_slice(rr < nrows ? rr : nrows - 1);
    }
  }
  ScoreRound<> first;
  // (with a window, no branch around them either: the compiler's waits for
  // the block query's rows would then count every later load as pending)
  if (!kPipelined || chunk_select) load_round<!kPipelined, !Window::kActive>(0, d, ncand, chunk_row, first);
  window.queries_issued();

  // ---- 1. block query (float64)
  {
    double* part = reinterpret_cast<double*>(sm.key);   // [waves][d]
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    int r0 = ph;
    if constexpr (Window::kActive) {
#pragma unroll
      for (int u = 0; u < kRowsPerThread; ++u) {
        // the rows in registers as loaded (otherwise the compiler copies
        // them under the row condition and waits for every later load too)
        asm volatile("" : "+v"(v0[u].x), "+v"(v0[u].y), "+v"(v0[u].z), "+v"(v0[u].w));
        const unsigned keep = ph + u * phases < nrows ? 0xffffffffu : 0u;
        Slice<T>::add(uint4{v0[u].x & keep, v0[u].y & keep, v0[u].z & keep, v0[u].w & keep}, acc);
      }
      r0 += kRowsPerThread * phases;
    }
    for (int r = r0; r < nrows; r += kRowsPerThread * phases) {
      uint4 v[kRowsPerThread];
#pragma unroll
      for (int u = 0; u < kRowsPerThread; ++u) {
        const int rr = r + u * phases;
        v[u] = uint4{0u, 0u, 0u, 0u};
        if (rr < nrows) v[u] = *q_slice(rr);
      }
#pragma unroll
      for (int u = 0; u < kRowsPerThread; ++u) Slice<T>::add(v[u], acc);
    }
    // lanes of a wave with the same slice are P apart: fold them, then the
    // 8 wave partials through LDS
    for (int off = P; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += __shfl_xor(acc[e], off);
    if ((tid & 63) < P)
#pragma unroll
      for (int e = 0; e < E; ++e) part[wave * d + p * E + e] = acc[e];
    __syncthreads();
    if (tid < d) {
      double t = 0.0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) t += part[w * d + tid];
      sm.qbar[tid] = t / nrows;
    }
    __syncthreads();
  }
  after_query();

  if constexpr (kCache) {
    if (a.qbar_out && write_out && tid < d) a.qbar_out[((int64_t)b * S.hkv + h) * d + tid] = sm.qbar[tid];
  }
  const int64_t orow = (int64_t)b * S.hkv + h;
  // ---- 2-3. chunk stage
  if (chunk_select) {
    score_rows<kPipelined>(sm.qbar, d, ncand, chunk_row, sm.key, first, 0);
    __syncthreads();
    // the functors handed to the select capture by value: a by-reference
    // capture would keep the captured locals in scratch memory
    int* kept = sm.chunks;
    const int first_cand = (int)lo;
    if (wave == 0) {
      auto keep = [kept, first_cand](int rank, int pos) { kept[rank] = first_cand + pos; };
      if constexpr (kSelectMax > 0)
        wave_select_inline<kSelectMax>(sm.key, ncand, nsc, sm.hist, keep);
      else
        wave_select(sm.key, ncand, nsc, sm.hist, keep);
    }
  } else {
    for (int i = tid; i < nsc; i += kThreads) sm.chunks[i] = (int)(lo + i);
  }
  window.chunks_selected();
  __syncthreads();
  window.chunks_kept();
  // (with a window the kept chunks are written at the end: a store in flight
  // here holds its registers, and the compiler's wait before reusing them
  // would wait for the group summaries too)
  if (write_out && !Window::kActive)
    for (int i = tid; i < S.kc; i += kThreads) a.chunk_idx[orow * S.kc + i] = i < nsc ? sm.chunks[i] : -1;

  if constexpr (kCache) {
    if (a.chunks_only) {
      if (write_out && tid == 0) a.n_sel[orow * 2 + 0] = nsc;
      return nsc;
    }
  }
  // ---- 4. group stage over the groups of the kept chunks (ascending order)
  // (written out here rather than through group_stage below: the fused
  // kernel's registers are allocated better this way, 232 against 744 bytes
  // of spill space)
  const int gpc = S.c / S.g;
  const int ngc = nsc * gpc;
  const int nsg = ngc < S.kg ? ngc : S.kg;
  int32_t* gout = a.group_idx + orow * S.kg;   // written only with write_out
  const int* kept_chunks = sm.chunks;
  auto group_of = [kept_chunks, gpc](int c) { return kept_chunks[c / gpc] * gpc + c % gpc; };
  if (nsg > 0 && nsg < ngc) {
    const int64_t gsplit = a.split / S.g;          // groups held in host memory
    const int64_t ngl = S.kvs / S.g;
    auto group_row = [&](int c) -> const float* {
      const int64_t j = group_of(c);
      return j < gsplit ? a.gs_host + ((int64_t)h * gsplit + j) * d
                        : a.gs_dev + ((int64_t)h * (ngl - gsplit) + (j - gsplit)) * d;
    };
    // with a window an attention tile runs while these rows load: fewer
    // rows per round leave it its registers
    ScoreRound<Window::kActive ? kGroupRowsWindow : kRowsInFlight> g0;
    load_round<!kPipelined, !Window::kActive>(0, d, ngc, group_row, g0);
    window.groups_issued();
    score_rows<kPipelined>(sm.qbar, d, ngc, group_row, sm.key, g0, 0);
    window.scored();
    __syncthreads();
    if (wave == 0) {
      auto keep = [emit, group_of](int rank, int pos) { emit(rank, group_of(pos)); };
      if constexpr (kSelectMax > 0)
        wave_select_inline<kSelectMax>(sm.key, ngc, nsg, sm.hist, keep);
      else
        wave_select(sm.key, ngc, nsg, sm.hist, keep);
    }
  } else {
    for (int i = tid; i < nsg; i += kThreads) emit(i, group_of(i));
    if constexpr (Window::kActive) {
      window.groups_issued();
      window.scored();
      __syncthreads();
    }
  }
  window.selected();
  if (write_out) {
    if (Window::kActive)
      for (int i = tid; i < S.kc; i += kThreads) a.chunk_idx[orow * S.kc + i] = i < nsc ? sm.chunks[i] : -1;
    for (int i = nsg + tid; i < S.kg; i += kThreads) gout[i] = -1;
    if (tid == 0) {
      a.n_sel[orow * 2 + 0] = nsc;
      a.n_sel[orow * 2 + 1] = nsg;
    }
  }
  return nsg;
}

// Group stage of item (b, h) on its own (the persistent cache's group kernel,
// after the chunk stage ran alone), given its nsc kept chunks (ascending, in
// sm.chunks) and its block query (sm.qbar), with all kThreads threads:
// score the groups of the kept chunks, keep the top_groups (ties to the
// lower group index), emit them ascending (see route_item), and with
// write_out write the -1 padding and the kept count. gs_row(c, j) gives the
// d float32 values of the summary of group j, candidate c (group c % (c/g)
// of kept chunk c / (c/g)). Returns the number kept.
template <bool kPipelined, typename GroupEmit, typename RowFn>
__device__ __attribute__((always_inline)) int group_stage(const RouteArgs& a, int b, int h, RouteSmem& sm, int nsc,
                                                          bool write_out, GroupEmit emit, RowFn gs_row) {
  const Shape& S = a.s;
  const int d = S.d;
  const int gpc = S.c / S.g;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t orow = (int64_t)b * S.hkv + h;
  const int ngc = nsc * gpc;
  const int nsg = ngc < S.kg ? ngc : S.kg;
  int32_t* gout = a.group_idx + orow * S.kg;   // written only with write_out
  const int* kept_chunks = sm.chunks;
  auto group_of = [kept_chunks, gpc](int c) { return kept_chunks[c / gpc] * gpc + c % gpc; };
  if (nsg > 0 && nsg < ngc) {
    auto group_row = [gs_row, group_of](int c) -> const float* { return gs_row(c, (int64_t)group_of(c)); };
    ScoreRound<> g0;
    load_round<!kPipelined>(0, d, ngc, group_row, g0);
    score_rows<kPipelined>(sm.qbar, d, ngc, group_row, sm.key, g0, 0);
    __syncthreads();
    if (wave == 0) wave_select(sm.key, ngc, nsg, sm.hist, [emit, group_of](int rank, int pos) { emit(rank, group_of(pos)); });
  } else {
    for (int i = tid; i < nsg; i += kThreads) emit(i, group_of(i));
  }
  if (write_out) {
    for (int i = nsg + tid; i < S.kg; i += kThreads) gout[i] = -1;
    if (tid == 0) a.n_sel[orow * 2 + 1] = nsg;
  }
  return nsg;
}

// Emit function of the router kernels: stores the kept group and, with the
// persistent cache's marks, sets the group's bit in kv_need when it lies in
// the history and counts it in *hist (shared memory).
struct MarkingEmit {
  int32_t* gout;
  uint64_t* need;     // the KV head's row of kv_need, or null
  int g;
  int64_t split;
  int* hist;
  __device__ void operator()(int rank, int group) const {
    gout[rank] = group;
    const int64_t tok = (int64_t)group * g;
    if (need && tok < split) {
      atomicOr(reinterpret_cast<unsigned long long*>(&need[tok / kChunk]), 1ull << ((tok % kChunk) / g));
      atomicAdd(hist, 1);
    }
  }
};

// After the group stage of item (b, h) (every thread, after a barrier that
// follows the emits): mark the item's fixed chunks below need_split as whole
// chunks in kv_need and add the item's K/V requests (hist kept history
// groups plus the fixed chunks' groups) to the counters.
__device__ inline void mark_fixed_chunks(const RouteArgs& a, int b, int h, int hist) {
  const Shape& S = a.s;
  const int64_t ms = (S.q0 + (int64_t)b * S.B) / S.c;
  int64_t fa, fbb;
  fixed_windows(ms, S.sink_chunks, S.local_chunks, &fa, &fbb);
  const int64_t nch = a.need_split / kChunk;
  const int gpc = kChunk / S.g;
  const uint64_t full = gpc == 64 ? ~0ull : (1ull << gpc) - 1ull;
  const int nfix = (int)(fa + (ms - fbb));
  for (int t = threadIdx.x; t < nfix; t += blockDim.x) {
    const int64_t m = t < fa ? t : fbb + (t - fa);
    if (m < nch) atomicOr(reinterpret_cast<unsigned long long*>(&a.kv_need[(int64_t)h * nch + m]), full);
  }
  if (threadIdx.x == 0) {
    const int64_t sink_hist = fa < nch ? fa : nch;
    const int64_t lo = fbb > nch ? nch : fbb, hi = ms > nch ? nch : ms;
    const long long n = hist + (long long)gpc * (sink_hist + (hi - lo));
    if (n) atomicAdd(reinterpret_cast<unsigned long long*>(&a.counters[kTcKvRequests]), (unsigned long long)n);
  }
}

// After the chunk stage of item h (chunks_only, every thread): when its group
// stage will score summaries, mark its kept history chunks in gs_need and
// count them. `count` is a shared-memory int the caller zeroed before a
// barrier.
__device__ inline void mark_summary_chunks(const RouteArgs& a, int h, const RouteSmem& sm, int nsc, int* count) {
  const Shape& S = a.s;
  const int gpc = kChunk / S.g;
  if (!(S.kg > 0 && S.kg < nsc * gpc)) return;   // every group kept (or none): no summary is read
  const int64_t nch = a.need_split / kChunk;
  int n = 0;
  for (int i = threadIdx.x; i < nsc; i += blockDim.x) {
    const int m = sm.chunks[i];
    if (m >= 0 && m < nch) {
      atomicOr(reinterpret_cast<unsigned long long*>(&a.gs_need[(int64_t)h * nch + m]), 1ull);
      ++n;
    }
  }
  if (n) atomicAdd(count, n);
  __syncthreads();
  if (threadIdx.x == 0 && *count)
    atomicAdd(reinterpret_cast<unsigned long long*>(&a.counters[kTcGsRequests]), (unsigned long long)*count);
}

}  // namespace route
}  // namespace hga
