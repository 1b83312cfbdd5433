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
struct ScoreRound {
  int c[kRowsInFlight];
  float4 v[kQuadsPerLane][kRowsInFlight];
};

template <typename RowFn>
__device__ void load_round(int base, int d, int n, RowFn row, ScoreRound& rd) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / kLanesPerCand, lic = lane % kLanesPerCand;
  constexpr int per_wave = 64 / kLanesPerCand;
  constexpr int per_round = kWaves * per_wave;
  const float* r[kRowsInFlight];
#pragma unroll
  for (int u = 0; u < kRowsInFlight; ++u) {
    rd.c[u] = base + u * per_round + wave * per_wave + sub;
    r[u] = rd.c[u] < n ? row(rd.c[u]) : nullptr;
  }
#pragma unroll
  for (int i = 0; i < kQuadsPerLane; ++i)
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int q4 = lic + i * kLanesPerCand;
      rd.v[i][u] = float4{0.f, 0.f, 0.f, 0.f};
      if (r[u] && q4 < d / 4) rd.v[i][u] = *reinterpret_cast<const float4*>(r[u] + 4 * q4);
    }
}

__device__ inline void finish_round(const ScoreRound& rd, const double* qbar, int d, int n,
                                    unsigned long long* key) {
  const int lic = (threadIdx.x & 63) % kLanesPerCand;
  double acc[kRowsInFlight];
#pragma unroll
  for (int u = 0; u < kRowsInFlight; ++u) acc[u] = 0.0;
#pragma unroll
  for (int i = 0; i < kQuadsPerLane; ++i) {
    const int q4 = lic + i * kLanesPerCand;
    if (q4 >= d / 4) break;
    const double q0 = qbar[4 * q4], q1 = qbar[4 * q4 + 1], q2 = qbar[4 * q4 + 2], q3 = qbar[4 * q4 + 3];
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      acc[u] += q0 * (double)rd.v[i][u].x; acc[u] += q1 * (double)rd.v[i][u].y;
      acc[u] += q2 * (double)rd.v[i][u].z; acc[u] += q3 * (double)rd.v[i][u].w;
    }
  }
#pragma unroll
  for (int u = 0; u < kRowsInFlight; ++u) {
#pragma unroll
    for (int off = kLanesPerCand / 2; off > 0; off >>= 1) acc[u] += __shfl_xor(acc[u], off, kLanesPerCand);
    if (lic == 0 && rd.c[u] < n) key[rd.c[u]] = order_key(acc[u]);
  }
}

constexpr int kRoundRows = kRowsInFlight * kWaves * (64 / kLanesPerCand);   // rows per round

// Rounds from row `from` on (a multiple of kRoundRows), the loads of round
// `from` already issued into cur. With kPipelined the next round's loads are
// issued before a round is scored, so two rounds are in flight (their
// registers are left to the router kernel: inside the fused kernel they
// would push the attention's state out to scratch memory).
template <bool kPipelined, typename RowFn>
__device__ void score_rows(const double* qbar, int d, int n, RowFn row, unsigned long long* key, ScoreRound& cur,
                           int from) {
  if (!kPipelined) {
    finish_round(cur, qbar, d, n, key);
    for (int base = from + kRoundRows; base < n; base += kRoundRows) {
      load_round(base, d, n, row, cur);
      finish_round(cur, qbar, d, n, key);
    }
    return;
  }
  ScoreRound nxt;
  for (int base = from; base < n; base += 2 * kRoundRows) {
    const bool more = base + kRoundRows < n;
    if (more) load_round(base + kRoundRows, d, n, row, nxt);
    finish_round(cur, qbar, d, n, key);
    if (!more) break;
    if (base + 2 * kRoundRows < n) load_round(base + 2 * kRoundRows, d, n, row, cur);
    finish_round(nxt, qbar, d, n, key);
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
};

// Route item (query block b, KV head h) with all kThreads threads of the
// workgroup. emit(rank, group) is called once per kept group (ranks 0..n-1,
// ascending groups), by wave 0 or spread over the workgroup; the caller
// synchronises before reading what it stored. With write_out the item's rows
// of chunk_idx, group_idx (-1 padding; the kept entries are left to emit) and
// n_sel are written. Returns the number of kept groups. after_query() is
// called by every thread once the block query is formed (the fused kernel
// starts its first key/value tile loads there, behind the router's first
// loads).
struct NoHook {
  __device__ void operator()() const {}
};
template <typename T, bool kPipelined, typename GroupEmit, typename AfterQuery = NoHook>
__device__ int route_item(const RouteArgs& a, int b, int h, RouteSmem& sm, bool write_out, GroupEmit emit,
                          AfterQuery after_query = {}) {
  constexpr int E = Slice<T>::E;
  constexpr int kRowsPerThread = 8;   // block-query rows loaded per thread per round
  const Shape& S = a.s;
  const int d = S.d;
  const int64_t s = S.q0 + (int64_t)b * S.B;
  const int64_t ms = s / S.c;
  const int gpc = S.c / S.g;
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
  ScoreRound first;
  if (chunk_select) load_round(0, d, ncand, chunk_row, first);

  // ---- 1. block query (float64)
  {
    const int P = d / E;                       // 16-byte slices per row
    const int phases = kThreads / P;
    const int p = tid % P, ph = tid / P;
    double* part = reinterpret_cast<double*>(sm.key);   // [waves][d]
    const int nrows = S.G * S.B;
    const T* qbase = static_cast<const T*>(a.q);
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    for (int r = ph; r < nrows; r += kRowsPerThread * phases) {
      uint4 v[kRowsPerThread];
#pragma unroll
      for (int u = 0; u < kRowsPerThread; ++u) {
        const int rr = r + u * phases;
        v[u] = uint4{0u, 0u, 0u, 0u};
        if (rr < nrows) {
          const int64_t row = (int64_t)(h * S.G + rr / S.B) * S.qs + (s - S.q0) + rr % S.B;
          v[u] = *reinterpret_cast<const uint4*>(qbase + row * d + p * E);
        }
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

  const int64_t orow = (int64_t)b * S.hkv + h;
  // ---- 2-3. chunk stage
  if (chunk_select) {
    score_rows<kPipelined>(sm.qbar, d, ncand, chunk_row, sm.key, first, 0);
    __syncthreads();
    // the functors handed to the select capture by value: a by-reference
    // capture would keep the captured locals in scratch memory
    int* kept = sm.chunks;
    const int first_cand = (int)lo;
    if (wave == 0)
      wave_select(sm.key, ncand, nsc, sm.hist, [kept, first_cand](int rank, int pos) { kept[rank] = first_cand + pos; });
  } else {
    for (int i = tid; i < nsc; i += kThreads) sm.chunks[i] = (int)(lo + i);
  }
  __syncthreads();
  if (write_out)
    for (int i = tid; i < S.kc; i += kThreads) a.chunk_idx[orow * S.kc + i] = i < nsc ? sm.chunks[i] : -1;

  // ---- 4. group stage over the groups of the kept chunks (ascending order)
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
    ScoreRound g0;
    load_round(0, d, ngc, group_row, g0);
    score_rows<kPipelined>(sm.qbar, d, ngc, group_row, sm.key, g0, 0);
    __syncthreads();
    if (wave == 0) wave_select(sm.key, ngc, nsg, sm.hist, [emit, group_of](int rank, int pos) { emit(rank, group_of(pos)); });
  } else {
    for (int i = tid; i < nsg; i += kThreads) emit(i, group_of(i));
  }
  if (write_out) {
    for (int i = nsg + tid; i < S.kg; i += kThreads) gout[i] = -1;
    if (tid == 0) {
      a.n_sel[orow * 2 + 0] = nsc;
      a.n_sel[orow * 2 + 1] = nsg;
    }
  }
  return nsg;
}

}  // namespace route
}  // namespace hga
