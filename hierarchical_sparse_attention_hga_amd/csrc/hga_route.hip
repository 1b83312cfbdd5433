// Two-level HGA router ("Long-Context Fine-Tuning with Limited VRAM",
// section 2.1, "Chunk selection" and "Group selection").
//
// One 512-thread workgroup routes one (query block, KV head) item:
//   1. block query: mean of the block's queries over its 64 positions and the
//      G query heads of the KV head, accumulated in float64 (exact for
//      bfloat16 inputs, so independent of the summation order); every thread
//      issues all of its 16-byte row loads before adding;
//   2. chunk stage: the candidates are the closed chunks before the block
//      that are neither sink nor local (a contiguous range); each score is the
//      float64 dot of the block query with the float32 chunk summary, eight
//      lanes per candidate, two candidates per lane group in flight;
//   3. exact top-k by an 8-pass radix select (8 bits per pass, MSB first) on
//      64-bit order keys (ascending key = descending score): it finds the k-th
//      key T; the kept set is every key below T plus the first keys equal to
//      T in candidate order, which is the lower-index tie rule because
//      candidates are laid out in ascending index order. A block-wide scan
//      then compacts the kept positions, so the output is ascending;
//   4. group stage: the groups of the kept chunks (ascending) are scored the
//      same way against the group summaries (device or pinned host memory)
//      and selected the same way; when the budget covers every group of the
//      kept chunks, all are kept and their summaries are never read.
// Outputs are ascending and -1 padded.
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kLanesPerCand = 8;

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
  unsigned long long key[kMaxCand];    // order keys; also stages block-query partial sums
  int chunks[kMaxKeptChunks];          // kept chunks, ascending
  int hist[256];
  int scan[kWaves];
  int misc[2];
  double qbar[128];
};

// Block-wide exclusive prefix sum of one int per thread; *total gets the sum.
__device__ int block_exclusive_sum(int v, int* scan, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scan[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = scan[w];
    pre += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return pre + x - v;
}

// Score candidates c in [0, n): row(c) points at d float32 values.
template <typename RowFn>
__device__ void score_rows(const double* qbar, int d, int n, RowFn row, unsigned long long* key) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / kLanesPerCand, lic = lane % kLanesPerCand;
  constexpr int per_wave = 64 / kLanesPerCand;
  constexpr int per_round = kWaves * per_wave;
  const int quads = d / 4;
  for (int base = 0; base < n; base += 2 * per_round) {
    const int c0 = base + wave * per_wave + sub, c1 = c0 + per_round;
    double a0 = 0.0, a1 = 0.0;
    const float* r0 = c0 < n ? row(c0) : nullptr;
    const float* r1 = c1 < n ? row(c1) : nullptr;
    for (int q4 = lic; q4 < quads; q4 += kLanesPerCand) {
      float4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
      if (r0) v0 = *reinterpret_cast<const float4*>(r0 + 4 * q4);
      if (r1) v1 = *reinterpret_cast<const float4*>(r1 + 4 * q4);
      const double* qb = qbar + 4 * q4;
      a0 += qb[0] * (double)v0.x; a0 += qb[1] * (double)v0.y; a0 += qb[2] * (double)v0.z; a0 += qb[3] * (double)v0.w;
      a1 += qb[0] * (double)v1.x; a1 += qb[1] * (double)v1.y; a1 += qb[2] * (double)v1.z; a1 += qb[3] * (double)v1.w;
    }
#pragma unroll
    for (int off = kLanesPerCand / 2; off > 0; off >>= 1) {
      a0 += __shfl_xor(a0, off, kLanesPerCand);
      a1 += __shfl_xor(a1, off, kLanesPerCand);
    }
    if (lic == 0) {
      if (c0 < n) key[c0] = order_key(a0);
      if (c1 < n) key[c1] = order_key(a1);
    }
  }
}

// Keep the k smallest of key[0..n) in (key, position) order (0 < k < n) and
// call emit(rank, position) for each kept position, ranks ascending with the
// position. Ends with a barrier.
template <typename EmitFn>
__device__ void select_smallest(const unsigned long long* key, int n, int k, RouteSmem& sm, EmitFn emit) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned long long prefix = 0ull, mask = 0ull;
  int kk = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = tid; i < 256; i += kThreads) sm.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const unsigned long long x = key[i];
      if ((x & mask) == prefix) atomicAdd(&sm.hist[(x >> shift) & 255], 1);
    }
    __syncthreads();
    if (wave == 0) {
      const int h0 = sm.hist[4 * lane], h1 = sm.hist[4 * lane + 1];
      const int h2 = sm.hist[4 * lane + 2], h3 = sm.hist[4 * lane + 3];
      const int sum = h0 + h1 + h2 + h3;
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const int excl = incl - sum;
      if (excl < kk && kk <= incl) {
        int r = kk - excl, dg = 4 * lane;
        if (r > h0) { r -= h0; ++dg; if (r > h1) { r -= h1; ++dg; if (r > h2) { r -= h2; ++dg; } } }
        sm.misc[0] = dg;
        sm.misc[1] = r;
      }
    }
    __syncthreads();
    prefix |= (unsigned long long)sm.misc[0] << shift;
    mask |= 255ull << shift;
    kk = sm.misc[1];
    __syncthreads();
  }
  // kept: key < T, or key == T among the first kk such keys by position
  const unsigned long long T = prefix;
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = tid * per, hi = lo + per < n ? lo + per : n;
  int eq = 0;
  for (int i = lo; i < hi; ++i) eq += key[i] == T;
  int tot;
  int eq_before = block_exclusive_sum(eq, sm.scan, &tot);
  int kept = 0;
  {
    int e = eq_before;
    for (int i = lo; i < hi; ++i) {
      const unsigned long long x = key[i];
      if (x < T || (x == T && e++ < kk)) ++kept;
    }
  }
  int rank = block_exclusive_sum(kept, sm.scan, &tot);
  {
    int e = eq_before;
    for (int i = lo; i < hi; ++i) {
      const unsigned long long x = key[i];
      if (x < T || (x == T && e++ < kk)) emit(rank++, i);
    }
  }
  __syncthreads();
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

template <typename T>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  __shared__ RouteSmem sm;
  constexpr int E = Slice<T>::E;
  const Shape& S = a.s;
  const int b = blockIdx.x / S.hkv;
  const int h = blockIdx.x % S.hkv;
  const int d = S.d;
  const int64_t s = S.q0 + (int64_t)b * S.B;
  const int64_t ms = s / S.c;
  const int gpc = S.c / S.g;
  const int tid = threadIdx.x;

  // ---- 1. block query (float64)
  {
    const int P = d / E;                   // 16-byte slices per row
    const int phases = kThreads / P;
    const int p = tid % P, ph = tid / P;
    double* part = reinterpret_cast<double*>(sm.key);   // [phases][d]
    const int nrows = S.G * S.B;
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    const T* qbase = static_cast<const T*>(a.q);
    int r = ph;
    for (; r + 3 * phases < nrows; r += 4 * phases) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rr = r + u * phases;
        const int64_t row = (int64_t)(h * S.G + rr / S.B) * S.nq + (s - S.q0) + rr % S.B;
        v[u] = *reinterpret_cast<const uint4*>(qbase + row * d + p * E);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) Slice<T>::add(v[u], acc);
    }
    for (; r < nrows; r += phases) {
      const int64_t row = (int64_t)(h * S.G + r / S.B) * S.nq + (s - S.q0) + r % S.B;
      Slice<T>::add(*reinterpret_cast<const uint4*>(qbase + row * d + p * E), acc);
    }
    if (ph < phases) {
#pragma unroll
      for (int e = 0; e < E; ++e) part[ph * d + p * E + e] = acc[e];
    }
    __syncthreads();
    if (tid < d) {
      double t = 0.0;
      for (int q = 0; q < phases; ++q) t += part[q * d + tid];
      sm.qbar[tid] = t / nrows;
    }
    __syncthreads();
  }

  const int64_t orow = (int64_t)b * S.hkv + h;
  // ---- 2-3. chunk stage
  int64_t lo, hi;
  fixed_windows(ms, S.sink_chunks, S.local_chunks, &lo, &hi);
  const int ncand = (int)(hi - lo);
  const int nsc = ncand < S.kc ? ncand : S.kc;
  if (nsc > 0 && nsc < ncand) {
    const float* csh = a.cs + (int64_t)h * (S.L / S.c) * d;
    score_rows(sm.qbar, d, ncand, [&](int c) { return csh + (lo + c) * d; }, sm.key);
    __syncthreads();
    select_smallest(sm.key, ncand, nsc, sm, [&](int rank, int pos) { sm.chunks[rank] = (int)(lo + pos); });
  } else {
    for (int i = tid; i < nsc; i += kThreads) sm.chunks[i] = (int)(lo + i);
    __syncthreads();
  }
  for (int i = tid; i < S.kc; i += kThreads) a.chunk_idx[orow * S.kc + i] = i < nsc ? sm.chunks[i] : -1;

  // ---- 4. group stage over the groups of the kept chunks (ascending order)
  const int ngc = nsc * gpc;
  const int nsg = ngc < S.kg ? ngc : S.kg;
  int32_t* gout = a.group_idx + orow * S.kg;
  auto group_of = [&](int c) { return (int)((int64_t)sm.chunks[c / gpc] * gpc + c % gpc); };
  if (nsg > 0 && nsg < ngc) {
    const int64_t gsplit = a.split / S.g;          // groups held in host memory
    const int64_t ngl = S.L / S.g;
    score_rows(sm.qbar, d, ngc, [&](int c) -> const float* {
      const int64_t j = group_of(c);
      return j < gsplit ? a.gs_host + ((int64_t)h * gsplit + j) * d
                        : a.gs_dev + ((int64_t)h * (ngl - gsplit) + (j - gsplit)) * d;
    }, sm.key);
    __syncthreads();
    select_smallest(sm.key, ngc, nsg, sm, [&](int rank, int pos) { gout[rank] = group_of(pos); });
  } else {
    for (int i = tid; i < nsg; i += kThreads) gout[i] = group_of(i);
  }
  for (int i = nsg + tid; i < S.kg; i += kThreads) gout[i] = -1;
  if (tid == 0) {
    a.n_sel[orow * 2 + 0] = nsc;
    a.n_sel[orow * 2 + 1] = nsg;
  }
}

}  // namespace

hipError_t launch_route(const Shape& s, const void* q, const float* cs, const float* gs_host,
                        const float* gs_dev, int64_t split, int32_t* chunk_idx, int32_t* group_idx,
                        int32_t* n_sel, hipStream_t st) {
  const int64_t items = s.nb * s.hkv;
  if (items == 0) return hipSuccess;
  RouteArgs a{q, cs, gs_host, gs_dev, split, chunk_idx, group_idx, n_sel, s};
  if (s.dtype == HGA_BF16)
    route_kernel<uint16_t><<<dim3((unsigned)items), dim3(kThreads), 0, st>>>(a);
  else
    route_kernel<float><<<dim3((unsigned)items), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hga
