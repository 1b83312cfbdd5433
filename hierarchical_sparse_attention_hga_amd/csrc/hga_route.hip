// Two-level HGA router ("Long-Context Fine-Tuning with Limited VRAM",
// section 2.1, "Chunk selection" and "Group selection").
//
// One workgroup of 256 threads routes one (query block, KV head) item:
//   1. block query: mean of the block's queries over its 64 positions and the
//      G query heads of the KV head, accumulated in float64 (exact for
//      bfloat16 inputs, so independent of the summation order);
//   2. chunk stage: the candidates are the closed chunks before the block
//      that are neither sink nor local (a contiguous range); each score is the
//      float64 dot of the block query with the float32 chunk summary, eight
//      lanes per candidate;
//   3. exact top-k: 64-bit order keys (score descending) with the index as a
//      tie-breaker (lower index first) are sorted by a bitonic network in LDS;
//   4. group stage: the groups of the kept chunks are scored the same way
//      against the group summaries (read from device or pinned host memory)
//      and the top-k is taken again; when the budget covers every group of the
//      kept chunks, all of them are kept without reading their summaries.
// Outputs are ascending and -1 padded.
#include <limits.h>

#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerCand = 8;

template <typename T>
struct Row4;

template <>
struct Row4<float> {
  __device__ static void load(const float* p, double* x) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
};

template <>
struct Row4<uint16_t> {
  __device__ static void load(const uint16_t* p, double* x) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(v.x << 16);
    x[1] = __uint_as_float(v.x & 0xffff0000u);
    x[2] = __uint_as_float(v.y << 16);
    x[3] = __uint_as_float(v.y & 0xffff0000u);
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
  unsigned long long key[kMaxCand];
  int idx[kMaxCand];
  int chunks[kMaxKeptChunks];
  double qbar[128];
};

__device__ inline bool before(unsigned long long ka, int ia, unsigned long long kb, int ib) {
  return ka < kb || (ka == kb && ia < ib);
}

// Sort key[0..n) (with idx as tie-breaker) ascending; entries [n, npad) are
// padded with the largest key.
__device__ void bitonic_sort_pairs(unsigned long long* key, int* idx, int n) {
  int npad = 1;
  while (npad < n) npad <<= 1;
  for (int i = n + threadIdx.x; i < npad; i += blockDim.x) {
    key[i] = ~0ull;
    idx[i] = INT_MAX;
  }
  __syncthreads();
  for (int k = 2; k <= npad; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < npad; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool up = (i & k) == 0;
          const bool swap = up ? before(key[ixj], idx[ixj], key[i], idx[i])
                               : before(key[i], idx[i], key[ixj], idx[ixj]);
          if (swap) {
            const unsigned long long tk = key[i]; key[i] = key[ixj]; key[ixj] = tk;
            const int ti = idx[i]; idx[i] = idx[ixj]; idx[ixj] = ti;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Sort idx[0..n) ascending (entries [n, npad) are overwritten with padding).
__device__ void bitonic_sort_int(int* idx, int n) {
  int npad = 1;
  while (npad < n) npad <<= 1;
  for (int i = n + threadIdx.x; i < npad; i += blockDim.x) idx[i] = INT_MAX;
  __syncthreads();
  for (int k = 2; k <= npad; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < npad; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool up = (i & k) == 0;
          if ((idx[i] > idx[ixj]) == up) {
            const int t = idx[i]; idx[i] = idx[ixj]; idx[ixj] = t;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Score summary rows against qbar: candidate c (0 <= c < n) reads the d floats
// at row(c). Eight lanes per candidate, float64 partial dots reduced by
// butterfly shuffles. Writes key/idx for each candidate.
template <typename RowFn, typename IdxFn>
__device__ void score_rows(const double* qbar, int d, int n, RowFn row, IdxFn index,
                           unsigned long long* key, int* idx) {
  const int lane = threadIdx.x & 63;
  const int sub = lane / kLanesPerCand;        // candidate slot within the wave
  const int lic = lane % kLanesPerCand;        // lane within the candidate
  const int wave = threadIdx.x >> 6;
  const int per_round = (kThreads / 64) * (64 / kLanesPerCand);
  const int quads = d / 4;
  for (int base = 0; base < n; base += per_round) {
    const int c = base + wave * (64 / kLanesPerCand) + sub;
    double acc = 0.0;
    if (c < n) {
      const float* r = row(c);
      for (int q4 = lic; q4 < quads; q4 += kLanesPerCand) {
        const float4 v = *reinterpret_cast<const float4*>(r + 4 * q4);
        acc += qbar[4 * q4 + 0] * (double)v.x;
        acc += qbar[4 * q4 + 1] * (double)v.y;
        acc += qbar[4 * q4 + 2] * (double)v.z;
        acc += qbar[4 * q4 + 3] * (double)v.w;
      }
    }
#pragma unroll
    for (int off = kLanesPerCand / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kLanesPerCand);
    if (c < n && lic == 0) {
      key[c] = order_key(acc);
      idx[c] = index(c);
    }
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

template <typename T>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  __shared__ RouteSmem sm;
  const Shape& S = a.s;
  const int b = blockIdx.x / S.hkv;
  const int h = blockIdx.x % S.hkv;
  const int d = S.d;
  const int64_t s = S.q0 + (int64_t)b * S.B;
  const int64_t ms = s / S.c;
  const int gpc = S.c / S.g;

  // ---- 1. block query (float64), partial sums staged through the key array
  {
    const int quads = d / 4;
    const int phases = kThreads / quads;
    const int q4 = threadIdx.x % quads;
    const int ph = threadIdx.x / quads;
    double* part = reinterpret_cast<double*>(sm.key);   // [phases][d]
    const int nrows = S.G * S.B;
    if (ph < phases) {
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      const T* qbase = static_cast<const T*>(a.q);
      for (int r = ph; r < nrows; r += phases) {
        const int head = h * S.G + r / S.B;
        const int64_t row = (s - S.q0) + r % S.B;
        double x[4];
        Row4<T>::load(qbase + ((int64_t)head * S.nq + row) * d + 4 * q4, x);
        acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
      }
      for (int e = 0; e < 4; ++e) part[ph * d + 4 * q4 + e] = acc[e];
    }
    __syncthreads();
    if (threadIdx.x < d) {
      double t = 0.0;
      for (int p = 0; p < phases; ++p) t += part[p * d + threadIdx.x];
      sm.qbar[threadIdx.x] = t / nrows;
    }
    __syncthreads();
  }

  // ---- 2-3. chunk stage
  int64_t lo, hi;
  fixed_windows(ms, S.sink_chunks, S.local_chunks, &lo, &hi);
  const int ncand = (int)(hi - lo);
  const int nsc = ncand < S.kc ? ncand : S.kc;
  const float* csh = a.cs + (int64_t)h * (S.L / S.c) * d;
  if (nsc > 0) {
    if (nsc < ncand) {
      score_rows(sm.qbar, d, ncand, [&](int c) { return csh + (lo + c) * d; },
                 [&](int c) { return (int)(lo + c); }, sm.key, sm.idx);
      __syncthreads();
      bitonic_sort_pairs(sm.key, sm.idx, ncand);
      bitonic_sort_int(sm.idx, nsc);
    } else {
      for (int i = threadIdx.x; i < nsc; i += kThreads) sm.idx[i] = (int)(lo + i);
      __syncthreads();
    }
  }
  const int64_t orow = (int64_t)b * S.hkv + h;
  for (int i = threadIdx.x; i < S.kc; i += kThreads)
    a.chunk_idx[orow * S.kc + i] = i < nsc ? sm.idx[i] : -1;
  __syncthreads();

  // ---- 4. group stage over the groups of the kept chunks (ascending order)
  const int ngc = nsc * gpc;
  const int nsg = ngc < S.kg ? ngc : S.kg;
  int* chunks = sm.chunks;   // kept chunks, ascending
  for (int i = threadIdx.x; i < nsc; i += kThreads) chunks[i] = sm.idx[i];
  __syncthreads();
  if (nsg > 0 && nsg < ngc) {
    const int64_t gsplit = a.split / S.g;          // groups held in host memory
    const int64_t ngl = S.L / S.g;
    auto grow = [&](int c) -> const float* {
      const int64_t j = (int64_t)chunks[c / gpc] * gpc + c % gpc;
      return j < gsplit ? a.gs_host + ((int64_t)h * gsplit + j) * d
                        : a.gs_dev + ((int64_t)h * (ngl - gsplit) + (j - gsplit)) * d;
    };
    score_rows(sm.qbar, d, ngc, grow,
               [&](int c) { return (int)((int64_t)chunks[c / gpc] * gpc + c % gpc); }, sm.key, sm.idx);
    __syncthreads();
    bitonic_sort_pairs(sm.key, sm.idx, ngc);
    bitonic_sort_int(sm.idx, nsg);
  } else {
    for (int i = threadIdx.x; i < nsg; i += kThreads)
      sm.idx[i] = (int)((int64_t)chunks[i / gpc] * gpc + i % gpc);
    __syncthreads();
  }
  for (int i = threadIdx.x; i < S.kg; i += kThreads)
    a.group_idx[orow * S.kg + i] = i < nsg ? sm.idx[i] : -1;
  if (threadIdx.x == 0) {
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
