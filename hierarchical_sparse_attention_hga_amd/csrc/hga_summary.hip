// Key summaries for HGA routing ("Long-Context Fine-Tuning with Limited VRAM",
// section 2.1: two levels of key summaries built from the model's projected
// keys; base HGA abstract: compact RoPE-aware chunk summaries).
//
// The operator is the mean of the post-RoPE keys. One workgroup owns one
// chunk of one KV head; each thread sums one group's keys over one 16-byte
// slice of the head dimension (g independent 16-byte loads), in float64 (exact
// for bfloat16 keys), and writes that group's mean rounded once to float32.
// The chunk mean is the float64 sum of its group sums, reduced through LDS in
// a fixed order, rounded once. One pass over K: the kernel is HBM-bound.
#include "hga_internal.h"

namespace hga {
namespace {

template <typename T>
struct Slice;  // one 16-byte slice of a key row, widened to double

template <>
struct Slice<float> {
  static constexpr int E = 4;
  __device__ static uint4 load(const float* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void add(uint4 v, double* acc) {
    acc[0] += __uint_as_float(v.x); acc[1] += __uint_as_float(v.y);
    acc[2] += __uint_as_float(v.z); acc[3] += __uint_as_float(v.w);
  }
};

template <>
struct Slice<uint16_t> {
  static constexpr int E = 8;
  __device__ static uint4 load(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void add(uint4 v, double* acc) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// Rows per head of k, gs and cs: kvs, kvs / g, kvs / 64; block x covers chunk c0 + x.
template <typename T>
__global__ __launch_bounds__(1024) void summary_kernel(const T* __restrict__ k, float* __restrict__ gs,
                                                       float* __restrict__ cs, int64_t kvs, int64_t c0, int d,
                                                       int g) {
  constexpr int E = Slice<T>::E;
  extern __shared__ double part[];   // [groups per chunk][d] group sums
  const int P = d / E;               // slices per row
  const int gpc = kChunk / g;
  const int64_t m = c0 + blockIdx.x, h = blockIdx.y;
  const int64_t nchunk = kvs / kChunk;
  for (int w = threadIdx.x; w < gpc * P; w += blockDim.x) {
    const int p = w % P, u = w / P;
    const T* src = k + (h * kvs + m * kChunk + (int64_t)u * g) * d + p * E;
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    if (g % 8 == 0) {
      // eight rows' loads issued together, then added in row order
      for (int t0 = 0; t0 < g; t0 += 8) {
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = Slice<T>::load(src + (int64_t)(t0 + j) * d);
#pragma unroll
        for (int j = 0; j < 8; ++j) Slice<T>::add(v[j], acc);
      }
    } else {
      for (int t = 0; t < g; ++t) Slice<T>::add(Slice<T>::load(src + (int64_t)t * d), acc);
    }
    float* dst = gs + (h * (kvs / g) + m * gpc + u) * d + p * E;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      float4 o;
      o.x = (float)(acc[e] / g); o.y = (float)(acc[e + 1] / g);
      o.z = (float)(acc[e + 2] / g); o.w = (float)(acc[e + 3] / g);
      *reinterpret_cast<float4*>(dst + e) = o;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) part[u * d + p * E + e] = acc[e];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < d; e += blockDim.x) {
    double s = 0.0;
    for (int u = 0; u < gpc; ++u) s += part[u * d + e];
    cs[(h * nchunk + m) * d + e] = (float)(s / kChunk);
  }
}

}  // namespace

hipError_t launch_summaries(const Shape& s, const void* k, float* gs, float* cs, int64_t c0, int64_t c1,
                            hipStream_t st) {
  const int64_t nchunk = c1 - c0;
  if (nchunk <= 0) return hipSuccess;
  const int gpc = kChunk / s.g;
  const size_t lds = (size_t)gpc * s.d * sizeof(double);
  const dim3 grid((unsigned)nchunk, (unsigned)s.hkv);
  if (s.dtype == HGA_BF16) {
    const int threads = gpc * (s.d / 8) < 1024 ? gpc * (s.d / 8) : 1024;
    summary_kernel<uint16_t><<<grid, dim3(threads), lds, st>>>(static_cast<const uint16_t*>(k), gs, cs, s.kvs,
                                                              c0, s.d, s.g);
  } else {
    const int threads = gpc * (s.d / 4) < 1024 ? gpc * (s.d / 4) : 1024;
    summary_kernel<float><<<grid, dim3(threads), lds, st>>>(static_cast<const float*>(k), gs, cs, s.kvs, c0,
                                                           s.d, s.g);
  }
  return hipGetLastError();
}

}  // namespace hga
