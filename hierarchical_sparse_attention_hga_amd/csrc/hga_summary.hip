// Key summaries for HGA routing ("Long-Context Fine-Tuning with Limited VRAM",
// section 2.1: two levels of key summaries built from the model's projected
// keys; base HGA abstract: compact RoPE-aware chunk summaries).
//
// The operator is the mean of the post-RoPE keys. Each thread owns four
// dimensions of one chunk of one KV head: it streams the chunk's 64 key rows
// once, accumulates every group and the whole chunk in float64 (exact for
// bfloat16 keys) and rounds each mean once to float32. One pass over K, one
// write of each summary: the kernel is HBM-bound.
#include "hga_internal.h"

namespace hga {
namespace {

template <typename T>
struct Quad;  // four consecutive key elements, widened to double

template <>
struct Quad<float> {
  __device__ static void load(const float* p, double* x) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
};

template <>
struct Quad<uint16_t> {
  __device__ static void load(const uint16_t* p, double* x) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(v.x << 16);
    x[1] = __uint_as_float(v.x & 0xffff0000u);
    x[2] = __uint_as_float(v.y << 16);
    x[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};

template <typename T>
__global__ __launch_bounds__(256) void summary_kernel(const T* __restrict__ k, float* __restrict__ gs,
                                                      float* __restrict__ cs, int hkv, int64_t L, int d,
                                                      int g) {
  const int quads = d / 4;
  const int64_t nchunk = L / kChunk;
  const int64_t total = (int64_t)hkv * nchunk * quads;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int e = (int)(idx % quads) * 4;
  const int64_t rest = idx / quads;
  const int64_t m = rest % nchunk;
  const int64_t h = rest / nchunk;
  const int gpc = kChunk / g;
  const T* src = k + (h * L + m * kChunk) * d + e;
  float* gdst = gs + (h * (L / g) + m * gpc) * d + e;
  double csum[4] = {0.0, 0.0, 0.0, 0.0};
  for (int u = 0; u < gpc; ++u) {
    double gsum[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int t = 0; t < g; ++t) {
      double x[4];
      Quad<T>::load(src + (int64_t)(u * g + t) * d, x);
      gsum[0] += x[0]; gsum[1] += x[1]; gsum[2] += x[2]; gsum[3] += x[3];
    }
    float4 o;
    o.x = (float)(gsum[0] / g); o.y = (float)(gsum[1] / g);
    o.z = (float)(gsum[2] / g); o.w = (float)(gsum[3] / g);
    *reinterpret_cast<float4*>(gdst + (int64_t)u * d) = o;
    csum[0] += gsum[0]; csum[1] += gsum[1]; csum[2] += gsum[2]; csum[3] += gsum[3];
  }
  float4 o;
  o.x = (float)(csum[0] / kChunk); o.y = (float)(csum[1] / kChunk);
  o.z = (float)(csum[2] / kChunk); o.w = (float)(csum[3] / kChunk);
  *reinterpret_cast<float4*>(cs + (h * nchunk + m) * d + e) = o;
}

}  // namespace

hipError_t launch_summaries(const Shape& s, const void* k, float* gs, float* cs, hipStream_t st) {
  const int64_t total = (int64_t)s.hkv * (s.L / kChunk) * (s.d / 4);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (s.dtype == HGA_BF16)
    summary_kernel<uint16_t><<<dim3((unsigned)blocks), dim3(threads), 0, st>>>(
        static_cast<const uint16_t*>(k), gs, cs, s.hkv, s.L, s.d, s.g);
  else
    summary_kernel<float><<<dim3((unsigned)blocks), dim3(threads), 0, st>>>(
        static_cast<const float*>(k), gs, cs, s.hkv, s.L, s.d, s.g);
  return hipGetLastError();
}

}  // namespace hga
