// Exact-token routed attention for HGA ("Long-Context Fine-Tuning with Limited
// VRAM", section 2.1, "Exact-token attention": only the exact token K/V of the
// kept groups is attended, summaries never are; the sink and local windows and
// the block's own tokens are always attended, with causal masking).
//
// Token set of one (query block b, KV head h) item, as 64-token tiles:
//   [fixed sink/local chunks, one tile each][kept groups, 64/g per tile,
//    the last tile possibly partial][the block's own chunk, causal].
// The order of tiles does not change the result (softmax is a sum over the
// set); each tile is one LDS-staged K/V tile of the flash-style loop.
//
// bfloat16 path (attend_bf16_kernel): one 512-thread workgroup per item and
// 256 query rows (G heads x 64 positions); each of the 8 waves owns 32 rows.
// Per 64-token tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (K from LDS as the A operand, its queries held in registers as B), keeps the
// online-softmax state of its own query column per lane, and accumulates
// O^T += V^T P^T with the same MFMA (V^T from LDS, P^T straight from the
// S^T accumulators after rounding to bfloat16). K/V tiles are gathered by
// group index from HBM, double-buffered through LDS (K row-major, V
// transposed), with the next tile's global loads in flight during the MFMAs.
//
// float32 path (attend_f32_kernel): SIMT, a few lanes per query row, for the
// float32 configurations.
//
// Host-tier path: K/V rows in pinned host memory are first gathered tile by
// tile into a device staging buffer (gather_kernel); the attention kernels
// then read the staged tiles contiguously.
#include <limits.h>

#include "hga_internal.h"

namespace hga {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const void* q;
  KVSrc kv;
  const void* k_stage;     // staged tiles [item][tile][64][d] (host-tier path)
  const void* v_stage;
  const int32_t* gidx;
  const int32_t* nsel;
  void* out;
  float* lse;
  int64_t tiles_per_item;  // staging stride in tiles
  int wg_per_item;
  Shape s;
};

// ------------------------------------------------------------ token-set plan
struct Plan {
  int64_t s;      // first position of the block
  int64_t a, bb;  // fixed chunks are [0, a) and [bb, ms)
  int nfix;       // fixed chunks (tiles)
  int nrouted;    // kept groups after validation (their first tokens in runs[])
  int nrt;        // routed tiles
  int ntiles;
};

// Block-wide exclusive scan (sum or max) of one int per thread.
template <bool kMax>
__device__ int block_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x = kMax ? (y > x ? y : x) : x + y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  const int ident = kMax ? INT_MIN : 0;
  int pre = ident, tot = ident;
  for (int w = 0; w < nw; ++w) {
    const int t = lds[w];
    if (w < wave) pre = kMax ? (t > pre ? t : pre) : pre + t;
    tot = kMax ? (t > tot ? t : tot) : tot + t;
  }
  int ex = __shfl_up(x, 1);
  if (lane == 0) ex = ident;
  __syncthreads();
  *total = tot;
  return kMax ? (ex > pre ? ex : pre) : pre + ex;
}

// Validate and compact the kept groups of item (b, h) into runs[] (first token
// of each group). An entry is usable when it is >= 0, its group ends by the
// block start and it is not inside a fixed chunk; a usable entry is used when
// it is greater than every earlier usable entry of the row, so each token is
// used once and ascending rows are taken whole.
__device__ Plan make_plan(const Shape& S, int b, int h, const int32_t* gidx, const int32_t* nsel,
                          int* runs, int* lds) {
  Plan P;
  P.s = S.q0 + (int64_t)b * S.B;
  const int64_t ms = P.s / S.c;
  fixed_windows(ms, S.sink_chunks, S.local_chunks, &P.a, &P.bb);
  P.nfix = (int)(P.a + (ms - P.bb));
  const int64_t row = (int64_t)b * S.hkv + h;
  int n = nsel[row * 2 + 1];
  n = n < 0 ? 0 : (n > S.kg ? S.kg : n);
  int carry_max = INT_MIN, count = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int i = base + threadIdx.x;
    const int j = i < n ? gidx[row * S.kg + i] : -1;
    bool usable = i < n && j >= 0 && ((int64_t)j + 1) * S.g <= P.s;
    if (usable) {
      const int64_t m = (int64_t)j * S.g / S.c;
      usable = m >= P.a && m < P.bb;
    }
    int bmax;
    int pm = block_scan<true>(usable ? j : INT_MIN, lds, &bmax);
    pm = pm > carry_max ? pm : carry_max;
    const bool ok = usable && j > pm;
    int tot;
    const int pos = block_scan<false>(ok ? 1 : 0, lds, &tot);
    if (ok && count + pos < kMaxRouted) runs[count + pos] = j * S.g;
    carry_max = bmax > carry_max ? bmax : carry_max;
    count += tot;
  }
  P.nrouted = count < kMaxRouted ? count : kMaxRouted;
  const int per_tile = kChunk / S.g;
  P.nrt = (P.nrouted + per_tile - 1) / per_tile;
  P.ntiles = P.nfix + P.nrt + 1;
  __syncthreads();
  return P;
}

// Token position of slot `slot` of tile t, or -1 for an empty slot.
__device__ inline int64_t tile_token(const Plan& P, const int* runs, int g, int t, int slot) {
  if (t < P.nfix) {
    const int64_t m = t < P.a ? t : P.bb + (t - P.a);
    return m * kChunk + slot;
  }
  if (t < P.nfix + P.nrt) {
    const int r = (t - P.nfix) * (kChunk / g) + slot / g;
    return r < P.nrouted ? (int64_t)runs[r] + slot % g : -1;
  }
  return P.s + slot;
}

// Number of leading valid slots of tile t (the rest are empty).
__device__ inline int tile_limit(const Plan& P, int g, int t) {
  if (t >= P.nfix && t < P.nfix + P.nrt) {
    const int rem = P.nrouted * g - (t - P.nfix) * kChunk;
    return rem < kChunk ? rem : kChunk;
  }
  return kChunk;
}

// Address of the d-wide row of token `tok` of KV head h in a tiered tensor.
template <typename T>
__device__ inline const T* kv_row(const void* host, const void* dev, int64_t split, int64_t L, int d,
                                  int h, int64_t tok) {
  if (tok < split) return static_cast<const T*>(host) + ((int64_t)h * split + tok) * d;
  return static_cast<const T*>(dev) + ((int64_t)h * (L - split) + (tok - split)) * d;
}

// Item and workgroup slot of this workgroup. Consecutive items of one KV head
// (neighbouring query blocks, which share sink, local and often routed
// chunks) are kept on the same XCD: the dispatcher deals workgroups to the 8
// XCDs round-robin, so block id x runs on XCD x % 8.
__device__ inline void item_of_block(const Shape& S, int wpi, int* b, int* h, int* z) {
  const int nwg = (int)(S.nb * S.hkv) * wpi;
  int lid = blockIdx.x;
  if (nwg % 8 == 0) lid = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
  *z = lid % wpi;
  const int item = lid / wpi;       // head-major: item = h * nb + b
  *h = item / (int)S.nb;
  *b = item % (int)S.nb;
}

// ------------------------------------------------------------ bf16 MFMA kernel
template <int D, bool kStaged>
__global__ __launch_bounds__(512) void attend_bf16_kernel(AttnArgs A) {
  constexpr int NT = 512;
  constexpr int KROW = D + 8;          // bf16 per LDS row of K (16 B pad: conflict-free 16 B reads)
  constexpr int VROW = kChunk + 4;     // bf16 per LDS row of V^T (8 B pad: conflict-free 8 B reads)
  constexpr int DP = D / 8;            // 16-byte pieces per token row
  constexpr int KPT = kChunk * DP / NT;        // K pieces per thread per tile
  constexpr int VPAIRS = kChunk / 2;           // token pairs per tile
  constexpr int VTHREADS = VPAIRS * DP;        // threads that load V
  static_assert(KPT >= 1 && VTHREADS <= NT, "tile shape");
  __shared__ __align__(16) uint16_t sK[2][kChunk * KROW];
  __shared__ __align__(16) uint16_t sV[2][D * VROW];
  __shared__ int sRuns[kMaxRouted];
  __shared__ int sScan[16];

  const Shape& S = A.s;
  int b, h, z;
  item_of_block(S, A.wg_per_item, &b, &h, &z);
  const Plan P = make_plan(S, b, h, A.gidx, A.nsel, sRuns, sScan);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5;                  // lane half
  const int col = lane & 31;                 // query column of this lane
  const int rb = z * 8 + wave;               // 32-row block of the item
  const bool active = rb < 2 * S.G;
  const int head = h * S.G + (rb >> 1);
  const int qi = (rb & 1) * 32 + col;        // position within the block
  const int64_t qrow = (int64_t)b * S.B + qi;  // row of Q / O
  const int64_t item_lin = (int64_t)h * S.nb + b;

  // queries of this lane's column as MFMA B operands (d = 16 ks + 8 hl + e)
  bf16x8 qf[D / 16];
  if (active) {
    const uint16_t* qp = static_cast<const uint16_t*>(A.q) + ((int64_t)head * S.nq + qrow) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
  }

  // tile loader: K as pieces (token sl, 8 dims), V as token pairs (2 sl, 8 dims)
  u32x4 kreg[KPT], vreg[2];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int p = tid + NT * r, sl = p / DP, dp = p % DP;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (kStaged) {
        x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(A.k_stage) +
                                           ((item_lin * A.tiles_per_item + t) * kChunk + sl) * D + dp * 8);
      } else {
        const int64_t tok = tile_token(P, sRuns, S.g, t, sl);
        if (tok >= 0)
          x = *reinterpret_cast<const u32x4*>(
              kv_row<uint16_t>(A.kv.k_host, A.kv.k_dev, A.kv.split, S.L, D, h, tok) + dp * 8);
      }
      kreg[r] = x;
    }
    if (tid < VTHREADS) {
      const int sp = tid % VPAIRS, dp = tid / VPAIRS;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int sl = 2 * sp + u;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (kStaged) {
          x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(A.v_stage) +
                                             ((item_lin * A.tiles_per_item + t) * kChunk + sl) * D + dp * 8);
        } else {
          const int64_t tok = tile_token(P, sRuns, S.g, t, sl);
          if (tok >= 0)
            x = *reinterpret_cast<const u32x4*>(
                kv_row<uint16_t>(A.kv.v_host, A.kv.v_dev, A.kv.split, S.L, D, h, tok) + dp * 8);
        }
        vreg[u] = x;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int p = tid + NT * r, sl = p / DP, dp = p % DP;
      *reinterpret_cast<u32x4*>(&sK[buf][sl * KROW + dp * 8]) = kreg[r];
    }
    if (tid < VTHREADS) {
      const int sp = tid % VPAIRS, dp = tid / VPAIRS;
      uint32_t* vt = reinterpret_cast<uint32_t*>(&sV[buf][0]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = vreg[0][e >> 1], w1 = vreg[1][e >> 1];
        const uint32_t lo = (e & 1) ? (w0 >> 16) : (w0 & 0xffffu);
        const uint32_t hi = (e & 1) ? (w1 & 0xffff0000u) : (w1 << 16);
        vt[((dp * 8 + e) * VROW + 2 * sp) >> 1] = lo | hi;
      }
    }
  };

  const float sl2 = S.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < P.ntiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < P.ntiles) load_tile(t + 1);
    if (active) {
      // S^T = K Q^T: two 32-token blocks
      f32x16 sacc[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        sacc[tb] = f32x16{};
        const uint16_t* kp = &sK[cur][(32 * tb + col) * KROW + 8 * hl];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kp + 16 * ks));
          sacc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[tb], 0, 0, 0);
        }
      }
      // scale, mask, online softmax (this lane: query column qi, 32 tokens)
      const bool diag = t == P.ntiles - 1;
      const int lim = tile_limit(P, S.g, t);
      float mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int slot = 32 * tb + 8 * (r >> 2) + 4 * hl + (r & 3);
          float zz = sacc[tb][r] * sl2;
          if (slot >= lim || (diag && slot > qi)) zz = -INFINITY;
          sacc[tb][r] = zz;
          mx = fmaxf(mx, zz);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float psum = 0.0f;
      bf16x8 pf[2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(sacc[tb][r] - m_new);
          psum += p;
          pf[tb][r >> 3][r & 7] = (__bf16)p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      // O^T += V^T P^T: token slot of (half hl, element e) in 16-token step mm
      // of block tb is 32 tb + 16 mm + 4 hl + (e & 3) + 8 (e >> 2)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t* vp = &sV[cur][(32 * db + col) * VROW + 4 * hl];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vp + 32 * tb + 16 * mm);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 32 * tb + 16 * mm + 8);
            const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[tb][mm],
                                                             o[db], 0, 0, 0);
          }
      }
    }
    if (t + 1 < P.ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  if (active) {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    uint16_t* op = static_cast<uint16_t*>(A.out) + ((int64_t)head * S.nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4 v4;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) v4[ii] = (__bf16)(o[db][4 * jj + ii] * inv);
        *reinterpret_cast<u32x2*>(op + 32 * db + 8 * jj + 4 * hl) = __builtin_bit_cast(u32x2, v4);
      }
    if (A.lse && hl == 0) A.lse[(int64_t)head * S.nq + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ------------------------------------------------------------ float32 SIMT kernel
// 256 threads; TPR lanes per query row, each owning D / TPR dimensions.
template <int D, bool kStaged>
__global__ __launch_bounds__(256) void attend_f32_kernel(AttnArgs A) {
  constexpr int NT = 256;
  constexpr int TPR = D <= 32 ? 1 : D / 32;   // lanes per row
  constexpr int DPT = D / TPR;                // dims per lane
  constexpr int ROWS = NT / TPR;              // rows per workgroup
  constexpr int HALF = 32;                    // tokens per LDS sub-tile
  __shared__ __align__(16) float sK[HALF * D];
  __shared__ __align__(16) float sV[HALF * D];
  __shared__ int sRuns[kMaxRouted];
  __shared__ int sScan[16];

  const Shape& S = A.s;
  int b, h, z;
  item_of_block(S, A.wg_per_item, &b, &h, &z);
  const Plan P = make_plan(S, b, h, A.gidx, A.nsel, sRuns, sScan);
  const int tid = threadIdx.x;
  const int row = z * ROWS + tid / TPR;       // row of the item: head-local * 64 + qi
  const int part = tid % TPR;
  const bool active = row < S.G * S.B;
  const int head = h * S.G + row / S.B;
  const int qi = row % S.B;
  const int64_t qrow = (int64_t)b * S.B + qi;
  const int64_t item_lin = (int64_t)h * S.nb + b;

  float q[DPT], o[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    q[e] = active ? static_cast<const float*>(A.q)[((int64_t)head * S.nq + qrow) * D + part * DPT + e] : 0.0f;
    o[e] = 0.0f;
  }
  const float sl2 = S.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.0f;

  for (int t = 0; t < P.ntiles; ++t) {
    const bool diag = t == P.ntiles - 1;
    const int lim = tile_limit(P, S.g, t);
    for (int half = 0; half < 2; ++half) {
      __syncthreads();
      for (int i = tid; i < HALF * (D / 4); i += NT) {
        const int sl = i / (D / 4), e4 = i % (D / 4);
        const int slot = half * HALF + sl;
        float4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
        if (kStaged) {
          const int64_t off = ((item_lin * A.tiles_per_item + t) * kChunk + slot) * D + 4 * e4;
          kx = *reinterpret_cast<const float4*>(static_cast<const float*>(A.k_stage) + off);
          vx = *reinterpret_cast<const float4*>(static_cast<const float*>(A.v_stage) + off);
        } else {
          const int64_t tok = tile_token(P, sRuns, S.g, t, slot);
          if (tok >= 0) {
            kx = *reinterpret_cast<const float4*>(kv_row<float>(A.kv.k_host, A.kv.k_dev, A.kv.split, S.L, D, h, tok) + 4 * e4);
            vx = *reinterpret_cast<const float4*>(kv_row<float>(A.kv.v_host, A.kv.v_dev, A.kv.split, S.L, D, h, tok) + 4 * e4);
          }
        }
        *reinterpret_cast<float4*>(&sK[sl * D + 4 * e4]) = kx;
        *reinterpret_cast<float4*>(&sV[sl * D + 4 * e4]) = vx;
      }
      __syncthreads();
      float zz[HALF];
      float mx = -INFINITY;
#pragma unroll 4
      for (int sl = 0; sl < HALF; ++sl) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < DPT; ++e) acc = fmaf(q[e], sK[sl * D + part * DPT + e], acc);
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
        const int slot = half * HALF + sl;
        float v = acc * sl2;
        if (slot >= lim || (diag && slot > qi)) v = -INFINITY;
        zz[sl] = v;
        mx = fmaxf(mx, v);
      }
      const float m_new = fmaxf(m_run, mx);
      if (m_new == -INFINITY) continue;   // nothing visible in this half yet
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < DPT; ++e) o[e] *= alpha;
      for (int sl = 0; sl < HALF; ++sl) {
        const float p = exp2f(zz[sl] - m_new);
        l_run += p;
#pragma unroll
        for (int e = 0; e < DPT; ++e) o[e] = fmaf(p, sV[sl * D + part * DPT + e], o[e]);
      }
      m_run = m_new;
    }
  }
  if (active) {
    const float inv = 1.0f / l_run;
    float* op = static_cast<float*>(A.out) + ((int64_t)head * S.nq + qrow) * D + part * DPT;
#pragma unroll
    for (int e = 0; e < DPT; ++e) op[e] = o[e] * inv;
    if (A.lse && part == 0) A.lse[(int64_t)head * S.nq + qrow] = (m_run + log2f(l_run)) * kLn2;
  }
}

// ------------------------------------------------------------ host-tier gather
// One workgroup per (item, tile): copies the tile's 64 K and V rows (empty
// slots as zeros) from pinned host or device memory into the staging buffer.
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(AttnArgs A) {
  __shared__ int sRuns[kMaxRouted];
  __shared__ int sScan[16];
  const Shape& S = A.s;
  const int64_t item_lin = blockIdx.x;            // h * nb + b
  const int h = (int)(item_lin / S.nb), b = (int)(item_lin % S.nb);
  const Plan P = make_plan(S, b, h, A.gidx, A.nsel, sRuns, sScan);
  const int d = S.d;
  constexpr int EPV = 16 / sizeof(T);             // elements per 16-byte piece
  const int pieces = kChunk * d / EPV;
  for (int t = blockIdx.y; t < P.ntiles; t += gridDim.y) {
    T* kd = static_cast<T*>(const_cast<void*>(A.k_stage)) + (item_lin * A.tiles_per_item + t) * kChunk * d;
    T* vd = static_cast<T*>(const_cast<void*>(A.v_stage)) + (item_lin * A.tiles_per_item + t) * kChunk * d;
    for (int p = threadIdx.x; p < pieces; p += blockDim.x) {
      const int sl = p / (d / EPV), dp = p % (d / EPV);
      const int64_t tok = tile_token(P, sRuns, S.g, t, sl);
      u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (tok >= 0) {
        kx = *reinterpret_cast<const u32x4*>(kv_row<T>(A.kv.k_host, A.kv.k_dev, A.kv.split, S.L, d, h, tok) + dp * EPV);
        vx = *reinterpret_cast<const u32x4*>(kv_row<T>(A.kv.v_host, A.kv.v_dev, A.kv.split, S.L, d, h, tok) + dp * EPV);
      }
      *reinterpret_cast<u32x4*>(kd + (int64_t)sl * d + dp * EPV) = kx;
      *reinterpret_cast<u32x4*>(vd + (int64_t)sl * d + dp * EPV) = vx;
    }
  }
}

template <int D, bool kStaged>
hipError_t launch_bf16(const AttnArgs& a, int64_t items, hipStream_t st) {
  attend_bf16_kernel<D, kStaged><<<dim3((unsigned)(items * a.wg_per_item)), dim3(512), 0, st>>>(a);
  return hipGetLastError();
}

template <int D, bool kStaged>
hipError_t launch_f32(const AttnArgs& a, int64_t items, hipStream_t st) {
  attend_f32_kernel<D, kStaged><<<dim3((unsigned)(items * a.wg_per_item)), dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

template <bool kStaged>
hipError_t dispatch_f32(const AttnArgs& a, int64_t items, hipStream_t st) {
  switch (a.s.d) {
    case 4: return launch_f32<4, kStaged>(a, items, st);
    case 8: return launch_f32<8, kStaged>(a, items, st);
    case 16: return launch_f32<16, kStaged>(a, items, st);
    case 32: return launch_f32<32, kStaged>(a, items, st);
    case 64: return launch_f32<64, kStaged>(a, items, st);
    case 128: return launch_f32<128, kStaged>(a, items, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t staging_bytes(const Shape& s) {
  const size_t esz = s.dtype == HGA_BF16 ? 2 : 4;
  return 2 * (size_t)(s.nb * s.hkv) * (size_t)max_tiles(s) * kChunk * (size_t)s.d * esz;
}

hipError_t launch_attend(const Shape& s, const void* q, const KVSrc& kv, const int32_t* group_idx,
                         const int32_t* n_sel, void* out, float* lse, void* staging, hipStream_t st) {
  const int64_t items = s.nb * s.hkv;
  if (items == 0) return hipSuccess;
  AttnArgs a{};
  a.q = q; a.kv = kv; a.gidx = group_idx; a.nsel = n_sel; a.out = out; a.lse = lse; a.s = s;
  a.tiles_per_item = max_tiles(s);
  const bool staged = kv.split > 0;
  if (staged) {
    const size_t esz = s.dtype == HGA_BF16 ? 2 : 4;
    a.k_stage = staging;
    a.v_stage = static_cast<char*>(staging) + (size_t)items * a.tiles_per_item * kChunk * s.d * esz;
    const int64_t ty = a.tiles_per_item < 64 ? a.tiles_per_item : 64;
    if (s.dtype == HGA_BF16)
      gather_kernel<uint16_t><<<dim3((unsigned)items, (unsigned)ty), dim3(256), 0, st>>>(a);
    else
      gather_kernel<float><<<dim3((unsigned)items, (unsigned)ty), dim3(256), 0, st>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (s.dtype == HGA_BF16) {
    a.wg_per_item = (2 * s.G + 7) / 8;
    if (s.d == 128) return staged ? launch_bf16<128, true>(a, items, st) : launch_bf16<128, false>(a, items, st);
    if (s.d == 64) return staged ? launch_bf16<64, true>(a, items, st) : launch_bf16<64, false>(a, items, st);
    return hipErrorInvalidValue;
  }
  const int tpr = s.d <= 32 ? 1 : s.d / 32;
  const int rows = 256 / tpr;
  a.wg_per_item = (s.G * s.B + rows - 1) / rows;
  return staged ? dispatch_f32<true>(a, items, st) : dispatch_f32<false>(a, items, st);
}

}  // namespace hga
