// Device code shared by the attention kernels (forward and backward) of the
// HGA routed attention ("Long-Context Fine-Tuning with Limited VRAM",
// section 2.1, "Exact-token attention"): the token-set plan of one (query
// block, KV head) item as 64-token tiles, its validation of the kept groups,
// the host-tier source-row encoding, and the LDS staging helpers (direct
// global-to-LDS loads, swizzles, cross-lane reductions) of the bfloat16 MFMA
// kernels. The tile order and the plan are documented in hga_attend.hip.
#pragma once

#include <limits.h>

#include "hga_route_impl.h"

namespace hga {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const void* q;
  KVSrc kv;
  const void* k_cache;     // host-tier path: cached history chunks, [Hkv][nch][64][d] by slot
  const void* v_cache;
  const int32_t* slot;     // [Hkv][nch]: cache slot of history chunk m of head h (-1: not needed)
  int nch;                 // chunks in the host tier (split / 64)
  int nslots;              // cache slots per KV head (the cache is [Hkv][nslots][64][d])
  const uint64_t* pending; // [Hkv][nch]: groups of history chunks copied by a concurrent kernel (null: none)
  int pass;                // with pending: 1 attends the items that read none of them, 2 the others
  int* done;               // [workgroups]: set by pass 1 for each workgroup that attended its item
  const int32_t* gidx;
  const int32_t* nsel;
  void* out;
  float* lse;
  int wg_per_item;
  Shape s;
};

// Source rows of the host-tier path are encoded in one int: with kCacheFlag
// set, a row of the cache ((h nch + slot) 64 + offset); without it, a row of
// the head's device part (token - split). Without a host tier a source row is
// the token itself.
constexpr int kCacheFlag = 1 << 30;

// ------------------------------------------------------------ token-set plan
struct Plan {
  int64_t s;      // first position of the block
  int64_t c0;     // first token of the block's chunk ms (the last tile's first token)
  int off;        // s - c0: the block's first slot in the last tile
  int dlim;       // off + B: slots of the last tile at or after it are empty
  int64_t a, bb;  // fixed chunks are [0, a) and [bb, ms)
  int nfix;       // fixed chunks (tiles)
  int nrouted;    // kept groups after validation (their first tokens in runs[])
  int nrt;        // routed tiles
  int ntiles;
};

// The parts of the plan of block b that need no routing.
__device__ inline void plan_windows(const Shape& S, int b, Plan* P) {
  P->s = S.q0 + (int64_t)b * S.B;
  const int64_t ms = P->s / S.c;
  P->c0 = ms * S.c;
  P->off = (int)(P->s - P->c0);
  P->dlim = P->off + S.B;
  fixed_windows(ms, S.sink_chunks, S.local_chunks, &P->a, &P->bb);
  P->nfix = (int)(P->a + (ms - P->bb));
}

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
__device__ inline Plan make_plan(const Shape& S, int b, int h, const int32_t* gidx, const int32_t* nsel,
                          int* runs, int* lds, int cap) {
  Plan P;
  plan_windows(S, b, &P);
  const int64_t row = (int64_t)b * S.hkv + h;
  // the first entries load together with the count (one memory round trip)
  const int j0 = (int)threadIdx.x < S.kg ? gidx[row * S.kg + threadIdx.x] : -1;
  int n = nsel[row * 2 + 1];
  n = n < 0 ? 0 : (n > S.kg ? S.kg : n);
  int carry_max = INT_MIN, count = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int i = base + threadIdx.x;
    const int j = i < n ? (base == 0 ? j0 : gidx[row * S.kg + i]) : -1;
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
    if (ok && count + pos < cap) runs[count + pos] = j * S.g;
    carry_max = bmax > carry_max ? bmax : carry_max;
    count += tot;
  }
  P.nrouted = count < cap ? count : cap;
  const int per_tile = kChunk / S.g;
  P.nrt = (P.nrouted + per_tile - 1) / per_tile;
  P.ntiles = P.nfix + P.nrt + 1;
  __syncthreads();
  return P;
}

// Source row of slot sl of tile t (see kCacheFlag), or -1 for an empty slot.
// runs hold the kept groups' first rows and fixsrc the fixed chunks' first
// rows (both encoded on the host-tier path, see translate_plan).
__device__ inline int tile_src(const Plan& P, const int* runs, const int* fixsrc, int g, bool tiered, int64_t split,
                               int t, int sl) {
  if (t < P.nfix) {
    if (tiered) return fixsrc[t] + sl;
    return (int)((t < P.a ? t : P.bb + (t - P.a)) * kChunk) + sl;
  }
  if (t < P.nfix + P.nrt) {
    const int r = (t - P.nfix) * (kChunk / g) + sl / g;
    return r < P.nrouted ? runs[r] + sl % g : -1;
  }
  // the last tile: empty slots (past the block) read the chunk's first row
  return (int)(tiered ? P.c0 - split : P.c0) + (sl < P.dlim ? sl : 0);
}

// Number of leading valid slots of tile t (the rest are empty).
__device__ inline int tile_limit(const Plan& P, int g, int t) {
  if (t >= P.nfix && t < P.nfix + P.nrt) {
    const int rem = P.nrouted * g - (t - P.nfix) * kChunk;
    return rem < kChunk ? rem : kChunk;
  }
  return t == P.ntiles - 1 ? P.dlim : kChunk;
}


// Host-tier path: rewrite the kept groups' first tokens in runs[] and the
// fixed chunks' first tokens into encoded source rows (fixsrc[t] for fixed
// tile t), given the cache slots (slot[h nch + m], -1: not cached) of the
// nch history chunks below split, in a cache of nslots chunk slots per KV
// head. Every history chunk used here was given a slot. With pending (the
// groups of each history chunk still being copied, as group bits) in pass 1,
// returns whether the item reads a pending group, so that the workgroup must
// leave it to pass 2, and records in done[workgroup] whether it attends it
// (pass 2 runs the workgroups pass 1 did not). The result is the same in
// every thread.
__device__ inline bool translate_plan(int64_t split, int nch, int nslots, const int32_t* slot, int h, const Plan& P,
                                      int* runs, int* fixsrc, int g = 8, const uint64_t* pending = nullptr,
                                      int pass = 0, int* done = nullptr) {
  // Each token's table entries are read unconditionally at a clamped chunk
  // (history chunk 0 for rows above the split; every table holds nch >= 1
  // entries per head), all of a thread's reads before any is used: with the
  // reads under their conditions the compiler waited for each on its own.
  const uint64_t* ph = pending && pass == 1 ? pending + (int64_t)h * nch : nullptr;
  const int32_t* sh = slot + (int64_t)h * nch;
  auto enc = [&](int64_t tok, int sl) -> int {
    // every chunk used here was marked; an unmarked one would read device
    // row 0 rather than outside the cache
    if (tok < split) return sl >= 0 ? kCacheFlag | (int)(((int64_t)h * nslots + sl) * kChunk + tok % kChunk) : 0;
    return (int)(tok - split);
  };
  int busy = 0;
  for (int base = 0; base < P.nrouted || base < P.nfix; base += blockDim.x) {
    const int i = base + threadIdx.x;
    const bool rt = i < P.nrouted, fx = i < P.nfix;
    const int64_t tok = rt ? runs[i] : 0;
    const int64_t mf = fx ? (i < P.a ? i : P.bb + (i - P.a)) : 0;
    const int64_t mr = tok < split ? tok / kChunk : 0;
    const int64_t mfc = mf < nch ? mf : 0;
    const int sr = sh[mr], sf = sh[mfc];
    const uint64_t pr = ph ? ph[mr] : 0ull, pf = ph ? ph[mfc] : 0ull;
    if (rt) {
      if (tok < split && ((pr >> ((tok % kChunk) / g)) & 1ull)) busy = 1;
      runs[i] = enc(tok, sr);
    }
    if (fx) {
      if (mf < nch && pf) busy = 1;
      fixsrc[i] = enc(mf * kChunk, sf);
    }
  }
  busy = __syncthreads_or(busy);
  if (ph && threadIdx.x == 0) done[blockIdx.x] = busy ? 0 : 1;
  return busy != 0;
}

// K or V row of a source row: the cache, or the head's device rows.
template <typename T>
__device__ inline const T* src_ptr(const T* dev_head, const T* cache, int src, int d) {
  return (src & kCacheFlag) ? cache + (int64_t)(src & ~kCacheFlag) * d : dev_head + (int64_t)src * d;
}

// Item and workgroup slot of this workgroup. Consecutive items of one KV head
// (neighbouring query blocks, which share sink, local and often routed
// chunks) are kept on the same XCD: the dispatcher deals workgroups to the 8
// XCDs round-robin, so block id x runs on XCD x % 8.
__device__ inline int xcd_index(int n) {
  int lid = blockIdx.x;
  if (n % 8 == 0) lid = (blockIdx.x % 8) * (n / 8) + blockIdx.x / 8;
  return lid;
}
__device__ inline void item_of_index(const Shape& S, int wpi, int lid, int* b, int* h, int* z) {
  *z = lid % wpi;
  const int item = lid / wpi;       // head-major: item = h * nb + b
  *h = item / (int)S.nb;
  *b = item % (int)S.nb;
}
__device__ inline void item_of_block(const Shape& S, int wpi, int* b, int* h, int* z) {
  item_of_index(S, wpi, xcd_index((int)(S.nb * S.hkv) * wpi), b, h, z);
}

// ------------------------------------------------------------ bf16 MFMA kernel

// The running max used by the exponentials is raised only when a row's new
// scores exceed it by more than 2^8 (in the log2 domain): probabilities then
// stay below 256, exact in float32 and in bfloat16's range, and the O/l
// rescale runs only when some row of the wave needs it.
constexpr float kRescaleSlack = 8.0f;

// bfloat16 attention workgroup: 8 waves of 32 query rows (256 rows: the G
// heads x 64 positions of one item for G = 4). K/V tiles stream through a ring
// of kAttnStages LDS stages filled by direct global-to-LDS loads, so the
// gathered rows of the next tiles are in flight while a tile is computed.
constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kAttnStages = 2;

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Tiles live in LDS row-major (one token row of D bf16 per row) with the
// 16-byte pieces of each row permuted by XOR:
//   K: piece p of row r at position p ^ (r % NP). The QK^T reads take one
//      piece from 16 consecutive rows at once: all 16 positions differ.
//   V: piece p of row r at position p ^ (4 (r % 4) % NP). The transposing reads
//      take an aligned block of 4 pieces from 4 consecutive rows at once: the
//      4 rows land in 4 different blocks.
// Both keep every LDS read of the tile loop free of bank conflicts.
// A tile read both ways (the backward's K, Q and dO) takes the XOR of the
// two: for D = 128 it maps 16 consecutive rows to 16 different positions and
// any 4 consecutive rows starting at a multiple of 4 to 4 different blocks,
// so both kinds of read stay free of conflicts.
template <int D>
__device__ inline int k_swizzle(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ inline int v_swizzle(int r) { return ((r & 3) << 2) & (D / 8 - 1); }
template <int D>
__device__ inline int kv_swizzle(int r) { return k_swizzle<D>(r) ^ v_swizzle<D>(r); }

// Swizzle by kind: 0 row reads (k_swizzle), 1 transposing reads (v_swizzle),
// 2 both (kv_swizzle).
template <int D, int kKind>
__device__ inline int swizzle(int r) {
  return kKind == 0 ? k_swizzle<D>(r) : kKind == 1 ? v_swizzle<D>(r) : kv_swizzle<D>(r);
}

// Direct global-to-LDS copy of 16 bytes per lane: lane i's 16 bytes at src
// land at LDS byte address lds_base + 16 i (lds_base uniform across the wave).
// The instruction writes no register, so the compiler never waits on it; the
// kernel waits for it itself (s_waitcnt vmcnt) before the barrier that
// publishes a stage.
// M0 is declared clobbered so the compiler sets it again before its own uses;
// clang warns about clobbering a reserved register, which is the intent here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_dma16(const void* src, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory", "m0");
}
// The same with a uniform 64-bit base in SGPRs and a 32-bit byte offset per
// lane (the global address is base + off): one vector instruction less per
// load, and no 64-bit address arithmetic per lane.
// base must be the same in every lane; it is taken from the first active
// lane, so that it is held in scalar registers even where the compiler keeps
// the pointer in vector registers.
__device__ inline void lds_dma16_off(const void* base, uint32_t off, uint32_t lds_base) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  // (the builtin returns int: each half goes through uint32_t, so the low
  // half is not sign-extended into the high one)
  const uint64_t sbase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) << 32) |
                         (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory", "m0");
}
// The same for 4 bytes per lane, with a uniform base and 32-bit lane offsets.
__device__ inline void lds_dma4_off(const void* base, uint32_t off, uint32_t lds_base) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint64_t sbase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) << 32) |
                         (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(off), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory", "m0");
}
// The same for 4 bytes per lane: lane i's word lands at lds_base + 4 i.
__device__ inline void lds_dma4(const void* src, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate that waits for vector memory only: vmcnt(n) with the
// LDS and export counters left at their "don't wait" maxima. vmcnt is split
// over bits 3:0 and 15:14.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
static_assert(vmcnt_imm(5) == (0x0F70 | 5), "waitcnt encoding");

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Max and sum of x over lanes l and l ^ 32, by one swap of the wave's halves:
// the two results of the swap are this lane's value and its partner's.
__device__ inline float pair_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ inline float pair_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Shared memory of the bfloat16 attention: the K and V stage rings (NS
// stages: the loop's two, and a third in the fused route-and-attend kernel
// for a fixed tile that loads during routing), the item's routed run list
// and, after it, the fixed chunks' source rows of the host-tier path.
template <int D, int NS = kAttnStages>
struct AttnSmem {
  uint16_t k[NS][kChunk * D];
  uint16_t v[NS][kChunk * D];
  int runs[kMaxRoutedAttn + kMaxFixedTiered];
  int scan[16];
};

// K/V rows of KV head h: its device rows (rows [split, L) on the host-tier
// path), and the cache of the host-tier path.
struct KVRows {
  const uint16_t *k_dev, *v_dev, *k_cache, *v_cache;
};
template <int D, bool kTiered>
__device__ inline KVRows kv_rows(const AttnArgs& A, int h) {
  const int64_t per_head = kTiered ? A.s.kvs - A.kv.split : A.s.kvs;
  return KVRows{static_cast<const uint16_t*>(A.kv.k_dev) + (int64_t)h * per_head * D,
                static_cast<const uint16_t*>(A.kv.v_dev) + (int64_t)h * per_head * D,
                static_cast<const uint16_t*>(A.k_cache), static_cast<const uint16_t*>(A.v_cache)};
}

// This wave's share of one tile load: rows [RPW w, RPW w + RPW) of the tile,
// each lane one 16-byte piece of K and of V written at its swizzled position
// (swizzle kinds kKS and kVS, see swizzle) in the stage at LDS byte addresses
// k_lds / v_lds. src(i, sl) is the source row (see kCacheFlag) of slot sl, the
// row of this lane in the wave's i-th load.
template <int D, bool kTiered, int kKS = 0, int kVS = 1, typename SrcFn>
__device__ inline void issue_tile(const KVRows& kv, uint32_t k_lds, uint32_t v_lds, SrcFn src) {
  constexpr int NP = D / 8;                   // 16-byte pieces per token row
  constexpr int RPI = 64 / NP;                // rows per direct-to-LDS wave load
  constexpr int RPW = kChunk / kAttnWaves;    // rows each wave loads per tile
  // the wave index is made scalar, so the LDS destinations are scalar
  // arithmetic and each load needs no lane-to-scalar move before setting M0
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < RPW / RPI; ++i) {
    const int row0 = wave * RPW + i * RPI;
    const int rr = row0 + lane / NP;
    const int sr = src(i, rr);
    if (kTiered) {
      lds_dma16(src_ptr(kv.k_dev, kv.k_cache, sr, D) + ((lane % NP) ^ swizzle<D, kKS>(rr)) * 8,
                k_lds + (uint32_t)(row0 * D * 2));
      lds_dma16(src_ptr(kv.v_dev, kv.v_cache, sr, D) + ((lane % NP) ^ swizzle<D, kVS>(rr)) * 8,
                v_lds + (uint32_t)(row0 * D * 2));
    } else {
      // device rows only: byte offsets from the head's rows (a head holds
      // at most 262,144 rows of at most 256 bytes, well below 2^32)
      const uint32_t row = (uint32_t)sr * (uint32_t)(D * 2);
      lds_dma16_off(kv.k_dev, row + ((uint32_t)((lane % NP) ^ swizzle<D, kKS>(rr)) << 4),
                    k_lds + (uint32_t)(row0 * D * 2));
      lds_dma16_off(kv.v_dev, row + ((uint32_t)((lane % NP) ^ swizzle<D, kVS>(rr)) << 4),
                    v_lds + (uint32_t)(row0 * D * 2));
    }
  }
}

}  // namespace
}  // namespace hga
