// Internal declarations of the gfx950 HGA routed-attention library.
// Kernel sources and the C-ABI layer include this; nothing outside csrc/ does.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hga.h"

namespace hga {

// Chunk size the kernels are built for (the pages' 64-token chunks). A query
// block is one chunk or a divisor of it (down to one token when decoding).
constexpr int kChunk = 64;
// Largest number of routing candidates of one stage for one (block, KV head).
constexpr int kMaxCand = 4096;
// Largest number of routed groups per (block, KV head) the library accepts.
constexpr int kMaxRouted = 4096;
// Routed groups the bfloat16 attention workgroup keeps in LDS (bounds
// top_groups for bfloat16).
constexpr int kMaxRoutedAttn = 2048;
// Most chunks the router may keep per item (LDS list of the group stage).
constexpr int kMaxKeptChunks = 2048;
// Most fixed (sink + local) chunks per item when the history is in host
// memory (LDS table of their cached source rows).
constexpr int kMaxFixedTiered = 256;

// Validated problem shape shared by the launchers.
struct Shape {
  int hq, hkv, G, d;
  int c, g, B;          // chunk, group, query block
  int kc, kg;           // top chunks, top groups
  int sink_chunks, local_chunks;
  int dtype;            // element type of Q, K and V (HGA_F32 or HGA_BF16)
  bool out_f32;         // O in float32 whatever dtype is (HGA_BF16_F32OUT)
  float scale;          // softmax scale (resolved)
  int64_t L, q0, nq, nb;
  int64_t qs;           // rows per head of Q, O and LSE (n_q; more when they cover a longer sequence)
  int64_t kvs;          // rows per head of K and V, and of the summaries in tokens (L; more when
                        // the tensors hold a longer sequence than the one attended)
};

// Fixed sink/local windows of a block whose first token is in chunk ms: the
// fixed chunks are [0, a) and [bb, ms) with a <= bb <= ms; the chunk-stage
// candidates are [a, bb).
__host__ __device__ inline void fixed_windows(int64_t ms, int sink_chunks, int local_chunks,
                                              int64_t* a, int64_t* bb) {
  int64_t aa = sink_chunks < ms ? sink_chunks : ms;
  int64_t lo = ms - local_chunks;
  *a = aa;
  *bb = lo > aa ? lo : aa;
}

// Summaries of chunks [c0, c1) of every KV head.
hipError_t launch_summaries(const Shape& s, const void* k, float* gs, float* cs, int64_t c0, int64_t c1,
                            hipStream_t st);

hipError_t launch_route(const Shape& s, const void* q, const float* cs, const float* gs_host,
                        const float* gs_dev, int64_t split, int32_t* chunk_idx, int32_t* group_idx,
                        int32_t* n_sel, hipStream_t st);

// K/V sources of the attention: device rows [split, L) and host rows [0, split).
struct KVSrc {
  const void* k_host;
  const void* k_dev;
  const void* v_host;
  const void* v_dev;
  int64_t split;
};

// Workspace bytes of the host-tier path for a history of `split` tokens in
// host memory: chunk flags and slots, and an HBM cache able to hold every
// history chunk of K and V.
size_t tier_cache_bytes(const Shape& s, int64_t split);

// Host-tier cache of one call: the cache slot of each history chunk of each
// KV head (-1: not needed) and the HBM copies of the needed chunks' K and V,
// in the workspace (tier_cache_bytes). The copy runs on st.
struct TierCache {
  const int32_t* slot;   // [Hkv][nch]: slot of history chunk m (-1: none)
  int nch;
  int nslots;            // slots per KV head of k_cache / v_cache ([Hkv][nslots][64][d])
  const void* k_cache;
  const void* v_cache;
  // [Hkv][nch]: groups of each needed history chunk that this call copies
  // (null: none). pass 1 attends only the items that need none of them,
  // pass 2 only the others, pass 0 every item.
  const uint64_t* pending;
  int pass;
  int* done;             // [workgroups of the attention launch]: written by pass 1, read by pass 2
};
hipError_t prepare_tier_cache(const Shape& s, const KVSrc& kv, const int32_t* group_idx, const int32_t* n_sel,
                              void* workspace, TierCache* tc, hipStream_t st);

// With `cached` (K/V split > 0) the history rows are read from that cache,
// whose slots the caller has filled, instead of a per-call cache built in the
// workspace.
hipError_t launch_attend(const Shape& s, const void* q, const KVSrc& kv, const int32_t* group_idx,
                         const int32_t* n_sel, void* out, float* lse, void* workspace, size_t ws_bytes,
                         hipStream_t st, const TierCache* cached = nullptr);
// Ranges per item when launch_attend spreads each item's tiles over several
// workgroups (1: one workgroup per item), and the workspace that takes.
int attend_split_count(const Shape& s);
size_t attend_split_bytes(const Shape& s);

// Routing and attention in one kernel (bfloat16, K/V all on the device).
bool fused_route_attend_supported(const Shape& s, int64_t kv_split);
hipError_t launch_route_attend(const Shape& s, const void* q, const float* cs, const float* gs_host,
                               const float* gs_dev, int64_t gs_split, const KVSrc& kv, int32_t* chunk_idx,
                               int32_t* group_idx, int32_t* n_sel, void* out, float* lse, hipStream_t st);

// ---------------------------------------------------------------- persistent host-tier cache
// Counters at the start of the cache memory (int64 each).
enum {
  kTcCalls = 0,         // calls made through the cache (each call's stamp)
  kTcKvRequests,        // history groups the calls' query blocks attended (summed over blocks and KV heads)
  kTcKvMisses,          // of those, groups copied from host memory (not resident at the call)
  kTcKvBytes,           // K and V bytes copied from host memory
  kTcKvEvictions,       // chunks whose K/V slots were given to other chunks
  kTcGsRequests,        // kept history chunks whose group summaries the group stage scored
  kTcGsMisses,          // of those, chunks whose summaries were copied from host memory
  kTcGsBytes,           // group-summary bytes copied
  kTcGsEvictions,       // chunks whose summary slots were given to other chunks
  kTierCounters = 16
};

// Byte offsets of the parts of a cache (see hga_tier_cache.hip).
struct TierCacheLayout {
  int nch, S, Sg;
  size_t slot, owner, used, valid, hand;        // K/V slot tables
  size_t gslot, gowner, gused, gvalid, ghand;   // group-summary slot tables
  size_t need, gneed;                           // [Hkv][nch] marks of the running call (zero between calls)
  size_t k, v, gs;                              // [Hkv][S][64][d], [Hkv][S][64][d], [Hkv][Sg][c/g][d]
  size_t total;
};
// Byte offsets of one call's workspace of the cached path.
struct TierCallLayout {
  size_t pend, list, count, glist, gcount, qbar, done, total;
};
// A chunk whose groups (mask) are copied into a slot.
struct CopyEntry {
  int32_t m, slot;
  uint64_t mask;
};
size_t tier_cache_layout(const Shape& s, int64_t split, int kv_slots, int gs_slots, TierCacheLayout* L);
size_t tier_call_layout(const Shape& s, int64_t split, TierCallLayout* W);
hipError_t tier_cache_init(const Shape& s, int64_t split, int kv_slots, int gs_slots, void* mem, hipStream_t st);
hipError_t launch_route_attend_cached(const Shape& s, const void* q, const float* cs, const float* gs_host,
                                      const float* gs_dev, int64_t gs_split, const KVSrc& kv, int kv_slots,
                                      int gs_slots, void* cache_mem, int32_t* chunk_idx, int32_t* group_idx,
                                      int32_t* n_sel, void* out, float* lse, void* workspace, hipStream_t st,
                                      hipStream_t copy_st);

// Backward of the attention (bfloat16): workspace bytes (without the
// host-tier cache, which follows them when kv.split > 0), and the launch of
// its kernels.
size_t backward_workspace_bytes(const Shape& s);
hipError_t launch_attend_backward(const Shape& s, const void* q, const KVSrc& kv, const int32_t* group_idx,
                                  const int32_t* n_sel, const void* out, const float* lse, const void* dout,
                                  void* dq, void* dk, void* dv, void* workspace, hipStream_t st);

}  // namespace hga
