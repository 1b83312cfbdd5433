// Persistent HBM cache of the host tier ("Long-Context Fine-Tuning with
// Limited VRAM", section 2.1, "Group selection": group summaries are kept in
// a larger VRAM cache and missing ones are fetched from host memory; section
// 2.1, "Exact-token attention": only the exact token K/V of the kept groups
// is loaded into the routed working set; section 4.5, table 8: the cache hit
// rate).
//
// The caller owns the cache memory (hga_tier_cache); the library keeps no
// state of its own. The cache holds, per KV head, chunk slots of two kinds:
//   K/V slots   the K and V rows of one 64-token history chunk; a slot holds
//               any subset of the chunk's groups (a 64-bit mask per slot),
//               so only the groups a call needs are ever copied;
//   GS slots    the group summaries of one history chunk (all its groups),
//               read by the group stage.
// Each kind has a table: the slot of every history chunk (-1: absent), the
// chunk of every slot (-1: empty), the call that last used each slot, a ring
// position, and one word per history chunk in which the router marks what
// the call's query blocks need (group bits for K/V, one bit for summaries).
// One workgroup per KV head then reads and clears the marks, stamps the
// resident chunks, gives the absent ones the next slots in ring order that
// this call does not use (evicting their chunks), and lists what to copy;
// copy kernels move those rows from pinned host memory into the slots. Every
// chunk a call needs is resident before its attention reads it, so results
// do not depend on what the cache held. Counters of requests, misses, bytes
// and evictions accumulate in the cache's first bytes.
//
// With a second stream the K/V copies run there while the attention of the
// query blocks whose history groups were all resident runs on the call's
// stream; the other blocks are attended once the copies are done.
#include "hga_attend_impl.h"

namespace hga {

size_t tier_cache_layout(const Shape& s, int64_t split, int kv_slots, int gs_slots, TierCacheLayout* L) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nch = (size_t)(split / kChunk), hkv = (size_t)s.hkv, S = (size_t)kv_slots, Sg = (size_t)gs_slots;
  const size_t esz = s.dtype == HGA_BF16 ? 2 : 4;
  const size_t gpc = (size_t)(kChunk / s.g);
  size_t o = up(kTierCounters * sizeof(long long));
  L->nch = (int)nch;
  L->S = kv_slots;
  L->Sg = gs_slots;
  L->slot = o;   o = up(o + hkv * nch * 4);
  L->owner = o;  o = up(o + hkv * S * 4);
  L->used = o;   o = up(o + hkv * S * 4);
  L->valid = o;  o = up(o + hkv * S * 8);
  L->hand = o;   o = up(o + hkv * 4);
  L->gslot = o;  o = up(o + hkv * nch * 4);
  L->gowner = o; o = up(o + hkv * Sg * 4);
  L->gused = o;  o = up(o + hkv * Sg * 4);
  L->gvalid = o; o = up(o + hkv * Sg * 8);
  L->ghand = o;  o = up(o + hkv * 4);
  L->need = o;   o = up(o + hkv * nch * 8);
  L->gneed = o;  o = up(o + hkv * nch * 8);
  L->k = o;      o = up(o + hkv * S * kChunk * (size_t)s.d * esz);
  L->v = o;      o = up(o + hkv * S * kChunk * (size_t)s.d * esz);
  L->gs = o;     o = up(o + hkv * Sg * gpc * (size_t)s.d * 4);
  L->total = o;
  return o;
}

size_t tier_call_layout(const Shape& s, int64_t split, TierCallLayout* W) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nch = (size_t)(split / kChunk), hkv = (size_t)s.hkv;
  size_t o = 0;
  W->pend = o;   o = up(o + hkv * nch * 8);
  W->list = o;   o = up(o + hkv * nch * sizeof(CopyEntry));
  W->count = o;  o = up(o + hkv * 4);
  W->glist = o;  o = up(o + hkv * nch * sizeof(CopyEntry));
  W->gcount = o; o = up(o + hkv * 4);
  W->qbar = o;   o = up(o + (size_t)s.nb * hkv * (size_t)s.d * 8);
  // one flag per attention workgroup (at least 32 query rows each)
  W->done = o;   o = up(o + (size_t)s.nb * hkv * (size_t)((s.G * s.B + 31) / 32) * 4);
  W->total = o;
  return o;
}

namespace {

// One kind of slot table of the cache (K/V or group summaries), with the
// call's needs and copy list in the workspace.
struct SlotTable {
  int32_t* slot;       // [Hkv][nch]
  int32_t* owner;      // [Hkv][S]
  int32_t* used;       // [Hkv][S]: the call that last needed the slot
  uint64_t* valid;     // [Hkv][S]: groups of the slot's chunk that are present
  int32_t* hand;       // [Hkv]: ring position of the next slot to give out
  int nch, S;
  uint64_t* need;         // [Hkv][nch]: groups of each chunk the call needs (0: chunk not needed); cleared here
  uint64_t* pend;         // [Hkv][nch] or null: groups of each needed chunk this call copies
  CopyEntry* list;        // [Hkv][nch]
  int32_t* count;         // [Hkv]
  long long* evictions;   // counter
};

template <typename T>
__global__ __launch_bounds__(256) void fill_kernel(T* p, int64_t n, T value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// Sum of one value per thread over the workgroup, added to *dst by thread 0.
__device__ void block_add(long long v, long long* dst, long long* lds) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long t = 0;
    for (int w = 0; w < nw; ++w) t += lds[w];
    if (t) atomicAdd(reinterpret_cast<unsigned long long*>(dst), (unsigned long long)t);
  }
  __syncthreads();
}

// Slot assignment of one KV head (one 1024-thread workgroup per head); the
// call's stamp is the call counter plus one (the K/V copy kernel raises the
// counter):
//  1. every needed chunk (its mark read and cleared) with a slot is stamped
//     with this call; the groups it still lacks go to the copy list;
//  2. every needed chunk without a slot takes the next slot in ring order
//     from the head's ring position that this call does not use (an empty
//     slot, or the slot of a chunk this call does not need, which is
//     evicted), and all its needed groups go to the copy list.
// The host guarantees enough slots for the chunks one call can need.
constexpr int kAssignThreads = 1024;
constexpr int kAssignPer = kMaxCand / kAssignThreads;   // chunks (and ring positions) per thread

__global__ __launch_bounds__(kAssignThreads) void assign_kernel(SlotTable T, const long long* counters) {
  __shared__ int sScan[16];
  __shared__ int sVict[kMaxCand];
  __shared__ long long sSum[16];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int stamp = (int)counters[kTcCalls] + 1;
  int32_t* slot = T.slot + (int64_t)h * T.nch;
  int32_t* owner = T.owner + (int64_t)h * T.S;
  int32_t* used = T.used + (int64_t)h * T.S;
  uint64_t* valid = T.valid + (int64_t)h * T.S;
  uint64_t* need = T.need + (int64_t)h * T.nch;
  uint64_t* pend = T.pend ? T.pend + (int64_t)h * T.nch : nullptr;
  CopyEntry* list = T.list + (int64_t)h * T.nch;
  // 1. needed chunks: hits stamped, their missing groups listed; misses counted
  uint64_t nd[kAssignPer];
  int sl[kAssignPer];
  int nfill = 0, nalloc = 0;
#pragma unroll
  for (int k = 0; k < kAssignPer; ++k) {
    const int m = tid * kAssignPer + k;
    nd[k] = m < T.nch ? need[m] : 0ull;
    if (nd[k]) need[m] = 0ull;   // the next call's marks start from zero
    sl[k] = nd[k] ? slot[m] : -1;
    if (nd[k] && sl[k] >= 0) {
      used[sl[k]] = stamp;
      if (nd[k] & ~valid[sl[k]]) ++nfill;
    } else if (nd[k]) {
      ++nalloc;
    }
  }
  int tot_fill, tot_alloc;
  int pos_fill = block_scan<false>(nfill, sScan, &tot_fill);
  int pos_alloc = block_scan<false>(nalloc, sScan, &tot_alloc);
  // 2. victims: the first tot_alloc ring positions (from the head's hand)
  // whose slots this call does not use (the stamps of step 1 are visible)
  const int hand = T.hand[h];
  int fr[kAssignPer], nfree = 0;
#pragma unroll
  for (int k = 0; k < kAssignPer; ++k) {
    const int i = tid * kAssignPer + k;
    fr[k] = 0;
    if (i < T.S) {
      const int v = (hand + i) % T.S;
      fr[k] = used[v] != stamp;
      nfree += fr[k];
    }
  }
  int tot_free;
  int rank = block_scan<false>(nfree, sScan, &tot_free);
#pragma unroll
  for (int k = 0; k < kAssignPer; ++k) {
    const int i = tid * kAssignPer + k;
    if (fr[k]) {
      if (rank < tot_alloc) sVict[rank] = (hand + i) % T.S;
      if (rank == tot_alloc - 1) T.hand[h] = (hand + i + 1) % T.S;
      ++rank;
    }
  }
  __syncthreads();
  // 3. list the copies; give each missing chunk its victim slot
  long long evict = 0;
#pragma unroll
  for (int k = 0; k < kAssignPer; ++k) {
    const int m = tid * kAssignPer + k;
    if (!nd[k]) continue;
    if (sl[k] >= 0) {
      const uint64_t miss = nd[k] & ~valid[sl[k]];
      if (pend) pend[m] = miss;
      if (miss) list[pos_fill++] = CopyEntry{m, sl[k], miss};
    } else if (pos_alloc < tot_free) {   // (the host sizes the cache so that this always holds)
      if (pend) pend[m] = nd[k];
      const int v = sVict[pos_alloc];
      const int old = owner[v];
      if (old >= 0) {
        slot[old] = -1;
        ++evict;
      }
      owner[v] = m;
      slot[m] = v;
      valid[v] = 0ull;
      used[v] = stamp;
      list[tot_fill + pos_alloc] = CopyEntry{m, v, nd[k]};
      ++pos_alloc;
    }
  }
  if (tid == 0) T.count[h] = tot_fill + tot_alloc;
  block_add(evict, T.evictions, sSum);
}

// Copy the listed groups of K and V (g rows each) from pinned host memory
// into their slots; one workgroup per list entry (grid-stride over the
// head's list). Every thread issues all its loads before its stores. The
// first workgroup raises the call counter (the call's stamp).
template <typename T>
__global__ __launch_bounds__(256) void copy_kv_kernel(AttnArgs A, const CopyEntry* list, const int32_t* count,
                                                      uint64_t* valid, int S, long long* counters) {
  const int h = blockIdx.y;
  const int n = count[h];
  const int d = A.s.d, g = A.s.g;
  const int64_t split = A.kv.split;
  constexpr int EPV = 16 / sizeof(T);             // elements per 16-byte piece
  const int per_group = g * d / EPV;               // pieces per group and tensor
  long long groups = 0;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) counters[kTcCalls] += 1;
  for (int e = blockIdx.x; e < n; e += gridDim.x) {
    const CopyEntry ce = list[(int64_t)h * A.nch + e];
    const int ng = __popcll(ce.mask);
    // the j-th set bit of the mask for piece p of the entry
    const T* ks = static_cast<const T*>(A.kv.k_host) + ((int64_t)h * split + (int64_t)ce.m * kChunk) * d;
    const T* vs = static_cast<const T*>(A.kv.v_host) + ((int64_t)h * split + (int64_t)ce.m * kChunk) * d;
    T* kd = static_cast<T*>(const_cast<void*>(A.k_cache)) + ((int64_t)h * S + ce.slot) * kChunk * d;
    T* vd = static_cast<T*>(const_cast<void*>(A.v_cache)) + ((int64_t)h * S + ce.slot) * kChunk * d;
    constexpr int kPer = 8;
    for (int base = threadIdx.x; base < ng * per_group; base += blockDim.x * kPer) {
      u32x4 kx[kPer], vx[kPer];
      int64_t off[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int p = base + u * blockDim.x;
        off[u] = -1;
        if (p < ng * per_group) {
          // group = the (p / per_group)-th set bit of the mask
          uint64_t msk = ce.mask;
          for (int j = p / per_group; j > 0; --j) msk &= msk - 1;
          const int grp = __ffsll((long long)msk) - 1;
          off[u] = (int64_t)grp * g * d + (int64_t)(p % per_group) * EPV;
          kx[u] = *reinterpret_cast<const u32x4*>(ks + off[u]);
          vx[u] = *reinterpret_cast<const u32x4*>(vs + off[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (off[u] >= 0) {
          *reinterpret_cast<u32x4*>(kd + off[u]) = kx[u];
          *reinterpret_cast<u32x4*>(vd + off[u]) = vx[u];
        }
    }
    if (threadIdx.x == 0) {
      valid[(int64_t)h * S + ce.slot] |= ce.mask;
      groups += ng;
    }
  }
  if (threadIdx.x == 0 && groups) {
    atomicAdd(reinterpret_cast<unsigned long long*>(&counters[kTcKvMisses]), (unsigned long long)groups);
    atomicAdd(reinterpret_cast<unsigned long long*>(&counters[kTcKvBytes]),
              (unsigned long long)(groups * 2 * g * d * (long long)sizeof(T)));
  }
}

// Copy the group summaries of the listed chunks (all c/g groups, d float32
// each) from pinned host memory into their slots.
__global__ __launch_bounds__(256) void copy_gs_kernel(const float* gs_host, int64_t gsplit, float* gs_cache,
                                                      const CopyEntry* list, const int32_t* count, uint64_t* gvalid,
                                                      int nch, int Sg, int gpc, int d, long long* counters) {
  const int h = blockIdx.y;
  const int n = count[h];
  long long chunks = 0;
  for (int e = blockIdx.x; e < n; e += gridDim.x) {
    const CopyEntry ce = list[(int64_t)h * nch + e];
    const float4* src = reinterpret_cast<const float4*>(gs_host + ((int64_t)h * gsplit + (int64_t)ce.m * gpc) * d);
    float4* dst = reinterpret_cast<float4*>(gs_cache + ((int64_t)h * Sg + ce.slot) * gpc * d);
    const int pieces = gpc * d / 4;
    for (int p = threadIdx.x; p < pieces; p += blockDim.x) dst[p] = src[p];
    if (threadIdx.x == 0) {
      gvalid[(int64_t)h * Sg + ce.slot] = 1ull;
      ++chunks;
    }
  }
  if (threadIdx.x == 0 && chunks) {
    atomicAdd(reinterpret_cast<unsigned long long*>(&counters[kTcGsMisses]), (unsigned long long)chunks);
    atomicAdd(reinterpret_cast<unsigned long long*>(&counters[kTcGsBytes]),
              (unsigned long long)(chunks * gpc * d * 4));
  }
}

// Group stage of every item after the chunk stage (route_kernel with
// chunks_only): the block query and the kept chunks come back from memory,
// the group summaries of history chunks from the cache's GS slots, the rest
// from the device rows.
struct GroupArgs {
  route::RouteArgs r;
  const double* qbar;      // [nb][Hkv][d]
  const int32_t* gslot;    // [Hkv][nch]
  const float* gs_cache;   // [Hkv][Sg][c/g][d]
  int nch, Sg;
};

__global__ __launch_bounds__(route::kThreads) void route_groups_kernel(GroupArgs G) {
  __shared__ route::RouteSmem sm;
  __shared__ const float* sBase[kMaxKeptChunks];   // summary row of each kept chunk's first group
  __shared__ int sMarked;                          // kept history groups marked for the K/V slots
  const route::RouteArgs& a = G.r;
  const Shape& S = a.s;
  const int nwg = (int)(S.nb * S.hkv);
  int lid = blockIdx.x;
  if (nwg % 8 == 0) lid = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
  const int h = lid / (int)S.nb, b = lid % (int)S.nb;
  const int64_t row = (int64_t)b * S.hkv + h;
  const int d = S.d, gpc = S.c / S.g;
  int nsc = a.n_sel[row * 2];
  nsc = nsc < 0 ? 0 : (nsc > S.kc ? S.kc : nsc);
  const int64_t gsplit = a.split / S.g;
  const int64_t ngl = S.kvs / S.g;
  if (threadIdx.x == 0) sMarked = 0;
  for (int i = threadIdx.x; i < d; i += blockDim.x) sm.qbar[i] = G.qbar[row * d + i];
  for (int i = threadIdx.x; i < nsc; i += blockDim.x) {
    const int m = a.chunk_idx[row * S.kc + i];
    sm.chunks[i] = m;
    const int64_t j0 = (int64_t)m * gpc;
    sBase[i] = j0 < gsplit ? G.gs_cache + ((int64_t)h * G.Sg + G.gslot[(int64_t)h * G.nch + m]) * gpc * d
                           : a.gs_dev + ((int64_t)h * (ngl - gsplit) + (j0 - gsplit)) * d;
  }
  __syncthreads();
  int32_t* gout = a.group_idx + row * S.kg;
  uint64_t* need = a.kv_need + (int64_t)h * (a.need_split / kChunk);
  route::group_stage<true>(a, b, h, sm, nsc, true, route::MarkingEmit{gout, need, S.g, a.need_split, &sMarked},
                           [gpc, d, base = &sBase[0]](int c, int64_t) -> const float* {
                             return base[c / gpc] + (int64_t)(c % gpc) * d;
                           });
  __syncthreads();
  route::mark_fixed_chunks(a, b, h, sMarked);
}

}  // namespace

hipError_t tier_cache_init(const Shape& s, int64_t split, int kv_slots, int gs_slots, void* mem, hipStream_t st) {
  TierCacheLayout L;
  tier_cache_layout(s, split, kv_slots, gs_slots, &L);
  char* base = static_cast<char*>(mem);
  const int64_t hkv = s.hkv;
  auto fill32 = [&](size_t off, int64_t n, int32_t v) {
    if (n > 0)
      fill_kernel<int32_t><<<dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)), dim3(256), 0, st>>>(
          reinterpret_cast<int32_t*>(base + off), n, v);
  };
  auto fill64 = [&](size_t off, int64_t n) {
    if (n > 0)
      fill_kernel<unsigned long long><<<dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)), dim3(256), 0,
                                        st>>>(reinterpret_cast<unsigned long long*>(base + off), n, 0ull);
  };
  fill64(0, kTierCounters);
  fill32(L.slot, hkv * L.nch, -1);
  fill32(L.owner, hkv * L.S, -1);
  fill32(L.used, hkv * L.S, -1);
  fill64(L.valid, hkv * L.S);
  fill32(L.hand, hkv, 0);
  fill32(L.gslot, hkv * L.nch, -1);
  fill32(L.gowner, hkv * L.Sg, -1);
  fill32(L.gused, hkv * L.Sg, -1);
  fill64(L.gvalid, hkv * L.Sg);
  fill32(L.ghand, hkv, 0);
  fill64(L.need, hkv * L.nch);
  fill64(L.gneed, hkv * L.nch);
  return hipGetLastError();
}

// Routing and attention of one call through the cache (history K/V and
// group summaries in pinned host memory, split at kv.split). With copy_st
// the K/V copies overlap the attention of the items that need none.
hipError_t launch_route_attend_cached(const Shape& s, const void* q, const float* cs, const float* gs_host,
                                      const float* gs_dev, int64_t gs_split, const KVSrc& kv, int kv_slots,
                                      int gs_slots, void* cache_mem, int32_t* chunk_idx, int32_t* group_idx,
                                      int32_t* n_sel, void* out, float* lse, void* workspace, hipStream_t st,
                                      hipStream_t copy_st) {
  const int64_t items = s.nb * s.hkv;
  if (items == 0) return hipSuccess;
  TierCacheLayout L;
  tier_cache_layout(s, kv.split, kv_slots, gs_slots, &L);
  TierCallLayout W;
  tier_call_layout(s, kv.split, &W);
  char* cb = static_cast<char*>(cache_mem);
  char* wb = static_cast<char*>(workspace);
  long long* counters = reinterpret_cast<long long*>(cb);
  const int nch = L.nch;
  uint64_t* need = reinterpret_cast<uint64_t*>(cb + L.need);
  uint64_t* gneed = reinterpret_cast<uint64_t*>(cb + L.gneed);

  // ---- routing, marking what each item needs; when the group stage must
  // choose, the group summaries of the kept history chunks go through the
  // cache's GS slots
  const int gpc = kChunk / s.g;
  const bool groups_choose = s.kg < s.kc * gpc && gs_split > 0;
  route::RouteArgs ra{q, cs, gs_host, gs_dev, gs_split, chunk_idx, group_idx, n_sel, s};
  ra.counters = counters;
  ra.need_split = kv.split;
  if (groups_choose) {
    ra.chunks_only = true;
    ra.qbar_out = reinterpret_cast<double*>(wb + W.qbar);
    ra.gs_need = gneed;
  } else {
    ra.kv_need = need;
  }
  hipError_t e = launch_route_args(ra, st);
  if (e != hipSuccess) return e;
  if (groups_choose) {
    SlotTable G{reinterpret_cast<int32_t*>(cb + L.gslot), reinterpret_cast<int32_t*>(cb + L.gowner),
                reinterpret_cast<int32_t*>(cb + L.gused), reinterpret_cast<uint64_t*>(cb + L.gvalid),
                reinterpret_cast<int32_t*>(cb + L.ghand), nch, gs_slots, gneed, nullptr,
                reinterpret_cast<CopyEntry*>(wb + W.glist), reinterpret_cast<int32_t*>(wb + W.gcount),
                &counters[kTcGsEvictions]};
    assign_kernel<<<dim3((unsigned)s.hkv), dim3(kAssignThreads), 0, st>>>(G, counters);
    copy_gs_kernel<<<dim3(64, (unsigned)s.hkv), dim3(256), 0, st>>>(
        gs_host, gs_split / s.g, reinterpret_cast<float*>(cb + L.gs), G.list, G.count, G.valid, nch, gs_slots, gpc,
        s.d, counters);
    GroupArgs ga{ra, reinterpret_cast<const double*>(wb + W.qbar), G.slot, reinterpret_cast<const float*>(cb + L.gs),
                 nch, gs_slots};
    ga.r.chunks_only = false;
    ga.r.qbar_out = nullptr;
    ga.r.gs_need = nullptr;
    ga.r.kv_need = need;
    route_groups_kernel<<<dim3((unsigned)items), dim3(route::kThreads), 0, st>>>(ga);
  }

  // ---- the history groups every item attends, through the K/V slots
  AttnArgs a{};
  a.kv = kv; a.gidx = group_idx; a.nsel = n_sel; a.s = s; a.nch = nch; a.nslots = kv_slots;
  a.k_cache = cb + L.k;
  a.v_cache = cb + L.v;
  uint64_t* pend = reinterpret_cast<uint64_t*>(wb + W.pend);
  SlotTable T{reinterpret_cast<int32_t*>(cb + L.slot), reinterpret_cast<int32_t*>(cb + L.owner),
              reinterpret_cast<int32_t*>(cb + L.used), reinterpret_cast<uint64_t*>(cb + L.valid),
              reinterpret_cast<int32_t*>(cb + L.hand), nch, kv_slots, need, pend,
              reinterpret_cast<CopyEntry*>(wb + W.list), reinterpret_cast<int32_t*>(wb + W.count),
              &counters[kTcKvEvictions]};
  assign_kernel<<<dim3((unsigned)s.hkv), dim3(kAssignThreads), 0, st>>>(T, counters);
  auto copy = [&](hipStream_t cs_) {
    if (s.dtype == HGA_BF16)
      copy_kv_kernel<uint16_t><<<dim3(64, (unsigned)s.hkv), dim3(256), 0, cs_>>>(a, T.list, T.count, T.valid,
                                                                                  kv_slots, counters);
    else
      copy_kv_kernel<float><<<dim3(64, (unsigned)s.hkv), dim3(256), 0, cs_>>>(a, T.list, T.count, T.valid,
                                                                               kv_slots, counters);
    return hipGetLastError();
  };
  TierCache tc{T.slot, nch, kv_slots, a.k_cache, a.v_cache, pend, 0, reinterpret_cast<int*>(wb + W.done)};
  if (!copy_st) {
    if ((e = copy(st)) != hipSuccess) return e;
    return launch_attend(s, q, kv, group_idx, n_sel, out, lse, nullptr, 0, st, &tc);
  }
  // fork the copies onto copy_st; attend the items that need no copy (pass
  // 1) meanwhile; join; attend the rest (pass 2)
  hipEvent_t assigned = nullptr, copied = nullptr;
  if ((e = hipEventCreateWithFlags(&assigned, hipEventDisableTiming)) != hipSuccess) return e;
  if ((e = hipEventCreateWithFlags(&copied, hipEventDisableTiming)) != hipSuccess) {
    (void)hipEventDestroy(assigned);
    return e;
  }
  if ((e = hipEventRecord(assigned, st)) == hipSuccess && (e = hipStreamWaitEvent(copy_st, assigned, 0)) == hipSuccess &&
      (e = copy(copy_st)) == hipSuccess && (e = hipEventRecord(copied, copy_st)) == hipSuccess) {
    tc.pass = 1;
    if ((e = launch_attend(s, q, kv, group_idx, n_sel, out, lse, nullptr, 0, st, &tc)) == hipSuccess &&
        (e = hipStreamWaitEvent(st, copied, 0)) == hipSuccess) {
      tc.pass = 2;
      e = launch_attend(s, q, kv, group_idx, n_sel, out, lse, nullptr, 0, st, &tc);
    }
  }
  // (an event recorded but not yet reached is released once it completes)
  (void)hipEventDestroy(assigned);
  (void)hipEventDestroy(copied);
  return e;
}

}  // namespace hga
