// Two-level HGA router ("Long-Context Fine-Tuning with Limited VRAM",
// section 2.1, "Chunk selection" and "Group selection").
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
#include "hga_route_impl.h"


namespace hga {
namespace {

using route::RouteArgs;
using route::kThreads;

// kCache: the persistent cache's variant (block queries kept, chunk stage
// alone, the history each item needs marked); a kernel of its own, so that
// the plain router's code and registers are those of the plain path.
// kSelectMax: both selections take at most that many candidates (512 or
// 1024, see select_fits), and the selection is inlined (0: any number, the
// selection is a function call).
template <typename T, bool kCache, int kSelectMax = 0>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  __shared__ route::RouteSmem sm;
  __shared__ int sMarked;   // the item's kept history groups (or chunks) marked for the cache
  const Shape& S = a.s;
  // the workgroups of one KV head stay on one XCD (block id x runs on XCD
  // x % 8), so its summaries stay in that XCD's L2
  const int nwg = (int)(S.nb * S.hkv);
  int lid = blockIdx.x;
  if (nwg % 8 == 0) lid = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
  const int h = lid / (int)S.nb;
  const int b = lid % (int)S.nb;
  int32_t* gout = a.group_idx + ((int64_t)b * S.hkv + h) * S.kg;
  if constexpr (!kCache) {
    auto emit = [gout](int rank, int group) { gout[rank] = group; };
    route::route_item<T, true, false, decltype(emit), route::NoHook, kSelectMax>(a, b, h, sm, true, emit);
    return;
  }
  // with the persistent cache's marks (route_item's first barrier orders
  // this store before every use)
  if (threadIdx.x == 0) sMarked = 0;
  uint64_t* need = a.kv_need ? a.kv_need + (int64_t)h * (a.need_split / kChunk) : nullptr;
  const int n = route::route_item<T, true, true>(a, b, h, sm, true,
                                                 route::MarkingEmit{gout, need, S.g, a.need_split, &sMarked});
  __syncthreads();
  if (a.chunks_only) {
    if (a.gs_need) route::mark_summary_chunks(a, h, sm, n, &sMarked);
  } else if (a.kv_need) {
    route::mark_fixed_chunks(a, b, h, sMarked);
  }
}

}  // namespace

hipError_t launch_route(const Shape& s, const void* q, const float* cs, const float* gs_host,
                        const float* gs_dev, int64_t split, int32_t* chunk_idx, int32_t* group_idx,
                        int32_t* n_sel, hipStream_t st) {
  return launch_route_args(RouteArgs{q, cs, gs_host, gs_dev, split, chunk_idx, group_idx, n_sel, s}, st);
}

hipError_t launch_route_args(const RouteArgs& a, hipStream_t st) {
  const Shape& s = a.s;
  const int64_t items = s.nb * s.hkv;
  if (items == 0) return hipSuccess;
  const bool cache = a.kv_need || a.gs_need || a.qbar_out || a.chunks_only;
  const int sel = route::select_fits(s, 512) ? 512 : route::select_fits(s, 1024) ? 1024 : 0;
  const dim3 grid((unsigned)items), block(kThreads);
  if (s.dtype == HGA_BF16) {
    if (cache) route_kernel<uint16_t, true><<<grid, block, 0, st>>>(a);
    else if (sel == 512) route_kernel<uint16_t, false, 512><<<grid, block, 0, st>>>(a);
    else if (sel == 1024) route_kernel<uint16_t, false, 1024><<<grid, block, 0, st>>>(a);
    else route_kernel<uint16_t, false><<<grid, block, 0, st>>>(a);
  } else {
    if (cache) route_kernel<float, true><<<grid, block, 0, st>>>(a);
    else if (sel == 512) route_kernel<float, false, 512><<<grid, block, 0, st>>>(a);
    else route_kernel<float, false><<<grid, block, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace hga
