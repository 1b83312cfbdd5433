// C ABI of the HGA routed-attention library: argument validation on the host,
// then kernel launches on the caller's stream. See include/hga.h for the
// contract of each entry point.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <initializer_list>
#include <mutex>

#include "hga_internal.h"

namespace {

thread_local char g_err[512] = "";

hga_status fail(hga_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

hga_status ok() {
  g_err[0] = '\0';
  return HGA_OK;
}

hga_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HGA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Validate the config and the sequence geometry; fill the derived shape.
hga_status make_shape(const hga_config* cfg, int64_t seq_len, int64_t q_start, int64_t n_q,
                      hga::Shape* s) {
  using namespace hga;
  if (!cfg) return fail(HGA_ERR_INVALID_ARGUMENT, "cfg is NULL");
  if (cfg->n_q_heads < 1 || cfg->n_kv_heads < 1 || cfg->n_q_heads % cfg->n_kv_heads != 0)
    return fail(HGA_ERR_INVALID_ARGUMENT, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                cfg->n_q_heads, cfg->n_kv_heads);
  if (cfg->dtype != HGA_F32 && cfg->dtype != HGA_BF16 && cfg->dtype != HGA_BF16_F32OUT)
    return fail(HGA_ERR_INVALID_ARGUMENT, "unknown dtype %d", cfg->dtype);
  const int dt = cfg->dtype == HGA_BF16_F32OUT ? HGA_BF16 : cfg->dtype;   // element type of Q, K, V
  if (cfg->summary_op != HGA_SUMMARY_MEAN)
    return fail(HGA_ERR_INVALID_ARGUMENT, "unknown summary_op %d", cfg->summary_op);
  if (cfg->head_dim < 1) return fail(HGA_ERR_INVALID_ARGUMENT, "head_dim must be positive");
  if (cfg->chunk_size < 1 || cfg->group_size < 1 || cfg->q_block < 1)
    return fail(HGA_ERR_INVALID_ARGUMENT, "chunk_size, group_size and q_block must be positive");
  if (cfg->chunk_size % cfg->group_size != 0)
    return fail(HGA_ERR_INVALID_ARGUMENT, "group_size (%d) must divide chunk_size (%d)", cfg->group_size,
                cfg->chunk_size);
  if (cfg->top_chunks < 0 || cfg->top_groups < 0 || cfg->sink_tokens < 0 || cfg->local_tokens < 0)
    return fail(HGA_ERR_INVALID_ARGUMENT, "budgets and window sizes must be >= 0");
  if (!(cfg->softmax_scale >= 0.0f) || !isfinite(cfg->softmax_scale))
    return fail(HGA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  if (seq_len < 0 || q_start < 0 || n_q < 0 || q_start + n_q > seq_len)
    return fail(HGA_ERR_INVALID_ARGUMENT, "need 0 <= q_start, 0 <= n_q, q_start + n_q <= seq_len");
  if (cfg->chunk_size != kChunk)
    return fail(HGA_ERR_UNSUPPORTED, "chunk_size must be %d", kChunk);
  if (cfg->q_block > kChunk || kChunk % cfg->q_block)
    return fail(HGA_ERR_UNSUPPORTED, "q_block must divide %d (got %d)", kChunk, cfg->q_block);
  if (cfg->sink_tokens % kChunk || cfg->local_tokens % kChunk)
    return fail(HGA_ERR_UNSUPPORTED, "sink_tokens and local_tokens must be multiples of %d", kChunk);
  if (seq_len % kChunk)
    return fail(HGA_ERR_UNSUPPORTED, "seq_len must be a multiple of %d", kChunk);
  if (q_start % cfg->q_block || n_q % cfg->q_block)
    return fail(HGA_ERR_UNSUPPORTED, "q_start and n_q must be multiples of q_block (%d)", cfg->q_block);
  const int d = cfg->head_dim;
  if (dt == HGA_BF16 && d != 64 && d != 128)
    return fail(HGA_ERR_UNSUPPORTED, "bfloat16 needs head_dim 64 or 128 (got %d)", d);
  if (dt == HGA_F32 && !(d == 4 || d == 8 || d == 16 || d == 32 || d == 64 || d == 128))
    return fail(HGA_ERR_UNSUPPORTED, "float32 needs head_dim in {4, 8, 16, 32, 64, 128} (got %d)", d);
  if (seq_len / kChunk > kMaxCand)
    return fail(HGA_ERR_UNSUPPORTED, "seq_len above %lld", (long long)kMaxCand * kChunk);
  const int gpc = kChunk / cfg->group_size;
  if (cfg->top_chunks > kMaxKeptChunks || (int64_t)cfg->top_chunks * gpc > kMaxCand)
    return fail(HGA_ERR_UNSUPPORTED, "top_chunks too large (at most %d and %d groups)", kMaxKeptChunks,
                kMaxCand);
  if (cfg->top_groups > kMaxRouted)
    return fail(HGA_ERR_UNSUPPORTED, "top_groups above %d", kMaxRouted);
  if (dt == HGA_BF16 && cfg->top_groups > kMaxRoutedAttn)
    return fail(HGA_ERR_UNSUPPORTED, "top_groups above %d for bfloat16", kMaxRoutedAttn);
  s->hq = cfg->n_q_heads;
  s->hkv = cfg->n_kv_heads;
  s->G = s->hq / s->hkv;
  s->d = d;
  s->c = kChunk;
  s->g = cfg->group_size;
  s->B = cfg->q_block;
  s->kc = cfg->top_chunks;
  s->kg = cfg->top_groups;
  s->sink_chunks = cfg->sink_tokens / kChunk;
  s->local_chunks = cfg->local_tokens / kChunk;
  s->dtype = dt;
  s->out_f32 = cfg->dtype == HGA_BF16_F32OUT;
  s->scale = cfg->softmax_scale > 0.0f ? cfg->softmax_scale : 1.0f / sqrtf((float)d);
  s->L = seq_len;
  s->q0 = q_start;
  s->nq = n_q;
  s->nb = n_q / cfg->q_block;
  s->qs = n_q;
  s->kvs = seq_len;
  return HGA_OK;
}

// The kernels move rows 16 bytes at a time: every tensor and workspace
// address must be a multiple of 16.
bool misaligned(const void* p) { return ((uintptr_t)p & 15) != 0; }

hga_status check_aligned(const char* names, std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (misaligned(p)) return fail(HGA_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", names);
  return HGA_OK;
}

hga_status check_tier(const hga_tiered* t, const char* name, int64_t seq_len, int64_t q_start) {
  if (!t) return fail(HGA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (misaligned(t->host) || misaligned(t->dev))
    return fail(HGA_ERR_INVALID_ARGUMENT, "%s.host and %s.dev must be 16-byte aligned", name, name);
  if (t->split < 0 || t->split > q_start)
    return fail(HGA_ERR_INVALID_ARGUMENT, "%s.split must be in [0, q_start]", name);
  if (t->split % hga::kChunk) return fail(HGA_ERR_UNSUPPORTED, "%s.split must be a multiple of 64", name);
  if (t->split > 0 && !t->host) return fail(HGA_ERR_INVALID_ARGUMENT, "%s.host is NULL", name);
  if (t->split < seq_len && !t->dev) return fail(HGA_ERR_INVALID_ARGUMENT, "%s.dev is NULL", name);
  return HGA_OK;
}

// K and V tiers of one call: same split; with a host part, a bounded number
// of fixed chunks and the workspace of the host-tier cache.
hga_status check_kv_tier(const hga::Shape& s, const hga_tiered* k, const hga_tiered* v, void* workspace,
                         size_t ws_bytes) {
  if (k->split != v->split) return fail(HGA_ERR_INVALID_ARGUMENT, "k.split and v.split differ");
  if (k->split == 0) return HGA_OK;
  if (s.sink_chunks + s.local_chunks > hga::kMaxFixedTiered)
    return fail(HGA_ERR_UNSUPPORTED, "with a host tier, sink and local windows may span at most %d chunks",
                hga::kMaxFixedTiered);
  const size_t need = hga::tier_cache_bytes(s, k->split);
  if (!workspace || ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  return HGA_OK;
}

// ---------------------------------------------------------------- static scratch
// Scratch memory of hga_route_attend_noalloc: the partial softmax states of
// the spread attention (attend_split_bytes), at most 256 ranges of 8 waves x
// (d / 2 + 2) x 64 floats at d = 128, i.e. 33 MiB. Each device the library
// runs on holds its own copy until the process ends. Its device address is
// taken once per device with hipGetSymbolAddress; host code passes that
// address (never the array's name, which is a host-side stand-in) to the
// kernels.
constexpr size_t kScratchBytes = (size_t)256 * 8 * (128 / 2 + 2) * 64 * sizeof(float);
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on that device, with that device current).
hga_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HGA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(HGA_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return HGA_OK;
}

// Most distinct history chunks (below split) one call of this shape can need
// per KV head, for K/V (the sink, local and kept chunks of every block) or
// for group summaries (the kept chunks).
int64_t cache_need_bound(const hga::Shape& s, int64_t split, int which) {
  const int64_t nch = split / hga::kChunk;
  const int64_t per = which == HGA_TC_KV ? (int64_t)s.kc + s.sink_chunks + s.local_chunks : (int64_t)s.kc;
  const int64_t b = s.nb * per;
  return b < nch ? b : nch;
}

// Whether the group stage of some block may choose (read group summaries).
bool group_stage_chooses(const hga::Shape& s) { return s.kg > 0 && (int64_t)s.kg < (int64_t)s.kc * (hga::kChunk / s.g); }

hga_status check_cache(const hga::Shape& s, const hga_tier_cache* c) {
  if (!c) return fail(HGA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!c->mem || ((uintptr_t)c->mem & 255))
    return fail(HGA_ERR_INVALID_ARGUMENT, "cache->mem must be non-NULL and 256-byte aligned");
  if (c->split <= 0 || c->split % hga::kChunk)
    return fail(HGA_ERR_INVALID_ARGUMENT, "cache->split must be a positive multiple of 64");
  if (c->split / hga::kChunk > hga::kMaxCand)
    return fail(HGA_ERR_UNSUPPORTED, "cache->split above %lld tokens", (long long)hga::kMaxCand * hga::kChunk);
  if (c->kv_slots < 1 || c->kv_slots > hga::kMaxCand || c->gs_slots < 0 || c->gs_slots > hga::kMaxCand)
    return fail(HGA_ERR_INVALID_ARGUMENT, "cache slots must be in [1, %d] (K/V) and [0, %d] (summaries)",
                hga::kMaxCand, hga::kMaxCand);
  hga::TierCacheLayout L;
  const size_t need = hga::tier_cache_layout(s, c->split, c->kv_slots, c->gs_slots, &L);
  if (c->bytes < need) return fail(HGA_ERR_WORKSPACE, "cache of %zu bytes needed, %zu given", need, c->bytes);
  return HGA_OK;
}

}  // namespace

extern "C" {

size_t hga_tier_cache_size(const hga_config* cfg, int64_t split, int32_t kv_slots, int32_t gs_slots) {
  hga::Shape s;
  if (make_shape(cfg, split, 0, 0, &s) != HGA_OK || split <= 0 || split / hga::kChunk > hga::kMaxCand ||
      kv_slots < 1 || kv_slots > hga::kMaxCand || gs_slots < 0 || gs_slots > hga::kMaxCand)
    return (size_t)-1;
  hga::TierCacheLayout L;
  return hga::tier_cache_layout(s, split, kv_slots, gs_slots, &L);
}

int32_t hga_tier_cache_min_slots(const hga_config* cfg, int64_t seq_len, int64_t n_q, int32_t which) {
  hga::Shape s;
  if (make_shape(cfg, seq_len, seq_len - n_q, n_q, &s) != HGA_OK || (which != HGA_TC_KV && which != HGA_TC_GS))
    return -1;
  if (which == HGA_TC_GS && !group_stage_chooses(s)) return 0;
  return (int32_t)cache_need_bound(s, seq_len - n_q, which);
}

hga_status hga_tier_cache_init(const hga_config* cfg, const hga_tier_cache* cache, void* stream) {
  if (!cache) return fail(HGA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (cache->split <= 0 || cache->split % hga::kChunk)
    return fail(HGA_ERR_INVALID_ARGUMENT, "cache->split must be a positive multiple of 64");
  hga::Shape s;
  hga_status st = make_shape(cfg, cache->split, 0, 0, &s);
  if (st != HGA_OK) return st;
  if ((st = check_cache(s, cache)) != HGA_OK) return st;
  return device_status(hga::tier_cache_init(s, cache->split, cache->kv_slots, cache->gs_slots, cache->mem,
                                            (hipStream_t)stream),
                       "hga_tier_cache_init launch");
}

hga_status hga_route_attend_cached(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q,
                                   int64_t seq_len, const float* chunk_sum, const hga_tiered* group_sum,
                                   const hga_tiered* k, const hga_tiered* v, const hga_tier_cache* cache,
                                   int32_t* chunk_idx, int32_t* group_idx, int32_t* n_sel, void* out, float* lse,
                                   void* workspace, size_t ws_bytes, void* stream, void* copy_stream) {
  hga::Shape s;
  hga_status st = make_shape(cfg, seq_len, q_start, n_q, &s);
  if (st != HGA_OK) return st;
  if (n_q == 0) return ok();
  if (!q || !chunk_sum || !n_sel || !out || (s.kc > 0 && !chunk_idx) || (s.kg > 0 && !group_idx))
    return fail(HGA_ERR_INVALID_ARGUMENT,
                "q, chunk_sum, n_sel, out, chunk_idx and group_idx must be non-NULL");
  if ((st = check_aligned("q, chunk_sum, out and workspace", {q, chunk_sum, out, workspace})) != HGA_OK) return st;
  if ((st = check_tier(group_sum, "group_sum", seq_len, q_start)) != HGA_OK) return st;
  if ((st = check_tier(k, "k", seq_len, q_start)) != HGA_OK) return st;
  if ((st = check_tier(v, "v", seq_len, q_start)) != HGA_OK) return st;
  if ((st = check_cache(s, cache)) != HGA_OK) return st;
  if (copy_stream && copy_stream == stream)
    return fail(HGA_ERR_INVALID_ARGUMENT, "copy_stream must be NULL or a stream other than stream");
  if (k->split != cache->split || v->split != cache->split || group_sum->split != cache->split)
    return fail(HGA_ERR_INVALID_ARGUMENT, "group_sum, k and v must be split at cache->split");
  if (s.sink_chunks + s.local_chunks > hga::kMaxFixedTiered)
    return fail(HGA_ERR_UNSUPPORTED, "with a host tier, sink and local windows may span at most %d chunks",
                hga::kMaxFixedTiered);
  if (cache->kv_slots < cache_need_bound(s, cache->split, HGA_TC_KV) ||
      (group_stage_chooses(s) && cache->gs_slots < cache_need_bound(s, cache->split, HGA_TC_GS)))
    return fail(HGA_ERR_UNSUPPORTED, "the cache has too few slots for calls of %lld queries (K/V %lld, summaries %lld)",
                (long long)n_q, (long long)cache_need_bound(s, cache->split, HGA_TC_KV),
                (long long)(group_stage_chooses(s) ? cache_need_bound(s, cache->split, HGA_TC_GS) : 0));
  hga::TierCallLayout W;
  const size_t need = hga::tier_call_layout(s, cache->split, &W);
  if (!workspace || ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  const hga::KVSrc kv{k->host, k->dev, v->host, v->dev, k->split};
  return device_status(hga::launch_route_attend_cached(s, q, chunk_sum, static_cast<const float*>(group_sum->host),
                                                       static_cast<const float*>(group_sum->dev), group_sum->split, kv,
                                                       cache->kv_slots, cache->gs_slots, cache->mem, chunk_idx,
                                                       group_idx, n_sel, out, lse, workspace, (hipStream_t)stream,
                                                       (hipStream_t)copy_stream),
                       "hga_route_attend_cached launch");
}

size_t hga_workspace_size(const hga_config* cfg, int64_t seq_len, int64_t n_q, int32_t which) {
  hga::Shape s;
  if (make_shape(cfg, seq_len, seq_len - n_q, n_q, &s) != HGA_OK) return (size_t)-1;
  switch (which) {
    case HGA_WS_ROUTE: return 0;
    case HGA_WS_ATTEND: return hga::attend_split_bytes(s);
    case HGA_WS_ATTEND_TIERED: return hga::tier_cache_bytes(s, seq_len - n_q);
    case HGA_WS_BACKWARD: return hga::backward_workspace_bytes(s);
    case HGA_WS_BACKWARD_TIERED:
      return hga::backward_workspace_bytes(s) + hga::tier_cache_bytes(s, seq_len - n_q);
    case HGA_WS_ATTEND_CACHED: {
      hga::TierCallLayout W;
      return hga::tier_call_layout(s, seq_len - n_q, &W);
    }
    default: fail(HGA_ERR_INVALID_ARGUMENT, "unknown workspace kind %d", which); return (size_t)-1;
  }
}

hga_status hga_build_summaries(const hga_config* cfg, const void* k, int64_t seq_len, float* group_sum,
                               float* chunk_sum, void* stream) {
  hga::Shape s;
  hga_status st = make_shape(cfg, seq_len, 0, 0, &s);
  if (st != HGA_OK) return st;
  if (seq_len == 0) return ok();
  if (!k || !group_sum || !chunk_sum)
    return fail(HGA_ERR_INVALID_ARGUMENT, "k, group_sum and chunk_sum must be non-NULL");
  if ((st = check_aligned("k, group_sum and chunk_sum", {k, group_sum, chunk_sum})) != HGA_OK) return st;
  return device_status(hga::launch_summaries(s, k, group_sum, chunk_sum, 0, seq_len / hga::kChunk,
                                             (hipStream_t)stream),
                       "hga_build_summaries launch");
}

hga_status hga_build_summaries_range(const hga_config* cfg, const void* k, int64_t seq_len, int64_t chunk_begin,
                                     int64_t chunk_end, float* group_sum, float* chunk_sum, void* stream) {
  hga::Shape s;
  hga_status st = make_shape(cfg, seq_len, 0, 0, &s);
  if (st != HGA_OK) return st;
  if (chunk_begin < 0 || chunk_begin > chunk_end || chunk_end > seq_len / hga::kChunk)
    return fail(HGA_ERR_INVALID_ARGUMENT, "need 0 <= chunk_begin <= chunk_end <= seq_len / 64");
  if (chunk_begin == chunk_end) return ok();
  if (!k || !group_sum || !chunk_sum)
    return fail(HGA_ERR_INVALID_ARGUMENT, "k, group_sum and chunk_sum must be non-NULL");
  if ((st = check_aligned("k, group_sum and chunk_sum", {k, group_sum, chunk_sum})) != HGA_OK) return st;
  return device_status(hga::launch_summaries(s, k, group_sum, chunk_sum, chunk_begin, chunk_end, (hipStream_t)stream),
                       "hga_build_summaries_range launch");
}

hga_status hga_stream_forward(const hga_config* cfg, const void* q, const void* k, const void* v, int64_t seq_len,
                              int64_t segment, float* chunk_sum, float* group_sum, int32_t* chunk_idx,
                              int32_t* group_idx, int32_t* n_sel, void* out, float* lse, void* stream) {
  hga::Shape full;
  hga_status st = make_shape(cfg, seq_len, 0, seq_len, &full);
  if (st != HGA_OK) return st;
  if (segment <= 0 || segment % hga::kChunk)
    return fail(HGA_ERR_INVALID_ARGUMENT, "segment must be a positive multiple of 64");
  if (seq_len == 0) return ok();
  if (!q || !k || !v || !chunk_sum || !group_sum || !n_sel || !out || (full.kc > 0 && !chunk_idx) ||
      (full.kg > 0 && !group_idx))
    return fail(HGA_ERR_INVALID_ARGUMENT,
                "q, k, v, chunk_sum, group_sum, n_sel, out, chunk_idx and group_idx must be non-NULL");
  if ((st = check_aligned("q, k, v, chunk_sum, group_sum and out", {q, k, v, chunk_sum, group_sum, out})) != HGA_OK)
    return st;
  const hipStream_t hs = (hipStream_t)stream;
  const size_t esz = full.dtype == HGA_BF16 ? 2 : 4;
  const size_t oesz = full.out_f32 ? 4 : esz;   // output elements
  const hga::KVSrc kv{nullptr, k, nullptr, v, 0};
  for (int64_t s0 = 0; s0 < seq_len; s0 += segment) {
    const int64_t s1 = s0 + segment < seq_len ? s0 + segment : seq_len;
    // the segment's chunks close: their summaries join the history's
    st = device_status(hga::launch_summaries(full, k, group_sum, chunk_sum, s0 / hga::kChunk, s1 / hga::kChunk, hs),
                       "hga_stream_forward summary launch");
    if (st != HGA_OK) return st;
    // the segment's queries against the committed history and themselves
    hga::Shape seg;
    if ((st = make_shape(cfg, s1, s0, s1 - s0, &seg)) != HGA_OK) return st;
    seg.qs = seq_len;
    seg.kvs = seq_len;
    const void* qs = static_cast<const char*>(q) + (size_t)s0 * full.d * esz;
    void* os = static_cast<char*>(out) + (size_t)s0 * full.d * oesz;
    float* ls = lse ? lse + s0 : nullptr;
    const int64_t b0 = s0 / full.B;   // first query block of the segment
    int32_t* ci = full.kc > 0 ? chunk_idx + b0 * full.hkv * full.kc : chunk_idx;
    int32_t* gi = full.kg > 0 ? group_idx + b0 * full.hkv * full.kg : group_idx;
    int32_t* ns = n_sel + b0 * full.hkv * 2;
    if (hga::fused_route_attend_supported(seg, 0)) {
      st = device_status(hga::launch_route_attend(seg, qs, chunk_sum, nullptr, group_sum, 0, kv, ci, gi, ns, os, ls, hs),
                         "hga_stream_forward launch");
    } else {
      st = device_status(hga::launch_route(seg, qs, chunk_sum, nullptr, group_sum, 0, ci, gi, ns, hs),
                         "hga_stream_forward routing launch");
      if (st == HGA_OK)
        st = device_status(hga::launch_attend(seg, qs, kv, gi, ns, os, ls, nullptr, 0, hs),
                           "hga_stream_forward attention launch");
    }
    if (st != HGA_OK) return st;
  }
  return ok();
}

hga_status hga_route(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q, int64_t seq_len,
                     const float* chunk_sum, const hga_tiered* group_sum, int32_t* chunk_idx,
                     int32_t* group_idx, int32_t* n_sel, void* workspace, size_t ws_bytes, void* stream) {
  (void)workspace;
  (void)ws_bytes;
  hga::Shape s;
  hga_status st = make_shape(cfg, seq_len, q_start, n_q, &s);
  if (st != HGA_OK) return st;
  if (n_q == 0) return ok();
  if (!q || !chunk_sum || !n_sel || (s.kc > 0 && !chunk_idx) || (s.kg > 0 && !group_idx))
    return fail(HGA_ERR_INVALID_ARGUMENT, "q, chunk_sum, n_sel, chunk_idx and group_idx must be non-NULL");
  if ((st = check_aligned("q and chunk_sum", {q, chunk_sum})) != HGA_OK) return st;
  if ((st = check_tier(group_sum, "group_sum", seq_len, q_start)) != HGA_OK) return st;
  return device_status(
      hga::launch_route(s, q, chunk_sum, static_cast<const float*>(group_sum->host),
                        static_cast<const float*>(group_sum->dev), group_sum->split, chunk_idx, group_idx,
                        n_sel, (hipStream_t)stream),
      "hga_route launch");
}

hga_status hga_attend(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q, int64_t seq_len,
                      const hga_tiered* k, const hga_tiered* v, const int32_t* group_idx,
                      const int32_t* n_sel, void* out, float* lse, void* workspace, size_t ws_bytes,
                      void* stream) {
  hga::Shape s;
  hga_status st = make_shape(cfg, seq_len, q_start, n_q, &s);
  if (st != HGA_OK) return st;
  if (n_q == 0) return ok();
  if (!q || !out || !n_sel || (s.kg > 0 && !group_idx))
    return fail(HGA_ERR_INVALID_ARGUMENT, "q, out, n_sel and group_idx must be non-NULL");
  if ((st = check_aligned("q, out and workspace", {q, out, workspace})) != HGA_OK) return st;
  if ((st = check_tier(k, "k", seq_len, q_start)) != HGA_OK) return st;
  if ((st = check_tier(v, "v", seq_len, q_start)) != HGA_OK) return st;
  if ((st = check_kv_tier(s, k, v, workspace, ws_bytes)) != HGA_OK) return st;
  hga::KVSrc kv{k->host, k->dev, v->host, v->dev, k->split};
  return device_status(hga::launch_attend(s, q, kv, group_idx, n_sel, out, lse, workspace, ws_bytes, (hipStream_t)stream),
                       "hga_attend launch");
}

hga_status hga_route_attend(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q, int64_t seq_len,
                            const float* chunk_sum, const hga_tiered* group_sum, const hga_tiered* k,
                            const hga_tiered* v, int32_t* chunk_idx, int32_t* group_idx, int32_t* n_sel,
                            void* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  hga::Shape s;
  hga_status st = make_shape(cfg, seq_len, q_start, n_q, &s);
  if (st != HGA_OK) return st;
  if (n_q == 0) return ok();
  if (!q || !chunk_sum || !n_sel || !out || (s.kc > 0 && !chunk_idx) || (s.kg > 0 && !group_idx))
    return fail(HGA_ERR_INVALID_ARGUMENT,
                "q, chunk_sum, n_sel, out, chunk_idx and group_idx must be non-NULL");
  if ((st = check_aligned("q, chunk_sum, out and workspace", {q, chunk_sum, out, workspace})) != HGA_OK) return st;
  if ((st = check_tier(group_sum, "group_sum", seq_len, q_start)) != HGA_OK) return st;
  if ((st = check_tier(k, "k", seq_len, q_start)) != HGA_OK) return st;
  if ((st = check_tier(v, "v", seq_len, q_start)) != HGA_OK) return st;
  if ((st = check_kv_tier(s, k, v, workspace, ws_bytes)) != HGA_OK) return st;
  const hipStream_t hs = (hipStream_t)stream;
  const float* gs_host = static_cast<const float*>(group_sum->host);
  const float* gs_dev = static_cast<const float*>(group_sum->dev);
  hga::KVSrc kv{k->host, k->dev, v->host, v->dev, k->split};
  // the fused kernel, unless the workspace lets the attention spread few
  // items over more workgroups
  const bool split = k->split == 0 && hga::attend_split_count(s) > 1 && workspace &&
                     ws_bytes >= hga::attend_split_bytes(s);
  if (!split && hga::fused_route_attend_supported(s, k->split))
    return device_status(hga::launch_route_attend(s, q, chunk_sum, gs_host, gs_dev, group_sum->split, kv,
                                                  chunk_idx, group_idx, n_sel, out, lse, hs),
                         "hga_route_attend launch");
  st = device_status(hga::launch_route(s, q, chunk_sum, gs_host, gs_dev, group_sum->split, chunk_idx, group_idx,
                                       n_sel, hs),
                     "hga_route_attend routing launch");
  if (st != HGA_OK) return st;
  return device_status(hga::launch_attend(s, q, kv, group_idx, n_sel, out, lse, workspace, ws_bytes, hs),
                       "hga_route_attend attention launch");
}

hga_status hga_route_attend_noalloc(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q,
                                    int64_t seq_len, const float* chunk_sum, const hga_tiered* group_sum,
                                    const hga_tiered* k, const hga_tiered* v, int32_t* chunk_idx, int32_t* group_idx,
                                    int32_t* n_sel, void* out, float* lse, void* stream) {
  hga::Shape s;
  hga_status st = make_shape(cfg, seq_len, q_start, n_q, &s);
  if (st != HGA_OK) return st;
  if (n_q == 0) return ok();
  if (!k || !v) return fail(HGA_ERR_INVALID_ARGUMENT, "k and v must be non-NULL");
  if (k->split != 0 || v->split != 0)
    return fail(HGA_ERR_UNSUPPORTED, "hga_route_attend_noalloc needs K and V on the device (split 0)");
  const size_t need = hga::attend_split_bytes(s);
  if (need > kScratchBytes)
    return fail(HGA_ERR_UNSUPPORTED, "the call needs %zu bytes of scratch; the static scratch holds %zu", need,
                kScratchBytes);
  void* ptr = nullptr;
  if ((st = scratch_of_current_device(&ptr)) != HGA_OK) return st;
  return hga_route_attend(cfg, q, q_start, n_q, seq_len, chunk_sum, group_sum, k, v, chunk_idx, group_idx, n_sel,
                          out, lse, need > 0 ? ptr : nullptr, need, stream);
}

hga_status hga_attend_backward(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q,
                               int64_t seq_len, const hga_tiered* k, const hga_tiered* v,
                               const int32_t* group_idx, const int32_t* n_sel, const void* out, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                               void* stream) {
  hga::Shape s;
  hga_status st = make_shape(cfg, seq_len, q_start, n_q, &s);
  if (st != HGA_OK) return st;
  if (n_q == 0) return ok();
  if (!q || !n_sel || !out || !lse || !dout || !dq || !dk || !dv || (s.kg > 0 && !group_idx))
    return fail(HGA_ERR_INVALID_ARGUMENT, "q, group_idx, n_sel, out, lse, dout, dq, dk and dv must be non-NULL");
  if (s.out_f32) return fail(HGA_ERR_UNSUPPORTED, "the backward takes the forward's bfloat16 output (dtype HGA_BF16)");
  if ((st = check_aligned("q, out, dout, dq, dk, dv and workspace", {q, out, dout, dq, dk, dv, workspace})) != HGA_OK)
    return st;
  if ((st = check_tier(k, "k", seq_len, q_start)) != HGA_OK) return st;
  if ((st = check_tier(v, "v", seq_len, q_start)) != HGA_OK) return st;
  if (k->split != v->split) return fail(HGA_ERR_INVALID_ARGUMENT, "k.split and v.split differ");
  if (k->split > 0 && s.sink_chunks + s.local_chunks > hga::kMaxFixedTiered)
    return fail(HGA_ERR_UNSUPPORTED, "with a host tier, sink and local windows may span at most %d chunks",
                hga::kMaxFixedTiered);
  // the dK/dV kernel addresses Q and dO rows by 32-bit byte offsets
  if ((int64_t)s.hq * s.qs * s.d * (s.dtype == HGA_BF16 ? 2 : 4) > (int64_t)UINT32_MAX)
    return fail(HGA_ERR_UNSUPPORTED, "q and dout must be under 4 GiB each");
  const size_t need = hga::backward_workspace_bytes(s) + (k->split > 0 ? hga::tier_cache_bytes(s, k->split) : 0);
  if (!workspace || ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  const hga::KVSrc kv{k->host, k->dev, v->host, v->dev, k->split};
  return device_status(hga::launch_attend_backward(s, q, kv, group_idx, n_sel, out, lse, dout, dq, dk, dv,
                                                   workspace, (hipStream_t)stream),
                       "hga_attend_backward launch");
}

const char* hga_status_string(hga_status status) {
  switch (status) {
    case HGA_OK: return "ok";
    case HGA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case HGA_ERR_UNSUPPORTED: return "unsupported";
    case HGA_ERR_WORKSPACE: return "workspace too small";
    case HGA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* hga_last_error(void) { return g_err; }

int32_t hga_version(void) { return 110; }

}  // extern "C"
