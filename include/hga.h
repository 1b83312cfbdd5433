/*
 * hga.h -- C ABI of the MI355X (gfx950) HGA routed-attention forward.
 *
 * Hierarchical Global Attention (HGA) replaces dense causal attention. The
 * operation follows "Long-Context Fine-Tuning with Limited VRAM", section 2.1
 * "Exact-token hierarchical routing", and the base HGA abstract:
 *
 *   hga_build_summaries  key summaries of every 8-token group and every closed
 *                        64-token chunk, built from the model's projected,
 *                        RoPE-applied keys (section 2.1, first paragraph;
 *                        abstract: "compact RoPE-aware summaries"). The
 *                        operator is the mean of the post-RoPE keys.
 *   hga_route            per query block and KV head: score chunk summaries
 *                        with the block's mean query, keep the top chunks in
 *                        addition to fixed sink and local windows, open them
 *                        into groups and keep the top groups (section 2.1,
 *                        "Chunk selection" and "Group selection"). Indices
 *                        only; no gradient (section 2.1, last paragraph).
 *   hga_attend           exact causal softmax attention of each query over
 *                        the exact token K/V of the kept groups, the fixed
 *                        windows and its own block (section 2.1, "Exact-token
 *                        attention"); summaries are never attended.
 *
 * Conventions shared by every entry point
 *   Layout     head-major, row-major: Q and O are [Hq][n_q][d], K and V are
 *              [Hkv][seq_len][d]; query row i of Q holds position q_start + i.
 *              Query head r reads KV head r / (Hq / Hkv).
 *   Element    Q, K, V and O use cfg->dtype (float32 or bfloat16);
 *              summaries are float32; indices are int32.
 *   Ownership  the caller allocates every buffer and the workspace and keeps
 *              them alive until the work on `stream` has finished. The library
 *              allocates nothing and keeps no state between calls, except the
 *              static scratch array of hga_route_attend_noalloc (see there).
 *   Memory     "device" pointers are GPU memory of the current HIP device;
 *              "host" pointers of an hga_tiered are pinned host memory
 *              allocated with hipHostMalloc (mapped, readable by kernels).
 *   Alignment  the kernels move rows 16 bytes at a time: every tensor
 *              pointer (Q, K, V, O, the summaries, the gradients, both parts
 *              of an hga_tiered) and the workspace must be 16-byte aligned
 *              (index, count and LSE arrays need only their element's
 *              alignment); otherwise HGA_ERR_INVALID_ARGUMENT before any
 *              launch.
 *   Streams    `stream` is a hipStream_t (NULL = the default stream). All work
 *              is enqueued on it; nothing synchronizes.
 *   Errors     arguments are validated on the host before any launch; on an
 *              error nothing is enqueued and a status other than HGA_OK is
 *              returned. hga_last_error() gives a message (thread-local).
 *              Kernel launch failures return HGA_ERR_DEVICE.
 *   Support    chunk_size == 64; q_block divides 64 (1 routes every token
 *              on its own, as when decoding); group_size divides 64; sink and
 *              local sizes are multiples of chunk_size; seq_len is a multiple
 *              of chunk_size; q_start and n_q are multiples of q_block.
 *              Rows of K, V and the summaries past q_start + n_q are never
 *              read, so seq_len may be the capacity of a decoding cache.
 *              bfloat16 needs
 *              head_dim 64 or 128; float32 needs head_dim % 4 == 0 and
 *              head_dim <= 128. Anything else returns HGA_ERR_UNSUPPORTED.
 */
#ifndef HGA_H
#define HGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HGA_OK = 0,
  HGA_ERR_INVALID_ARGUMENT = 1,  /* null pointer, negative or inconsistent size */
  HGA_ERR_UNSUPPORTED = 2,       /* valid, but outside what this build implements */
  HGA_ERR_WORKSPACE = 3,         /* workspace missing or smaller than hga_workspace_size */
  HGA_ERR_DEVICE = 4             /* a HIP launch or runtime call failed */
} hga_status;

/* Element types. HGA_BF16_F32OUT takes bfloat16 Q, K and V like HGA_BF16 and
 * writes the attention output O in float32 (the value before any rounding to
 * bfloat16: the output a parity check compares with a float64 reference
 * without the output's own storage rounding). Every entry point that writes
 * O accepts it (O then has 4-byte elements); hga_attend_backward does not
 * (HGA_ERR_UNSUPPORTED). The LSE is float32 in every mode. */
typedef enum { HGA_F32 = 0, HGA_BF16 = 1, HGA_BF16_F32OUT = 2 } hga_dtype;

/* Summary operator. The pages call the chunk summaries "RoPE-aware" without
 * defining them; the mean of the post-RoPE keys is the operator built here. */
typedef enum { HGA_SUMMARY_MEAN = 0 } hga_summary_op;

typedef struct {
  int32_t n_q_heads;     /* Hq >= 1, a multiple of n_kv_heads */
  int32_t n_kv_heads;    /* Hkv >= 1 */
  int32_t head_dim;      /* d */
  int32_t chunk_size;    /* tokens per chunk (64) */
  int32_t group_size;    /* tokens per group (8); divides chunk_size */
  int32_t q_block;       /* B: queries per routing block, a divisor of chunk_size */
  int32_t top_chunks;    /* kc >= 0: routed chunks kept per block and KV head */
  int32_t top_groups;    /* kg >= 0: routed groups kept per block and KV head */
  int32_t sink_tokens;   /* S: the first S tokens are always attended */
  int32_t local_tokens;  /* W: the W tokens before the block are always attended */
  int32_t summary_op;    /* hga_summary_op */
  int32_t dtype;         /* hga_dtype of Q, K, V and O */
  float softmax_scale;   /* 0 selects 1/sqrt(head_dim) */
} hga_config;

/* A [H][seq_len][width] tensor split between two tiers at token `split`:
 * rows [0, split) live in `host` as [H][split][width] (pinned host memory),
 * rows [split, seq_len) live in `dev` as [H][seq_len - split][width].
 * split == 0 means everything is in `dev` (then `host` may be NULL). For group
 * summaries the split is counted in tokens and the rows are groups. */
typedef struct {
  const void* host;
  const void* dev;
  int64_t split;
} hga_tiered;

enum {
  HGA_WS_ROUTE = 0, HGA_WS_ATTEND = 1, HGA_WS_ATTEND_TIERED = 2, HGA_WS_BACKWARD = 3, HGA_WS_BACKWARD_TIERED = 4,
  HGA_WS_ATTEND_CACHED = 5
};

/* Bytes of device workspace that hga_route (which = HGA_WS_ROUTE) or
 * hga_attend / hga_route_attend (HGA_WS_ATTEND with everything on the device,
 * HGA_WS_ATTEND_TIERED with K/V split at a token > 0) needs for this shape.
 * HGA_WS_ATTEND is 0 unless the call has few (block, KV head) items (bf16, at
 * most 128 attention workgroups, as when decoding a few sequences): then it
 * is the room for each item's tiles to be cut into ranges attended by
 * separate workgroups, whose partial softmax states are merged per query row.
 * The outputs then differ from the one-workgroup result by the rounding of
 * the probabilities to bfloat16 before the PV product, which each range takes
 * against its own running maximum (about 2^-9 relative, within the output
 * tolerance); the LSE differs by float32 rounding order only. Given less, the
 * calls attend each item in one workgroup.
 * The tiered figure holds for every split <= seq_len - n_q: it covers chunk
 * flags and slots and an HBM cache as large as the whole host part of K and V
 * (the attention copies each history chunk any query block needs into it once
 * per call). HGA_WS_BACKWARD is the workspace of hga_attend_backward with K/V
 * on the device, HGA_WS_BACKWARD_TIERED the same plus that cache (any split).
 * HGA_WS_ATTEND_CACHED is the per-call workspace of hga_route_attend_cached
 * for a host tier of seq_len - n_q tokens or fewer.
 * Returns 0 when no workspace is needed, and (size_t)-1 when the config or
 * sizes are invalid. */
size_t hga_workspace_size(const hga_config* cfg, int64_t seq_len, int64_t n_q, int32_t which);

/* Key summaries (section 2.1, first paragraph).
 *   k          device, [Hkv][seq_len][d] of cfg->dtype, post-RoPE keys.
 *   group_sum  device, [Hkv][seq_len / group_size][d] float32: the mean of
 *              each group's keys, rounded once to float32.
 *   chunk_sum  device, [Hkv][seq_len / chunk_size][d] float32: the mean of
 *              each chunk's keys, rounded once to float32.
 * Means are accumulated in float64 before the single rounding. */
hga_status hga_build_summaries(const hga_config* cfg, const void* k, int64_t seq_len,
                               float* group_sum, float* chunk_sum, void* stream);

/* Summaries of chunks [chunk_begin, chunk_end) only (section 2.1, first
 * paragraph: summaries are kept resident and a chunk's are built once, when it
 * closes). Layouts as in hga_build_summaries; rows of other chunks are left
 * untouched. 0 <= chunk_begin <= chunk_end <= seq_len / chunk_size, else
 * HGA_ERR_INVALID_ARGUMENT; an empty range is a no-op. */
hga_status hga_build_summaries_range(const hga_config* cfg, const void* k, int64_t seq_len,
                                     int64_t chunk_begin, int64_t chunk_end,
                                     float* group_sum, float* chunk_sum, void* stream);

/* Two-level routing (section 2.1, "Chunk selection", "Group selection").
 * For query block b (positions s = q_start + B b .. s + B - 1, B = q_block)
 * and KV head h, with c0 = 64 floor(s / 64) the first token of the block's
 * chunk:
 *   block query   mean of Q over the block's B positions and the
 *                 Hq/Hkv query heads of h (float64 accumulation);
 *   fixed chunks  sink: chunks before sink_tokens; local: the chunks holding
 *                 the local_tokens before c0 (only chunks that end by c0);
 *   chunk stage   candidates are the chunks ending by c0 that are not fixed;
 *                 score = block query . chunk_sum (float64 dot of the float32
 *                 summary); keep the top_chunks highest, ties to the lower
 *                 chunk index;
 *   group stage   candidates are the groups of the kept chunks; score =
 *                 block query . group_sum; keep the top_groups highest, ties to
 *                 the lower group index.
 *   q          device, [Hq][n_q][d] of cfg->dtype.
 *   chunk_sum  device, as written by hga_build_summaries.
 *   group_sum  group summaries, tiered at a token split (a multiple of
 *              chunk_size, <= q_start); host rows are read only when the group
 *              stage must choose (top_groups < groups of the kept chunks).
 *   chunk_idx  device, [n_q/B][Hkv][top_chunks] int32, ascending, -1 padded.
 *   group_idx  device, [n_q/B][Hkv][top_groups] int32, ascending, -1 padded.
 *   n_sel      device, [n_q/B][Hkv][2] int32: kept chunks, kept groups.
 *   workspace  unused (hga_workspace_size returns 0); may be NULL. */
hga_status hga_route(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q,
                     int64_t seq_len, const float* chunk_sum, const hga_tiered* group_sum,
                     int32_t* chunk_idx, int32_t* group_idx, int32_t* n_sel,
                     void* workspace, size_t ws_bytes, void* stream);

/* Exact-token routed attention (section 2.1, "Exact-token attention").
 * Query at position p of block b attends, with causal masking t <= p, to the
 * token set: the fixed sink and local chunks, the kept groups, and the
 * block's own chunk from its first token c0 up to the block's last position
 * (for B = 64 the block itself; for smaller blocks the chunk is still open,
 * has no summary, and its earlier tokens are kept whole). out = softmax(scale * q . k_t) @ v_t; lse = log-sum-exp of the
 * scaled scores (natural log).
 *   q          device, [Hq][n_q][d] of cfg->dtype.
 *   k, v       [Hkv][seq_len][d] of cfg->dtype, tiered at a token split
 *              (a multiple of chunk_size, <= q_start). With split > 0 the
 *              history chunks that any query block of the call needs (its
 *              sink and local chunks, the chunks of its kept groups) are
 *              copied once each into an HBM cache in the workspace, and the
 *              attention reads history rows from there (the pages' VRAM cache
 *              of routed sets shared across query blocks, section 2.1); sink
 *              and local windows may then span at most 256 chunks
 *              (HGA_ERR_UNSUPPORTED otherwise).
 *   group_idx  device, [n_q/B][Hkv][top_groups] as written by hga_route.
 *              An entry is usable when it is >= 0, its group ends by the
 *              block start and it lies outside the sink and local chunks; a usable
 *              entry that is not greater than every earlier usable entry of
 *              its row is skipped, so each token counts once and an ascending
 *              row is taken whole.
 *   n_sel      device, [n_q/B][Hkv][2]; the second value (clamped to
 *              [0, top_groups]) is how many entries of the row to read.
 *   out        device, [Hq][n_q][d] of cfg->dtype (float32 for HGA_BF16_F32OUT).
 *   lse        device, [Hq][n_q] float32, or NULL.
 *   workspace  device, at least hga_workspace_size(...) bytes (with split 0,
 *              NULL or fewer bytes than HGA_WS_ATTEND asks for is accepted:
 *              each item is then attended by one workgroup). */
hga_status hga_attend(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q,
                      int64_t seq_len, const hga_tiered* k, const hga_tiered* v,
                      const int32_t* group_idx, const int32_t* n_sel,
                      void* out, float* lse, void* workspace, size_t ws_bytes, void* stream);

/* Routing and attention of the same query rows in one call (section 2.1,
 * "Chunk selection", "Group selection" and "Exact-token attention" in
 * sequence): the results are those of hga_route followed by hga_attend on
 * its chunk_idx / group_idx / n_sel, which are written as well. Arguments
 * have the meaning, layout and ownership they have in those two calls; the
 * workspace is the one hga_attend needs for this K/V split. With bfloat16,
 * K/V entirely on the device (split 0), at most 256 query rows per block and
 * KV head (Hq/Hkv x q_block) and at most 512 chunk candidates per block
 * (closed chunks outside the sink and local windows: sequences up to about
 * 32K tokens), both steps run in one kernel, each workgroup routing its own
 * query block before attending over the groups it kept; otherwise the call
 * runs the two steps one after the other (the results are the same either
 * way). When the workspace holds what HGA_WS_ATTEND asks for (nonzero only
 * for few items) the two steps run one after the other and the attention
 * spreads each item over several workgroups. Errors are those of either
 * call. */
hga_status hga_route_attend(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q,
                            int64_t seq_len, const float* chunk_sum, const hga_tiered* group_sum,
                            const hga_tiered* k, const hga_tiered* v,
                            int32_t* chunk_idx, int32_t* group_idx, int32_t* n_sel,
                            void* out, float* lse, void* workspace, size_t ws_bytes, void* stream);

/* hga_route_attend for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same routing and attention, with the same results, taking
 * no workspace. Where hga_route_attend would spread few items over several
 * workgroups given its HGA_WS_ATTEND workspace (decoding a few sequences), the
 * partial softmax states go to a static device array of the library instead:
 * at most 33 MiB (256 ranges of 8 waves x (head_dim / 2 + 2) x 64 floats at
 * head_dim 128), held by each device the library runs on until the process
 * ends; shapes that would need more return HGA_ERR_UNSUPPORTED. The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * on its first call on a device it looks the array's device address up once.
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (each range writes its partial state before the merge reads
 * it, so nothing needs clearing): calls that overlap on one device, on
 * different streams or from different threads, race and must be ordered by
 * the caller. K and V must be entirely on the device (split 0, else
 * HGA_ERR_UNSUPPORTED). Other arguments, layouts and errors are those of
 * hga_route_attend. */
hga_status hga_route_attend_noalloc(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q,
                                    int64_t seq_len, const float* chunk_sum, const hga_tiered* group_sum,
                                    const hga_tiered* k, const hga_tiered* v, int32_t* chunk_idx, int32_t* group_idx,
                                    int32_t* n_sel, void* out, float* lse, void* stream);

/* Persistent cache in device memory of a host tier (the pages' VRAM cache:
 * "Long-Context Fine-Tuning with Limited VRAM", section 2.1, "Group
 * selection": group summaries are kept in a larger VRAM cache and missing
 * ones are fetched from host memory; "Exact-token attention": only the exact
 * token K/V of the selected groups is loaded; section 4.5, table 8: the cache
 * hit rate). It lives across calls: a call copies from host memory only what
 * its query blocks need and the cache does not hold. The caller owns the
 * memory; the library keeps no state of its own.
 *   mem        device memory of hga_tier_cache_size(...) bytes, 256-byte
 *              aligned. Its first HGA_TC_COUNTERS int64 are the counters
 *              below (read them with a device-to-host copy).
 *   split      the host tier it caches: tokens [0, split) of K, V and the
 *              group summaries, in the hga_tiered layouts of the calls (a
 *              multiple of 64). The host memory must not change while the
 *              cache holds its rows (call hga_tier_cache_init after a change).
 *   kv_slots   chunk slots per KV head for K and V rows: a slot holds any of
 *              the 64 / group_size groups of one history chunk (only needed
 *              groups are copied). At least hga_tier_cache_min_slots(...,
 *              HGA_TC_KV) and at most 4096.
 *   gs_slots   chunk slots per KV head for the group summaries of one history
 *              chunk each; at least hga_tier_cache_min_slots(..., HGA_TC_GS)
 *              (0 when top_groups >= top_chunks * 64 / group_size: the group
 *              stage then keeps every group and reads no summary) and at most
 *              4096.
 * Replacement: a chunk a call needs and the cache lacks takes the next slot
 * in ring order (per KV head and kind) that the call itself does not use,
 * evicting the chunk there. */
typedef struct {
  void* mem;
  size_t bytes;
  int64_t split;
  int32_t kv_slots;
  int32_t gs_slots;
} hga_tier_cache;

enum { HGA_TC_KV = 0, HGA_TC_GS = 1 };

/* Counters (int64) at the start of the cache memory. Requests are summed
 * over the calls' (query block, KV head) items: a group (or chunk) that
 * several blocks use counts once per block; a miss is a group (or chunk)
 * copied from host memory because the cache did not hold it at the call. */
enum {
  HGA_TC_CALLS = 0,          /* calls made through the cache */
  HGA_TC_KV_REQUESTS = 1,    /* history groups attended */
  HGA_TC_KV_MISSES = 2,      /* groups whose K and V rows were copied */
  HGA_TC_KV_BYTES = 3,       /* K and V bytes copied */
  HGA_TC_KV_EVICTIONS = 4,   /* chunks whose K/V slots were reused */
  HGA_TC_GS_REQUESTS = 5,    /* history chunks whose group summaries the group stage scored */
  HGA_TC_GS_MISSES = 6,      /* chunks whose group summaries were copied */
  HGA_TC_GS_BYTES = 7,       /* group-summary bytes copied */
  HGA_TC_GS_EVICTIONS = 8,   /* chunks whose summary slots were reused */
  HGA_TC_COUNTERS = 16
};

/* Bytes of device memory of a cache of this shape; (size_t)-1 if invalid. */
size_t hga_tier_cache_size(const hga_config* cfg, int64_t split, int32_t kv_slots, int32_t gs_slots);

/* Fewest slots per KV head of one kind (HGA_TC_KV or HGA_TC_GS) a cache must
 * have for calls of n_q queries against a history of seq_len - n_q tokens in
 * host memory: the most distinct history chunks such a call can need per KV
 * head (the sink, local and kept chunks of all its query blocks), at most the
 * history's chunks. -1 if invalid. */
int32_t hga_tier_cache_min_slots(const hga_config* cfg, int64_t seq_len, int64_t n_q, int32_t which);

/* Empty the cache and zero its counters (kernels on `stream`). */
hga_status hga_tier_cache_init(const hga_config* cfg, const hga_tier_cache* cache, void* stream);

/* hga_route_attend with the history (tokens below cache->split) in pinned
 * host memory, through the persistent cache: the chunk stage reads the chunk
 * summaries in HBM; when the group stage must choose, the group summaries of
 * the kept history chunks are brought into the cache's summary slots (those
 * missing are copied) and scored from there; then the K and V rows of every
 * history group a query block attends (its kept groups and its sink and local
 * chunks) are brought into the K/V slots (those missing are copied) and the
 * attention reads them from there. Results equal those of hga_route_attend
 * with everything in HBM, whatever the cache held.
 *   group_sum, k, v   tiered at cache->split (> 0, <= q_start).
 *   cache      initialized by hga_tier_cache_init for this configuration and
 *              split, with enough slots for calls of n_q queries (see
 *              hga_tier_cache_min_slots); else HGA_ERR_UNSUPPORTED.
 *   workspace  device, hga_workspace_size(..., HGA_WS_ATTEND_CACHED) bytes.
 *   copy_stream  NULL, or a stream other than `stream` (default priority):
 *              the copies of missing K/V groups then run on it while the
 *              attention of the query blocks (per KV head) that need none of
 *              them runs on `stream`; the rest are attended once the copies
 *              are done. Work enqueued on `stream` after the call follows all
 *              of it; work on copy_stream is not ordered after the call. The
 *              call creates and destroys two HIP events (no device memory).
 *              Results do not depend on copy_stream.
 * Other arguments as in hga_route_attend. Calls that share a cache must be
 * ordered (one stream, or the caller's synchronization). */
hga_status hga_route_attend_cached(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q,
                                   int64_t seq_len, const float* chunk_sum, const hga_tiered* group_sum,
                                   const hga_tiered* k, const hga_tiered* v, const hga_tier_cache* cache,
                                   int32_t* chunk_idx, int32_t* group_idx, int32_t* n_sel, void* out, float* lse,
                                   void* workspace, size_t ws_bytes, void* stream, void* copy_stream);

/* Forward pass over a whole sequence in segments, in the pages' execution
 * order (section 2.1 with the segment-by-segment processing of section 2.2):
 * for each segment [s0, s0 + segment) in turn (the last may be shorter), the
 * summaries of the chunks it closes are built, then its queries are routed
 * and attended against the committed history and the segment itself
 * (hga_route_attend with q_start = s0 and seq_len = the segment's end). The
 * results equal one hga_build_summaries over the sequence followed by one
 * hga_route_attend over all of its queries.
 *   q, out     device, [Hq][seq_len][d] of cfg->dtype (every position queries; out
 *              float32 for HGA_BF16_F32OUT).
 *   k, v       device, [Hkv][seq_len][d] of cfg->dtype.
 *   chunk_sum, group_sum   device, as written by hga_build_summaries (every
 *              row is written).
 *   chunk_idx, group_idx, n_sel   device, [seq_len/B][Hkv][...] as in hga_route.
 *   lse        device, [Hq][seq_len] float32, or NULL.
 *   segment    a positive multiple of chunk_size, else HGA_ERR_INVALID_ARGUMENT.
 * Everything is on the device (no host tier); no workspace is needed. */
hga_status hga_stream_forward(const hga_config* cfg, const void* q, const void* k, const void* v,
                              int64_t seq_len, int64_t segment, float* chunk_sum, float* group_sum,
                              int32_t* chunk_idx, int32_t* group_idx, int32_t* n_sel,
                              void* out, float* lse, void* stream);

/* Backward of the exact-token attention (section 2.1: the routing is not
 * differentiated, the gather and the attention are; section 2.2: only the
 * active segment is differentiable, the history's K and V are detached).
 * With the token sets of hga_attend fixed by group_idx / n_sel, it returns
 * the gradients of a loss whose gradient with respect to `out` is `dout`:
 *   dq         for every query row of the call;
 *   dk, dv     for the keys and values at the call's own positions
 *              q_start .. q_start + n_q - 1 (the segment): the sums of the
 *              contributions of every query of the call that attends them.
 *              Keys before q_start (the history) receive no gradient.
 * Arguments:
 *   q, k, v, group_idx, n_sel   as hga_attend took them. With a host tier
 *              (split > 0) the history chunks the call attends are copied
 *              once each into an HBM cache in the workspace, as in hga_attend.
 *   out, lse   device, the forward's outputs for these queries (lse required).
 *   dout, dq   device, [Hq][n_q][d] of cfg->dtype.
 *   dk, dv     device, [Hkv][n_q][d] of cfg->dtype: row i is position q_start + i.
 *   workspace  device, at least hga_workspace_size(..., HGA_WS_BACKWARD) bytes
 *              for split 0, HGA_WS_BACKWARD_TIERED with a host tier.
 * bfloat16 and float32 (head dims as for hga_attend); q and dout of 4 GiB or
 * more each return HGA_ERR_UNSUPPORTED. The gradient of each key is summed
 * in one workgroup in a fixed order: repeated calls give identical bits. */
hga_status hga_attend_backward(const hga_config* cfg, const void* q, int64_t q_start, int64_t n_q,
                               int64_t seq_len, const hga_tiered* k, const hga_tiered* v,
                               const int32_t* group_idx, const int32_t* n_sel, const void* out, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                               void* stream);

/* Static description of a status code. */
const char* hga_status_string(hga_status status);

/* Message of the last failed call on this thread ("" if none). */
const char* hga_last_error(void);

/* ABI version of this library (major * 100 + minor). */
int32_t hga_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HGA_H */
