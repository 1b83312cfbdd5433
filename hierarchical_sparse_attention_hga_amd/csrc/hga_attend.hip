// Exact-token routed attention for HGA ("Long-Context Fine-Tuning with Limited
// VRAM", section 2.1, "Exact-token attention": only the exact token K/V of the
// kept groups is attended, summaries never are; the sink and local windows and
// the block's own tokens are always attended, with causal masking).
//
// Token set of one (query block b, KV head h) item, as 64-token tiles:
//   [fixed sink/local chunks, one tile each][kept groups, 64/g per tile,
//    the last tile possibly partial][the block's own chunk from its first
//    token up to the block's last position, causal]. A block smaller than a
//    chunk (one token when decoding) lies inside a chunk that is still open:
//    it has no summary, so the chunk's earlier tokens are kept whole.
// The order of tiles does not change the result (softmax is a sum over the
// set); each tile is one LDS-staged K/V tile of the flash-style loop.
//
// bfloat16 path (attend_bf16_kernel): 512-thread workgroups, each of the 8
// waves owning 32 of the item's G B query rows (G heads x B positions; 256
// rows for G = 4 and B = 64, one workgroup).
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
// Host-tier path (history rows [0, split) in pinned host memory): the chunks
// of the history that any item of the call needs (its fixed windows and the
// chunks of its kept groups) are marked, given slots in an HBM cache in the
// caller's workspace, and copied there once each, so a chunk shared by many
// query blocks crosses the host link once per call (the pages' VRAM cache of
// routed sets shared across query blocks, "Long-Context Fine-Tuning with
// Limited VRAM", section 2.1). The attention kernels then read history rows
// from the cache and the rest from HBM.
#include "hga_attend_impl.h"

namespace hga {
namespace {

// Queries of this lane's column of item (b, h), slot z, as MFMA B operands
// (d = 16 ks + 8 hl + e); zero on the columns past the item's rows.
template <int D>
__device__ inline void load_q_operands(const AttnArgs& A, int b, int h, int z, bf16x8* qf) {
  const Shape& S = A.s;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, col = lane & 31;
  const int row = 32 * (z * kAttnWaves + wave) + col;
  const int lgB = __ffs(S.B) - 1;
  const int head = h * S.G + (row >> lgB);
  const int64_t qrow = (int64_t)b * S.B + (row & (S.B - 1));
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = bf16x8{};
  if (row < S.G * S.B) {
    const uint16_t* qp = static_cast<const uint16_t*>(A.q) + ((int64_t)head * S.qs + qrow) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
  }
}

// Per wave of a split workgroup, the partial state of its 32 query columns:
// the unnormalized O^T accumulators (D / 2 per lane), the running maximum
// (log2 units) and the row sum, each as 64 lane-contiguous floats.
template <int D>
constexpr int kPartFloats = (D / 2 + 2) * 64;

template <int D, int NS>
__device__ __attribute__((always_inline)) void store_output(const AttnArgs& A, int b, int h, int z, AttnSmem<D, NS>& sm,
                                                            const f32x16* o, float m_run, float l_tot,
                                                            int free_stage = -1);

// No routing inside the attention body: the plan is complete.
struct NoRoute {};

// Attention of item (b, h), workgroup slot z, over tiles [ta, te) of the
// token set of plan P (runs in sm.runs). The caller has loaded the queries
// (qpre) and already issued the loads of the range's first pre_tiles tiles
// (at most kAttnStages), the range's tile i into stage i. With part == NULL
// the range is the whole set and the output is stored; otherwise each wave
// leaves its partial state at part + wave * kPartFloats<D>.
//
// With a router (route(window) routes the item and returns its kept groups
// after a barrier; the plan then holds only its fixed windows, te is ignored
// and the range is the whole set): the first fixed tiles are computed while
// the router's group selection runs (one wave selects, the others would
// wait). route calls window.scored() before the barrier that follows the
// group scores (each wave waits for its tile loads there, so the tiles are
// visible after it) and window.selected() right after the selecting wave is
// done; there every wave computes the early tiles from the LDS stages
// without a barrier and without issuing loads. One fixed tile is kept back
// to run while the first tile after routing loads; with three fixed tiles or
// more it is tile 2, which loads into a third stage once the chunks are kept
// (window.chunks_kept()). The order of the tiles is unchanged, so the
// results equal the separate route and attention calls bit for bit.
template <int D, bool kTiered, int NS = kAttnStages, typename Route = NoRoute>
__device__ __attribute__((always_inline)) void attend_bf16_body(const AttnArgs& A, int b, int h, int z,
                                                                Plan P, AttnSmem<D, NS>& sm, int pre_tiles,
                                                                const bf16x8* qpre, int ta, int te,
                                                                float* part, Route route = {}) {
  constexpr int NP = D / 8;
  constexpr int RPI = 64 / NP;
  constexpr int RPW = kChunk / kAttnWaves;
  constexpr int KI = RPW / RPI;               // loads per wave per tensor per tile
  constexpr int kPerTile = 2 * KI;            // K and V
  constexpr int kAhead = kAttnStages - 2;     // most tiles in flight beyond t at the top of iteration t
  static_assert(KI >= 1 && kAttnStages >= 2 && kAttnStages <= 4 && kPerTile * kAhead <= 63, "tile shape");
  constexpr bool kRouted = !std::is_same<Route, NoRoute>::value;
  const Shape& S = A.s;
  int nt = P.ntiles;
  int nl = te - ta;                          // tiles of the range

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;                  // lane half
  const int col = lane & 31;                 // query column of this lane
  // item rows are head-major (row = B * head-local index + position); wave
  // rb owns rows [32 rb, 32 rb + 32), lane column col row 32 rb + col
  const int nrows = S.G * S.B;
  const int rb = z * kAttnWaves + wave;      // 32-row block of the item
  const bool active = 32 * rb < nrows;       // the wave has rows of the item
  const int row = 32 * rb + col;
  const int qi = row & (S.B - 1);            // position within the block

  // queries of this lane's column, loaded by the caller (load_q_operands),
  // or with a router once the router's first loads are issued
  bf16x8 qf[D / 16];
  if constexpr (!kRouted)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = qpre[ks];

  const int lg = __ffs(S.g) - 1;
  const KVRows kv = kv_rows<D, kTiered>(A, h);
  // Source row of slot sl of tile t (see kCacheFlag). Empty slots read row 0
  // of the head's device rows: their probabilities are exactly zero, so any
  // finite row will do. The table entry a row needs (a kept group's first
  // row, or on the host-tier path a fixed chunk's) is read one tile ahead, at
  // an index clamped into the table, and only used when that tile's loads
  // issue (after a barrier): the reads never stall the loop.
  constexpr int KIr = (kChunk / kAttnWaves) / (64 / (D / 8));   // loads per wave per tensor per tile
  int raw[KIr];
  auto run_of = [&](int t, int sl) { return ((t - P.nfix) << (6 - lg)) + (sl >> lg); };
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < KIr; ++i) {
      const int rr = wave * (kChunk / kAttnWaves) + i * (64 / (D / 8)) + lane / (D / 8);
      const int idx = kTiered && t < P.nfix ? kMaxRoutedAttn + (t & (kMaxFixedTiered - 1))
                                            : run_of(t, rr) & (kMaxRoutedAttn - 1);
      raw[i] = sm.runs[idx];
    }
  };
  const int diag0 = (int)(kTiered ? P.c0 - A.kv.split : P.c0);   // source row of the last tile's first slot
  const int dlim = P.dlim;
  auto issue_to = [&](int t, int st) {
    const uint32_t off = (uint32_t)(st * kChunk * D * 2);
    issue_tile<D, kTiered>(kv, lds_addr(&sm.k[0][0]) + off, lds_addr(&sm.v[0][0]) + off, [&](int i, int sl) -> int {
      if (t < P.nfix) return kTiered ? raw[i] + sl : (int)((t < P.a ? t : P.bb + (t - P.a)) * kChunk) + sl;
      if (t < P.nfix + P.nrt) return run_of(t, sl) < P.nrouted ? raw[i] + (sl & ((1 << lg) - 1)) : 0;
      return diag0 + (sl < dlim ? sl : 0);   // empty slots past the block read the chunk's first row
    });
  };
  auto issue = [&](int t) { issue_to(t, (t - ta) % kAttnStages); };

  const float sl2 = S.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};

  // Per-lane byte offsets of the tile-loop LDS reads inside a stage. K: lane
  // (col, hl) reads piece 2 ks + hl of row col (+ 32 for the second half).
  // V (transposing reads): lane j of 16-lane group g points at row
  // vrow = 4 hl + j / 4 (+ 32 tb + 16 mm, + 8 for the upper four tokens) and
  // columns vcol = 16 (g % 2) + 4 (j % 4) (+ 32 db), and receives its column's
  // four tokens. The row additions are multiples of 4 and leave both swizzles
  // unchanged, so they fold into the instructions' constant offsets.
  constexpr int RB = D * 2;                        // bytes per LDS row
  uint32_t koff[D / 16], voff[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    koff[ks] = (uint32_t)(col * RB + (((2 * ks + hl) ^ k_swizzle<D>(col)) << 4));
  {
    const int vj = lane & 15, vg = lane >> 4;
    const int vcol = 16 * (vg & 1) + 4 * (vj & 3);
    const int vrow = 4 * hl + (vj >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = 32 * db + vcol;
      voff[db] = (uint32_t)(vrow * RB + ((((c >> 3) ^ v_swizzle<D>(vrow))) << 4) + ((c & 7) << 1));
    }
  }
  const char* sKb = reinterpret_cast<const char*>(&sm.k[0][0]);
  const char* sVb = reinterpret_cast<const char*>(&sm.v[0][0]);

  // Tiles 0 .. kAttnStages - 2 are in flight before the loop (the caller's
  // pre_tiles among them). At iteration t, once tile t has landed, tile
  // t + kAttnStages - 1 goes into the stage tile t - 1 left; the run-table
  // entries of the next tile to issue are always read one issue ahead.
  // One tile per call; the stage is a compile-time constant (the loop below
  // takes the tiles two at a time), so it folds into the LDS reads' offsets.
  static_assert(kAttnStages == 2, "the tile loop alternates two stages");
  auto compute = [&](int t, auto stage_c) __attribute__((always_inline)) {
    constexpr uint32_t stage = (uint32_t)(decltype(stage_c)::value * kChunk * RB);
    const char* kt = sKb + stage;
    const char* vt = sVb + stage;
    // S^T = K Q^T for both 32-token halves of the tile
    // All K operands of the tile, then the 16 score MFMAs, then the V^T
    // operands of both halves: the scheduling fences keep the compiler from
    // interleaving each read right before its use (which exposed the LDS
    // latency before every MFMA); measured 3% faster at 16K and 64K.
    f32x16 sacc[2];
    {
      bf16x8 kf[2][D / 16];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
          kf[tb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kt + koff[ks] + 32 * tb * RB));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        sacc[tb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
          sacc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[tb][ks], qf[ks], sacc[tb], 0, 0, 0);
      }
    }
    // V^T operands of both halves, read while the score MFMAs run
    bf16x8 vfa[2][D / 32][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const char* vp = vt + voff[db] + (32 * tb + 16 * mm) * RB;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)vp);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vp + 8 * RB));
          const s16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          vfa[tb][db][mm] = __builtin_bit_cast(bf16x8, w);
        }
    __builtin_amdgcn_sched_barrier(0);
    // masking only on the block's own tile and on a partial routed tile;
    // slot of accumulator r of half tb: 32 tb + 8 (r >> 2) + 4 hl + (r & 3).
    // A slot is masked when it reaches the tile's limit or, on the block's
    // own tile, passes the query's position (slot off + qi); thr is that
    // bound shifted by this lane's 4 hl.
    const bool diag = t == nt - 1;
    const int lim = tile_limit(P, S.g, t);
    if (diag || lim < kChunk) {
      const int thr = (diag ? P.off + qi + 1 : lim) - 4 * hl;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * tb + 8 * (r >> 2) + (r & 3) >= thr) sacc[tb][r] = -INFINITY;
    }
    float mx = __builtin_fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(__builtin_fmaxf(mx, sacc[0][r]), sacc[1][r]);
    mx = pair_max(mx) * sl2;
    const bool upd = mx > m_run + kRescaleSlack;
    if (__ballot(upd)) {
      const float m_new = upd ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    const float neg_m = -m_run;   // finite: the first slot of every tile is visible to every row
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      bf16x8 pf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[tb][r], sl2, neg_m));
        l_run += p;
        pf[r >> 3][r & 7] = (__bf16)p;
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfa[tb][db][mm], pf[mm], o[db], 0, 0, 0);
    }
  };

  int i0 = 0;   // tiles of the range already computed
  if constexpr (kRouted) {
    static_assert(!kTiered && NS == 3, "the routing body reads device rows and has a third stage");
    // fixed tiles [0, nearly) run in the group selection's window; the
    // caller issued tiles [0, pre_tiles), one per stage. A fixed tile is
    // kept back to run while the first tile after routing loads: with three
    // fixed tiles or more, tile 2 loads into the third stage once the chunks
    // are kept (its loads then come before the group summaries').
    int nearly = P.nfix - 1 < pre_tiles ? P.nfix - 1 : pre_tiles;
    nearly = nearly > 0 ? nearly : 0;
    const bool third = nearly == 2;
    P.nrouted = 0;
    P.nrt = 0;
    P.ntiles = P.nfix + 1;   // only fixed tiles are computed before routing ends
    nt = P.ntiles;
    auto chunks_kept = [&]() __attribute__((always_inline)) {
      if (third) issue_to(ta + 2, 2);
    };
    auto scored = [nearly]() __attribute__((always_inline)) {
      if (nearly > 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    };
    auto chunks_selected = [nearly]() __attribute__((always_inline)) {
      if (nearly > 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    };
    auto groups_issued = [&]() __attribute__((always_inline)) {
      if (active && nearly > 0) compute(0, std::integral_constant<int, 0>{});
    };
    auto selected = [&]() __attribute__((always_inline)) {
      if (active && nearly > 1) compute(1, std::integral_constant<int, 1>{});
    };
    auto queries_issued = [&]() __attribute__((always_inline)) { load_q_operands<D>(A, b, h, z, qf); };
    const int nsg = route(route::EarlyWindow<decltype(queries_issued), decltype(chunks_kept), decltype(scored),
                                             decltype(selected), decltype(chunks_selected), decltype(groups_issued)>{
        queries_issued, chunks_kept, scored, selected, chunks_selected, groups_issued});
    P.nrouted = nsg;
    P.nrt = (nsg + kChunk / S.g - 1) / (kChunk / S.g);
    P.ntiles = P.nfix + P.nrt + 1;
    nt = P.ntiles;
    nl = nt;
    i0 = nearly;
    if (third) {
      // route returned after a barrier: stage 1 is free; tile 2 has landed
      // (the group scores waited for it) and every wave saw it at the
      // barrier before the group selection
      fetch(ta + 3);
      issue(ta + 3);
      fetch(ta + 4);
      if (active) compute(ta + 2, std::integral_constant<int, 2>{});
      i0 = 3;
      pre_tiles = 4;
    }
  }
  for (int u = i0; u < i0 + kAttnStages - 1 && u < nl; ++u)
    if (u >= pre_tiles) {
      fetch(ta + u);
      issue(ta + u);
    }
  fetch(ta + i0 + kAttnStages - 1);
  auto step = [&](int i, auto stage_c) __attribute__((always_inline)) {
    const int t = ta + i;   // tile i of the range
    // this thread's loads of tile t are done once only newer tiles are pending
    const int ahead = nl - 1 - i < kAhead ? nl - 1 - i : kAhead;
    if (kAhead >= 2 && ahead >= 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kPerTile));
    else if (kAhead >= 1 && ahead >= 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPerTile));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();   // every wave's loads of tile t landed; tile t - 1 is free
    if (i + kAttnStages - 1 < nl) {
      if (i + kAttnStages - 1 >= pre_tiles) issue(t + kAttnStages - 1);
      fetch(t + kAttnStages);
    }
    if (!active) return;
    compute(t, stage_c);
  };
  int i = i0;
  if (i & 1) {
    step(i, std::integral_constant<int, 1>{});
    ++i;
  }
  for (; i < nl; i += 2) {
    step(i, std::integral_constant<int, 0>{});
    if (i + 1 < nl) step(i + 1, std::integral_constant<int, 1>{});
  }
  if (part) {
    if (active) {
      float* pw = part + (size_t)wave * kPartFloats<D>;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) pw[(db * 16 + r) * 64 + lane] = o[db][r];
      pw[(D / 2) * 64 + lane] = m_run;
      pw[(D / 2 + 1) * 64 + lane] = pair_sum(l_run);
    }
    return;
  }
  // the stage the last tile did not use is free: no wave reads it any more
  store_output<D>(A, b, h, z, sm, o, m_run, active ? pair_sum(l_run) : 0.0f, 1 - ((nl - 1) & 1));
}

// Normalize and store the output rows of item (b, h), slot z, from each
// wave's O^T accumulators, running maximum and row sum.
template <int D, int NS>
__device__ __attribute__((always_inline)) void store_output(const AttnArgs& A, int b, int h, int z, AttnSmem<D, NS>& sm,
                                                            const f32x16* o, float m_run, float l_tot,
                                                            int free_stage) {
  constexpr int NP = D / 8;
  constexpr int RB = D * 2;
  const Shape& S = A.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, col = lane & 31;
  const int nrows = S.G * S.B;
  const int rb = z * kAttnWaves + wave;
  const bool active = 32 * rb < nrows;
  const int row = 32 * rb + col;
  const bool live = row < nrows;
  const int lgB = __ffs(S.B) - 1;
  const int head = h * S.G + (row >> lgB);
  const int64_t qrow = (int64_t)b * S.B + (row & (S.B - 1));

  if (S.out_f32) {
    // float32 output: each lane stores its column's four consecutive values
    // of each accumulator quarter as they are (16-byte stores)
    if (active && live) {
      const float inv = 1.0f / l_tot;
      float* op = static_cast<float*>(A.out) + ((int64_t)head * S.qs + qrow) * D + 4 * hl;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<float4*>(op + 32 * db + 8 * jj) =
              float4{o[db][4 * jj] * inv, o[db][4 * jj + 1] * inv, o[db][4 * jj + 2] * inv, o[db][4 * jj + 3] * inv};
      if (A.lse && hl == 0) A.lse[(int64_t)head * S.qs + qrow] = (m_run + __log2f(l_tot)) * kLn2;
    }
    return;
  }
  // Output: each wave writes its normalized 32 x D tile to LDS (the stage
  // ring is free once every wave has left the loop), then stores it back
  // row by row, 64 / (D / 8) whole rows per instruction, so every store
  // writes contiguous rows instead of 16 bytes of each of 32 rows. Pieces of
  // 16 bytes are XOR-swizzled by row in LDS (conflict-free both ways).
  static_assert(kAttnWaves * 32 * RB <= sizeof(sm.k) + sizeof(sm.v), "output tiles fit in the stage ring");
  if (free_stage >= 0) {
    // With one stage known free (after the tile loop), no barrier: each wave
    // stages its tile through its own quarter of that stage's K or V half,
    // one half of the head dimension at a time (half rows of D bytes).
    static_assert(kAttnWaves * 32 * D <= 2 * kChunk * D * 2, "half tiles fit in one stage");
    if (!active) return;
    constexpr int NH = D / 16;   // 16-byte pieces per half row
    const float inv = 1.0f / l_tot;
    char* tile = (wave < kAttnWaves / 2 ? reinterpret_cast<char*>(&sm.k[free_stage][0])
                                        : reinterpret_cast<char*>(&sm.v[free_stage][0])) +
                 (wave % (kAttnWaves / 2)) * (32 * D);
    uint16_t* outp = static_cast<uint16_t*>(A.out);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int dq = 0; dq < D / 64; ++dq)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int db = half * (D / 64) + dq;
          bf16x4 v4;
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) v4[ii] = (__bf16)(o[db][4 * jj + ii] * inv);
          const int piece = 4 * dq + jj;   // of the half row
          *reinterpret_cast<u32x2*>(tile + col * D + ((piece ^ (col & (NH - 1))) << 4) + 8 * hl) =
              __builtin_bit_cast(u32x2, v4);
        }
      constexpr int RPR = 64 / NH;   // half rows per store instruction
#pragma unroll
      for (int i = 0; i < 32 / RPR; ++i) {
        const int r = i * RPR + lane / NH, pc = lane % NH;
        const u32x4 val = *reinterpret_cast<const u32x4*>(tile + r * D + ((pc ^ (r & (NH - 1))) << 4));
        const int R = 32 * rb + r;   // item row
        if (R < nrows) {
          const int64_t orow = (int64_t)(h * S.G + (R >> lgB)) * S.qs + (int64_t)b * S.B + (R & (S.B - 1));
          *reinterpret_cast<u32x4*>(outp + orow * D + half * (D / 2) + pc * 8) = val;
        }
      }
    }
    if (A.lse && hl == 0 && live) A.lse[(int64_t)head * S.qs + qrow] = (m_run + __log2f(l_tot)) * kLn2;
    return;
  }
  __syncthreads();
  if (active) {
    const float inv = 1.0f / l_tot;   // columns past the item's rows are never stored
    char* tile = reinterpret_cast<char*>(&sm.k[0][0]) + wave * (32 * RB);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4 v4;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) v4[ii] = (__bf16)(o[db][4 * jj + ii] * inv);
        const int piece = 4 * db + jj;   // dims 8 piece .. 8 piece + 7; this lane holds half 4 hl
        *reinterpret_cast<u32x2*>(tile + col * RB + ((piece ^ (col & (NP - 1))) << 4) + 8 * hl) =
            __builtin_bit_cast(u32x2, v4);
      }
    constexpr int RPR = 64 / NP;   // rows per store instruction
    uint16_t* outp = static_cast<uint16_t*>(A.out);
#pragma unroll
    for (int i = 0; i < 32 / RPR; ++i) {
      const int r = i * RPR + lane / NP, pc = lane % NP;
      const u32x4 val = *reinterpret_cast<const u32x4*>(tile + r * RB + ((pc ^ (r & (NP - 1))) << 4));
      const int R = 32 * rb + r;   // item row
      if (R < nrows) {
        const int64_t orow = (int64_t)(h * S.G + (R >> lgB)) * S.qs + (int64_t)b * S.B + (R & (S.B - 1));
        *reinterpret_cast<u32x4*>(outp + orow * D + pc * 8) = val;
      }
    }
    if (A.lse && hl == 0 && live) A.lse[(int64_t)head * S.qs + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// bfloat16 attention of items whose kept groups come from group_idx.
template <int D, bool kTiered>
__global__ __launch_bounds__(kAttnThreads) void attend_bf16_kernel(AttnArgs A) {
  __shared__ AttnSmem<D> sm;
  if (kTiered && A.pass == 2 && A.done[blockIdx.x]) return;   // attended by pass 1
  int b, h, z;
  item_of_block(A.s, A.wg_per_item, &b, &h, &z);
  // the queries and, with every row on the device, the first fixed tiles
  // (which need no plan) load while the plan is built
  int pre = 0;
  if (!kTiered) {
    Plan W;
    plan_windows(A.s, b, &W);
    pre = W.nfix < kAttnStages ? W.nfix : kAttnStages;
    for (int t = 0; t < pre; ++t) {
      const int m = t < W.a ? t : (int)(W.bb + (t - W.a));   // chunk of fixed tile t
      const uint32_t off = (uint32_t)(t * kChunk * D * 2);
      issue_tile<D, false>(kv_rows<D, false>(A, h), lds_addr(&sm.k[0][0]) + off, lds_addr(&sm.v[0][0]) + off,
                           [&](int, int sl) -> int { return m * kChunk + sl; });
    }
  }
  bf16x8 qf[D / 16];
  load_q_operands<D>(A, b, h, z, qf);
  const Plan P = make_plan(A.s, b, h, A.gidx, A.nsel, sm.runs, sm.scan, kMaxRoutedAttn);
  if (kTiered && translate_plan(A.kv.split, A.nch, A.nslots, A.slot, h, P, sm.runs, sm.runs + kMaxRoutedAttn,
                                A.s.g, A.pending, A.pass, A.done))
    return;   // pass 2 attends this item
  attend_bf16_body<D, kTiered>(A, b, h, z, P, sm, pre, qf, 0, P.ntiles, nullptr);
}

// Route, then attend, in one workgroup per (item, slot): the router's kept
// groups go straight into the run list (they are ascending and every one is
// usable, so the run list is exactly the one built from the router's output),
// and the loads of the first fixed tiles, which need no routing, are in
// flight while the router runs. Slot 0 writes the router's outputs.
struct FusedArgs {
  route::RouteArgs r;
  AttnArgs a;
};

template <int D>
__global__ __launch_bounds__(kAttnThreads) void route_attend_bf16_kernel(FusedArgs F) {
  static_assert(kAttnThreads == route::kThreads, "one workgroup size for both phases");
  __shared__ AttnSmem<D, 3> sm;
  __shared__ route::RouteSmem rsm;
  const Shape& S = F.a.s;
  int b, h, z;
  item_of_block(S, F.a.wg_per_item, &b, &h, &z);
  Plan P;
  plan_windows(S, b, &P);
  // fixed tiles need no routing: the first two (one per stage) load while
  // the router runs, once its block query is formed (issued earlier, the
  // tiles' bytes delayed the router's first loads)
  const int pre = P.nfix < kAttnStages ? P.nfix : kAttnStages;
  // (captures by value: captured references would keep the locals in
  // scratch memory)
  auto prefetch = [pre, pa = (int)P.a, pbb = (int)P.bb, kvr = kv_rows<D, false>(F.a, h),
                   kl = lds_addr(&sm.k[0][0]), vl = lds_addr(&sm.v[0][0])]() {
    for (int t = 0; t < pre; ++t) {
      const int m = t < pa ? t : pbb + (t - pa);   // chunk of fixed tile t
      const uint32_t off = (uint32_t)(t * kChunk * D * 2);
      issue_tile<D, false>(kvr, kl + off, vl + off, [m](int, int sl) -> int { return m * kChunk + sl; });
    }
  };
  const bool wr = z == 0;
  int32_t* gout = F.r.group_idx + ((int64_t)b * S.hkv + h) * S.kg;
  const int g = S.g;
  int* runs = sm.runs;
  auto emit = [runs, wr, gout, g](int rank, int group) {
    runs[rank] = group * g;
    if (wr) gout[rank] = group;
  };
  auto route = [&](auto window) __attribute__((always_inline)) -> int {
    const int nsg = route::route_item<uint16_t, false, false, decltype(emit), decltype(prefetch), 512,
                                      decltype(window)>(F.r, b, h, rsm, wr, emit, prefetch, window);
    __syncthreads();
    return nsg;
  };
  attend_bf16_body<D, false, 3>(F.a, b, h, z, P, sm, pre, nullptr, 0, 0, nullptr, route);
}

// ------------------------------------------------------------ split items
constexpr int kSplitMax = 32;   // ranges per item at most
// For calls with few items (decoding a few sequences), each item's tile list
// is cut into nsplit contiguous ranges, one workgroup each; every workgroup
// leaves its waves' partial softmax states (relative to their own running
// maxima) in the workspace, and attend_combine_kernel merges them per query
// row: m = max m_s, O = sum O_s 2^(m_s - m), l = sum l_s 2^(m_s - m).
template <int D>
__global__ __launch_bounds__(kAttnThreads) void attend_split_bf16_kernel(AttnArgs A, float* part, int nsplit) {
  __shared__ AttnSmem<D> sm;
  const int nwg = (int)(A.s.nb * A.s.hkv) * A.wg_per_item;
  const int lid = xcd_index(nwg * nsplit);   // the ranges of one item stay on one XCD
  const int wgi = lid / nsplit, sidx = lid % nsplit;
  int b, h, z;
  item_of_index(A.s, A.wg_per_item, wgi, &b, &h, &z);
  bf16x8 qf[D / 16];
  load_q_operands<D>(A, b, h, z, qf);
  const Plan P = make_plan(A.s, b, h, A.gidx, A.nsel, sm.runs, sm.scan, kMaxRoutedAttn);
  const int per = (P.ntiles + nsplit - 1) / nsplit;
  const int ta = sidx * per < P.ntiles ? sidx * per : P.ntiles;
  const int te = ta + per < P.ntiles ? ta + per : P.ntiles;
  attend_bf16_body<D, false>(A, b, h, z, P, sm, 0, qf, ta, te,
                             part + ((size_t)wgi * nsplit + sidx) * kAttnWaves * kPartFloats<D>);
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attend_combine_kernel(AttnArgs A, const float* part, int nsplit) {
  __shared__ AttnSmem<D> sm;
  int b, h, z;
  item_of_block(A.s, A.wg_per_item, &b, &h, &z);
  const int nwg = (int)(A.s.nb * A.s.hkv) * A.wg_per_item;
  const int wgi = xcd_index(nwg);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const bool active = 32 * (z * kAttnWaves + wave) < A.s.G * A.s.B;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.0f;
  if (active) {
    const float* pw = part + (size_t)wgi * nsplit * kAttnWaves * kPartFloats<D> + (size_t)wave * kPartFloats<D>;
    const size_t stride = (size_t)kAttnWaves * kPartFloats<D>;   // from one range to the next
    float mv[kSplitMax];   // the ranges' maxima, all loads in flight at once
#pragma unroll
    for (int sp = 0; sp < kSplitMax; ++sp)
      mv[sp] = sp < nsplit ? __builtin_nontemporal_load(pw + sp * stride + (D / 2) * 64 + lane) : -INFINITY;
#pragma unroll
    for (int sp = 0; sp < kSplitMax; ++sp) m = __builtin_fmaxf(m, mv[sp]);
    // every row sees the first slot of the item's first tile, so m is finite
    for (int sp = 0; sp < nsplit; ++sp) {
      const float* ps = pw + sp * stride;
      float v[D / 2 + 2];   // all of the range's loads in flight at once
#pragma unroll
      for (int j = 0; j < D / 2 + 2; ++j) v[j] = __builtin_nontemporal_load(ps + j * 64 + lane);
      const float ms = v[D / 2];
      const float w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - m);   // ranges with no tile
      l = fmaf(v[D / 2 + 1], w, l);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = fmaf(v[db * 16 + r], w, o[db][r]);
    }
  }
  store_output<D>(A, b, h, z, sm, o, m, l);
}

// ------------------------------------------------------------ float32 SIMT kernel
// 256 threads; TPR lanes per query row, each owning D / TPR dimensions.
template <int D, bool kTiered>
__global__ __launch_bounds__(256) void attend_f32_kernel(AttnArgs A) {
  constexpr int NT = 256;
  constexpr int TPR = D <= 32 ? 1 : D / 32;   // lanes per row
  constexpr int DPT = D / TPR;                // dims per lane
  constexpr int ROWS = NT / TPR;              // rows per workgroup
  constexpr int HALF = 32;                    // tokens per LDS sub-tile
  __shared__ __align__(16) float sK[HALF * D];
  __shared__ __align__(16) float sV[HALF * D];
  __shared__ int sRuns[kMaxRouted + kMaxFixedTiered];
  __shared__ int sScan[16];

  if (kTiered && A.pass == 2 && A.done[blockIdx.x]) return;   // attended by pass 1
  const Shape& S = A.s;
  int b, h, z;
  item_of_block(S, A.wg_per_item, &b, &h, &z);
  const Plan P = make_plan(S, b, h, A.gidx, A.nsel, sRuns, sScan, kMaxRouted);
  if (kTiered && translate_plan(A.kv.split, A.nch, A.nslots, A.slot, h, P, sRuns, sRuns + kMaxRouted, S.g,
                                A.pending, A.pass, A.done))
    return;   // pass 2 attends this item
  const int64_t per_head = kTiered ? S.kvs - A.kv.split : S.kvs;
  const float* kdev = static_cast<const float*>(A.kv.k_dev) + (int64_t)h * per_head * D;
  const float* vdev = static_cast<const float*>(A.kv.v_dev) + (int64_t)h * per_head * D;
  const float* kc = static_cast<const float*>(A.k_cache);
  const float* vc = static_cast<const float*>(A.v_cache);
  const int tid = threadIdx.x;
  const int row = z * ROWS + tid / TPR;       // row of the item: head-local * B + qi
  const int part = tid % TPR;
  const bool active = row < S.G * S.B;
  const int head = h * S.G + row / S.B;
  const int qi = row % S.B;
  const int64_t qrow = (int64_t)b * S.B + qi;

  float q[DPT], o[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    q[e] = active ? static_cast<const float*>(A.q)[((int64_t)head * S.qs + qrow) * D + part * DPT + e] : 0.0f;
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
        const int src = tile_src(P, sRuns, sRuns + kMaxRouted, S.g, kTiered, A.kv.split, t, slot);
        if (src >= 0) {
          kx = *reinterpret_cast<const float4*>(src_ptr(kdev, kc, src, D) + 4 * e4);
          vx = *reinterpret_cast<const float4*>(src_ptr(vdev, vc, src, D) + 4 * e4);
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
        if (slot >= lim || (diag && slot > P.off + qi)) v = -INFINITY;
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
    float* op = static_cast<float*>(A.out) + ((int64_t)head * S.qs + qrow) * D + part * DPT;
#pragma unroll
    for (int e = 0; e < DPT; ++e) op[e] = o[e] * inv;
    if (A.lse && part == 0) A.lse[(int64_t)head * S.qs + qrow] = (m_run + log2f(l_run)) * kLn2;
  }
}

// ------------------------------------------------------------ host-tier cache
__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// Mark the history chunks (below split) item (b, h) needs: its fixed chunks
// and the chunks of its usable kept groups. One workgroup per item; every
// writer stores the same 1.
__global__ __launch_bounds__(256) void mark_kernel(AttnArgs A, int32_t* need) {
  __shared__ int sRuns[kMaxRouted];
  __shared__ int sScan[16];
  const Shape& S = A.s;
  const int h = (int)(blockIdx.x / S.nb), b = (int)(blockIdx.x % S.nb);
  const Plan P = make_plan(S, b, h, A.gidx, A.nsel, sRuns, sScan, kMaxRouted);
  int32_t* nh = need + (int64_t)h * A.nch;
  for (int i = threadIdx.x; i < P.nrouted; i += blockDim.x)
    if (sRuns[i] < A.kv.split) nh[sRuns[i] / kChunk] = 1;
  for (int t = threadIdx.x; t < P.nfix; t += blockDim.x) {
    const int64_t m = t < P.a ? t : P.bb + (t - P.a);
    if (m < A.nch) nh[m] = 1;
  }
}

// Cache slots of the marked chunks: per head (one workgroup each), an
// exclusive scan of the flags in chunk order; -1 for unmarked chunks.
__global__ __launch_bounds__(1024) void slot_kernel(const int32_t* need, int32_t* slot, int nch) {
  __shared__ int sScan[16];
  constexpr int kPer = kMaxCand / 1024;
  const int32_t* nh = need + (int64_t)blockIdx.x * nch;
  int32_t* sh = slot + (int64_t)blockIdx.x * nch;
  const int c0 = threadIdx.x * kPer;
  int f[kPer], cnt = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    f[k] = c0 + k < nch ? nh[c0 + k] : 0;
    cnt += f[k];
  }
  int tot;
  int next = block_scan<false>(cnt, sScan, &tot);
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    if (c0 + k < nch) {
      sh[c0 + k] = f[k] ? next : -1;
      next += f[k];
    }
}

// Copy each marked history chunk of K and V (64 rows) from pinned host memory
// into its cache slot. One workgroup per (chunk, KV head); unmarked chunks
// return at once. Every thread issues all its loads before its stores.
template <typename T>
__global__ __launch_bounds__(256) void copy_kernel(AttnArgs A) {
  const int m = blockIdx.x, h = blockIdx.y;
  const int sl = A.slot[(int64_t)h * A.nch + m];
  if (sl < 0) return;
  const int d = A.s.d;
  const int64_t split = A.kv.split;
  constexpr int EPV = 16 / sizeof(T);             // elements per 16-byte piece
  constexpr int kPer = 8;
  const int pieces = kChunk * d / EPV;
  const T* ks = static_cast<const T*>(A.kv.k_host) + ((int64_t)h * split + (int64_t)m * kChunk) * d;
  const T* vs = static_cast<const T*>(A.kv.v_host) + ((int64_t)h * split + (int64_t)m * kChunk) * d;
  T* kd = static_cast<T*>(const_cast<void*>(A.k_cache)) + ((int64_t)h * A.nch + sl) * kChunk * d;
  T* vd = static_cast<T*>(const_cast<void*>(A.v_cache)) + ((int64_t)h * A.nch + sl) * kChunk * d;
  for (int base = threadIdx.x; base < pieces; base += blockDim.x * kPer) {
    u32x4 kx[kPer], vx[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int p = base + u * blockDim.x;
      if (p < pieces) {
        kx[u] = *reinterpret_cast<const u32x4*>(ks + (int64_t)p * EPV);
        vx[u] = *reinterpret_cast<const u32x4*>(vs + (int64_t)p * EPV);
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int p = base + u * blockDim.x;
      if (p < pieces) {
        *reinterpret_cast<u32x4*>(kd + (int64_t)p * EPV) = kx[u];
        *reinterpret_cast<u32x4*>(vd + (int64_t)p * EPV) = vx[u];
      }
    }
  }
}

template <int D, bool kTiered>
hipError_t launch_bf16(const AttnArgs& a, int64_t items, hipStream_t st) {
  attend_bf16_kernel<D, kTiered><<<dim3((unsigned)(items * a.wg_per_item)), dim3(kAttnThreads), 0, st>>>(a);
  return hipGetLastError();
}

template <int D, bool kTiered>
hipError_t launch_f32(const AttnArgs& a, int64_t items, hipStream_t st) {
  attend_f32_kernel<D, kTiered><<<dim3((unsigned)(items * a.wg_per_item)), dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

template <bool kTiered>
hipError_t dispatch_f32(const AttnArgs& a, int64_t items, hipStream_t st) {
  switch (a.s.d) {
    case 4: return launch_f32<4, kTiered>(a, items, st);
    case 8: return launch_f32<8, kTiered>(a, items, st);
    case 16: return launch_f32<16, kTiered>(a, items, st);
    case 32: return launch_f32<32, kTiered>(a, items, st);
    case 64: return launch_f32<64, kTiered>(a, items, st);
    case 128: return launch_f32<128, kTiered>(a, items, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t tier_cache_bytes(const Shape& s, int64_t split) {
  const int64_t nch = split / kChunk;
  const size_t esz = s.dtype == HGA_BF16 ? 2 : 4;
  const size_t flags = ((2 * (size_t)s.hkv * nch * sizeof(int32_t)) + 255) & ~(size_t)255;
  return flags + 2 * (size_t)s.hkv * nch * kChunk * (size_t)s.d * esz;
}

// Workgroups of the bfloat16 kernels per item: one wave per 32 query rows.
static int bf16_wg_per_item(const Shape& s) {
  const int waves = (s.G * s.B + 31) / 32;
  return (waves + kAttnWaves - 1) / kAttnWaves;
}

// Host-tier cache of one call (workspace: [need][slot] int32 [Hkv][nch], then
// the K and V caches): mark the history chunks the call's items need, give
// them slots, copy them once each.
hipError_t prepare_tier_cache(const Shape& s, const KVSrc& kv, const int32_t* group_idx, const int32_t* n_sel,
                              void* workspace, TierCache* tc, hipStream_t st) {
  const int64_t items = s.nb * s.hkv;
  AttnArgs a{};
  a.kv = kv; a.gidx = group_idx; a.nsel = n_sel; a.s = s;
  const int nch = (int)(kv.split / kChunk);
  const size_t esz = s.dtype == HGA_BF16 ? 2 : 4;
  int32_t* need = static_cast<int32_t*>(workspace);
  int32_t* slot = need + (int64_t)s.hkv * nch;
  char* cache = static_cast<char*>(workspace) + (((2 * (size_t)s.hkv * nch * sizeof(int32_t)) + 255) & ~(size_t)255);
  a.slot = slot;
  a.nch = nch;
  a.nslots = nch;
  a.k_cache = cache;
  a.v_cache = cache + (size_t)s.hkv * nch * kChunk * s.d * esz;
  *tc = TierCache{slot, nch, nch, a.k_cache, a.v_cache};
  const int64_t nflags = (int64_t)s.hkv * nch;
  fill_zero_kernel<<<dim3((unsigned)((nflags + 255) / 256)), dim3(256), 0, st>>>(need, nflags);
  mark_kernel<<<dim3((unsigned)items), dim3(256), 0, st>>>(a, need);
  slot_kernel<<<dim3((unsigned)s.hkv), dim3(1024), 0, st>>>(need, slot, nch);
  if (s.dtype == HGA_BF16)
    copy_kernel<uint16_t><<<dim3((unsigned)nch, (unsigned)s.hkv), dim3(256), 0, st>>>(a);
  else
    copy_kernel<float><<<dim3((unsigned)nch, (unsigned)s.hkv), dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

// Ranges per item of the split attention: with at most kSplitMaxWgs
// workgroups the items alone leave most of the 256 compute units idle, so
// each item's tiles are cut into ranges of about kSplitTiles tiles, up to
// about 256 workgroups in all. 1 = no split. The tile count is bounded by
// the fixed chunks, the kept groups' tiles and the block's own chunk.
constexpr int64_t kSplitMaxWgs = 128;
constexpr int kSplitTiles = 4;
int attend_split_count(const Shape& s) {
  if (s.dtype != HGA_BF16 || (s.d != 128 && s.d != 64)) return 1;
  const int64_t wgs = s.nb * s.hkv * bf16_wg_per_item(s);
  if (wgs == 0 || wgs > kSplitMaxWgs) return 1;
  const int64_t max_tiles = s.sink_chunks + s.local_chunks + ((int64_t)s.kg * s.g + kChunk - 1) / kChunk + 1;
  int64_t n = (max_tiles + kSplitTiles - 1) / kSplitTiles;
  if (n > 256 / wgs) n = 256 / wgs;
  if (n > kSplitMax) n = kSplitMax;
  return n >= 2 ? (int)n : 1;
}

size_t attend_split_bytes(const Shape& s) {
  const int n = attend_split_count(s);
  if (n == 1) return 0;
  const size_t per = (size_t)kAttnWaves * (s.d / 2 + 2) * 64 * sizeof(float);
  return (size_t)(s.nb * s.hkv * bf16_wg_per_item(s)) * n * per;
}

hipError_t launch_attend(const Shape& s, const void* q, const KVSrc& kv, const int32_t* group_idx,
                         const int32_t* n_sel, void* out, float* lse, void* workspace, size_t ws_bytes,
                         hipStream_t st, const TierCache* cached) {
  const int64_t items = s.nb * s.hkv;
  if (items == 0) return hipSuccess;
  AttnArgs a{};
  a.q = q; a.kv = kv; a.gidx = group_idx; a.nsel = n_sel; a.out = out; a.lse = lse; a.s = s;
  const bool tiered = kv.split > 0;
  const int nsplit = tiered ? 1 : attend_split_count(s);
  if (nsplit > 1 && workspace && ws_bytes >= attend_split_bytes(s)) {
    a.wg_per_item = bf16_wg_per_item(s);
    float* part = static_cast<float*>(workspace);
    const unsigned nwg = (unsigned)(items * a.wg_per_item);
    if (s.d == 128) {
      attend_split_bf16_kernel<128><<<dim3(nwg * nsplit), dim3(kAttnThreads), 0, st>>>(a, part, nsplit);
      attend_combine_kernel<128><<<dim3(nwg), dim3(kAttnThreads), 0, st>>>(a, part, nsplit);
    } else {
      attend_split_bf16_kernel<64><<<dim3(nwg * nsplit), dim3(kAttnThreads), 0, st>>>(a, part, nsplit);
      attend_combine_kernel<64><<<dim3(nwg), dim3(kAttnThreads), 0, st>>>(a, part, nsplit);
    }
    return hipGetLastError();
  }
  if (tiered) {
    TierCache tc;
    if (cached) {
      tc = *cached;
    } else {
      const hipError_t e = prepare_tier_cache(s, kv, group_idx, n_sel, workspace, &tc, st);
      if (e != hipSuccess) return e;
    }
    a.slot = tc.slot;
    a.nch = tc.nch;
    a.nslots = tc.nslots;
    a.k_cache = tc.k_cache;
    a.v_cache = tc.v_cache;
    a.pending = tc.pending;
    a.pass = tc.pass;
    a.done = tc.done;
  }
  if (s.dtype == HGA_BF16) {
    a.wg_per_item = bf16_wg_per_item(s);
    if (s.d == 128) return tiered ? launch_bf16<128, true>(a, items, st) : launch_bf16<128, false>(a, items, st);
    if (s.d == 64) return tiered ? launch_bf16<64, true>(a, items, st) : launch_bf16<64, false>(a, items, st);
    return hipErrorInvalidValue;
  }
  const int tpr = s.d <= 32 ? 1 : s.d / 32;
  const int rows = 256 / tpr;
  a.wg_per_item = (s.G * s.B + rows - 1) / rows;
  return tiered ? dispatch_f32<true>(a, items, st) : dispatch_f32<false>(a, items, st);
}

// One kernel when one workgroup holds every query row of an item (G B <= 8
// waves of 32 rows): with more, each of an item's workgroups would route it
// again, and the separate router is cheaper. Also the separate router when a
// block has more than two scoring rounds of chunk candidates: the router
// kernel keeps two rounds in flight, the fused kernel (whose registers hold
// the attention's state) one, and at 64K and beyond the router kernel then
// attention kernel are faster (measured: 128K 200 -> 183 us, 64K decoding
// 83 -> 70 us). Both selections then take at most 512 candidates (two rounds
// of chunk summaries; the kept chunks' groups, bounded as well), which the
// kernel's inlined selection requires.
bool fused_route_attend_supported(const Shape& s, int64_t kv_split) {
  static_assert(2 * route::kRoundRows == 512, "two rounds of chunk candidates: the fused kernel's selection bound");
  return s.dtype == HGA_BF16 && kv_split == 0 && (s.d == 128 || s.d == 64) && bf16_wg_per_item(s) == 1 &&
         route::select512_fits(s);
}

hipError_t launch_route_attend(const Shape& s, const void* q, const float* cs, const float* gs_host,
                               const float* gs_dev, int64_t gs_split, const KVSrc& kv, int32_t* chunk_idx,
                               int32_t* group_idx, int32_t* n_sel, void* out, float* lse, hipStream_t st) {
  const int64_t items = s.nb * s.hkv;
  if (items == 0) return hipSuccess;
  if (!fused_route_attend_supported(s, kv.split)) return hipErrorInvalidValue;
  FusedArgs f{};
  f.r = route::RouteArgs{q, cs, gs_host, gs_dev, gs_split, chunk_idx, group_idx, n_sel, s};
  f.a.q = q; f.a.kv = kv; f.a.out = out; f.a.lse = lse; f.a.s = s;
  f.a.wg_per_item = 1;
  const dim3 grid((unsigned)(items * f.a.wg_per_item)), block(kAttnThreads);
  if (s.d == 128)
    route_attend_bf16_kernel<128><<<grid, block, 0, st>>>(f);
  else
    route_attend_bf16_kernel<64><<<grid, block, 0, st>>>(f);
  return hipGetLastError();
}

}  // namespace hga
