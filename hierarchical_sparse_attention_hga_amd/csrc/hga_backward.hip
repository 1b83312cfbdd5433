// Backward of the HGA exact-token attention ("Long-Context Fine-Tuning with
// Limited VRAM", section 2.1: the selection is not differentiated, the gather
// and the exact-token attention are; section 2.2: only the active segment is
// differentiable, the history's K and V are detached, so gradients are formed
// for the call's queries and for the keys and values at the call's own
// positions).
//
// The token set of every (query block, KV head) item is fixed by the kept
// groups the forward used. For a query row with weights P_t (recomputed
// exactly from the forward's log-sum-exp) and output gradient dO:
//   dP_t = dO . v_t,   D = dO . O,   dS_t = P_t (dP_t - D),
//   dQ = scale sum_t dS_t k_t,   dK_t = scale sum dS_t q,   dV_t = sum P_t dO.
// Two kernels run on the call's stream:
//   bwd_dq_kernel    per item, laid out like the forward kernel: it validates
//                    the kept groups as the forward does (so both see the
//                    same token set), computes D = dO . O of its rows, and
//                    leaves both in the workspace for the second kernel; the
//                    item's K/V tiles stream through LDS; S^T = K Q^T, P^T
//                    from the LSE, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T, all
//                    with v_mfma_f32_32x32x16_bf16 (K read both row-wise and
//                    transposed, hence kv_swizzle);
//   bwd_dkv_kernel   per (KV head, chunk holding positions of the call): the
//                    chunk's K and V stay in registers as MFMA operands while
//                    the query rows of every block that attends the chunk
//                    stream through LDS in 64-row tiles (Q and dO, with their
//                    LSE and D): S = Q K^T, P, dP = dO V^T, dS, then
//                    dV^T += dO^T P and dK^T += Q^T dS. A key's gradient is
//                    summed inside one workgroup, in block order: no atomics,
//                    and the result does not depend on scheduling.
#include "hga_attend_impl.h"

namespace hga {
namespace {

struct BwdArgs {
  const void* q;
  KVSrc kv;           // K/V: device rows [split, L), host rows [0, split)
  TierCache tc;       // host-tier cache of the history chunks the call attends (split > 0)
  const void* out;
  const float* lse;
  const void* dout;
  const int32_t* gidx;
  const int32_t* nsel;
  float* dd;          // workspace [Hq][n_q]: D = dO . O
  unsigned long long* cmask;   // workspace [nb][Hkv][nchunks]: tokens of chunk m0 + c kept as
                               // routed groups of the item (bit t: token 64 (m0 + c) + t)
  void* dq;
  void* dk;
  void* dv;
  int wg_per_item;    // bwd_dq_kernel workgroups per item
  int64_t m0;         // first chunk holding a position of the call
  int nchunks;        // chunks holding positions of the call
  Shape s;
};

// For the dK/dV pass: the kept routed tokens of item (b, h) in each chunk of
// the call's positions, from its ascending run list (first tokens of the
// kept groups, before any host-tier translation).
__device__ void write_chunk_masks(const BwdArgs& A, int b, int h, const Plan& P, const int* runs) {
  const Shape& S = A.s;
  const int64_t it = (int64_t)b * S.hkv + h;
  const unsigned long long gmask = S.g >= 64 ? ~0ull : ((1ull << S.g) - 1ull);
  for (int c = threadIdx.x; c < A.nchunks; c += blockDim.x) {
    const int first = (int)((A.m0 + c) * kChunk);
    int lo = 0, hi = P.nrouted;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (runs[mid] < first) lo = mid + 1; else hi = mid;
    }
    unsigned long long msk = 0ull;
    for (int i = lo; i < P.nrouted && runs[i] < first + kChunk; ++i) msk |= gmask << (runs[i] - first);
    A.cmask[it * A.nchunks + c] = msk;
  }
}

// Whether block b attends chunk m of KV head h: code b (| kDiagBit for the
// chunk's own blocks) or -1, and the chunk's tokens in the block's token set.
constexpr int kDiagBit = 1 << 30;
struct Attending {
  int code;
  unsigned long long msk;
};
__device__ Attending attending(const BwdArgs& A, int h, int64_t m, int b) {
  const Shape& S = A.s;
  Attending x{-1, 0ull};
  if (b < S.nb) {
    const int64_t s = S.q0 + (int64_t)b * S.B, ms = s / kChunk;
    if (m == ms) {
      x = {b | kDiagBit, ~0ull};
    } else if (m < ms) {
      int64_t a, bb;
      fixed_windows(ms, S.sink_chunks, S.local_chunks, &a, &bb);
      if (m < a || m >= bb) {
        x = {b, ~0ull};
      } else {
        x.msk = A.cmask[((int64_t)b * S.hkv + h) * A.nchunks + (m - A.m0)];
        if (x.msk) x.code = b;
      }
    }
  }
  return x;
}

// The attending blocks among one per thread, in thread (block) order, into lb
// and lmask; returns their count.
__device__ int list_compact(Attending x, int* lb, unsigned long long* lmask, int* scan) {
  int tot;
  const int pos = block_scan<false>(x.code >= 0 ? 1 : 0, scan, &tot);
  if (x.code >= 0) {
    lb[pos] = x.code;
    lmask[pos] = x.msk;
  }
  __syncthreads();
  return tot;
}

// The blocks of [b0, b0 + blockDim.x) that attend chunk m of KV head h.
__device__ int list_attending(const BwdArgs& A, int h, int64_t m, int b0, int* lb, unsigned long long* lmask,
                              int* scan) {
  return list_compact(attending(A, h, m, b0 + (int)threadIdx.x), lb, lmask, scan);
}

// ------------------------------------------------------------ dQ
template <int D>
struct BwdQSmem {
  uint16_t k[2][kChunk * D];   // kv_swizzle: read row-wise and transposed
  uint16_t v[2][kChunk * D];   // k_swizzle: read row-wise
  int runs[kMaxRoutedAttn + kMaxFixedTiered];   // kept groups' rows, then (host tier) the fixed chunks'
  int scan[16];
};

// One workgroup slot z of item (b, h): 8 waves of 32 query rows, the item's
// token-set tiles in the forward's order through a 2-stage LDS ring.
template <int D, bool kTiered>
__global__ __launch_bounds__(kAttnThreads) void bwd_dq_kernel(BwdArgs A) {
  __shared__ BwdQSmem<D> sm;
  constexpr int NP = D / 8;
  constexpr int RPI = 64 / NP;
  constexpr int RPW = kChunk / kAttnWaves;
  constexpr int KI = RPW / RPI;   // loads per wave per tensor per tile
  const Shape& S = A.s;
  int b, h, z;
  item_of_block(S, A.wg_per_item, &b, &h, &z);
  const Plan P = make_plan(S, b, h, A.gidx, A.nsel, sm.runs, sm.scan, kMaxRoutedAttn);
  if (z == 0) write_chunk_masks(A, b, h, P, sm.runs);
  if (kTiered) {   // rows of the history come from the host-tier cache
    __syncthreads();   // the masks above read the token runs
    translate_plan(A.kv.split, A.tc.nch, A.tc.nslots, A.tc.slot, h, P, sm.runs, sm.runs + kMaxRoutedAttn);
  }
  const int nt = P.ntiles;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, col = lane & 31;
  const int nrows = S.G * S.B;
  const int rb = z * kAttnWaves + wave;
  const bool active = 32 * rb < nrows;
  const int row = 32 * rb + col;
  const bool live = row < nrows;
  const int lgB = __ffs(S.B) - 1;
  const int head = h * S.G + (row >> lgB);
  const int qi = row & (S.B - 1);
  const int64_t qrow = (int64_t)head * S.qs + (int64_t)b * S.B + qi;

  // queries and output gradients of this lane's column as MFMA B operands
  // (d = 16 ks + 8 hl + e); zero on columns past the item's rows
  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = gf[ks] = bf16x8{};
  float lse2 = 0.0f, dpart = 0.0f;
  if (live) {
    const uint16_t* qp = static_cast<const uint16_t*>(A.q) + qrow * D + 8 * hl;
    const uint16_t* gp = static_cast<const uint16_t*>(A.dout) + qrow * D + 8 * hl;
    const uint16_t* op = static_cast<const uint16_t*>(A.out) + qrow * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
      gf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(gp + 16 * ks));
      const bf16x8 of = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(op + 16 * ks));
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart = fmaf((float)gf[ks][e], (float)of[e], dpart);
    }
    lse2 = A.lse[qrow] * kLog2e;
  }
  // D = dO . O of this lane's row: the two lane halves hold the two halves of d
  const float dterm = active ? pair_sum(dpart) : 0.0f;
  if (live && hl == 0) A.dd[qrow] = dterm;

  const int lg = __ffs(S.g) - 1;
  const int64_t per_head = S.kvs - A.kv.split;   // device rows per head
  const KVRows kv{static_cast<const uint16_t*>(A.kv.k_dev) + (int64_t)h * per_head * D,
                  static_cast<const uint16_t*>(A.kv.v_dev) + (int64_t)h * per_head * D,
                  static_cast<const uint16_t*>(A.tc.k_cache), static_cast<const uint16_t*>(A.tc.v_cache)};
  // run-table entries one tile ahead, as in the forward
  int raw[KI];
  auto run_of = [&](int t, int sl) { return ((t - P.nfix) << (6 - lg)) + (sl >> lg); };
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int rr = wave * RPW + i * RPI + lane / NP;
      const int idx = kTiered && t < P.nfix ? kMaxRoutedAttn + (t & (kMaxFixedTiered - 1))
                                            : run_of(t, rr) & (kMaxRoutedAttn - 1);
      raw[i] = sm.runs[idx];
    }
  };
  const int diag0 = (int)(P.c0 - A.kv.split);   // source row of the last tile's first slot
  const int dlim = P.dlim;
  auto issue = [&](int t) {
    const uint32_t off = (uint32_t)((t & 1) * kChunk * D * 2);
    issue_tile<D, kTiered, 2, 0>(kv, lds_addr(&sm.k[0][0]) + off, lds_addr(&sm.v[0][0]) + off, [&](int i, int sl) -> int {
      if (t < P.nfix) return kTiered ? raw[i] + sl : (int)((t < P.a ? t : P.bb + (t - P.a)) * kChunk) + sl;
      if (t < P.nfix + P.nrt) return run_of(t, sl) < P.nrouted ? raw[i] + (sl & ((1 << lg) - 1)) : 0;
      return diag0 + (sl < dlim ? sl : 0);
    });
  };

  constexpr int RB = D * 2;
  // row reads of K (kv_swizzle) and V (k_swizzle): lane (col, hl) reads piece
  // 2 ks + hl of row col (+ 32 for the second half)
  uint32_t koff[D / 16], voff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    koff[ks] = (uint32_t)(col * RB + (((2 * ks + hl) ^ kv_swizzle<D>(col)) << 4));
    voff[ks] = (uint32_t)(col * RB + (((2 * ks + hl) ^ k_swizzle<D>(col)) << 4));
  }
  // transposing reads of K: lane j of 16-lane group g reads row vrow (lo) and
  // vrow + 8 (hi), columns vcol (+ 32 db); kv_swizzle differs between the two
  // rows, and is unchanged by the row additions (multiples of 16)
  uint32_t tlo[D / 32], thi[D / 32];
  {
    const int vj = lane & 15, vg = lane >> 4;
    const int vcol = 16 * (vg & 1) + 4 * (vj & 3);
    const int vrow = 4 * hl + (vj >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = 32 * db + vcol;
      tlo[db] = (uint32_t)(vrow * RB + (((c >> 3) ^ kv_swizzle<D>(vrow)) << 4) + ((c & 7) << 1));
      thi[db] = (uint32_t)((vrow + 8) * RB + (((c >> 3) ^ kv_swizzle<D>(vrow + 8)) << 4) + ((c & 7) << 1));
    }
  }
  const char* sKb = reinterpret_cast<const char*>(&sm.k[0][0]);
  const char* sVb = reinterpret_cast<const char*>(&sm.v[0][0]);
  const float sl2 = S.scale * kLog2e;
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  fetch(0);
  issue(0);
  fetch(1);
  for (int t = 0; t < nt; ++t) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();   // every wave's loads of tile t landed; tile t - 1 is free
    if (t + 1 < nt) {
      issue(t + 1);
      fetch(t + 2);
    }
    if (!active) continue;
    const uint32_t stage = (uint32_t)((t & 1) * kChunk * RB);
    const char* kt = sKb + stage;
    const char* vt = sVb + stage;
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        kf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kt + koff[ks] + 32 * tb * RB));
        vf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vt + voff[ks] + 32 * tb * RB));
      }
      sacc[tb] = f32x16{};
      pacc[tb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        sacc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], sacc[tb], 0, 0, 0);
        pacc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks], gf[ks], pacc[tb], 0, 0, 0);
      }
    }
    // the forward's masks: slot of accumulator r of half tb is
    // 32 tb + 8 (r >> 2) + 4 hl + (r & 3)
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
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      bf16x8 sf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[tb][r], sl2, -lse2));
        sf[r >> 3][r & 7] = (__bf16)(p * (pacc[tb][r] - dterm));
      }
      // dQ^T += K^T dS^T: the A operand of lane (half hl, column kd) holds K
      // at tokens 32 tb + 16 mm + 4 hl + {0..3, 8..11}
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const char* base = kt + (32 * tb + 16 * mm) * RB;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + tlo[db]));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + thi[db]));
          const s16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), sf[mm], acc[db], 0, 0, 0);
        }
    }
  }
  // dQ: each wave's 32 x D tile goes through LDS (the stages are free once
  // every wave has left the loop) and is stored as whole rows, 64 / (D / 8)
  // rows per instruction; 16-byte pieces XOR-swizzled by row.
  static_assert(kAttnWaves * 32 * RB <= sizeof(sm.k) + sizeof(sm.v), "dQ tiles fit in the stages");
  __syncthreads();
  if (!active) return;
  char* tile = reinterpret_cast<char*>(&sm.k[0][0]) + wave * (32 * RB);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      bf16x4 v4;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) v4[ii] = (__bf16)(acc[db][4 * jj + ii] * S.scale);
      const int piece = 4 * db + jj;
      *reinterpret_cast<u32x2*>(tile + col * RB + ((piece ^ (col & (NP - 1))) << 4) + 8 * hl) =
          __builtin_bit_cast(u32x2, v4);
    }
  constexpr int RPR = 64 / NP;   // rows per store instruction
  uint16_t* dqp = static_cast<uint16_t*>(A.dq);
#pragma unroll
  for (int i = 0; i < 32 / RPR; ++i) {
    const int r = i * RPR + lane / NP, pc = lane % NP;
    const u32x4 val = *reinterpret_cast<const u32x4*>(tile + r * RB + ((pc ^ (r & (NP - 1))) << 4));
    const int R = 32 * rb + r;   // item row
    if (R < nrows) {
      const int64_t orow = (int64_t)(h * S.G + (R >> lgB)) * S.qs + (int64_t)b * S.B + (R & (S.B - 1));
      *reinterpret_cast<u32x4*>(dqp + orow * D + pc * 8) = val;
    }
  }
}

// ------------------------------------------------------------ dK, dV
constexpr int kKVThreads = 256;                // float32 kernel: 64 tokens x 4 lanes
constexpr int kKVListCap = kKVThreads;         // float32 kernel: attending blocks listed per pass
constexpr int kKV16Threads = 512;              // bf16 kernel: 8 waves, two per SIMD
constexpr int kKV16Waves = kKV16Threads / 64;
constexpr int kKV16ListCap = kKV16Threads;     // bf16 kernel: attending blocks listed per pass
constexpr int kKVStages = 3;                   // query tiles in the LDS ring: scored, summed, loading

template <int D>
struct BwdKVSmem {
  uint16_t q[kKVStages][kChunk * D];   // 64-row tiles of Q and dO (kv_swizzle); after
  uint16_t g[kKVStages][kChunk * D];   // the loop, the cross-wave reduction buffer
  u32x4 pds[2][4][2][2][64];           // [tile parity][th, rw][P, dS][mm][lane]: bf16 MFMA operands
  float lse[kKVStages][kChunk];
  float dd[kKVStages][kChunk];
  int lb[kKV16ListCap];        // attending block, | kDiagBit for the chunk's own blocks
  unsigned long long lmask[kKV16ListCap];   // tokens of the chunk in the block's token set
  int scan[16];
};

// One workgroup per (KV head h, chunk m holding positions of the call), eight
// waves in two roles, a pipeline over the query tiles of the attending
// blocks. Wave w: token half th = w & 1 (tokens 32 th .. 32 th + 31 of the
// chunk, this lane's token is column col), row half rw = (w >> 1) & 1 of each
// 64-row tile, role w >> 2. At step u the scoring waves (role 0) form S^T and
// dP^T of tile u for their (th, rw), then P and dS as bf16 MFMA operands in
// LDS; the summing waves (role 1, sharing a SIMD with the scoring wave of the
// same (th, rw)) accumulate dV^T += dO^T P and dK^T += Q^T dS of tile u - 1
// over the whole head dimension. The two row halves are summed at the end.
template <int D>
__global__ __launch_bounds__(kKV16Threads) void bwd_dkv_kernel(BwdArgs A) {
  __shared__ BwdKVSmem<D> sm;
  constexpr int NP = D / 8;
  constexpr int RPI = 64 / NP;
  constexpr int RPW = kChunk / kKV16Waves;   // tile rows each wave loads
  constexpr int KI = RPW / RPI;
  constexpr int RB = D * 2;
  static_assert(KI >= 1 && KI * RPI == RPW, "tile rows split evenly over the waves");
  const Shape& S = A.s;
  const int h = (int)(blockIdx.x / A.nchunks);
  const int64_t m = A.m0 + blockIdx.x % A.nchunks;
  const int64_t t0 = m * kChunk;
  const int64_t lq = S.q0 + S.nq;          // no query of the call attends a token at or past lq
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, col = lane & 31;
  const int th = wave & 1, rw = (wave >> 1) & 1, role = wave >> 2, pair = wave & 3;
  const int tok = 32 * th + col;
  const int64_t tpos = t0 + tok;
  // the first pass's list entry of this thread, read before anything else loads
  const Attending first = attending(A, h, m, tid);

  const uint16_t* qg = static_cast<const uint16_t*>(A.q);
  const uint16_t* gg = static_cast<const uint16_t*>(A.dout);
  const int nrows = S.G * S.B;
  const int ntl = (nrows + kChunk - 1) / kChunk;   // 64-row query tiles per attending block
  // source row (in Q / dO / LSE / D) of row ir of block bq; rows past the
  // item's read its first row (masked). B is a power of two. Rows index
  // arrays of at most 2^32 bytes (checked by the caller), so byte offsets
  // from the arrays' bases are 32-bit and the bases stay in scalar registers.
  const int lgB = __ffs(S.B) - 1;
  auto src_row = [&](int bq, int ir) -> uint32_t {
    const int r = ir < nrows ? ir : 0;
    return (uint32_t)(h * S.G + (r >> lgB)) * (uint32_t)S.qs + (uint32_t)((bq << lgB) + (r & (S.B - 1)));
  };
  // tile u (query tile pt of attending block bq) into stage u mod kKVStages:
  // every wave loads RPW rows of Q and dO; wave 0 loads the rows' LSE, wave 1
  // their D
  auto issue = [&](int u, int bq, int pt) {
    const uint32_t off = (uint32_t)((u % kKVStages) * kChunk * D * 2);
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int row0 = wave * RPW + i * RPI;
      const int rr = row0 + lane / NP;
      const uint32_t bo = src_row(bq, kChunk * pt + rr) * (uint32_t)(D * 2) +
                          ((uint32_t)((lane % NP) ^ kv_swizzle<D>(rr)) << 4);
      lds_dma16_off(qg, bo, lds_addr(&sm.q[0][0]) + off + (uint32_t)(row0 * RB));
      lds_dma16_off(gg, bo, lds_addr(&sm.g[0][0]) + off + (uint32_t)(row0 * RB));
    }
    if (wave < 2) {
      const int st = u % kKVStages;
      lds_dma4_off(wave == 1 ? A.dd : A.lse, src_row(bq, kChunk * pt + lane) * 4u,
                   lds_addr(wave == 1 ? &sm.dd[st][0] : &sm.lse[st][0]));
    }
  };
  auto issue_listed = [&](int u) {
    const int e = u / ntl;
    issue(u, sm.lb[e] & (kDiagBit - 1), u - e * ntl);
  };
  // The first attending block is known before the list: the first block of
  // the call starting in chunk m (blocks lie within one chunk; every earlier
  // block ends before the chunk). Its first tile loads while the list is built.
  const int b_first = (int)(((t0 > S.q0 ? t0 : S.q0) - S.q0) >> lgB);
  // The passes over the attending blocks, kKV16ListCap at a time: step u
  // (0 .. T) waits for tile u, starts tile u + 1 into the stage tile u - 2
  // left, and runs the role's work of the step. Both roles run the same
  // barriers.
  auto passes = [&](auto&& step) {
    for (int b0 = 0; b0 < S.nb; b0 += kKV16ListCap) {
      const bool pre = b0 <= b_first && b_first < b0 + kKV16ListCap;
      if (pre) issue(0, b_first, 0);
      const int tot = list_compact(b0 == 0 ? first : attending(A, h, m, b0 + tid), sm.lb, sm.lmask, sm.scan);
      const int T = tot * ntl;
      if (!pre && T > 0) issue_listed(0);
      for (int u = 0; T > 0 && u <= T; ++u) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this thread's loads of tile u
        __syncthreads();   // every wave's; steps u - 1 done (tile u - 2's stage, the P/dS buffer of u - 2)
        if (u + 1 < T) issue_listed(u + 1);
        step(u, T);
      }
      __syncthreads();   // the list and the stages are reused by the next pass
    }
  };
  // Transposing-read offsets: rows vrow and vrow + 8 (+ 32 rw + 16 mm),
  // columns vcol (+ 32 db).
  auto tr_offsets = [&](uint32_t* tlo, uint32_t* thi) {
    const int vj = lane & 15, vg = lane >> 4;
    const int vcol = 16 * (vg & 1) + 4 * (vj & 3);
    const int vrow = 4 * hl + (vj >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = 32 * db + vcol;
      tlo[db] = (uint32_t)(vrow * RB + (((c >> 3) ^ kv_swizzle<D>(vrow)) << 4) + ((c & 7) << 1));
      thi[db] = (uint32_t)((vrow + 8) * RB + (((c >> 3) ^ kv_swizzle<D>(vrow + 8)) << 4) + ((c & 7) << 1));
    }
  };
  const char* sQb = reinterpret_cast<const char*>(&sm.q[0][0]);
  const char* sGb = reinterpret_cast<const char*>(&sm.g[0][0]);
  // the row-half partial sums (row half 1 of both token halves, a lane's 16
  // accumulators as four lane-contiguous 16-byte pieces), then the output
  // tiles, in the stage ring once both roles have left the passes
  constexpr size_t kRed = sizeof(float) * 2 * 2 * (D / 32) * 16 * 64;
  static_assert(kRed + 2 * kChunk * RB <= sizeof(sm.q) + sizeof(sm.g),
                "the row-half buffer and the output tiles fit in the stage ring");
  float4* red = reinterpret_cast<float4*>(&sm.q[0][0]);
  char* otile = reinterpret_cast<char*>(&sm.q[0][0]) + kRed;

  if (role == 0) {
    // scoring: K and V of this lane's token as MFMA B operands
    // (d = 16 ks + 8 hl + e); zero past lq, where rows may hold anything
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kf[ks] = vf[ks] = bf16x8{};
    if (tpos < lq) {   // the call's positions lie in the device rows (split <= 64 m0)
      const int64_t drow = (int64_t)h * (S.kvs - A.kv.split) + (tpos - A.kv.split);
      const uint16_t* kp = static_cast<const uint16_t*>(A.kv.k_dev) + drow * D + 8 * hl;
      const uint16_t* vp = static_cast<const uint16_t*>(A.kv.v_dev) + drow * D + 8 * hl;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        kf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kp + 16 * ks));
        vf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vp + 16 * ks));
      }
    }
    // row reads of a Q or dO tile: lane (col, hl) reads piece 2 ks + hl of
    // row col (+ 32 rw)
    uint32_t qoff[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qoff[ks] = (uint32_t)(col * RB + (((2 * ks + hl) ^ kv_swizzle<D>(col)) << 4));
    const float sl2 = S.scale * kLog2e;
    passes([&](int u, int T) {
      if (u >= T) return;
      const int e = u / ntl, pt = u - e * ntl;
      const int code_e = sm.lb[e];
      const bool diag = (code_e & kDiagBit) != 0;
      const int64_t sq = S.q0 + (int64_t)(code_e & (kDiagBit - 1)) * S.B;
      const bool tok_ok = ((sm.lmask[e] >> tok) & 1ull) && tpos < lq;
      const int su = u % kKVStages;
      const uint32_t stage = (uint32_t)(su * kChunk * RB);
      const char* qt = sQb + stage + 32 * rw * RB;
      const char* gt = sGb + stage + 32 * rw * RB;
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qt + qoff[ks]));
        const bf16x8 c = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(gt + qoff[ks]));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ks], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c, vf[ks], pacc, 0, 0, 0);
      }
      // accumulator r of this lane: tile row 32 rw + 8 (r >> 2) + 4 hl + (r & 3)
      float lr[16], dr[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 l4 = *reinterpret_cast<const float4*>(&sm.lse[su][32 * rw + 8 * a4 + 4 * hl]);
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.dd[su][32 * rw + 8 * a4 + 4 * hl]);
        lr[4 * a4] = l4.x; lr[4 * a4 + 1] = l4.y; lr[4 * a4 + 2] = l4.z; lr[4 * a4 + 3] = l4.w;
        dr[4 * a4] = d4.x; dr[4 * a4 + 1] = d4.y; dr[4 * a4 + 2] = d4.z; dr[4 * a4 + 3] = d4.w;
      }
      // Accumulator r holds tile row ir = base + cr, cr = 8 (r >> 2) + (r & 3).
      // The pair is visible when the token is in the block's set, the row
      // exists, and on the block's own chunk the row's position is at or past
      // the token's (position sq + (ir & (B - 1)), the token at tpos). A
      // hidden score becomes -inf, so its probability and dS are zero.
      const int base = kChunk * pt + 32 * rw + 4 * hl;
      const int rlim = tok_ok ? nrows - base : 0;
      const int dpos = diag ? (int)(tpos - sq) : INT_MIN;
      bf16x8 pf[2], sf[2];
      // (the accumulators' slots cr reach 27: with rlim >= 28 off the own
      // chunk every pair of the lane is visible, and the wave takes the
      // plain form when that holds in every lane)
      if (__all(!diag && rlim >= 28)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], sl2, -lr[r] * kLog2e));
          pf[r >> 3][r & 7] = (__bf16)p;
          sf[r >> 3][r & 7] = (__bf16)(p * (pacc[r] - dr[r]));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = 8 * (r >> 2) + (r & 3);
          const bool vis = cr < rlim && ((base + cr) & (S.B - 1)) >= dpos;
          const float p = __builtin_amdgcn_exp2f(fmaf(vis ? sacc[r] : -INFINITY, sl2, -lr[r] * kLog2e));
          pf[r >> 3][r & 7] = (__bf16)p;
          sf[r >> 3][r & 7] = (__bf16)(p * (pacc[r] - dr[r]));
        }
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        sm.pds[u & 1][pair][0][mm][lane] = __builtin_bit_cast(u32x4, pf[mm]);
        sm.pds[u & 1][pair][1][mm][lane] = __builtin_bit_cast(u32x4, sf[mm]);
      }
    });
    __syncthreads();   // the summing waves' row-half exchange
    __syncthreads();   // ... and their output tiles
  } else {
    // summing: dK^T and dV^T of the wave's tokens over its row half
    uint32_t tlo[D / 32], thi[D / 32];
    tr_offsets(tlo, thi);
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dk[i] = dv[i] = f32x16{};
    passes([&](int u, int T) {
      if (u == 0) return;
      const int t = u - 1;
      const uint32_t stage = (uint32_t)((t % kKVStages) * kChunk * RB);
      const char* qt = sQb + stage + 32 * rw * RB;
      const char* gt = sGb + stage + 32 * rw * RB;
      // dV^T += dO^T P and dK^T += Q^T dS: A operands of lane (half hl,
      // column kd) hold dO / Q at tile rows 32 rw + 16 mm + 4 hl + {0..3, 8..11}
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const bf16x8 pf = __builtin_bit_cast(bf16x8, sm.pds[t & 1][pair][0][mm][lane]);
        const bf16x8 sf = __builtin_bit_cast(bf16x8, sm.pds[t & 1][pair][1][mm][lane]);
        const char* gb = gt + 16 * mm * RB;
        const char* qb = qt + 16 * mm * RB;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const s16x4 glo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(gb + tlo[db]));
          const s16x4 ghi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(gb + thi[db]));
          const s16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(qb + tlo[db]));
          const s16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(qb + thi[db]));
          const s16x8 wg = {glo[0], glo[1], glo[2], glo[3], ghi[0], ghi[1], ghi[2], ghi[3]};
          const s16x8 wq = {qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]};
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wg), pf, dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wq), sf, dk[db], 0, 0, 0);
        }
      }
    });
    auto slot = [&](int which, int db, int a4) { return (((th * 2 + which) * (D / 32) + db) * 4 + a4) * 64 + lane; };
    if (rw == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          red[slot(0, db, a4)] = float4{dk[db][4 * a4], dk[db][4 * a4 + 1], dk[db][4 * a4 + 2], dk[db][4 * a4 + 3]};
          red[slot(1, db, a4)] = float4{dv[db][4 * a4], dv[db][4 * a4 + 1], dv[db][4 * a4 + 2], dv[db][4 * a4 + 3]};
        }
    }
    __syncthreads();
    // the sums, as bfloat16 rows of the chunk's 64 tokens, into LDS after the
    // reduction buffer (16-byte pieces XOR-swizzled by token)
    if (rw == 0) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const float4 rk = red[slot(0, db, a4)], rv = red[slot(1, db, a4)];
          const float ak[4] = {rk.x, rk.y, rk.z, rk.w}, av[4] = {rv.x, rv.y, rv.z, rv.w};
          bf16x4 k4, v4;
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            k4[ii] = (__bf16)((dk[db][4 * a4 + ii] + ak[ii]) * S.scale);
            v4[ii] = (__bf16)(dv[db][4 * a4 + ii] + av[ii]);
          }
          const int off = tok * RB + (((4 * db + a4) ^ (tok & (NP - 1))) << 4) + 8 * hl;
          *reinterpret_cast<u32x2*>(otile + off) = __builtin_bit_cast(u32x2, k4);
          *reinterpret_cast<u32x2*>(otile + kChunk * RB + off) = __builtin_bit_cast(u32x2, v4);
        }
    }
    __syncthreads();
  }
  // every wave stores whole rows: dK at rows tpos - q0 of dk, dV of dv
  constexpr int RPR = 64 / NP;   // token rows per store instruction
  static_assert((2 * kChunk) % (kKV16Waves * RPR) == 0, "the output rows split evenly over the waves");
#pragma unroll
  for (int i = 0; i < 2 * kChunk / (kKV16Waves * RPR); ++i) {
    const int rowi = (i * kKV16Waves + wave) * RPR + lane / NP;   // 0 .. 127: dK rows, then dV rows
    const int tk = rowi & (kChunk - 1), pc = lane % NP;
    const int64_t p = t0 + tk;
    if (p < S.q0 || p >= lq) continue;
    const u32x4 val = *reinterpret_cast<const u32x4*>(otile + rowi * RB + ((pc ^ (tk & (NP - 1))) << 4));
    uint16_t* dst = static_cast<uint16_t*>(rowi < kChunk ? A.dk : A.dv) + ((int64_t)h * S.nq + (p - S.q0)) * D;
    *reinterpret_cast<u32x4*>(dst + pc * 8) = val;
  }
}

// ------------------------------------------------------------ float32 (SIMT)
// The same two passes for float32 inputs, as the float32 forward computes:
// TPR lanes per query row, each owning D / TPR dimensions, and the token set
// in 32-token LDS sub-tiles.
template <int D, bool kTiered>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(BwdArgs A) {
  constexpr int NT = 256;
  constexpr int TPR = D <= 32 ? 1 : D / 32;   // lanes per row
  constexpr int DPT = D / TPR;                // dims per lane
  constexpr int ROWS = NT / TPR;              // rows per workgroup
  constexpr int HALF = 32;                    // tokens per LDS sub-tile
  __shared__ __align__(16) float sK[HALF * D];
  __shared__ __align__(16) float sV[HALF * D];
  __shared__ int sRuns[kMaxRouted + kMaxFixedTiered];
  __shared__ int sScan[16];
  const Shape& S = A.s;
  int b, h, z;
  item_of_block(S, A.wg_per_item, &b, &h, &z);
  const Plan P = make_plan(S, b, h, A.gidx, A.nsel, sRuns, sScan, kMaxRouted);
  if (z == 0) write_chunk_masks(A, b, h, P, sRuns);
  if (kTiered) {
    __syncthreads();
    translate_plan(A.kv.split, A.tc.nch, A.tc.nslots, A.tc.slot, h, P, sRuns, sRuns + kMaxRouted);
  }
  const int64_t per_head = S.kvs - A.kv.split;
  const float* kdev = static_cast<const float*>(A.kv.k_dev) + (int64_t)h * per_head * D;
  const float* vdev = static_cast<const float*>(A.kv.v_dev) + (int64_t)h * per_head * D;
  const float* kc = static_cast<const float*>(A.tc.k_cache);
  const float* vc = static_cast<const float*>(A.tc.v_cache);
  const int tid = threadIdx.x;
  const int row = z * ROWS + tid / TPR;
  const int part = tid % TPR;
  const bool active = row < S.G * S.B;
  const int head = h * S.G + row / S.B;
  const int qi = row % S.B;
  const int64_t qrow = (int64_t)head * S.qs + (int64_t)b * S.B + qi;

  float q[DPT], g[DPT], dq[DPT];
  float dpart = 0.0f;
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    const int64_t at = qrow * D + part * DPT + e;
    q[e] = active ? static_cast<const float*>(A.q)[at] : 0.0f;
    g[e] = active ? static_cast<const float*>(A.dout)[at] : 0.0f;
    dpart = fmaf(g[e], active ? static_cast<const float*>(A.out)[at] : 0.0f, dpart);
    dq[e] = 0.0f;
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) dpart += __shfl_xor(dpart, off, TPR);
  const float dterm = dpart;
  if (active && part == 0) A.dd[qrow] = dterm;
  const float lse2 = active ? A.lse[qrow] * kLog2e : 0.0f;
  const float sl2 = S.scale * kLog2e;

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
      for (int sl = 0; sl < HALF; ++sl) {
        float sacc = 0.0f, pacc = 0.0f;
#pragma unroll
        for (int e = 0; e < DPT; ++e) {
          sacc = fmaf(q[e], sK[sl * D + part * DPT + e], sacc);
          pacc = fmaf(g[e], sV[sl * D + part * DPT + e], pacc);
        }
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) {
          sacc += __shfl_xor(sacc, off, TPR);
          pacc += __shfl_xor(pacc, off, TPR);
        }
        const int slot = half * HALF + sl;
        const bool vis = slot < lim && !(diag && slot > P.off + qi);
        const float p = vis ? exp2f(fmaf(sacc, sl2, -lse2)) : 0.0f;
        const float ds = p * (pacc - dterm);
#pragma unroll
        for (int e = 0; e < DPT; ++e) dq[e] = fmaf(ds, sK[sl * D + part * DPT + e], dq[e]);
      }
    }
  }
  if (active) {
    float* op = static_cast<float*>(A.dq) + qrow * D + part * DPT;
#pragma unroll
    for (int e = 0; e < DPT; ++e) op[e] = dq[e] * S.scale;
  }
}

// Per (KV head, chunk of the call's positions): 4 lanes per token of the
// chunk, each owning D / 4 dimensions of its key, value and their gradients;
// the query rows of every attending block stream through LDS 32 at a time.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkv_f32_kernel(BwdArgs A) {
  constexpr int TPT = 4;               // lanes per token
  constexpr int DPT = D / TPT;
  constexpr int RT = 32;               // query rows per LDS batch
  static_assert(D % TPT == 0 && kKVThreads == kChunk * TPT, "lane layout");
  __shared__ __align__(16) float sQ[RT * D];
  __shared__ __align__(16) float sG[RT * D];
  __shared__ float sL[RT], sD[RT];
  __shared__ int lb[kKVListCap];
  __shared__ unsigned long long lmask[kKVListCap];
  __shared__ int scan[16];
  const Shape& S = A.s;
  const int h = (int)(blockIdx.x / A.nchunks);
  const int64_t m = A.m0 + blockIdx.x % A.nchunks;
  const int64_t lq = S.q0 + S.nq;
  const int tid = threadIdx.x;
  const int tok = tid / TPT, part = tid % TPT;
  const int64_t tpos = m * kChunk + tok;
  float k[DPT], v[DPT], dk[DPT], dv[DPT];
  const int64_t drow = (int64_t)h * (S.kvs - A.kv.split) + (tpos - A.kv.split);
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    k[e] = tpos < lq ? static_cast<const float*>(A.kv.k_dev)[drow * D + part * DPT + e] : 0.0f;
    v[e] = tpos < lq ? static_cast<const float*>(A.kv.v_dev)[drow * D + part * DPT + e] : 0.0f;
    dk[e] = dv[e] = 0.0f;
  }
  const int nrows = S.G * S.B;
  const float sl2 = S.scale * kLog2e;
  const float* qg = static_cast<const float*>(A.q);
  const float* gg = static_cast<const float*>(A.dout);
  for (int b0 = 0; b0 < S.nb; b0 += kKVListCap) {
    const int tot = list_attending(A, h, m, b0, lb, lmask, scan);
    for (int e = 0; e < tot; ++e) {
      const bool diag = (lb[e] & kDiagBit) != 0;
      const int bq = lb[e] & (kDiagBit - 1);
      const int64_t sq = S.q0 + (int64_t)bq * S.B;
      const bool tok_ok = ((lmask[e] >> tok) & 1ull) && tpos < lq;
      for (int r0 = 0; r0 < nrows; r0 += RT) {
        __syncthreads();
        for (int i = tid; i < RT * (D / 4); i += kKVThreads) {
          const int rr = i / (D / 4), e4 = i % (D / 4);
          const int ir = r0 + rr < nrows ? r0 + rr : 0;
          const int64_t src = (int64_t)(h * S.G + ir / S.B) * S.qs + (int64_t)bq * S.B + ir % S.B;
          *reinterpret_cast<float4*>(&sQ[rr * D + 4 * e4]) = *reinterpret_cast<const float4*>(qg + src * D + 4 * e4);
          *reinterpret_cast<float4*>(&sG[rr * D + 4 * e4]) = *reinterpret_cast<const float4*>(gg + src * D + 4 * e4);
          if (e4 == 0) {
            sL[rr] = A.lse[src] * kLog2e;
            sD[rr] = A.dd[src];
          }
        }
        __syncthreads();
        const int nr = nrows - r0 < RT ? nrows - r0 : RT;
        for (int rr = 0; rr < nr; ++rr) {
          float sacc = 0.0f, pacc = 0.0f;
#pragma unroll
          for (int e2 = 0; e2 < DPT; ++e2) {
            sacc = fmaf(k[e2], sQ[rr * D + part * DPT + e2], sacc);
            pacc = fmaf(v[e2], sG[rr * D + part * DPT + e2], pacc);
          }
#pragma unroll
          for (int off = TPT / 2; off > 0; off >>= 1) {
            sacc += __shfl_xor(sacc, off, TPT);
            pacc += __shfl_xor(pacc, off, TPT);
          }
          const int ir = r0 + rr;
          const bool vis = tok_ok && (!diag || tpos <= sq + ir % S.B);
          const float p = vis ? exp2f(fmaf(sacc, sl2, -sL[rr])) : 0.0f;
          const float ds = vis ? p * (pacc - sD[rr]) : 0.0f;
#pragma unroll
          for (int e2 = 0; e2 < DPT; ++e2) {
            dk[e2] = fmaf(ds, sQ[rr * D + part * DPT + e2], dk[e2]);
            dv[e2] = fmaf(p, sG[rr * D + part * DPT + e2], dv[e2]);
          }
        }
      }
    }
    __syncthreads();   // the list is rebuilt by the next pass
  }
  if (tpos < S.q0 || tpos >= lq) return;
  float* ko = static_cast<float*>(A.dk) + ((int64_t)h * S.nq + (tpos - S.q0)) * D + part * DPT;
  float* vo = static_cast<float*>(A.dv) + ((int64_t)h * S.nq + (tpos - S.q0)) * D + part * DPT;
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    ko[e] = dk[e] * S.scale;
    vo[e] = dv[e];
  }
}

template <int D>
hipError_t launch_backward_f32(const BwdArgs& A, bool tiered, int64_t items, hipStream_t st) {
  const dim3 gq((unsigned)(items * A.wg_per_item)), gkv((unsigned)(A.s.hkv * A.nchunks));
  if (tiered) bwd_dq_f32_kernel<D, true><<<gq, dim3(256), 0, st>>>(A);
  else bwd_dq_f32_kernel<D, false><<<gq, dim3(256), 0, st>>>(A);
  bwd_dkv_f32_kernel<D><<<gkv, dim3(kKVThreads), 0, st>>>(A);
  return hipGetLastError();
}

}  // namespace

// D per query row, then the kept-token masks per (block, KV head, chunk of
// the call's positions); the chunk count is bounded for any q_start.
size_t backward_workspace_bytes(const Shape& s) {
  auto a256 = [](size_t n) { return (n + 255) & ~(size_t)255; };
  const size_t nchunks_max = (size_t)(s.nq + kChunk - 1) / kChunk + 1;
  return a256(4 * (size_t)s.hq * s.nq) + a256(8 * (size_t)s.nb * s.hkv * nchunks_max);
}

hipError_t launch_attend_backward(const Shape& s, const void* q, const KVSrc& kv, const int32_t* group_idx,
                                  const int32_t* n_sel, const void* out, const float* lse, const void* dout,
                                  void* dq, void* dk, void* dv, void* workspace, hipStream_t st) {
  if (s.nq == 0) return hipSuccess;
  auto a256 = [](size_t n) { return (n + 255) & ~(size_t)255; };
  BwdArgs A{};
  A.q = q; A.kv = kv; A.out = out; A.lse = lse; A.dout = dout; A.gidx = group_idx; A.nsel = n_sel;
  A.dq = dq; A.dk = dk; A.dv = dv; A.s = s;
  char* ws = static_cast<char*>(workspace);
  A.dd = reinterpret_cast<float*>(ws);
  A.cmask = reinterpret_cast<unsigned long long*>(ws + a256(4 * (size_t)s.hq * s.nq));
  if (s.dtype == HGA_BF16) {
    const int waves = (s.G * s.B + 31) / 32;
    A.wg_per_item = (waves + kAttnWaves - 1) / kAttnWaves;
  } else {
    const int rows = 256 / (s.d <= 32 ? 1 : s.d / 32);
    A.wg_per_item = (s.G * s.B + rows - 1) / rows;
  }
  A.m0 = s.q0 / kChunk;
  A.nchunks = (int)((s.q0 + s.nq - 1) / kChunk - A.m0 + 1);
  const bool tiered = kv.split > 0;
  if (tiered) {   // the host-tier cache follows the backward's own workspace
    const hipError_t e = prepare_tier_cache(s, kv, group_idx, n_sel, ws + backward_workspace_bytes(s), &A.tc, st);
    if (e != hipSuccess) return e;
  }
  const int64_t items = s.nb * s.hkv;
  if (s.dtype == HGA_F32) {
    switch (s.d) {
      case 4: return launch_backward_f32<4>(A, tiered, items, st);
      case 8: return launch_backward_f32<8>(A, tiered, items, st);
      case 16: return launch_backward_f32<16>(A, tiered, items, st);
      case 32: return launch_backward_f32<32>(A, tiered, items, st);
      case 64: return launch_backward_f32<64>(A, tiered, items, st);
      case 128: return launch_backward_f32<128>(A, tiered, items, st);
      default: return hipErrorInvalidValue;
    }
  }
  const dim3 gq((unsigned)(items * A.wg_per_item)), gkv((unsigned)(s.hkv * A.nchunks));
  if (s.d == 128) {
    if (tiered) bwd_dq_kernel<128, true><<<gq, dim3(kAttnThreads), 0, st>>>(A);
    else bwd_dq_kernel<128, false><<<gq, dim3(kAttnThreads), 0, st>>>(A);
    bwd_dkv_kernel<128><<<gkv, dim3(kKV16Threads), 0, st>>>(A);
  } else if (s.d == 64) {
    if (tiered) bwd_dq_kernel<64, true><<<gq, dim3(kAttnThreads), 0, st>>>(A);
    else bwd_dq_kernel<64, false><<<gq, dim3(kAttnThreads), 0, st>>>(A);
    bwd_dkv_kernel<64><<<gkv, dim3(kKV16Threads), 0, st>>>(A);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hga
