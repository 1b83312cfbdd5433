/*
 * hga_oracle.c -- plain, slow CPU oracle for the HGA routed-attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * does. It shares no code, header or constant with the HIP kernels.
 *
 * Source of the method: "Long-Context Fine-Tuning with Limited VRAM",
 * section 2.1 "Exact-token hierarchical routing" (chunk selection, group
 * selection, exact-token attention) and the base HGA abstract (compact
 * RoPE-aware chunk summaries, sink and local windows, ~3% routed budget).
 * Steps are taken in that order, in float64 unless stated:
 *
 *   1. summaries  GS[h][j] = mean of keys 8j..8j+7, CS[h][m] = mean of keys
 *                 64m..64m+63 (the pages leave the "RoPE-aware" operator open;
 *                 the reading taken is the mean of the post-RoPE keys).
 *   2. block query  qbar = mean of the block's queries over the B positions
 *                 and the G query heads sharing the KV head (reading: routing
 *                 is per KV head and scores with the block-mean query).
 *   3. fixed windows  sink = chunks holding the first S tokens, local = the
 *                 W tokens right before the block; both only if closed.
 *   4. chunk stage  candidates = closed chunks before the block that are not
 *                 fixed; keep the top kc by (score desc, chunk index asc).
 *   5. group stage  open the kept chunks into groups; keep the top kg by
 *                 (score desc, group index asc).
 *   6. token set  fixed chunks + kept groups + the block's own chunk up to
 *                 the block's last position (reading: the open chunk has no
 *                 summary, so its earlier tokens are kept whole; for a block
 *                 of one whole chunk this is the block's own tokens).
 *   7. attention  exact causal softmax attention over the token set.
 *   7'. backward  gradients of step 7 with respect to Q, K and V, the
 *                 routing held fixed (see orc_attend_backward).
 *
 * Steps 4 and 5 are decisions. Summaries are stored in float32 (the mean
 * rounded to nearest); a decision score is the float64 dot of the float64
 * block query with that float32 summary, as the HIP router computes it. The
 * gap between the k-th and (k+1)-th scores is reported with a bound on how far
 * any evaluation order can move a score, so that a test can tell a certified
 * boundary (one correct answer) from one where several answers are correct.
 *
 * Parity pins: every function here is pinned by the CPU tests (closed forms,
 * brute-force top-k, dense-attention equivalence, invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t hq, hkv, d;
  int32_t chunk, group, q_block;
  int32_t top_chunks, top_groups;
  int32_t sink, local;
  int64_t seq_len, n_q;
  double scale;
} orc_cfg;

/* Layout of the diagnostics row written per routed item. */
enum {
  DG_NCAND_C = 0, DG_GAP_C, DG_EPS_C, DG_UNROUNDED_EQ_C,
  DG_NCAND_G, DG_GAP_G, DG_EPS_G, DG_UNROUNDED_EQ_G,
  DG_NUM
};

static int64_t q_start(const orc_cfg* c) { return c->seq_len - c->n_q; }

/* ------------------------------------------------------------------ step 1 */
static int summaries(const orc_cfg* c, const double* k, double* gs, double* cs, int absval) {
  const int64_t L = c->seq_len, d = c->d;
  const int64_t ng = L / c->group, nc = L / c->chunk;
#pragma omp parallel for schedule(static, 1)
  for (int64_t h = 0; h < c->hkv; ++h) {
    for (int64_t j = 0; j < ng; ++j)
      for (int64_t e = 0; e < d; ++e) {
        double s = 0.0;
        for (int64_t t = j * c->group; t < (j + 1) * c->group; ++t)
          s += absval ? fabs(k[(h * L + t) * d + e]) : k[(h * L + t) * d + e];
        gs[(h * ng + j) * d + e] = s / c->group;
      }
    for (int64_t m = 0; m < nc; ++m)
      for (int64_t e = 0; e < d; ++e) {
        double s = 0.0;
        for (int64_t t = m * c->chunk; t < (m + 1) * c->chunk; ++t)
          s += absval ? fabs(k[(h * L + t) * d + e]) : k[(h * L + t) * d + e];
        cs[(h * nc + m) * d + e] = s / c->chunk;
      }
  }
  return 0;
}

int orc_summaries(const orc_cfg* c, const double* k, double* gs, double* cs) {
  return summaries(c, k, gs, cs, 0);
}

/* The same means taken over |K|: used only for the float32 error bound. */
int orc_abs_summaries(const orc_cfg* c, const double* k, double* ga, double* ca) {
  return summaries(c, k, ga, ca, 1);
}

/* ------------------------------------------------------------------ step 3 */
/* Is chunk m (closed, m < ms) a fixed sink or local chunk for a block whose
 * first token lies in chunk ms? */
static int is_fixed(const orc_cfg* c, int64_t m, int64_t ms) {
  if (m < 0 || m >= ms) return 0;
  if (m < c->sink / c->chunk) return 1;
  if (m >= ms - c->local / c->chunk) return 1;
  return 0;
}

/* ------------------------------------------------------------------ steps 4, 5 */
typedef struct { double dec, exact; int32_t idx; } cand_t;

/* decision order: score descending, then index ascending */
static int cmp_dec(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a; const cand_t* y = (const cand_t*)b;
  if (x->dec > y->dec) return -1;
  if (x->dec < y->dec) return 1;
  return (x->idx > y->idx) - (x->idx < y->idx);
}
/* the same order on scores taken with unrounded (float64) summaries */
static int cmp_exact(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a; const cand_t* y = (const cand_t*)b;
  if (x->exact > y->exact) return -1;
  if (x->exact < y->exact) return 1;
  return (x->idx > y->idx) - (x->idx < y->idx);
}
static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

static double gamma_n(double n, double u) { return n * u / (1.0 - n * u); }

/* Decision score of one summary row (float64 block query qb against the
 * summary rounded to float32, its storage precision), the same score with the
 * unrounded summary, and an update of the stage's error bound eps: a bound on
 * how far any float64 evaluation order of the block mean, of the summary mean
 * before its float32 rounding, and of the dot can move the decision score.
 * The float32 rounding of a summary can land one float32 ulp apart when its
 * float64 sum is inexact, hence the 2u32 term. */
static void score(const orc_cfg* c, const double* qb, const double* qabs, const double* srow,
                  const double* sabs, int N, int n_tok, double* dec, double* exact, double* eps) {
  const double u64 = ldexp(1.0, -53), u32 = ldexp(1.0, -24);
  double sd = 0.0, se = 0.0, bound = 0.0;
  for (int64_t e = 0; e < c->d; ++e) {
    const double s32 = (double)(float)srow[e];
    sd += qb[e] * s32;
    se += qb[e] * srow[e];
    bound += gamma_n(N + 1, u64) * qabs[e] * fabs(s32)
           + (2.0 * u32 + gamma_n(n_tok + 1, u64)) * fabs(qb[e]) * (fabs(s32) + sabs[e])
           + gamma_n(c->d + 1, u64) * fabs(qb[e]) * fabs(s32);
  }
  *dec = sd;
  *exact = se;
  if (bound > *eps) *eps = bound;
}

/* Keep the first k of cand[0..n) in decision order; write their indices
 * ascending into sel. Reports the gap between the k-th and (k+1)-th decision
 * scores and whether the unrounded-summary scores keep the same set.
 * Returns the number kept. */
static int select_topk(cand_t* cand, int n, int k, int32_t* sel, double* gap, int* same_unrounded) {
  const int kk = n < k ? n : k;
  *gap = INFINITY;
  *same_unrounded = 1;
  if (kk > 0 && kk < n) {
    int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)kk);
    qsort(cand, (size_t)n, sizeof(cand_t), cmp_exact);
    for (int i = 0; i < kk; ++i) a[i] = cand[i].idx;
    qsort(a, (size_t)kk, sizeof(int32_t), cmp_i32);
    qsort(cand, (size_t)n, sizeof(cand_t), cmp_dec);
    *gap = cand[kk - 1].dec - cand[kk].dec;
    for (int i = 0; i < kk; ++i) sel[i] = cand[i].idx;
    qsort(sel, (size_t)kk, sizeof(int32_t), cmp_i32);
    for (int i = 0; i < kk; ++i) if (a[i] != sel[i]) *same_unrounded = 0;
    free(a);
  } else {
    for (int i = 0; i < kk; ++i) sel[i] = cand[i].idx;
    qsort(sel, (size_t)kk, sizeof(int32_t), cmp_i32);
  }
  return kk;
}

/* Step 2: the block query of (block b, KV head h): the float64 mean of the
 * block's B queries over the G query heads of the KV head, and the mean |Q|
 * per dimension for the error bound. Both arrays hold d values. */
static void block_query(const orc_cfg* c, const double* q, int b, int h, double* qb, double* qabs) {
  const int64_t d = c->d, q0 = q_start(c);
  const int G = c->hq / c->hkv, B = c->q_block, N = G * B;
  const int64_t s = q0 + (int64_t)b * B;
  for (int64_t e = 0; e < d; ++e) { qb[e] = 0.0; qabs[e] = 0.0; }
  for (int r = 0; r < G; ++r)
    for (int i = 0; i < B; ++i) {
      const double* row = q + ((int64_t)(h * G + r) * c->n_q + (s - q0) + i) * d;
      for (int64_t e = 0; e < d; ++e) { qb[e] += row[e]; qabs[e] += fabs(row[e]); }
    }
  for (int64_t e = 0; e < d; ++e) { qb[e] /= N; qabs[e] /= N; }
}

/* Route one (block b, KV head h) item. */
static void route_item(const orc_cfg* c, const double* q, const double* ga, const double* ca,
                       const double* gs, const double* cs, int b, int h, int32_t* chunk_idx, int32_t* group_idx,
                       int32_t* n_sel, double* diag) {
  const int64_t L = c->seq_len, d = c->d, q0 = q_start(c);
  const int G = c->hq / c->hkv, B = c->q_block, N = G * B;
  const int64_t s = q0 + (int64_t)b * B, ms = s / c->chunk;
  const int64_t ng = L / c->group, nc = L / c->chunk, gpc = c->chunk / c->group;

  double* qb = (double*)calloc((size_t)d, sizeof(double));
  double* qabs = (double*)calloc((size_t)d, sizeof(double));
  block_query(c, q, b, h, qb, qabs);

  /* steps 3, 4: chunk candidates and chunk stage */
  cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)(ms > 0 ? ms : 1));
  int n = 0;
  double eps_c = 0.0;
  for (int64_t m = 0; m < ms; ++m) {
    if (is_fixed(c, m, ms)) continue;
    score(c, qb, qabs, cs + ((int64_t)h * nc + m) * d, ca + ((int64_t)h * nc + m) * d, N, c->chunk,
          &cand[n].dec, &cand[n].exact, &eps_c);
    cand[n].idx = (int32_t)m;
    ++n;
  }
  int32_t* selc = (int32_t*)malloc(sizeof(int32_t) * (size_t)(c->top_chunks > 0 ? c->top_chunks : 1));
  double gap_c; int eq_c;
  int nsc = select_topk(cand, n, c->top_chunks, selc, &gap_c, &eq_c);
  diag[DG_NCAND_C] = n; diag[DG_GAP_C] = gap_c; diag[DG_EPS_C] = eps_c; diag[DG_UNROUNDED_EQ_C] = eq_c;
  for (int i = 0; i < c->top_chunks; ++i) chunk_idx[i] = i < nsc ? selc[i] : -1;
  free(cand);

  /* step 5: group stage over the groups of the kept chunks */
  int ngc = (int)(nsc * gpc);
  cand_t* gc = (cand_t*)malloc(sizeof(cand_t) * (size_t)(ngc > 0 ? ngc : 1));
  double eps_g = 0.0;
  n = 0;
  for (int i = 0; i < nsc; ++i)
    for (int64_t u = 0; u < gpc; ++u) {
      const int64_t j = (int64_t)selc[i] * gpc + u;
      score(c, qb, qabs, gs + ((int64_t)h * ng + j) * d, ga + ((int64_t)h * ng + j) * d, N, c->group,
            &gc[n].dec, &gc[n].exact, &eps_g);
      gc[n].idx = (int32_t)j;
      ++n;
    }
  int32_t* selg = (int32_t*)malloc(sizeof(int32_t) * (size_t)(c->top_groups > 0 ? c->top_groups : 1));
  double gap_g; int eq_g;
  int nsg = select_topk(gc, n, c->top_groups, selg, &gap_g, &eq_g);
  diag[DG_NCAND_G] = n; diag[DG_GAP_G] = gap_g; diag[DG_EPS_G] = eps_g; diag[DG_UNROUNDED_EQ_G] = eq_g;
  for (int i = 0; i < c->top_groups; ++i) group_idx[i] = i < nsg ? selg[i] : -1;
  n_sel[0] = nsc; n_sel[1] = nsg;
  free(gc); free(selc); free(selg); free(qb); free(qabs);
}

/* Decision scores of every candidate of both stages of (block b, KV head h),
 * for checking a selection at a boundary that is not certified (where
 * several selections are correct): chunk_sc[m] for every closed chunk m
 * before the block that is not fixed (NaN for every other chunk), group_sc[j]
 * for every group j of those chunks (NaN otherwise), and the error bounds of
 * the two stages over all of these scores (eps[0]: chunks, eps[1]: groups).
 * chunk_sc holds seq_len / chunk values, group_sc seq_len / group. */
static void score_item(const orc_cfg* c, const double* q, const double* ga, const double* ca, const double* gs,
                       const double* cs, int b, int h, double* chunk_sc, double* group_sc, double* eps) {
  const int64_t L = c->seq_len, d = c->d, q0 = q_start(c);
  const int G = c->hq / c->hkv, B = c->q_block, N = G * B;
  const int64_t s = q0 + (int64_t)b * B, ms = s / c->chunk;
  const int64_t ng = L / c->group, nc = L / c->chunk, gpc = c->chunk / c->group;
  double* qb = (double*)calloc((size_t)d, sizeof(double));
  double* qabs = (double*)calloc((size_t)d, sizeof(double));
  block_query(c, q, b, h, qb, qabs);
  for (int64_t m = 0; m < nc; ++m) chunk_sc[m] = NAN;
  for (int64_t j = 0; j < ng; ++j) group_sc[j] = NAN;
  eps[0] = eps[1] = 0.0;
  for (int64_t m = 0; m < ms; ++m) {
    if (is_fixed(c, m, ms)) continue;
    double exact;
    score(c, qb, qabs, cs + ((int64_t)h * nc + m) * d, ca + ((int64_t)h * nc + m) * d, N, c->chunk,
          &chunk_sc[m], &exact, &eps[0]);
    for (int64_t u = 0; u < gpc; ++u) {
      const int64_t j = m * gpc + u;
      score(c, qb, qabs, gs + ((int64_t)h * ng + j) * d, ga + ((int64_t)h * ng + j) * d, N, c->group,
            &group_sc[j], &exact, &eps[1]);
    }
  }
  free(qb); free(qabs);
}

int orc_route_scores(const orc_cfg* c, const double* q, const double* ga, const double* ca,
                     const double* gs, const double* cs, int n_items, const int32_t* items,
                     double* chunk_sc, double* group_sc, double* eps) {
  const int64_t nc = c->seq_len / c->chunk, ng = c->seq_len / c->group;
#pragma omp parallel for schedule(dynamic, 1)
  for (int it = 0; it < n_items; ++it)
    score_item(c, q, ga, ca, gs, cs, items[2 * it], items[2 * it + 1], chunk_sc + (int64_t)it * nc,
               group_sc + (int64_t)it * ng, eps + 2 * (int64_t)it);
  return 0;
}

int orc_route(const orc_cfg* c, const double* q, const double* ga, const double* ca,
              const double* gs, const double* cs,
              int n_items, const int32_t* items, int32_t* chunk_idx, int32_t* group_idx,
              int32_t* n_sel, double* diag) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int it = 0; it < n_items; ++it)
    route_item(c, q, ga, ca, gs, cs, items[2 * it], items[2 * it + 1],
               chunk_idx + (int64_t)it * c->top_chunks, group_idx + (int64_t)it * c->top_groups,
               n_sel + 2 * (int64_t)it, diag + (int64_t)it * DG_NUM);
  return 0;
}

/* ------------------------------------------------------------------ step 6 */
/* Mark the token set of block b in mask[0 .. s+B). Entries of group_idx that
 * are out of range, inside a fixed chunk or not closed are ignored, so the
 * result is always a set. The block's own chunk ms is still open (it has no
 * summary, so it is neither a candidate nor a fixed window): its tokens from
 * the chunk start up to the block's last position are kept whole. For a block
 * that is a whole chunk these are exactly the block's own tokens; for a
 * smaller block (one token when decoding) they add the open chunk's earlier
 * tokens. */
static void token_mask(const orc_cfg* c, int b, const int32_t* group_idx, int n_groups, unsigned char* mask) {
  const int64_t s = q_start(c) + (int64_t)b * c->q_block, ms = s / c->chunk;
  memset(mask, 0, (size_t)(s + c->q_block));
  for (int64_t m = 0; m < ms; ++m)
    if (is_fixed(c, m, ms))
      for (int64_t t = m * c->chunk; t < (m + 1) * c->chunk; ++t) mask[t] = 1;
  for (int i = 0; i < n_groups; ++i) {
    int64_t j = group_idx[i];
    if (j < 0 || (j + 1) * c->group > s) continue;
    if (is_fixed(c, j * c->group / c->chunk, ms)) continue;
    for (int64_t t = j * c->group; t < (j + 1) * c->group; ++t) mask[t] = 1;
  }
  for (int64_t t = ms * c->chunk; t < s + c->q_block; ++t) mask[t] = 1;
}

int64_t orc_token_set(const orc_cfg* c, int b, const int32_t* group_idx, int n_groups,
                      int32_t* tokens, int64_t max_tokens) {
  const int64_t end = q_start(c) + (int64_t)(b + 1) * c->q_block;
  unsigned char* mask = (unsigned char*)malloc((size_t)end);
  token_mask(c, b, group_idx, n_groups, mask);
  int64_t n = 0;
  for (int64_t t = 0; t < end; ++t)
    if (mask[t]) { if (n < max_tokens) tokens[n] = (int32_t)t; ++n; }
  free(mask);
  return n;
}

/* ------------------------------------------------------------------ step 7 */
static void attend_item(const orc_cfg* c, const double* q, const double* k, const double* v,
                        int b, int h, const int32_t* group_idx, int n_groups, double* out, double* lse) {
  const int64_t L = c->seq_len, d = c->d, q0 = q_start(c);
  const int G = c->hq / c->hkv, B = c->q_block;
  const int64_t s = q0 + (int64_t)b * B;
  int32_t* T = (int32_t*)malloc(sizeof(int32_t) * (size_t)(s + B));
  int64_t nt = orc_token_set(c, b, group_idx, n_groups, T, s + B);
  double* z = (double*)malloc(sizeof(double) * (size_t)nt);
  for (int r = 0; r < G; ++r)
    for (int i = 0; i < B; ++i) {
      const int64_t pos = s + i;
      const double* qi = q + ((int64_t)(h * G + r) * c->n_q + (pos - q0)) * d;
      double mx = -INFINITY;
      int64_t nv = 0;
      for (int64_t a = 0; a < nt && T[a] <= pos; ++a) {
        const double* kt = k + ((int64_t)h * L + T[a]) * d;
        double dot = 0.0;
        for (int64_t e = 0; e < d; ++e) dot += qi[e] * kt[e];
        z[a] = c->scale * dot;
        if (z[a] > mx) mx = z[a];
        nv = a + 1;
      }
      double den = 0.0;
      for (int64_t a = 0; a < nv; ++a) den += exp(z[a] - mx);
      double* o = out + ((int64_t)r * B + i) * d;
      for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
      for (int64_t a = 0; a < nv; ++a) {
        const double w = exp(z[a] - mx) / den;
        const double* vt = v + ((int64_t)h * L + T[a]) * d;
        for (int64_t e = 0; e < d; ++e) o[e] += w * vt[e];
      }
      lse[(int64_t)r * B + i] = mx + log(den);
    }
  free(z); free(T);
}

/* out [n_items][G][B][d], lse [n_items][G][B] */
int orc_attend(const orc_cfg* c, const double* q, const double* k, const double* v, int n_items,
               const int32_t* items, const int32_t* group_idx, const int32_t* n_groups,
               double* out, double* lse) {
  const int G = c->hq / c->hkv, B = c->q_block;
#pragma omp parallel for schedule(dynamic, 1)
  for (int it = 0; it < n_items; ++it)
    attend_item(c, q, k, v, items[2 * it], items[2 * it + 1],
                group_idx + (int64_t)it * c->top_groups, n_groups[it],
                out + (int64_t)it * G * B * c->d, lse + (int64_t)it * G * B);
  return 0;
}

/* ------------------------------------------------------------------ backward of step 7 */
/* Gradients of step 7 with the routing held fixed: the pages keep routing out
 * of the gradient (no-grad selection) while the gather and the exact-token
 * attention stay differentiable ("Long-Context Fine-Tuning with Limited
 * VRAM", section 2.1). For one query row with token set T (causal, t <= p),
 * scores z_t = scale q . k_t and weights P_t = softmax(z)_t, and the output
 * gradient g = dO:
 *   dP_t = g . v_t,   D = sum_t P_t dP_t,   dS_t = P_t (dP_t - D),
 *   dq  = scale sum_t dS_t k_t,
 *   dk_t += scale dS_t q,   dv_t += P_t g.
 * Keys and values collect the contributions of every row of every block that
 * attends them. Items of different KV heads touch disjoint rows, so heads run
 * in parallel and the blocks of one head in order.
 *
 * For tolerances the same sums are also taken over magnitudes (when the abs
 * arrays are given), with |dS_t| replaced by P_t (|dP_t| + |D| + W), where
 * W = sum_e |g_e| |o_e| over the exact output o:
 *   dq_abs = scale sum_t P_t (|dP_t| + |D| + W) |k_t|,
 *   dk_abs_t += scale P_t (|dP_t| + |D| + W) |q|,   dv_abs_t += P_t |g|.
 * A relative perturbation e of each dS_t term, of D by e W, or of each P_t
 * moves a gradient element by at most e times its companion. */
static void backward_item(const orc_cfg* c, const double* q, const double* k, const double* v,
                          const double* dout, int b, int h, const int32_t* group_idx, int n_groups,
                          double* dq, double* dk, double* dv, double* dq_abs, double* dk_abs, double* dv_abs) {
  const int64_t L = c->seq_len, d = c->d, q0 = q_start(c);
  const int G = c->hq / c->hkv, B = c->q_block;
  const int64_t s = q0 + (int64_t)b * B;
  int32_t* T = (int32_t*)malloc(sizeof(int32_t) * (size_t)(s + B));
  const int64_t nt = orc_token_set(c, b, group_idx, n_groups, T, s + B);
  double* z = (double*)malloc(sizeof(double) * (size_t)nt);
  double* dp = (double*)malloc(sizeof(double) * (size_t)nt);
  for (int r = 0; r < G; ++r)
    for (int i = 0; i < B; ++i) {
      const int64_t pos = s + i, row = (int64_t)(h * G + r) * c->n_q + (pos - q0);
      const double* qi = q + row * d;
      const double* gi = dout + row * d;
      double mx = -INFINITY;
      int64_t nv = 0;
      for (int64_t a = 0; a < nt && T[a] <= pos; ++a) {
        const double* kt = k + ((int64_t)h * L + T[a]) * d;
        const double* vt = v + ((int64_t)h * L + T[a]) * d;
        double dot = 0.0, gdot = 0.0;
        for (int64_t e = 0; e < d; ++e) { dot += qi[e] * kt[e]; gdot += gi[e] * vt[e]; }
        z[a] = c->scale * dot;
        dp[a] = gdot;
        if (z[a] > mx) mx = z[a];
        nv = a + 1;
      }
      double den = 0.0;
      for (int64_t a = 0; a < nv; ++a) den += exp(z[a] - mx);
      double D = 0.0;
      for (int64_t a = 0; a < nv; ++a) D += exp(z[a] - mx) / den * dp[a];
      double W = 0.0;   /* sum_e |g_e| |o_e| */
      if (dq_abs)
        for (int64_t e = 0; e < d; ++e) {
          double o = 0.0;
          for (int64_t a = 0; a < nv; ++a) o += exp(z[a] - mx) / den * v[((int64_t)h * L + T[a]) * d + e];
          W += fabs(gi[e]) * fabs(o);
        }
      double* dqi = dq + row * d;
      for (int64_t e = 0; e < d; ++e) dqi[e] = 0.0;
      if (dq_abs)
        for (int64_t e = 0; e < d; ++e) dq_abs[row * d + e] = 0.0;
      for (int64_t a = 0; a < nv; ++a) {
        const double P = exp(z[a] - mx) / den;
        const double dS = P * (dp[a] - D);
        const double* kt = k + ((int64_t)h * L + T[a]) * d;
        double* dkt = dk + ((int64_t)h * L + T[a]) * d;
        double* dvt = dv + ((int64_t)h * L + T[a]) * d;
        for (int64_t e = 0; e < d; ++e) {
          dqi[e] += c->scale * dS * kt[e];
          dkt[e] += c->scale * dS * qi[e];
          dvt[e] += P * gi[e];
        }
        if (dq_abs) {
          const double m = P * (fabs(dp[a]) + fabs(D) + W);
          const int64_t kr = ((int64_t)h * L + T[a]) * d;
          for (int64_t e = 0; e < d; ++e) {
            dq_abs[row * d + e] += c->scale * m * fabs(kt[e]);
            dk_abs[kr + e] += c->scale * m * fabs(qi[e]);
            dv_abs[kr + e] += P * fabs(gi[e]);
          }
        }
      }
    }
  free(dp); free(z); free(T);
}

/* dq [Hq][n_q][d]; dk, dv [Hkv][L][d] (every key row, zero where no query
 * attends it). group_idx [nb][Hkv][kg] and n_groups [nb][Hkv] as the forward
 * takes them. dq_abs, dk_abs, dv_abs (same shapes) may all be NULL. */
int orc_attend_backward(const orc_cfg* c, const double* q, const double* k, const double* v,
                        const double* dout, const int32_t* group_idx, const int32_t* n_groups,
                        double* dq, double* dk, double* dv, double* dq_abs, double* dk_abs, double* dv_abs) {
  const int64_t nb = c->n_q / c->q_block;
  const size_t kv_bytes = sizeof(double) * (size_t)(c->hkv * c->seq_len * c->d);
  memset(dk, 0, kv_bytes);
  memset(dv, 0, kv_bytes);
  if (dq_abs) {
    memset(dk_abs, 0, kv_bytes);
    memset(dv_abs, 0, kv_bytes);
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < c->hkv; ++h)
    for (int64_t b = 0; b < nb; ++b)
      backward_item(c, q, k, v, dout, (int)b, h, group_idx + (b * c->hkv + h) * c->top_groups,
                    n_groups[b * c->hkv + h], dq, dk, dv, dq_abs, dk_abs, dv_abs);
  return 0;
}

int orc_diag_width(void) { return DG_NUM; }

/* Threads the OpenMP loops use. */
#ifdef _OPENMP
#include <omp.h>
int orc_threads(void) { return omp_get_max_threads(); }
/* Threads of the following OpenMP loops (n >= 1). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int orc_threads(void) { return 1; }
void orc_set_threads(int n) { (void)n; }
#endif
