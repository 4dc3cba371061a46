/*
 * oracle.c -- plain, slow CPU oracle for the Monodratic routed sparse causal
 * attention path.  TEST INFRASTRUCTURE ONLY: it is loaded by the test suite,
 * by the smoke check and by the CPU-baseline leg of the benchmark, never by
 * the product library, and it shares no code with the GPU path.
 *
 * Sources (the pages):
 *   [TR]  "Monodratic: a reproducible sparse attention mixer", technical
 *         report page (misul.org), sections "Mixer" (+ Figure 1), "Learned
 *         sparse route", "Capacity", "Finite-range scaling", "Evidence",
 *         "Limits".
 *   [NEWS] "Monodratic Claims Learned Routing Can Make Sparse Causal Attention
 *         More Selective" (remio.ai), sections "Monodratic Turns Sparse
 *         Attention Into a Retrieval Decision", "Learned Routing Faces Dense
 *         Attention's Reliability Advantage".
 *
 * What the pages fix, restated: after rotary position embedding, source
 * blocks get product addresses that combine the decisions of several learned
 * code components; addresses point at bounded causal posting lists; a query
 * probes addresses, gathers candidate blocks, reranks them and keeps a fixed
 * number of remote blocks; local blocks are added separately; attention over
 * the chosen tokens is ordinary causal softmax ([TR] "Mixer"; [NEWS]
 * "Retrieval Decision").  Overflow beyond capacity is counted ([TR]
 * "Capacity").  Everything else is a reading, listed in the design doc and at each
 * function below.
 *
 * Precision.  Routing decisions (key argmax, address ranking, rerank top-R)
 * turn floating point into integers; they are taken in fp32, the precision
 * of the kernels, with every step written as a plain sequential fp32
 * operation: products rounded before subtraction in the rotation, sums
 * accumulated in index order from 0.0f, dot products as a chain of fused
 * multiply-adds (fmaf) in index order.  Ties go to the lowest index.  The
 * attention output is computed in fp64 from the unrounded rotated inputs.
 * This file must be compiled with -ffp-contract=off so the compiler keeps
 * every fp32 rounding written here.
 *
 * Parity pins: every function below is pinned by tests under tests/ (brute
 * force, closed forms, library routines, invariants); none is "parity
 * unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int B, T, Hq, Hkv, d, beta, P, K, cap, n_probes, R, L;
} orc_shape;

/* ------------------------------------------------------------------------ */
/* Rotary table.  [TR] "Mixer": routing and attention happen after rotary
 * position embedding.  Reading: rotate-half pairing (dimension i with
 * i + d/2), frequency base^(-2i/d), positions 0..T-1 per sequence; angles in
 * fp64, cos/sin rounded once to fp32. */
void orc_rope_table(int T, int d, double base, float *cos_tab, float *sin_tab)
{
    int h = d / 2;
    for (int t = 0; t < T; ++t) {
        for (int i = 0; i < h; ++i) {
            double inv_freq = pow(base, -(2.0 * (double)i) / (double)d);
            double ang = (double)t * inv_freq;
            cos_tab[(size_t)t * h + i] = (float)cos(ang);
            sin_tab[(size_t)t * h + i] = (float)sin(ang);
        }
    }
}

/* fp32 rotation of one row x[0..d) at position t (routing precision). */
static void rope_row_f32(const float *x, int d, const float *c, const float *s,
                         float *out)
{
    int h = d / 2;
    for (int i = 0; i < h; ++i) {
        float a = x[i], b = x[i + h];
        float ac = a * c[i], bs = b * s[i];
        float bc = b * c[i], as = a * s[i];
        out[i] = ac - bs;
        out[i + h] = bc + as;
    }
}

/* fp64 rotation of one row (attention precision). */
static void rope_row_f64(const float *x, int d, const float *c, const float *s,
                         double *out)
{
    int h = d / 2;
    for (int i = 0; i < h; ++i) {
        double a = x[i], b = x[i + h];
        out[i] = a * (double)c[i] - b * (double)s[i];
        out[i + h] = b * (double)c[i] + a * (double)s[i];
    }
}

/* fp32 dot product as a chain of fmaf in index order. */
static float dot_f32(const float *a, const float *b, int n)
{
    float acc = 0.0f;
    for (int j = 0; j < n; ++j) acc = fmaf(a[j], b[j], acc);
    return acc;
}

static double rel_gap(double best, double second)
{
    double den = fabs(best);
    if (fabs(second) > den) den = fabs(second);
    if (den < 1e-30) den = 1e-30;
    return (best - second) / den;
}

/* ------------------------------------------------------------------------ */
/* Block summaries and key addresses.
 * [NEWS] "Retrieval Decision": after RoPE, source blocks receive learned
 * product addresses, each address combining the decisions of several code
 * components.
 * Readings: the block summary is the mean of the block's post-RoPE keys
 * (fp32 sum in token order, times 1/beta); the d dimensions split into P
 * contiguous sub-vectors of d/P, component p scores code k by the inner
 * product of sub-vector p with C[g][p][k]; the decision is the argmax (ties
 * to the lowest code); the address is the mixed-radix number
 * sum_p c_p * K^(P-1-p) (component 0 most significant).
 * k: [B][T][Hkv][d] values; codebooks: [Hkv][P][K][d/P]; kbar out:
 * [B][Hkv][NB][d]; addr out: [B][Hkv][NB]; gap out (optional):
 * [B][Hkv][NB][P], the relative gap between winner and runner-up. */
void orc_block_addresses(const orc_shape *sh, const float *k,
                         const float *cos_tab, const float *sin_tab,
                         const float *codebooks, float *kbar, int32_t *addr,
                         double *gap, int nthreads)
{
    const int B = sh->B, T = sh->T, Hkv = sh->Hkv, d = sh->d, beta = sh->beta;
    const int P = sh->P, K = sh->K, NB = T / beta, ds = d / P, h = d / 2;
    const float inv_beta = 1.0f / (float)beta;
#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 4)
#else
    (void)nthreads;
#endif
    for (long u = 0; u < (long)B * Hkv * NB; ++u) {
        int n = (int)(u % NB);
        int g = (int)((u / NB) % Hkv);
        int b = (int)(u / ((long)NB * Hkv));
        float *kb = kbar + (size_t)u * d;
        float rot[256];
        for (int j = 0; j < d; ++j) kb[j] = 0.0f;
        for (int i = 0; i < beta; ++i) {
            int t = n * beta + i;
            const float *row = k + (((size_t)b * T + t) * Hkv + g) * d;
            rope_row_f32(row, d, cos_tab + (size_t)t * h, sin_tab + (size_t)t * h, rot);
            for (int j = 0; j < d; ++j) kb[j] = kb[j] + rot[j];
        }
        for (int j = 0; j < d; ++j) kb[j] = kb[j] * inv_beta;

        int a = 0;
        for (int p = 0; p < P; ++p) {
            int best = 0;
            float bestv = 0.0f, second = -INFINITY;
            for (int c = 0; c < K; ++c) {
                const float *code = codebooks + (((size_t)g * P + p) * K + c) * ds;
                float s = dot_f32(kb + p * ds, code, ds);
                if (c == 0 || s > bestv) {
                    if (c != 0) second = bestv;
                    best = c;
                    bestv = s;
                } else if (s > second) {
                    second = s;
                }
            }
            a = a * K + best;
            if (gap) gap[(size_t)u * P + p] = (K > 1) ? rel_gap(bestv, second) : INFINITY;
        }
        addr[u] = a;
    }
}

/* ------------------------------------------------------------------------ */
/* Bounded causal posting lists for one (batch, kv-head).
 * [TR] "Mixer": product routing writes keys into bounded causal posting
 * lists; [NEWS] "Retrieval Decision": a posting list is a bounded set of
 * source blocks assigned to one address, a strict capacity bounds it, and
 * overflow may discard blocks; [TR] "Capacity" counts overflow events;
 * [TR] "Finite-range scaling": the index build is a stable sort.
 * Reading: blocks are visited in source order; each address keeps its first
 * cap blocks; every further block is dropped and counted; load is the count
 * before the clamp; offsets are the exclusive prefix sum of min(load, cap);
 * entries beyond the kept total are -1. */
void orc_posting_lists(int NB, int A, int cap, const int32_t *addr,
                       int32_t *offsets, int32_t *entries, int32_t *load,
                       int32_t *overflow)
{
    int32_t *kept = (int32_t *)calloc((size_t)A, sizeof(int32_t));
    for (int a = 0; a < A; ++a) load[a] = 0;
    *overflow = 0;
    for (int n = 0; n < NB; ++n) {
        int a = addr[n];
        load[a] += 1;
        if (load[a] <= cap) kept[a] += 1;
        else *overflow += 1;
    }
    offsets[0] = 0;
    for (int a = 0; a < A; ++a) offsets[a + 1] = offsets[a] + kept[a];
    for (int a = 0; a < A; ++a) kept[a] = 0;
    for (int n = 0; n < NB; ++n) entries[n] = -1;
    for (int n = 0; n < NB; ++n) {
        int a = addr[n];
        if (kept[a] < cap) {
            entries[offsets[a] + kept[a]] = n;
            kept[a] += 1;
        }
    }
    free(kept);
}

/* Whole index: addresses for every (b, g, n), then one posting-list build per
 * (b, g).  offsets: [B][Hkv][A+1]; entries: [B][Hkv][NB]; load: [B][Hkv][A];
 * overflow: [B][Hkv]. */
void orc_build_index(const orc_shape *sh, const float *k, const float *cos_tab,
                     const float *sin_tab, const float *codebooks, float *kbar,
                     int32_t *addr, int32_t *offsets, int32_t *entries,
                     int32_t *load, int32_t *overflow, double *gap, int nthreads)
{
    const int NB = sh->T / sh->beta;
    int A = 1;
    for (int p = 0; p < sh->P; ++p) A *= sh->K;
    orc_block_addresses(sh, k, cos_tab, sin_tab, codebooks, kbar, addr, gap, nthreads);
    for (int u = 0; u < sh->B * sh->Hkv; ++u)
        orc_posting_lists(NB, A, sh->cap, addr + (size_t)u * NB,
                          offsets + (size_t)u * (A + 1), entries + (size_t)u * NB,
                          load + (size_t)u * A, overflow + u);
}

/* ------------------------------------------------------------------------ */
/* Routing of one query token.
 * [NEWS] "Retrieval Decision": each query probes addresses, receives
 * candidates, reranks them and selects a fixed number of remote blocks; a
 * source block is never available to an earlier query; local blocks are
 * guaranteed.  [TR] "Learned sparse route": six blocks with one local block
 * leave five eligible remote blocks at the latest queries; "Capacity": when
 * every remote block is eligible the run does not exercise retrieval.
 * Readings:
 *  - query block qb = t / beta; the L local blocks are qb-L+1..qb (the own
 *    block counts); remote-eligible blocks are 0..qb-L, E = max(0, qb-L+1);
 *  - if E <= R the search is bypassed and the selection is blocks 0..E-1;
 *  - otherwise component scores s_p[k] = <q'_p, C[g][p][k]>, address score
 *    sigma(a) = s_0[a_0] + s_1[a_1] + ... (fp32, left to right); all
 *    addresses are ranked by (sigma descending, address ascending) and
 *    walked in that order, adding each list's causally eligible entries to
 *    the pool, until at least n_probes addresses were probed and the pool
 *    holds at least R blocks (or every address was probed);
 *  - rerank score rho(n) = <q', kbar_n>; keep the R best by (rho
 *    descending, block ascending); emit them ascending, -1 padded.
 * q' is the fp32-rotated query; queries of q-head h use kv-head h / (Hq/Hkv).
 * gaps (optional, 2 per route): relative gap of the pool boundary (last
 * probed address vs the next one) and of the rerank boundary (R-th kept vs
 * best dropped); +inf where no such decision was taken. */
typedef struct { float sig; int32_t a; } addr_key;

static int cmp_addr_key(const void *x, const void *y)
{
    const addr_key *p = (const addr_key *)x, *q = (const addr_key *)y;
    if (p->sig > q->sig) return -1;
    if (p->sig < q->sig) return 1;
    return (p->a < q->a) ? -1 : (p->a > q->a);
}

typedef struct { float rho; int32_t n; } blk_key;

static int cmp_blk_key(const void *x, const void *y)
{
    const blk_key *p = (const blk_key *)x, *q = (const blk_key *)y;
    if (p->rho > q->rho) return -1;
    if (p->rho < q->rho) return 1;
    return (p->n < q->n) ? -1 : (p->n > q->n);
}

static int cmp_i32(const void *x, const void *y)
{
    int32_t a = *(const int32_t *)x, b = *(const int32_t *)y;
    return (a > b) - (a < b);
}

static void route_one(const orc_shape *sh, int A, const float *q,
                      const float *cos_tab, const float *sin_tab,
                      const float *codebooks, const float *kbar,
                      const int32_t *offsets, const int32_t *entries,
                      long route, int32_t *sel_out, double *gap_out,
                      addr_key *order, blk_key *pool, float *scratch)
{
    const int T = sh->T, Hq = sh->Hq, Hkv = sh->Hkv, d = sh->d, beta = sh->beta;
    const int P = sh->P, K = sh->K, R = sh->R, L = sh->L, NB = T / beta;
    const int ds = d / P, h = d / 2, G = Hq / Hkv;
    int t = (int)(route % T);
    int hq = (int)((route / T) % Hq);
    int b = (int)(route / ((long)T * Hq));
    int g = hq / G;
    int qb = t / beta;
    int E = qb - L + 1;
    if (E < 0) E = 0;
    if (gap_out) { gap_out[0] = INFINITY; gap_out[1] = INFINITY; }

    if (E <= R) {
        for (int r = 0; r < R; ++r) sel_out[r] = (r < E) ? r : -1;
        return;
    }

    float *qr = scratch;          /* d   */
    float *sc = scratch + d;      /* P*K */
    const float *qrow = q + (((size_t)b * T + t) * Hq + hq) * d;
    rope_row_f32(qrow, d, cos_tab + (size_t)t * h, sin_tab + (size_t)t * h, qr);
    for (int p = 0; p < P; ++p)
        for (int c = 0; c < K; ++c)
            sc[p * K + c] = dot_f32(qr + p * ds,
                                    codebooks + (((size_t)g * P + p) * K + c) * ds, ds);
    for (int a = 0; a < A; ++a) {
        int rest = a, digit[16];
        for (int p = P - 1; p >= 0; --p) { digit[p] = rest % K; rest /= K; }
        float s = sc[0 * K + digit[0]];
        for (int p = 1; p < P; ++p) s = s + sc[p * K + digit[p]];
        order[a].sig = s;
        order[a].a = a;
    }
    qsort(order, (size_t)A, sizeof(addr_key), cmp_addr_key);

    const int32_t *off = offsets + ((size_t)b * Hkv + g) * (A + 1);
    const int32_t *ent = entries + ((size_t)b * Hkv + g) * NB;
    const float *kb = kbar + ((size_t)b * Hkv + g) * (size_t)NB * d;
    int last_eligible = qb - L;
    int npool = 0, probed = 0;
    for (int i = 0; i < A; ++i) {
        int a = order[i].a;
        for (int e = off[a]; e < off[a + 1]; ++e) {
            int n = ent[e];
            if (n > last_eligible) break; /* lists ascend: the rest is later */
            pool[npool].n = n;
            pool[npool].rho = dot_f32(qr, kb + (size_t)n * d, d);
            ++npool;
        }
        probed = i + 1;
        if (probed >= sh->n_probes && npool >= R) break;
    }
    if (gap_out && probed < A)
        gap_out[0] = rel_gap(order[probed - 1].sig, order[probed].sig);

    qsort(pool, (size_t)npool, sizeof(blk_key), cmp_blk_key);
    int nsel = npool < R ? npool : R;
    if (gap_out && npool > R) gap_out[1] = rel_gap(pool[R - 1].rho, pool[R].rho);
    for (int r = 0; r < R; ++r) sel_out[r] = (r < nsel) ? pool[r].n : -1;
    qsort(sel_out, (size_t)nsel, sizeof(int32_t), cmp_i32);
}

/* Route a list of routes (route id = (b*Hq + h)*T + t), or every route when
 * route_ids is NULL.  sel: [n_routes][R]; gaps: [n_routes][2] or NULL. */
void orc_route(const orc_shape *sh, const float *q, const float *cos_tab,
               const float *sin_tab, const float *codebooks, const float *kbar,
               const int32_t *offsets, const int32_t *entries,
               const int64_t *route_ids, long n_routes, int32_t *sel,
               double *gaps, int nthreads)
{
    int A = 1;
    for (int p = 0; p < sh->P; ++p) A *= sh->K;
    const int NB = sh->T / sh->beta;
#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads)
#else
    (void)nthreads;
#endif
    {
        addr_key *order = (addr_key *)malloc(sizeof(addr_key) * (size_t)A);
        blk_key *pool = (blk_key *)malloc(sizeof(blk_key) * (size_t)(NB + 1));
        float *scratch = (float *)malloc(sizeof(float) * (size_t)(sh->d + sh->P * sh->K));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 64)
#endif
        for (long i = 0; i < n_routes; ++i) {
            long route = route_ids ? (long)route_ids[i] : i;
            route_one(sh, A, q, cos_tab, sin_tab, codebooks, kbar, offsets, entries,
                      route, sel + (size_t)i * sh->R, gaps ? gaps + (size_t)i * 2 : NULL,
                      order, pool, scratch);
        }
        free(order);
        free(pool);
        free(scratch);
    }
}

/* ------------------------------------------------------------------------ */
/* Spherical codebook calibration.
 * [TR] "Capacity" (and Figure 3): calibrating the codebooks spherically on a
 * training split removes the held-out capacity overflow and lowers the
 * largest list load.  The pages name the method only.  Reading: spherical
 * k-means, separately for every kv-head g and component p, over the block
 * summaries of the training split restricted to component p's sub-vector
 * (exactly the vectors whose code decisions make the addresses):
 *   assignment  each point takes the code with the largest inner product
 *               (fmaf chain in dimension order, ties to the lowest code),
 *               the decision the address uses;
 *   update      every code with members becomes the sum of its members
 *               (fp32 additions in point order from 0.0f) divided by that
 *               sum's norm, sqrtf of its fmaf-chain square; a code without
 *               members keeps its value;
 *   n_iter rounds of assignment followed by update.
 * kbar: [B][Hkv][NB][d], points ordered batch-major then block; codebooks:
 * [Hkv][P][K][d/P], calibrated in place. */
void orc_calibrate(int B, int Hkv, int NB, int d, int P, int K, const float *kbar,
                   float *codebooks, int n_iter)
{
    const int ds = d / P;
    const long N = (long)B * NB;
    int32_t *asg = (int32_t *)malloc(sizeof(int32_t) * (size_t)N);
    float *sum = (float *)malloc(sizeof(float) * (size_t)K * ds);
    int32_t *cnt = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    for (int g = 0; g < Hkv; ++g) {
        for (int p = 0; p < P; ++p) {
            float *C = codebooks + ((size_t)g * P + p) * K * ds;
            for (int it = 0; it < n_iter; ++it) {
                for (long i = 0; i < N; ++i) {
                    long b = i / NB, n = i % NB;
                    const float *x = kbar + (((size_t)b * Hkv + g) * NB + n) * d + (size_t)p * ds;
                    int best = 0;
                    float bs = dot_f32(x, C, ds);
                    for (int c = 1; c < K; ++c) {
                        float v = dot_f32(x, C + (size_t)c * ds, ds);
                        if (v > bs) { bs = v; best = c; }
                    }
                    asg[i] = best;
                }
                for (size_t e = 0; e < (size_t)K * ds; ++e) sum[e] = 0.0f;
                for (int c = 0; c < K; ++c) cnt[c] = 0;
                for (long i = 0; i < N; ++i) {
                    long b = i / NB, n = i % NB;
                    const float *x = kbar + (((size_t)b * Hkv + g) * NB + n) * d + (size_t)p * ds;
                    float *sc = sum + (size_t)asg[i] * ds;
                    for (int j = 0; j < ds; ++j) sc[j] = sc[j] + x[j];
                    cnt[asg[i]] += 1;
                }
                for (int c = 0; c < K; ++c) {
                    if (cnt[c] == 0) continue;
                    const float *sc = sum + (size_t)c * ds;
                    float norm = sqrtf(dot_f32(sc, sc, ds));
                    for (int j = 0; j < ds; ++j) C[(size_t)c * ds + j] = sc[j] / norm;
                }
            }
        }
    }
    free(asg);
    free(sum);
    free(cnt);
}

/* ------------------------------------------------------------------------ */
/* Selected-set attention for a list of routes.
 * [TR] "Mixer": local blocks are added separately and attention over the
 * selected set is ordinary causal softmax; no value summary replaces the
 * selected values.  [NEWS] "Retrieval Decision": exact within the selected
 * set, causal mask applied.
 * Readings: the token set of query t is every token s <= t whose block is a
 * selected remote block or one of the L local blocks; logits are
 * <q'_t, k'_s> / sqrt(d) with fp64 rotation; values are not rotated.
 * sel: [n_routes][R] (the selection of each listed route); out:
 * [n_routes][d] fp64. */
void orc_attention(const orc_shape *sh, const float *q, const float *k,
                   const float *v, const float *cos_tab, const float *sin_tab,
                   const int32_t *sel, const int64_t *route_ids, long n_routes,
                   double *out, int nthreads)
{
    const int T = sh->T, Hq = sh->Hq, Hkv = sh->Hkv, d = sh->d, beta = sh->beta;
    const int R = sh->R, L = sh->L, h = d / 2, G = Hq / Hkv;
    const double scale = 1.0 / sqrt((double)d);
#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads)
#else
    (void)nthreads;
#endif
    {
        int maxtok = (R + L) * beta;
        double *qr = (double *)malloc(sizeof(double) * (size_t)d);
        double *kr = (double *)malloc(sizeof(double) * (size_t)d);
        double *logit = (double *)malloc(sizeof(double) * (size_t)maxtok);
        int32_t *tok = (int32_t *)malloc(sizeof(int32_t) * (size_t)maxtok);
        int32_t *blocks = (int32_t *)malloc(sizeof(int32_t) * (size_t)(R + L));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 64)
#endif
        for (long i = 0; i < n_routes; ++i) {
            long route = route_ids ? (long)route_ids[i] : i;
            int t = (int)(route % T);
            int hq = (int)((route / T) % Hq);
            int b = (int)(route / ((long)T * Hq));
            int g = hq / G, qb = t / beta;
            const float *qrow = q + (((size_t)b * T + t) * Hq + hq) * d;
            rope_row_f64(qrow, d, cos_tab + (size_t)t * h, sin_tab + (size_t)t * h, qr);

            /* the block set: selected remote blocks, then the local window */
            int nb = 0;
            for (int r = 0; r < R; ++r)
                if (sel[(size_t)i * R + r] >= 0) blocks[nb++] = sel[(size_t)i * R + r];
            int lo = qb - L + 1;
            if (lo < 0) lo = 0;
            for (int m = lo; m <= qb; ++m) {
                int dup = 0;
                for (int j = 0; j < nb; ++j) dup |= (blocks[j] == m);
                if (!dup) blocks[nb++] = m;
            }
            int ntok = 0;
            for (int j = 0; j < nb; ++j)
                for (int s = blocks[j] * beta; s < (blocks[j] + 1) * beta; ++s)
                    if (s <= t) tok[ntok++] = s;

            double mx = -INFINITY;
            for (int j = 0; j < ntok; ++j) {
                int s = tok[j];
                const float *krow = k + (((size_t)b * T + s) * Hkv + g) * d;
                rope_row_f64(krow, d, cos_tab + (size_t)s * h, sin_tab + (size_t)s * h, kr);
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += qr[c] * kr[c];
                logit[j] = dot * scale;
                if (logit[j] > mx) mx = logit[j];
            }
            double den = 0.0;
            for (int j = 0; j < ntok; ++j) { logit[j] = exp(logit[j] - mx); den += logit[j]; }
            double *o = out + (size_t)i * d;
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            for (int j = 0; j < ntok; ++j) {
                const float *vrow = v + (((size_t)b * T + tok[j]) * Hkv + g) * d;
                double w = logit[j] / den;
                for (int c = 0; c < d; ++c) o[c] += w * (double)vrow[c];
            }
        }
        free(qr);
        free(kr);
        free(logit);
        free(tok);
        free(blocks);
    }
}

/* Number of routes of a shape: B * Hq * T. */
long orc_num_routes(const orc_shape *sh) { return (long)sh->B * sh->Hq * sh->T; }

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
