/*
 * moe_oracle.c -- plain, slow, fp64 CPU evaluation of the sparse
 * Mixture-of-Experts FFN layer (router top-k softmax, token->expert
 * grouping, SwiGLU experts, weighted combine).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker against which the
 * HIP library is compared.  Only the test suite, the smoke entry point and
 * the benchmark's CPU-baseline leg may load it.  It shares no source,
 * header, table or helper with the HIP library (prefill_moe_router_amd/csrc).
 *
 * Source of what is computed:
 *   - "Decode 吞吐专项实验分析报告", section "2026-07-14：解除强制 eager /
 *     custom all-reduce 禁用验证", subsection "下一步 profiling 方向": the
 *     fused MoE layer is the sequence gate -> topk -> expert kernel ->
 *     activation -> sum.
 *   - "第 9 章 prefill：最大的瓶颈", §9.9: expert grouping happens on the
 *     device and a numeric-path switch must be checked against the old
 *     path's outputs; §9.5: entries past a fixed per-group limit must never
 *     be silently dropped.
 *   - The layer definition this repository implements: softmax over all
 *     experts, keep the k largest, renormalise the kept weights to sum to 1
 *     (optional), SwiGLU experts silu(x Wg^T) * (x Wu^T) projected by Wd,
 *     and a weighted sum over each token's k experts.
 *
 * Every stored input value is decoded exactly to fp64 and every sum is
 * taken in fp64, in ascending index order.  No blocking, fusion or
 * reordering beyond the definition.  Readings where the sources are silent
 * (tie rule, id order inside a token, near-tie rule) are stated at each
 * function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes used by this file's interface (independent of the HIP side) */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_MXFP4 2
#define ORC_NVFP4 3
#define ORC_MXINT8 4

typedef struct {
    int32_t T;          /* number of tokens */
    int32_t H;          /* hidden size */
    int32_t E;          /* number of experts */
    int32_t K;          /* experts kept per token (top-k) */
    int32_t I;          /* expert intermediate size */
    int32_t renorm;     /* 1: kept weights renormalised to sum 1 */
    int32_t act_dtype;  /* x and router weight: ORC_F32 or ORC_BF16 */
    int32_t w_dtype;    /* expert weights: ORC_F32, ORC_BF16, ORC_MXFP4, ORC_NVFP4 or ORC_MXINT8 */
    const void *x;      /* [T][H] */
    const void *wr;     /* [E][H] */
    const float *bias;  /* [E] or NULL */
    const void *wg;     /* [E][I][H]   (MXFP4: [E][I][H/2] bytes; MXINT8: [E][I][H] bytes) */
    const void *wu;     /* [E][I][H] */
    const void *wd;     /* [E][H][I]   (MXFP4: [E][H][I/2] bytes) */
    const uint8_t *sg;  /* MXFP4 scales [E][I][H/32]; NVFP4 [E][I][H/16] */
    const uint8_t *su;  /* [E][I][H/32] or [E][I][H/16] */
    const uint8_t *sd;  /* [E][H][I/32] or [E][H][I/16] */
    double tsg, tsu, tsd; /* NVFP4 tensor scales of gate, up and down */
} orc_layer;

/* ---- exact decoders of the stored formats ------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_decode_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP MX E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
 * exponent field 0 is subnormal (0.5 * mantissa). */
double orc_decode_e2m1(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double v = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -v : v;
}

/* OCP MX E8M0 shared scale: 2^(code-127); code 255 is NaN. */
double orc_decode_e8m0(uint8_t code)
{
    if (code == 255) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* OCP FP8 E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0; exponent
 * field 0 is subnormal (mantissa/8 * 2^-6); no infinities; S.1111.111 is NaN. */
double orc_decode_e4m3(uint8_t code)
{
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    if (e == 15u && m == 7u) return NAN;
    double v = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -v : v;
}

/* OCP MX INT8 element: an 8-bit two's complement integer with an implicit scale of
 * 2^-6 (so codes span -2 .. 127/64); the block's E8M0 scale multiplies it. */
double orc_decode_int8(uint8_t code)
{
    int v = (code & 0x80u) ? (int)code - 256 : (int)code;
    return ldexp((double)v, -6);
}

/* Every code's value, looked up per element instead of decoded again: entry c is
 * exactly what the decoder above returns for code c, so the lookups change no value
 * (they only spare the per-element ldexp calls of the 4-bit formats). */
static double tab_e2m1[16], tab_e8m0[256], tab_e4m3[256], tab_int8[256];

static void fill_code_tables(void)
{
    for (unsigned c = 0; c < 16; ++c) tab_e2m1[c] = orc_decode_e2m1(c);
    for (unsigned c = 0; c < 256; ++c) {
        tab_e8m0[c] = orc_decode_e8m0((uint8_t)c);
        tab_e4m3[c] = orc_decode_e4m3((uint8_t)c);
        tab_int8[c] = orc_decode_int8((uint8_t)c);
    }
}

static double act_at(const orc_layer *L, const void *base, size_t idx)
{
    if (L->act_dtype == ORC_F32) return (double)((const float *)base)[idx];
    return orc_decode_bf16(((const uint16_t *)base)[idx]);
}

/* element (row, col) of an expert matrix stored row-major [rows][cols]; ts is the
 * matrix's NVFP4 tensor scale */
static double wt_at(const orc_layer *L, const void *w, const uint8_t *s, double ts,
                    size_t row, size_t cols, size_t col)
{
    if (L->w_dtype == ORC_F32) return (double)((const float *)w)[row * cols + col];
    if (L->w_dtype == ORC_BF16) return orc_decode_bf16(((const uint16_t *)w)[row * cols + col]);
    if (L->w_dtype == ORC_MXINT8) /* one byte per element, one E8M0 scale per 32 elements */
        return tab_int8[((const uint8_t *)w)[row * cols + col]] * tab_e8m0[s[row * (cols / 32) + col / 32]];
    /* MXFP4 and NVFP4: two codes per byte, the even element in the low nibble */
    uint8_t byte = ((const uint8_t *)w)[row * (cols / 2) + col / 2];
    unsigned code = (col & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
    if (L->w_dtype == ORC_NVFP4) /* one E4M3 scale per 16 elements, then the tensor scale */
        return tab_e2m1[code] * tab_e4m3[s[row * (cols / 16) + col / 16]] * ts;
    /* MXFP4: one E8M0 scale per 32 consecutive elements of a row */
    return tab_e2m1[code] * tab_e8m0[s[row * (cols / 32) + col / 32]];
}

/* ---- a1: router logits -------------------------------------------------- */
/* s[e] = b[e] + sum_h x[t,h] * Wr[e,h]  (b = 0 when absent) */
static void router_logits(const orc_layer *L, int t, double *s)
{
    for (int e = 0; e < L->E; ++e) {
        double acc = 0.0;
        for (int h = 0; h < L->H; ++h)
            acc += act_at(L, L->x, (size_t)t * L->H + h) * act_at(L, L->wr, (size_t)e * L->H + h);
        s[e] = acc + (L->bias ? (double)L->bias[e] : 0.0);
    }
}

/* ---- a2: top-k, softmax, renormalisation --------------------------------- */
/* Order experts by (score descending, id ascending); keep the first k.
 * rank[] receives the full order's first min(k+1, E) entries. */
static void rank_experts(const double *s, int E, int n, int *rank)
{
    unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
    for (int r = 0; r < n; ++r) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || s[e] > s[best]) best = e; /* equal score: lower id stays */
        }
        rank[r] = best;
        taken[best] = 1;
    }
    free(taken);
}

static int cmp_int(const void *a, const void *b)
{
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

/* Weights of the kept set: p = softmax over all E scores; kept weights are
 * p restricted to the set, divided by their sum when renorm is on.
 * ids[] must already be in ascending order. */
static void gate_weights(const double *s, int E, int k, int renorm, const int *ids, double *w)
{
    double m = s[0];
    for (int e = 1; e < E; ++e) if (s[e] > m) m = s[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += exp(s[e] - m);
    double kept = 0.0;
    for (int j = 0; j < k; ++j) {
        w[j] = exp(s[ids[j]] - m) / z;
        kept += w[j];
    }
    if (renorm)
        for (int j = 0; j < k; ++j) w[j] /= kept;
}

/*
 * Router for a subset of tokens (tokens == NULL: all T tokens, n = T).
 * Outputs per evaluated token r: ids[r*k..] ascending, w[r*k..], near[r]
 * (1 when the k-th and (k+1)-th ranked scores differ by less than
 * 1e-5 * max(|s_k|, |s_k+1|, 1)), gap[r] = that absolute difference
 * (+inf when k == E), and the raw logits when logits != NULL.
 */
int orc_router(const orc_layer *L, const int32_t *tokens, int n,
               double *logits, int32_t *ids, double *w, uint8_t *near, double *gap)
{
    if (L->K < 1 || L->K > L->E) return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic)
    for (int r = 0; r < n; ++r) {
        int t = tokens ? tokens[r] : r;
        if (t < 0 || t >= L->T) { err = -1; continue; }
        double *s = (double *)malloc(sizeof(double) * (size_t)L->E);
        int nr = L->K < L->E ? L->K + 1 : L->K;
        int *rank = (int *)malloc(sizeof(int) * (size_t)nr);
        int *sel = (int *)malloc(sizeof(int) * (size_t)L->K);
        double *wk = (double *)malloc(sizeof(double) * (size_t)L->K);
        router_logits(L, t, s);
        rank_experts(s, L->E, nr, rank);
        for (int j = 0; j < L->K; ++j) sel[j] = rank[j];
        qsort(sel, (size_t)L->K, sizeof(int), cmp_int);
        gate_weights(s, L->E, L->K, L->renorm, sel, wk);
        for (int j = 0; j < L->K; ++j) {
            ids[(size_t)r * L->K + j] = sel[j];
            w[(size_t)r * L->K + j] = wk[j];
        }
        if (L->K < L->E) {
            double a = s[rank[L->K - 1]], b = s[rank[L->K]];
            double g = fabs(a - b), ref = fmax(fmax(fabs(a), fabs(b)), 1.0);
            if (gap) gap[r] = g;
            if (near) near[r] = g < 1e-5 * ref;
        } else {
            if (gap) gap[r] = INFINITY;
            if (near) near[r] = 0;
        }
        if (logits) memcpy(logits + (size_t)r * L->E, s, sizeof(double) * (size_t)L->E);
        free(s); free(rank); free(sel); free(wk);
    }
    return err;
}

/* ---- a3: token -> expert grouping ---------------------------------------- */
/*
 * Slot t*k+j is the j-th kept expert of token t.  cnt[e] = number of slots
 * routed to e; off[0] = 0, off[e+1] = off[e] + cnt[e]; slots are placed in
 * ascending slot order within each expert (a stable counting sort), and
 * slot_pos is the inverse map.  Returns -1 (and writes nothing beyond the
 * counts) when an id lies outside [0, E).
 */
int orc_group(int T, int k, int E, const int32_t *ids, int32_t *off, int32_t *sorted, int32_t *slot_pos)
{
    if (T < 0 || k < 1 || E < 1) return -1;
    size_t P = (size_t)T * (size_t)k;
    for (size_t p = 0; p < P; ++p)
        if (ids[p] < 0 || ids[p] >= E) return -1;
    for (int e = 0; e <= E; ++e) off[e] = 0;
    for (size_t p = 0; p < P; ++p) off[ids[p] + 1] += 1;
    for (int e = 0; e < E; ++e) off[e + 1] += off[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (size_t p = 0; p < P; ++p) {
        int e = ids[p];
        int32_t pos = off[e] + fill[e]++;
        sorted[pos] = (int32_t)p;
        slot_pos[p] = pos;
    }
    free(fill);
    return 0;
}

/* ---- a4 + a5: one expert applied to one token ----------------------------- */
/* g[i] = Wg[e,i,:].x ; u[i] = Wu[e,i,:].x ; a[i] = g/(1+exp(-g)) * u ;
 * o[n] = Wd[e,n,:].a */
static void expert_apply(const orc_layer *L, int t, int e, double *o, double *a)
{
    const int H = L->H, I = L->I;
    const int sc = (L->w_dtype == ORC_MXFP4 || L->w_dtype == ORC_NVFP4 || L->w_dtype == ORC_MXINT8);
    const size_t rows_gu = (size_t)e * I, rows_d = (size_t)e * H;
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
            double xv = act_at(L, L->x, (size_t)t * H + h);
            g += wt_at(L, L->wg, sc ? L->sg : NULL, L->tsg, rows_gu + i, (size_t)H, (size_t)h) * xv;
            u += wt_at(L, L->wu, sc ? L->su : NULL, L->tsu, rows_gu + i, (size_t)H, (size_t)h) * xv;
        }
        a[i] = g / (1.0 + exp(-g)) * u;
    }
    for (int n = 0; n < H; ++n) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i)
            acc += wt_at(L, L->wd, sc ? L->sd : NULL, L->tsd, rows_d + n, (size_t)I, (size_t)i) * a[i];
        o[n] = acc;
    }
}

/* Expert output for explicit (token, expert) pairs: o[p][H]. */
int orc_expert_pairs(const orc_layer *L, const int32_t *tok, const int32_t *exp_id, int npairs, double *o)
{
    int err = 0;
    fill_code_tables();
#pragma omp parallel for schedule(dynamic)
    for (int p = 0; p < npairs; ++p) {
        if (tok[p] < 0 || tok[p] >= L->T || exp_id[p] < 0 || exp_id[p] >= L->E) { err = -1; continue; }
        double *a = (double *)malloc(sizeof(double) * (size_t)L->I);
        expert_apply(L, tok[p], exp_id[p], o + (size_t)p * L->H, a);
        free(a);
    }
    return err;
}

/* ---- whole layer (a1..a6) for a subset of tokens ------------------------- */
/*
 * y[r][n] = sum_{j ascending} w[r,j] * o_{ids[r,j]}(x_t)[n] for token
 * t = tokens[r] (tokens == NULL: all).  When forced_ids != NULL its rows
 * (ascending ids, one row of k per evaluated token) replace the selection
 * and the weights are those of the forced set.  ids/w/near/gap as in
 * orc_router (for forced ids near/gap still describe the oracle's own
 * ranking).
 */
int orc_forward(const orc_layer *L, const int32_t *tokens, int n, const int32_t *forced_ids,
                double *y, int32_t *ids, double *w, uint8_t *near, double *gap)
{
    int err = orc_router(L, tokens, n, NULL, ids, w, near, gap);
    if (err) return err;
    fill_code_tables();
    const int H = L->H, E = L->E, k = L->K;
    if (forced_ids) {
        for (int r = 0; r < n; ++r)
            for (int j = 0; j < k; ++j) {
                int32_t e = forced_ids[(size_t)r * k + j];
                if (e < 0 || e >= E) return -1;
                if (j > 0 && forced_ids[(size_t)r * k + j - 1] >= e) return -1;
            }
    }
#pragma omp parallel for schedule(dynamic)
    for (int r = 0; r < n; ++r) {
        int t = tokens ? tokens[r] : r;
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        double *a = (double *)malloc(sizeof(double) * (size_t)L->I);
        if (forced_ids) {
            double *s = (double *)malloc(sizeof(double) * (size_t)E);
            int *sel = (int *)malloc(sizeof(int) * (size_t)k);
            double *wk = (double *)malloc(sizeof(double) * (size_t)k);
            router_logits(L, t, s);
            for (int j = 0; j < k; ++j) sel[j] = forced_ids[(size_t)r * k + j];
            gate_weights(s, E, k, L->renorm, sel, wk);
            for (int j = 0; j < k; ++j) {
                ids[(size_t)r * k + j] = sel[j];
                w[(size_t)r * k + j] = wk[j];
            }
            free(s); free(sel); free(wk);
        }
        double *yr = y + (size_t)r * H;
        for (int h = 0; h < H; ++h) yr[h] = 0.0;
        for (int j = 0; j < k; ++j) {
            expert_apply(L, t, ids[(size_t)r * k + j], o, a);
            double wj = w[(size_t)r * k + j];
            for (int h = 0; h < H; ++h) yr[h] += wj * o[h];
        }
        free(o); free(a);
    }
    return 0;
}

/* sets the number of OpenMP threads later calls use (no effect without OpenMP) */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* number of OpenMP threads the oracle will use (1 without OpenMP) */
int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
