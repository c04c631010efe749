/*
 * moe_oracle.c -- plain, slow, obviously correct CPU oracle for the prefill MoE expert layer.
 *
 * TEST INFRASTRUCTURE: see moe_oracle.h for who may load it, the page titles cited as
 * [G1] [G2] [QS] [CS], and the byte formats.  Floating point follows the precision the pages
 * fix (q8_1 = int8 with fp16 d and s; fp32 activations) and is fp64 everywhere else.
 * Built with -ffp-contract=off so that no multiply-add is fused behind the reader's back.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------------------------
 * fp16 (IEEE 754 binary16) from its definition: 1 sign bit, 5 exponent bits (bias 15),
 * 10 fraction bits; normal values (1024+m)*2^(e-25), subnormals m*2^-24.
 * Conversion from fp32 rounds to nearest, ties to even (nearbyint in the default rounding
 * mode), keeps subnormals, and overflows to infinity from 65520 (the midpoint between the
 * largest finite value 65504 and 65536).  Pinned in tests/test_oracle_formats.py against
 * numpy.float16 over every fp16 boundary, midpoint and subnormal.
 * ------------------------------------------------------------------------------------- */
uint16_t orc_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    double a = fabs((double)f);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    if (a < ldexp(1.0, -14)) {
        /* subnormal result in units of 2^-24; a count of 1024 is the smallest normal
         * number, whose encoding (exponent field 1, fraction 0) is the same integer */
        double m = nearbyint(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e2;
    frexp(a, &e2);                 /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;                /* unbiased exponent */
    double m = nearbyint(a * ldexp(1.0, 10 - E));   /* significand in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; E += 1; }
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(m - 1024.0));
}

double orc_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }

size_t orc_block_bytes(int wtype) { return wtype == ORC_Q4_1 ? 20 : 34; }

size_t orc_expert_bytes(int H, int F, int wtype)
{
    /* gate and up: F rows of H/32 blocks each; down: H rows of F/32 blocks */
    return ((size_t)2 * F * (H / 32) + (size_t)H * (F / 32)) * orc_block_bytes(wtype);
}

size_t orc_q8_1_row_bytes(int n) { return (size_t)(n / 128) * 144; }

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------------------
 * a0  top-K routing.  [QS] "Identity": routing is built as Prefill builds it, 10 of 512
 * experts per token; the pages give no formula.  Reading: each token takes the K experts
 * with the largest logits (equal logits: the lower expert id first), and its weights are the
 * softmax of those K logits -- the same as softmax over all E logits, then top-K, then
 * renormalising, because the full denominator cancels.  Weights in fp64, stored fp32.
 * Pinned in tests/test_oracle_route_maps.py (brute force with a stable numpy sort, ties,
 * weight closed forms).
 * ------------------------------------------------------------------------------------- */
void orc_route_topk(const float *logits, int T, int E, int K, int32_t *idx, float *w)
{
    char *taken = (char *)malloc((size_t)E);
    double *ex = (double *)malloc(sizeof(double) * (size_t)K);
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;   /* strict: a tie keeps the lower id */
            }
            taken[best] = 1;
            idx[(size_t)t * K + k] = best;
        }
        double lmax = (double)l[idx[(size_t)t * K]];
        double sum = 0.0;
        for (int k = 0; k < K; ++k) {
            ex[k] = exp((double)l[idx[(size_t)t * K + k]] - lmax);
            sum += ex[k];
        }
        for (int k = 0; k < K; ++k) w[(size_t)t * K + k] = (float)(ex[k] / sum);
    }
    free(ex);
    free(taken);
}

/* ---------------------------------------------------------------------------------------
 * a1  token -> row maps.  [QS] opening section: the quantizer runs over T x K rows in expert
 * order, src_dev names each row's source, and token t's k-th row is slot[t*K+k], the inverse
 * of src_dev.  Readings: src[r] = t*K+k (so the inverse is exact); rows are grouped by expert
 * id ascending and, inside an expert, keep ascending t*K+k (a stable counting sort).
 * order[] lists the experts that received rows, walking the ring from ring_start
 * ([G2] opening section and "What changes": the walk runs over ring entries; entries the
 * routing skipped hold no rows).  Groups of the walk are order[gs*g .. gs*g+gs-1].
 * Pinned in tests/test_oracle_route_maps.py.
 * ------------------------------------------------------------------------------------- */
void orc_build_maps(const int32_t *idx, int T, int K, int E, int ring_start,
                    int32_t *counts, int32_t *offsets, int32_t *src, int32_t *slot,
                    int32_t *order, int32_t *n_active)
{
    int R = T * K;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int i = 0; i < R; ++i) counts[idx[i]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int i = 0; i < R; ++i) {
        int e = idx[i];
        int r = offsets[e] + seen[e];
        seen[e] += 1;
        src[r] = i;
        slot[i] = r;
    }
    free(seen);
    int n = 0;
    for (int j = 0; j < E; ++j) {
        int e = (ring_start + j) % E;
        if (counts[e] > 0) order[n++] = e;
    }
    *n_active = n;
}

/* ---------------------------------------------------------------------------------------
 * a2 / a5  q8_1 quantisation of one block of 32 fp32 values.  [QS] opening section and
 * "Identity" (q8_1, and the DS4 layout carrying d and s that Q4_1 needs).  Readings:
 *   amax = max |v_j|; an all-zero block stores q = 0, d = s = +0.
 *   d = amax / 127 in fp32 (IEEE division); q_j = roundf(v_j / d) (IEEE division, then
 *   round half away from zero; |v_j/d| never exceeds 127 by more than rounding, so no clamp);
 *   S = sum q_j (exact); stored d16 = fp16(d), s16 = fp16(d * (float)S) (fp32 product).
 * Pinned in tests/test_oracle_q8_1.py.
 * ------------------------------------------------------------------------------------- */
void orc_q8_1_block(const float *v, int8_t *q, uint16_t *d16, uint16_t *s16)
{
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
        float a = fabsf(v[j]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int j = 0; j < 32; ++j) q[j] = 0;
        *d16 = 0;
        *s16 = 0;
        return;
    }
    float d = amax / 127.0f;
    int S = 0;
    for (int j = 0; j < 32; ++j) {
        float r = roundf(v[j] / d);
        q[j] = (int8_t)(int)r;
        S += q[j];
    }
    *d16 = orc_f32_to_f16(d);
    *s16 = orc_f32_to_f16(d * (float)S);
}

/* One row of n values (n a multiple of 128) in the DS4 layout: each 128 values make a
 * 144-byte group, (d16, s16) of its 4 blocks first, then the 4 blocks' q. */
void orc_q8_1_row(const float *v, int n, uint8_t *out)
{
    for (int g = 0; g < n / 128; ++g) {
        uint8_t *grp = out + (size_t)g * 144;
        for (int j = 0; j < 4; ++j) {
            int8_t q[32];
            uint16_t d16, s16;
            orc_q8_1_block(v + (size_t)g * 128 + 32 * j, q, &d16, &s16);
            wr16(grp + 4 * j, d16);
            wr16(grp + 4 * j + 2, s16);
            memcpy(grp + 16 + 32 * j, q, 32);
        }
    }
}

/* The D4 layout.  [QS] "Identity" names D4 as the q8_1 layout the MMQ uses for Q8_0 (and
 * Q2_0, IQ2_XS) beside DS4 for Q4_1, and gives nothing but the name.  Reading: "D4" = four d
 * per 128-value group, kept in fp32 (the scale before it is rounded to fp16), no s (only Q4_1's
 * min term needs one): per 128 values a 144-byte group of 4 x fp32 d, then the 4 blocks' q.
 * The q are those of the DS4 form (the same fp32 d divides the values).
 * Pinned in tests/test_oracle_q8_1.py. */
void orc_q8_1_row_d4(const float *v, int n, uint8_t *out)
{
    for (int g = 0; g < n / 128; ++g) {
        uint8_t *grp = out + (size_t)g * 144;
        for (int j = 0; j < 4; ++j) {
            const float *b = v + (size_t)g * 128 + 32 * j;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i)
                if (fabsf(b[i]) > amax) amax = fabsf(b[i]);
            float d = amax / 127.0f;
            int8_t q[32];
            for (int i = 0; i < 32; ++i) q[i] = amax == 0.0f ? 0 : (int8_t)(int)roundf(b[i] / d);
            memcpy(grp + 4 * j, &d, 4);
            memcpy(grp + 16 + 32 * j, q, 32);
        }
    }
}

static void q8_1_row_layout(int layout, const float *v, int n, uint8_t *out)
{
    if (layout == ORC_D4)
        orc_q8_1_row_d4(v, n, out);
    else
        orc_q8_1_row(v, n, out);
}

/* [QS] opening section: the per-row ("gather") form quantises the T x K rows in expert
 * order, reading token src[r]/K's input row once for every row r. */
void orc_quantize_gather(const float *x, int T, int H, int K, const int32_t *src, int layout,
                         uint8_t *q8)
{
    size_t rb = orc_q8_1_row_bytes(H);
    int R = T * K;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < R; ++r) {
        int t = src[r] / K;
        q8_1_row_layout(layout, x + (size_t)t * H, H, q8 + (size_t)r * rb);
    }
}

/* [QS] opening section: the scatter form quantises each token once and writes the same
 * bytes to each of its K rows slot[t*K+k]. */
void orc_quantize_scatter(const float *x, int T, int H, int K, const int32_t *slot, int layout,
                          uint8_t *q8)
{
    size_t rb = orc_q8_1_row_bytes(H);
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        uint8_t *row = q8 + (size_t)slot[(size_t)t * K] * rb;
        q8_1_row_layout(layout, x + (size_t)t * H, H, row);
        for (int k = 1; k < K; ++k)
            memcpy(q8 + (size_t)slot[(size_t)t * K + k] * rb, row, rb);
    }
}

/* ---------------------------------------------------------------------------------------
 * a3  gather.  [G1] "What": one copy per expert (the per-expert form) of the expert's bytes
 * into its position in the MMQ group buffer; the batched form must leave the buffer byte for
 * byte as the per-expert copies do.  [G1] "What" (new test) and [G2] "What changes" (skipped ring entries):
 * a batch may start mid-group, so positions begin at first_pos.
 * Pinned in tests/test_oracle_gather_dot.py.
 * ------------------------------------------------------------------------------------- */
void orc_gather(const uint8_t *pool, const int64_t *expert_off, const int32_t *experts, int n,
                size_t expert_bytes, uint8_t *group_buf, int first_pos, size_t pos_stride)
{
    for (int j = 0; j < n; ++j)
        memcpy(group_buf + (size_t)(first_pos + j) * pos_stride,
               pool + expert_off[experts[j]], expert_bytes);
}

/* ---------------------------------------------------------------------------------------
 * a4 / a6  block dots (MMQ).  [G2] "What changes" and [QS] opening section: the grouped
 * quantised matmul on q8_1 activations.  For weight block b of row n and activation block b
 * of row r:  I_b = sum_j qw_j * qx_j  (integer),
 *   Q8_0:  y_b = dw * dx * I_b                (dx: fp16 d of DS4, or fp32 d of D4)
 *   Q4_1:  y_b = dw * dx * I_b + mw * sx      (w_j = dw*qw_j + mw, and sx = d*sum qx is what
 *                                             the DS4 layout stores for exactly this term)
 * and the row result is sum_b y_b over b ascending, in fp64 (fp16 -> fp64 is exact and, with
 * DS4, dw*dx*I_b has at most 41 significant bits, so every y_b is exact; with D4's fp32 dx it
 * has up to 55 and dw*dx*I_b is rounded once, to 2^-53 relative).
 * Pinned in tests/test_oracle_gather_dot.py against an fp64 dequantised brute force.
 * ------------------------------------------------------------------------------------- */
int32_t orc_block_idot(int wtype, const uint8_t *wblock, const int8_t *xq)
{
    int32_t I = 0;
    if (wtype != ORC_Q4_1) {
        const int8_t *qw = (const int8_t *)(wblock + 2);
        for (int j = 0; j < 32; ++j) I += (int32_t)qw[j] * (int32_t)xq[j];
    } else {
        const uint8_t *qs = wblock + 4;
        for (int j = 0; j < 16; ++j) {
            I += (int32_t)(qs[j] & 15) * (int32_t)xq[j];
            I += (int32_t)(qs[j] >> 4) * (int32_t)xq[j + 16];
        }
    }
    return I;
}

double orc_row_dot(int wtype, const uint8_t *wrow, const uint8_t *xrow_q8, int k_in)
{
    size_t bb = orc_block_bytes(wtype);
    double acc = 0.0;
    for (int b = 0; b < k_in / 32; ++b) {
        const uint8_t *grp = xrow_q8 + (size_t)(b / 4) * 144;
        double dx, sx = 0.0;
        if (wtype == ORC_Q8_0_D4) {  /* fp32 d, no s */
            float d32;
            memcpy(&d32, grp + 4 * (b % 4), 4);
            dx = (double)d32;
        } else {
            dx = orc_f16_to_f64(rd16(grp + 4 * (b % 4)));
            sx = orc_f16_to_f64(rd16(grp + 4 * (b % 4) + 2));
        }
        const int8_t *xq = (const int8_t *)(grp + 16 + 32 * (b % 4));
        const uint8_t *blk = wrow + (size_t)b * bb;
        double dw = orc_f16_to_f64(rd16(blk));
        double I = (double)orc_block_idot(wtype, blk, xq);
        double y = dw * dx * I;
        if (wtype == ORC_Q4_1) y += orc_f16_to_f64(rd16(blk + 2)) * sx;
        acc += y;
    }
    return acc;
}

/* Raw integer block dots of n_rows activation rows against the n_out rows of one weight
 * matrix: out[(r*n_out + n)*(k_in/32) + b] = I_b. */
void orc_block_dots(int wtype, const uint8_t *wmat, int n_out, int k_in,
                    const uint8_t *act_q8, int n_rows, int32_t *out)
{
    size_t bb = orc_block_bytes(wtype), rb = orc_q8_1_row_bytes(k_in);
    int nb = k_in / 32;
    for (int r = 0; r < n_rows; ++r)
        for (int n = 0; n < n_out; ++n)
            for (int b = 0; b < nb; ++b) {
                const uint8_t *grp = act_q8 + (size_t)r * rb + (size_t)(b / 4) * 144;
                const int8_t *xq = (const int8_t *)(grp + 16 + 32 * (b % 4));
                out[((size_t)r * n_out + n) * nb + b] =
                    orc_block_idot(wtype, wmat + ((size_t)n * nb + b) * bb, xq);
            }
}

/* Products of n_rows activation rows with every row of one weight matrix (fp64):
 * out[r*n_out + n] = orc_row_dot(row n of wmat, activation row r). */
void orc_matrix_rows(int wtype, const uint8_t *wmat, int n_out, int k_in, const uint8_t *act_q8,
                  int n_rows, double *out)
{
    size_t wrb = (size_t)(k_in / 32) * orc_block_bytes(wtype), arb = orc_q8_1_row_bytes(k_in);
#pragma omp parallel for schedule(static)
    for (int r = 0; r < n_rows; ++r)
        for (int n = 0; n < n_out; ++n)
            out[(size_t)r * n_out + n] =
                orc_row_dot(wtype, wmat + (size_t)n * wrb, act_q8 + (size_t)r * arb, k_in);
}

/* ---------------------------------------------------------------------------------------
 * a4..a6  one routed row through one expert.  [QS] opening section: the down-projection
 * input is quantised to q8_1 again (the page lists these quantisations as unchanged).  The pages do not
 * name the activation; this reads it as SwiGLU: h_f = silu(g_f) * u_f with
 * silu(z) = z / (1 + e^-z), gate = the expert's first F rows, up = the next F, no bias.
 * g, u and h in fp64; h is stored fp32 and re-quantised along F with orc_q8_1_row; the down
 * product Dm_i = sum over F/32 blocks of the down matrix's row i (fp64).
 * Pinned in tests/test_oracle_layer.py (dense special case against numpy.matmul).
 * ------------------------------------------------------------------------------------- */
void orc_expert_row(int wtype, const uint8_t *expert, int H, int F, const uint8_t *xrow_q8,
                    float *h, uint8_t *hq8, double *dm)
{
    size_t bb = orc_block_bytes(wtype);
    size_t gu_row = (size_t)(H / 32) * bb, dn_row = (size_t)(F / 32) * bb;
    const uint8_t *gate = expert;
    const uint8_t *up = expert + (size_t)F * gu_row;
    const uint8_t *down = expert + (size_t)2 * F * gu_row;
    for (int f = 0; f < F; ++f) {
        double g = orc_row_dot(wtype, gate + (size_t)f * gu_row, xrow_q8, H);
        double u = orc_row_dot(wtype, up + (size_t)f * gu_row, xrow_q8, H);
        h[f] = (float)(g / (1.0 + exp(-g)) * u);
    }
    q8_1_row_layout(wtype == ORC_Q8_0_D4 ? ORC_D4 : ORC_DS4, h, F, hq8);
    for (int i = 0; i < H; ++i) dm[i] = orc_row_dot(wtype, down + (size_t)i * dn_row, hq8, F);
}

/* ---------------------------------------------------------------------------------------
 * a7  combine.  [CS] "What it does": Dm holds the expert rows without their routing weights,
 * which the combine applies.  out[t,i] = sum_{k<K} w[t,k] * Dm[slot[t*K+k], i], k ascending, fp64,
 * stored fp32.  Pinned in tests/test_oracle_layer.py.
 * ------------------------------------------------------------------------------------- */
void orc_combine(const double *Dm, const int32_t *slot, const float *w, int T, int K, int H,
                 float *out)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < H; ++i) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += (double)w[(size_t)t * K + k] * Dm[(size_t)slot[(size_t)t * K + k] * H + i];
            out[(size_t)t * H + i] = (float)acc;
        }
}

/* ---------------------------------------------------------------------------------------
 * a1..a7  the layer, as the plain definition: maps, one quantisation per token scattered to
 * its rows, every routed row through its expert's weights (read where the pool holds them:
 * a gather only moves those bytes), then the weighted combine.
 * ------------------------------------------------------------------------------------- */
int orc_prefill_layer(const float *x, int T, int H, int F, int E, int K,
                      const int32_t *idx, const float *w, int wtype,
                      const uint8_t *pool, const int64_t *expert_off,
                      float *out, uint8_t *q8x, float *h, uint8_t *hq8, double *Dm)
{
    if (T < 1 || K < 1 || K > E || H % 128 || F % 128) return -1;
    int R = T * K;
    size_t xrb = orc_q8_1_row_bytes(H), hrb = orc_q8_1_row_bytes(F);
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *src = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t n_active = 0;
    orc_build_maps(idx, T, K, E, 0, counts, offsets, src, slot, order, &n_active);

    uint8_t *q8 = q8x ? q8x : (uint8_t *)malloc(xrb * (size_t)R);
    double *dm = Dm ? Dm : (double *)malloc(sizeof(double) * (size_t)R * H);
    orc_quantize_scatter(x, T, H, K, slot, wtype == ORC_Q8_0_D4 ? ORC_D4 : ORC_DS4, q8);

#pragma omp parallel
    {
        float *hrow = (float *)malloc(sizeof(float) * (size_t)F);
        uint8_t *hqrow = (uint8_t *)malloc(hrb);
#pragma omp for schedule(dynamic, 4)
        for (int r = 0; r < R; ++r) {
            int e = idx[src[r]];
            orc_expert_row(wtype, pool + expert_off[e], H, F, q8 + (size_t)r * xrb, hrow, hqrow,
                           dm + (size_t)r * H);
            if (h) memcpy(h + (size_t)r * F, hrow, sizeof(float) * (size_t)F);
            if (hq8) memcpy(hq8 + (size_t)r * hrb, hqrow, hrb);
        }
        free(hqrow);
        free(hrow);
    }
    orc_combine(dm, slot, w, T, K, H, out);

    if (!Dm) free(dm);
    if (!q8x) free(q8);
    free(order);
    free(slot);
    free(src);
    free(offsets);
    free(counts);
    return 0;
}

void orc_token_out(const float *x_row, int H, int F, int K, const int32_t *idx_row,
                   const float *w_row, int wtype, const uint8_t *pool, const int64_t *expert_off,
                   float *out_row)
{
    uint8_t *xq = (uint8_t *)malloc(orc_q8_1_row_bytes(H));
    float *hrow = (float *)malloc(sizeof(float) * (size_t)F);
    uint8_t *hq = (uint8_t *)malloc(orc_q8_1_row_bytes(F));
    double *dm = (double *)malloc(sizeof(double) * (size_t)K * H);
    q8_1_row_layout(wtype == ORC_Q8_0_D4 ? ORC_D4 : ORC_DS4, x_row, H, xq);
    for (int k = 0; k < K; ++k)
        orc_expert_row(wtype, pool + expert_off[idx_row[k]], H, F, xq, hrow, hq,
                       dm + (size_t)k * H);
    for (int i = 0; i < H; ++i) {
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += (double)w_row[k] * dm[(size_t)k * H + i];
        out_row[i] = (float)acc;
    }
    free(dm);
    free(hq);
    free(hrow);
    free(xq);
}
