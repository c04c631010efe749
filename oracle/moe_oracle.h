/*
 * moe_oracle.h -- plain CPU oracle for the prompt-path (prefill) MoE expert layer.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or helper
 * with the HIP library under quantized_expert_grouped_amd/csrc, and neither includes
 * nor links the other.
 *
 * What it computes is taken from the pages on the Strata prompt path:
 *   [G1] "#439 prefill: a group's expert gathers in one launch (bit-identical, long prompts +4%)"
 *   [G2] "Prompt path: an MMQ group's experts gathered in one launch, after one wait, released
 *         by one event (-9% on a 32K prompt, same output)"
 *   [QS] "#1368 prefill: quantize each token's MoE input once and scatter it to its k rows
 *         (the same bytes)"
 *   [CS] "#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto hands a small chunk's least-routed experts
 *         to the idle CPU pool (opt-in)"
 * Where the pages are silent the plainest reading is taken; each such reading is named at the
 * function that makes it.
 *
 * Byte formats (little endian throughout):
 *   Q8_0 weight block, 34 B : fp16 d | int8 q[32]                     w_j = d*q_j
 *   Q4_1 weight block, 20 B : fp16 d | fp16 m | u8 qs[16]             w_j = d*q_j + m
 *                             qs[j] low nibble = element j, high nibble = element j+16
 *   q8_1 activation row     : per 128 values one 144 B group:
 *                             4 x (fp16 d, fp16 s) for its 4 blocks of 32, then 4 x 32 int8 q
 *   expert                  : gate [F rows x H/32 blocks] | up [F x H/32] | down [H x F/32],
 *                             every matrix row-major with blocks along the reduction dimension.
 *
 * Parity pins: every function below is pinned by a CPU test against something other than
 * itself (closed forms, an independent numpy brute force, library routines, invariants the
 * pages state).  The test file that pins each function is named in its comment.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight type, and with it the activations' q8_1 layout:
 *   ORC_Q8_0    Q8_0 weights, DS4 activations (4 x (fp16 d, fp16 s) per 128 values)
 *   ORC_Q4_1    Q4_1 weights, DS4 activations
 *   ORC_Q8_0_D4 Q8_0 weights, D4 activations (4 x fp32 d per 128 values, no s) */
enum { ORC_Q8_0 = 0, ORC_Q4_1 = 1, ORC_Q8_0_D4 = 2 };
enum { ORC_DS4 = 0, ORC_D4 = 1 };

/* --- number formats ------------------------------------------------------------------- */
uint16_t orc_f32_to_f16(float f);      /* IEEE binary16, round to nearest even, subnormals kept */
double   orc_f16_to_f64(uint16_t h);   /* exact */
size_t   orc_block_bytes(int wtype);   /* 34 (Q8_0) or 20 (Q4_1) */
size_t   orc_expert_bytes(int H, int F, int wtype);
size_t   orc_q8_1_row_bytes(int n);    /* n/128 * 144 */

/* --- threads -------------------------------------------------------------------------- */
void orc_set_threads(int n);
int  orc_get_threads(void);

/* --- a0 routing ------------------------------------------------------------------------- */
void orc_route_topk(const float *logits, int T, int E, int K, int32_t *idx, float *w);

/* --- a1 maps ---------------------------------------------------------------------------- */
void orc_build_maps(const int32_t *idx, int T, int K, int E, int ring_start,
                    int32_t *counts, int32_t *offsets, int32_t *src, int32_t *slot,
                    int32_t *order, int32_t *n_active);

/* --- a2 / a5 q8_1 ------------------------------------------------------------------------ */
void orc_q8_1_block(const float *v, int8_t *q, uint16_t *d16, uint16_t *s16);
void orc_q8_1_row(const float *v, int n, uint8_t *out);
void orc_q8_1_row_d4(const float *v, int n, uint8_t *out);
void orc_quantize_gather(const float *x, int T, int H, int K, const int32_t *src, int layout,
                         uint8_t *q8);
void orc_quantize_scatter(const float *x, int T, int H, int K, const int32_t *slot, int layout,
                          uint8_t *q8);

/* --- a3 gather ------------------------------------------------------------------------- */
void orc_gather(const uint8_t *pool, const int64_t *expert_off, const int32_t *experts, int n,
                size_t expert_bytes, uint8_t *group_buf, int first_pos, size_t pos_stride);

/* --- a4 / a6 block dots ----------------------------------------------------------------- */
int32_t orc_block_idot(int wtype, const uint8_t *wblock, const int8_t *xq);
double  orc_row_dot(int wtype, const uint8_t *wrow, const uint8_t *xrow_q8, int k_in);
void    orc_block_dots(int wtype, const uint8_t *wmat, int n_out, int k_in,
                       const uint8_t *act_q8, int n_rows, int32_t *out);
void    orc_matrix_rows(int wtype, const uint8_t *wmat, int n_out, int k_in,
                     const uint8_t *act_q8, int n_rows, double *out);

/* --- a4..a6 one routed row through one expert ------------------------------------------ */
void orc_expert_row(int wtype, const uint8_t *expert, int H, int F, const uint8_t *xrow_q8,
                    float *h, uint8_t *hq8, double *dm);

/* --- a7 combine --------------------------------------------------------------------------- */
void orc_combine(const double *Dm, const int32_t *slot, const float *w, int T, int K, int H,
                 float *out);

/* --- a1..a7 the layer ----------------------------------------------------------------------
 * Debug outputs may be NULL: q8x [R x H/128*144], h [R x F] fp32, hq8 [R x F/128*144], Dm [R x H]. */
int orc_prefill_layer(const float *x, int T, int H, int F, int E, int K,
                      const int32_t *idx, const float *w, int wtype,
                      const uint8_t *pool, const int64_t *expert_off,
                      float *out, uint8_t *q8x, float *h, uint8_t *hq8, double *Dm);

/* One token's output row at any size: out[t] computed from x[t] and its K routes alone. */
void orc_token_out(const float *x_row, int H, int F, int K, const int32_t *idx_row,
                   const float *w_row, int wtype, const uint8_t *pool, const int64_t *expert_off,
                   float *out_row);

#ifdef __cplusplus
}
#endif
#endif
