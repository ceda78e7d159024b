/*
 * qdr_oracle.h -- plain scalar CPU oracle for the quantized Delta-rule decode step.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py may load or call this library. The product library (HIP kernels
 * behind include/qdr.h) never links, includes or calls anything here, and the two
 * share no source: this file, qdr_oracle.c and oracle/__init__.py are written from
 * the arithmetic contract alone.
 *
 * Sources (cited by page title and section; figures/abstracts as labelled there):
 *  [DEV]   dev.to, "Uniform INT8 on recurrent states is a default, not a decision",
 *          section "The state is a running sum, not a buffer"  (the Delta-rule update
 *          S <- S(I - k k^T) + v k^T and its projection reading).
 *  [STEP]  "STEPQuant: When and Where Errors Matter in Delta-Rule Recurrent State
 *          Quantization" (signal-papers page): Fig. 1(b) and Fig. 4 / Figure B1 (gate
 *          half-life as the precision-allocation signal, longest-lived quarter),
 *          Fig. 5 / Figure B2 (128x128 states, row/column outliers), Key contributions
 *          (nominal 6-bit and 4-bit budgets).
 *  [ABS]   thelatestinai page titled "DAMP: Decay-Aware Mixed-Precision Recurrent-State
 *          Quantization": the STEPQuant abstract (key-row and value-column scales,
 *          lifetime-based precision), the LeapQuant abstract (per-window quantization
 *          with high-precision buffered updates) and the DASC abstract (GDN head-wise,
 *          KDA channel-wise decay).
 *  [MEAS]  freedom251, "Recurrent-state INT8 quantization: measure before you make it
 *          the default", section "Memory and speed gains are implementation-specific"
 *          (packed pages per request, 144 MiB FP32 vs 28.609 MiB packed).
 *
 * Conventions. One unit = one (request, head) state S in R^{dv x dk}, row i = value
 * index, column j = key channel, o = S q. The pages' "key row j" is column j of S and
 * their "value column i" is row i of S. All state-level quantities are IEEE fp32 (the
 * pages' baseline is an FP32 state with fp32 scales); the two dot products are
 * accumulated in fp64 and rounded once. Every floating-point operation below is one
 * IEEE rounding in the stated precision (built with -ffp-contract=off, no fast-math).
 *
 * parity unpinned: the pages give no formula for their fitted scales. The two-stage
 * absmax rule implemented here is the plainest reading of the scale-fitting passage;
 * its invariants (half-step bound, idempotence, full code range) are pinned by tests.
 */
#ifndef QDR_ORACLE_H
#define QDR_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OREF_GDN 0 /* scalar gate per (request, head)            */
#define OREF_KDA 1 /* diagonal gate, one value per key channel    */

/* S0: lifetime-based bit map. GDN: halflife[n_head] (one per head), every channel of a
 * head gets the head's width. KDA: halflife[n_head*dk], ranked within each head.
 * Ranking is by (half-life, index) ascending; the shortest-lived floor(n/4) units get
 * 4 bits, the longest-lived floor(n/4) get 8 bits, the rest 6 bits.
 * bits_out is [n_head][dk]. Returns 0, or -1 on bad arguments. */
int oref_assign_bits(int gate, int n_head, int dk, const double *halflife, uint8_t *bits_out);

/* Packed tile format (own implementation of the format spec). Physical key order:
 * channels sorted by width descending (8, 6, 4), ties by channel index. perm[p] is the
 * logical channel at physical position p. Width classes must come in multiples of 32
 * channels. seg_bits[s] is the width of physical positions 32s..32s+31.
 * Returns the tile size in bytes, or -1 if the bit map is not representable. */
long oref_layout(int dv, int dk, const uint8_t *bits, uint8_t *perm, uint8_t *seg_bits);

/* codes: [dv][dk] logical order, signed. tile: packed bytes. 0 / -1. */
int oref_pack(int dv, int dk, const uint8_t *bits, const int8_t *codes, uint8_t *tile);
int oref_unpack(int dv, int dk, const uint8_t *bits, const uint8_t *tile, int8_t *codes);

/* Scale refit + requantization (two-stage absmax, key axis first). S: [dv][dk] fp32.
 * Outputs codes [dv][dk], R[dk] (key-row scales, logical order), c[dv] (value-column). */
void oref_quantize(int dv, int dk, const uint8_t *bits, const float *S, int8_t *codes,
                   float *R, float *c);

/* Dequantized state S_hat[i][j] = fl(code * fl(R_j * c_i)): the code times the step of
 * its entry, the product of its key-row and value-column scales. */
void oref_dequantize(int dv, int dk, const int8_t *codes, const float *R, const float *c,
                     float *S);

/* Scale rules. STEP: the two-stage absmax of the STEPQuant reading (key rows, then value
 * columns). The comparison baselines of the dev.to page's "four options" section, in the
 * same (R_j, c_i) format with c = 1: KEYROW, per-row INT8 (one range per key row, the
 * first stage alone); TENSOR, uniform per-tensor INT8 (one range for the whole state,
 * symmetric: the zero point is the code 0). */
#define OREF_RULE_STEP 0
#define OREF_RULE_KEYROW 1
#define OREF_RULE_TENSOR 2

/* Quantize with a scale rule (oref_quantize is rule STEP). */
void oref_quantize_rule(int dv, int dk, const uint8_t *bits, const float *S, int8_t *codes,
                        float *R, float *c, int rule);

/* One decode step on one unit, in place on (codes, R, c).
 * a: GDN -> a[0]; KDA -> a[dk]. o[dv] receives S_new q.
 * S_new (optional, may be NULL) receives the fp32 state before requantization. */
void oref_step(int dv, int dk, int gate, const uint8_t *bits, int8_t *codes, float *R,
               float *c, const float *q, const float *k, const float *v, const float *a,
               float b, float *o, float *S_new);

/* oref_step with the requantization of a given scale rule (oref_step is rule STEP). */
void oref_step_rule(int dv, int dk, int gate, const uint8_t *bits, int8_t *codes, float *R,
                    float *c, const float *q, const float *k, const float *v, const float *a,
                    float b, float *o, float *S_new, int rule);

/* One window of W tokens on one unit (LeapQuant reading): the state is the dequantized
 * low-bit state at the window start; the exact recurrence runs in fp64 over the W
 * tokens, o_t = S_t q_t, and the state is requantized once at the end.
 * q,k: [W][dk]; v: [W][dv]; a: [W] (GDN) or [W][dk] (KDA); b: [W]; o: [W][dv].
 * S_end (optional) receives the fp32-rounded state before requantization. */
void oref_window(int dv, int dk, int gate, const uint8_t *bits, int8_t *codes, float *R,
                 float *c, int W, const float *q, const float *k, const float *v,
                 const float *a, const float *b, float *o, float *S_end);

/* One step of the unquantized recurrence in fp64 (pre-warm and error reference).
 * S: [dv][dk] fp64, updated in place. o (optional): [dv]. */
void oref_recur_fp64(int dv, int dk, int gate, double *S, const float *q, const float *k,
                     const float *v, const float *a, float b, float *o);

/* ---- batched drivers over the packed pool --------------------------------------
 * Pool layout: packed[n_req][req_bytes], heads concatenated in order inside a request;
 * row_scale[n_req][n_head][dk] in PHYSICAL key order; col_scale[n_req][n_head][dv];
 * q,k,a(KDA): [n_req][n_head][dk] logical order; v,o: [n_req][n_head][dv];
 * a(GDN), b: [n_req][n_head]. Units [u0, u1) of the flattened (req, head) index run.
 * Returns 0 or -1. */
long oref_request_bytes(int n_head, int dv, int dk, const uint8_t *bits);
int oref_quantize_pool(int n_req, int n_head, int dv, int dk, const uint8_t *bits,
                       const float *S, uint8_t *packed, float *row_scale, float *col_scale);
int oref_dequantize_pool(int n_req, int n_head, int dv, int dk, const uint8_t *bits,
                         const uint8_t *packed, const float *row_scale,
                         const float *col_scale, float *S);
int oref_step_pool(int n_req, int n_head, int dv, int dk, int gate, const uint8_t *bits,
                   uint8_t *packed, float *row_scale, float *col_scale, const float *q,
                   const float *k, const float *v, const float *a, const float *b, float *o,
                   long u0, long u1);
/* The pool drivers with a scale rule (the functions above use rule STEP). */
int oref_quantize_pool_rule(int n_req, int n_head, int dv, int dk, const uint8_t *bits,
                            const float *S, uint8_t *packed, float *row_scale, float *col_scale,
                            int rule);
int oref_step_pool_rule(int n_req, int n_head, int dv, int dk, int gate, const uint8_t *bits,
                        uint8_t *packed, float *row_scale, float *col_scale, const float *q,
                        const float *k, const float *v, const float *a, const float *b, float *o,
                        long u0, long u1, int rule);
/* Window over W tokens for every unit: token inputs are [W][n_req][n_head][...]. */
int oref_window_pool(int n_req, int n_head, int dv, int dk, int gate, const uint8_t *bits,
                     uint8_t *packed, float *row_scale, float *col_scale, int W,
                     const float *q, const float *k, const float *v, const float *a,
                     const float *b, float *o, long u0, long u1);

/* ---- compensator tokens ([ABS] LeapQuant abstract: the largest outliers kept as a few
 * high-precision tokens sharing the real tokens' update path; the residual quantized).
 * Reading: a token is one entry x at (i, j) in fp32 (the rank-one term x e_i e_j^T);
 * the m tokens are the m nonzero entries of largest |S| (equal magnitudes: smaller
 * flat index i*dk + j first), in that order; unused slots hold OREF_TOK_EMPTY and 0.
 * tok_idx / tok_val: [m] per unit (pools: [n_req][n_head][m]); flat index in logical
 * key order. dv*dk must be below 65535. */
#define OREF_TOK_EMPTY 0xFFFFu
/* selects the tokens of S and sets their entries to 0 in place (S becomes the residual) */
void oref_comp_select(int dv, int dk, int m, float *S, uint16_t *tok_idx, float *tok_val);
/* S += tokens */
void oref_comp_add(int m, const uint16_t *tok_idx, const float *tok_val, float *S);
/* tokens of S, then the residual quantized by rule STEP */
void oref_comp_quantize(int dv, int dk, const uint8_t *bits, const float *S, int m,
                        int8_t *codes, float *R, float *c, uint16_t *tok_idx, float *tok_val);
/* dequantized residual plus the tokens */
void oref_comp_dequantize(int dv, int dk, const int8_t *codes, const float *R, const float *c,
                          int m, const uint16_t *tok_idx, const float *tok_val, float *S);
/* oref_window started from the dequantized residual plus the tokens; at the end the new
 * tokens are selected from the fp32 state and the residual is quantized (in place on
 * codes, R, c, tok_idx, tok_val). S_end (optional): the state before the selection. */
void oref_comp_window(int dv, int dk, int gate, const uint8_t *bits, int8_t *codes, float *R,
                      float *c, int m, uint16_t *tok_idx, float *tok_val, int W, const float *q,
                      const float *k, const float *v, const float *a, const float *b, float *o,
                      float *S_end);
int oref_comp_quantize_pool(int n_req, int n_head, int dv, int dk, const uint8_t *bits,
                            const float *S, int m, uint8_t *packed, float *row_scale,
                            float *col_scale, uint16_t *tok_idx, float *tok_val);
int oref_comp_dequantize_pool(int n_req, int n_head, int dv, int dk, const uint8_t *bits,
                              const uint8_t *packed, const float *row_scale,
                              const float *col_scale, int m, const uint16_t *tok_idx,
                              const float *tok_val, float *S);
int oref_comp_window_pool(int n_req, int n_head, int dv, int dk, int gate, const uint8_t *bits,
                          uint8_t *packed, float *row_scale, float *col_scale, int m,
                          uint16_t *tok_idx, float *tok_val, int W, const float *q,
                          const float *k, const float *v, const float *a, const float *b,
                          float *o, long u0, long u1);

/* ---- DAMP-style storage variant ([MEAS] section "DAMP: accuracy depends on the task")
 * Per unit, 16 selected key channels are kept in IEEE binary16 and the other 112 in
 * INT8 with one range per key row and stochastic rounding. Physical positions 0..15 are
 * the selected channels, 16..127 the others, each in increasing channel order
 * (perm[p] = logical channel). Storage per unit: half[dv][16], codes[dv][112], R[112].
 * Arithmetic:
 *   dequantize   S = f32(h) (selected) or fl(code * R_j)
 *   gate         S' = fl(f32(h) * a_j) or fl(code * fl(a_j * R_j))   (GDN: a_j = a)
 *   u_i          fl32(sum_j S'_ij k_j), one fp64 sum over the key channels j = 0..127 in
 *                logical order; w_i = fl(b fl(v_i - u_i)); S_new = fma(w_i, k_j, S'_ij);
 *                o_i = fl32(sum_j S_new_ij q_j), the same way
 *   requantize   selected: binary16 round-to-nearest-even; others: A_j = max_i |S_ij|
 *                (1 if 0), R_j = fl(A_j/127), y = fl(S * fl(1/A_j)),
 *                code = clamp(floor(y*127 + u), +-127) in fp64, u = uniform [0, 1):
 *                byte p mod 16 (little-endian over the four words) of Philox4x32-7 for
 *                counter (i*8 + p/16, unit, step lo, step hi) and key seed, times 2^-8. */
#define OREF_DAMP_HALF 16
#define OREF_DAMP_PHILOX_ROUNDS 7

/* Philox4x32 with `rounds` rounds (the key bumped between rounds); _10 is the paper's
 * default, kept for its published known answers */
void oref_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int rounds, uint32_t out[4]);
void oref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint16_t oref_f32_to_f16(float x);
float oref_f16_to_f32(uint16_t h);
int oref_damp_perm(int dk, const uint8_t *sel, uint8_t *perm);
void oref_damp_dequantize(int dv, const uint8_t *perm, const uint16_t *half, const int8_t *codes,
                          const float *R, float *S);
void oref_damp_quantize(int dv, const uint8_t *perm, const float *S, uint16_t *half,
                        int8_t *codes, float *R, uint64_t seed, uint32_t unit, uint64_t step);
void oref_damp_step(int dv, int gate, const uint8_t *perm, uint16_t *half, int8_t *codes,
                    float *R, const float *q, const float *k, const float *v, const float *a,
                    float b, float *o, uint64_t seed, uint32_t unit, uint64_t step);
int oref_damp_quantize_pool(int n_unit, int n_head, int dv, const uint8_t *perm, const float *S,
                            uint16_t *half, int8_t *codes, float *R, uint64_t seed,
                            uint64_t step);
int oref_damp_dequantize_pool(int n_unit, int n_head, int dv, const uint8_t *perm,
                              const uint16_t *half, const int8_t *codes, const float *R,
                              float *S);
int oref_damp_step_pool(int n_unit, int n_head, int dv, int gate, const uint8_t *perm,
                        uint16_t *half, int8_t *codes, float *R, const float *q, const float *k,
                        const float *v, const float *a, const float *b, float *o, uint64_t seed,
                        uint64_t step, long u0, long u1);

#ifdef __cplusplus
}
#endif
#endif
