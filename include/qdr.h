/*
 * qdr.h -- C ABI of libqdr: the per-token decode step of a Delta-rule linear-attention
 * layer over a low-bit quantized recurrent state, on one MI355X (gfx950).
 *
 * Every (request, head) pair is one "unit": a state S in R^{dv x dk}, dv = dk = 128,
 * row i = value index, column j = key channel, readout o = S q. The pages' "key row j"
 * is column j of S and their "value column i" is row i of S.
 *
 * Sources, cited by page title and section:
 *  - dev.to, "Uniform INT8 on recurrent states is a default, not a decision", section
 *    "The state is a running sum, not a buffer": the Delta-rule update
 *    S <- S (I - k k^T) + v k^T.
 *  - thelatestinai page titled "DAMP: Decay-Aware Mixed-Precision Recurrent-State
 *    Quantization": the STEPQuant abstract (precision by error and memory lifetime;
 *    key-row and value-column scales), the LeapQuant abstract (per-window quantization:
 *    outputs from the fixed low-bit state plus high-precision buffered updates, one
 *    quantization at the window end) and the DASC abstract (GDN decays per head, KDA per
 *    key channel).
 *  - "STEPQuant: When and Where Errors Matter in Delta-Rule Recurrent State
 *    Quantization" (signal-papers page): Fig. 1(b) and Fig. 4 / Figure B1 (gate
 *    half-life orders the units; the longest-lived quarter matters most), Fig. 5 /
 *    Figure B2 (128x128 states with row and column outliers).
 *  - freedom251, "Recurrent-state INT8 quantization: measure before you make it the
 *    default", section "Memory and speed gains are implementation-specific": per-request
 *    packed pages; the checklist under "How to decide for a deployment" counts codes,
 *    scales and precision maps as state memory.
 *
 * Conventions shared by every entry point
 *  - Return value: QDR_OK (0) or a negative QDR_E* code. On error nothing is launched
 *    and qdr_last_error() (thread-local) describes the failure. No exception crosses
 *    the ABI.
 *  - Pointers: every array argument is a DEVICE pointer (memory of the GPU current on
 *    the calling thread) except qdr_desc.bits and the host arrays of qdr_assign_bits /
 *    qdr_state_bytes, which are HOST pointers. Device arrays must be 16-byte aligned
 *    and contiguous in the stated layout. The caller owns every buffer and the stream;
 *    the library allocates and frees nothing. Only qdr_init_state and qdr_damp_init
 *    synchronize (the stream, once, after copying their small host-built metadata
 *    table); every other call only enqueues work.
 *  - Host cost per call: the descriptor's bit map is validated and summarised once and
 *    the summary kept (the last 8 distinct maps, compared in full on every call, so an
 *    edited map is never taken for a cached one); a decode call with a known map does no
 *    per-head work and no heap allocation on the host.
 *  - stream: a hipStream_t passed as void* (NULL = the null stream). All device work
 *    is enqueued asynchronously on it in call order.
 *  - Non-finite inputs are undefined behaviour and are not checked.
 *  - Layouts (all fp32, row-major):
 *      q, k        [n_req][n_head][dk]   logical key-channel order
 *      v, o        [n_req][n_head][dv]
 *      a (GDN)     [n_req][n_head]       scalar gate
 *      a (KDA)     [n_req][n_head][dk]   per-key-channel gate, logical order
 *      b           [n_req][n_head]       write strength
 *      row_scale   [n_req][n_head][dk]   key-row scales R_j, PHYSICAL key order
 *      col_scale   [n_req][n_head][dv]   value-column scales c_i
 *      packed      [n_req][req_bytes]    heads concatenated inside a request
 *  - Packed tile of one head: key channels sorted by width (8, 6, 4; ties by index)
 *    give the physical order; physical positions 32s..32s+31 form segment s (one
 *    width b_s); segment s stores dv rows of 32 codes, each row 4*b_s bytes, code of
 *    position 32s+m in bits [m*b, m*b+b) of the row's little-endian bit stream, as the
 *    offset-binary field code + 2^(b-1). Tile bytes = 16 * sum_j bits_j.
 */
#ifndef QDR_H
#define QDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QDR_OK 0
#define QDR_EINVAL (-1)       /* null / negative / inconsistent argument            */
#define QDR_EUNSUPPORTED (-2) /* dims != 128, bits not in {4,6,8}, bad width counts,  */
                              /* window position out of range                       */
#define QDR_EALIGN (-3)       /* a device pointer is not 16-byte aligned              */
#define QDR_EHIP (-4)         /* HIP launch or runtime error (text in last_error)     */

#define QDR_GATE_GDN 0 /* scalar gate per (request, head) */
#define QDR_GATE_KDA 1 /* diagonal gate, one value per key channel */

/* Scale rules. STEP (default): the STEPQuant reading, key-row ranges then value-column
 * scales. The comparison baselines of the dev.to page's section on the quantization
 * options, in the same (R_j, c_i) format with every c_i = 1: KEYROW, per-row INT8 (one
 * range per key row); TENSOR, uniform per-tensor INT8 (one range per state; symmetric,
 * the zero point is code 0). */
#define QDR_RULE_STEP 0
#define QDR_RULE_KEYROW 1
#define QDR_RULE_TENSOR 2

typedef struct qdr_desc {
    int32_t n_req;        /* requests (>= 0; 0 makes every call a no-op)            */
    int32_t n_head;       /* heads per request (1..1024)                            */
    int32_t dk, dv;       /* must both be 128                                       */
    int32_t gate;         /* QDR_GATE_GDN or QDR_GATE_KDA                           */
    const uint8_t *bits;  /* HOST [n_head][dk], each in {4,6,8}; per head, the count */
                          /* of channels of each width is a multiple of 32           */
    int32_t window;       /* 1 <= W <= 256 for qdr_decode_window, 0 otherwise       */
    int32_t rule;         /* QDR_RULE_*: scale rule of qdr_quantize_state and          */
                          /* qdr_decode_step; window and chunk mode take QDR_RULE_STEP */
} qdr_desc;

/* S0 -- lifetime-based bit map (STEPQuant abstract; STEPQuant page Fig. 1(b), Fig. 4 /
 * Figure B1). HOST only. Units ranked by (half-life, index) ascending: the shortest
 * floor(n/4) get 4 bits, the longest floor(n/4) get 8 bits, the rest 6 bits.
 *   GDN: halflife[n_head], the unit is a head (all its channels share the width).
 *   KDA: halflife[n_head][dk], units are the key channels of each head.
 * bits_out: HOST [n_head][dk]. Errors: QDR_EINVAL. */
int qdr_assign_bits(int32_t gate, int32_t n_head, int32_t dk, const double *halflife,
                    uint8_t *bits_out);

/* Sizes of the caller-owned buffers for a descriptor (HOST outputs, any may be NULL).
 * The state is kept as per-request packed pages (freedom251 page, section "Memory and
 * speed gains are implementation-specific"), and its footprint counts the codes, the
 * scales and the precision map (the same page's checklist under "How to decide for a
 * deployment"):
 *   packed  -- n_req * req_bytes bytes (codes)
 *   scales  -- bytes of ONE of row_scale / col_scale (n_req*n_head*128*4)
 *   meta    -- bytes of the device metadata table written by qdr_init_state
 *   window_buf -- bytes of the window buffer (0 when desc->window == 0)
 * Errors: QDR_EINVAL, QDR_EUNSUPPORTED. */
int qdr_state_bytes(const qdr_desc *desc, size_t *packed, size_t *scales, size_t *meta,
                    size_t *window_buf);

/* Initialise: write the metadata table -- the precision map as the kernels read it
 * (per-head tile offsets, segment widths and the physical key order; freedom251 page,
 * checklist under "How to decide for a deployment") -- and the zero state (every code 0,
 * R_j = 1/Qmax_j, c_i = 1), i.e. the state that qdr_quantize_state gives for S = 0.
 * Copies the table from the host and synchronizes `stream` once. Errors: all codes. */
int qdr_init_state(const qdr_desc *desc, void *packed, float *row_scale, float *col_scale,
                   void *meta, void *stream);

/* Refit scales and quantize a caller fp32 state S [n_req][n_head][dv][dk] (logical key
 * order) into (packed, row_scale, col_scale): the scale rule of the STEPQuant abstract
 * read as a two-stage absmax, key axis first:
 *   A_j = max_i |S_ij| (1 if 0), R_j = A_j/Qmax_j, y_ij = S_ij*(1/A_j),
 *   c_i = max_j |y_ij| (1 if 0), code_ij = RNE(y_ij * (Qmax_j*(1/c_i))).
 * desc->rule = QDR_RULE_KEYROW keeps c_i = 1; QDR_RULE_TENSOR also replaces every A_j by
 * max_j A_j (1 if 0) before the rest.
 * meta must come from qdr_init_state with the same descriptor. Errors: all codes. */
int qdr_quantize_state(const qdr_desc *desc, const void *meta, const float *S,
                       void *packed, float *row_scale, float *col_scale, void *stream);

/* One decode step for every unit, in place on (packed, row_scale, col_scale):
 * dequantize, apply the gated delta update
 *   S <- S diag(a) (I - b k k^T) + b v k^T   (GDN: diag(a) = a I)
 * (dev.to page, running-sum section; gate families per the DASC abstract), read out
 * o = S q from the updated fp32 state, then refit the scales and requantize (same rule
 * as qdr_quantize_state). Arithmetic: S'_ij = fl(code * fl(cf_j*rf_i)) with GDN
 * cf_j = R_j, rf_i = fl(a c_i) and KDA cf_j = fl(a_j R_j), rf_i = c_i;
 * u_i = fl32(rf_i * sum_j code_ij (cf_j k_j)) accumulated in fp64;
 * w_i = fl(b fl(v_i - u_i)); S_new_ij = fma(w_i, k_j, S'_ij).
 * Each unit is read completely before it is written, by one work-group, so in-place
 * update is safe; calls on one stream are ordered. Errors: all codes. */
int qdr_decode_step(const qdr_desc *desc, const void *meta, void *packed, float *row_scale,
                    float *col_scale, const float *q, const float *k, const float *v,
                    const float *a, const float *b, float *o, void *stream);

/* One token of window mode (LeapQuant abstract): the packed state stays fixed for W
 * tokens; token t (0 <= t < W, the same for all units) reads it plus the buffered
 * high-precision updates of tokens 0..t-1 from window_buf, produces o_t, and appends
 * its own update. At t = W-1 the buffered updates are folded into the state and the
 * state is requantized once (same scale rule). window_buf is caller-owned, sized by
 * qdr_state_bytes; its contents at t = 0 are ignored. Errors: all codes;
 * QDR_EUNSUPPORTED if t is out of range, desc->window < 1 or desc->window > 256. */
int qdr_decode_window(const qdr_desc *desc, const void *meta, void *packed,
                      float *row_scale, float *col_scale, void *window_buf, int32_t t,
                      const float *q, const float *k, const float *v, const float *a,
                      const float *b, float *o, void *stream);

/* qdr_decode_window for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same call, with the
 * window buffer taken from a fixed 32 MiB device array of the library instead of a caller
 * argument. No allocation happens in the call. The array is one per GPU, allocated with the
 * library's code object and held until the process ends; it keeps the last call's contents,
 * which is what carries a window from token to token (nothing in it needs clearing: token
 * t = 0 ignores what it holds). Every call on one GPU shares it, so windows of different
 * states must not interleave on a GPU, and calls on one GPU that overlap (other streams,
 * other threads) race. Limit: n_req * n_head * (W * 1024 + 1024) bytes <= 32 MiB (e.g.
 * 504 units at W = 64); a larger pool returns QDR_EUNSUPPORTED with the sizes in the error
 * text. Errors: as qdr_decode_window. */
int qdr_decode_window_static(const qdr_desc *desc, const void *meta, void *packed,
                             float *row_scale, float *col_scale, int32_t t, const float *q,
                             const float *k, const float *v, const float *a, const float *b,
                             float *o, void *stream);

/* T known tokens for every unit in one call (teacher-forced replay, prefill, multi-token
 * verification): the chunked form of window mode (LeapQuant abstract: outputs from the
 * fixed low-bit state plus high-precision updates, one quantization at the end). The
 * result is that of T consecutive tokens of qdr_decode_window with W = T: the state is
 * dequantized once, the gated delta recurrence of qdr_decode_step runs over the T tokens
 * in fp32 (no requantization inside), o_t = S_t q_t for every token, and the state is
 * refit and requantized once after token T-1 (same scale rule). In place on
 * (packed, row_scale, col_scale).
 * Token-major inputs: q, k: [T][n_req][n_head][dk] (logical key order);
 * v, o: [T][n_req][n_head][dv]; a: GDN [T][n_req][n_head], KDA [T][n_req][n_head][dk];
 * b: [T][n_req][n_head]. desc->window is not used; no window buffer. Gates may take any
 * value in [0, 1]. T = 0 is a no-op. Errors: all codes; QDR_EINVAL if T < 0. */
int qdr_decode_chunk(const qdr_desc *desc, const void *meta, void *packed, float *row_scale,
                     float *col_scale, int32_t T, const float *q, const float *k,
                     const float *v, const float *a, const float *b, float *o, void *stream);

/* ---- compensator tokens (LeapQuant abstract: the state's largest outliers are kept as
 * a few high-precision tokens that share the update path of the real tokens; the
 * remaining residual is quantized) ----------------------------------------------------
 * A token is one state entry kept in fp32, the rank-one term x e_i e_j^T. At each
 * quantization the m nonzero entries of largest |S_ij| become the unit's tokens, listed
 * largest first (equal magnitudes: smaller flat index i*dk + j first; j is the logical key
 * channel), and are set to 0 in the residual, which the STEPQuant rule quantizes.
 * Unused slots hold index QDR_TOK_EMPTY and value 0. The stored state is the dequantized
 * residual plus the tokens; a window (one qdr_comp_chunk call, or W qdr_comp_window calls)
 * starts from it, so the tokens go through the same gated delta updates as the rest of the
 * state, and the tokens are selected afresh from the fp32 state at the window's end.
 * tok_idx: uint16 [n_req][n_head][m] (flat index i*128 + j); tok_val: fp32, same shape;
 * both caller-owned device buffers, 16-byte aligned. 0 <= m <= QDR_COMP_MAX; m = 0 is the
 * plain mode. Only QDR_RULE_STEP. Errors: all codes; QDR_EINVAL for m out of range;
 * QDR_EUNSUPPORTED for another rule. */
#define QDR_TOK_EMPTY 0xFFFFu
#define QDR_COMP_MAX 64

/* Tokens of the fp32 state S_in [n_req][n_head][dv][dk] (logical order), then the residual
 * quantized into (packed, row_scale, col_scale) as qdr_quantize_state does. */
int qdr_comp_quantize(const qdr_desc *desc, const void *meta, void *packed, float *row_scale,
                      float *col_scale, int32_t m, uint16_t *tok_idx, float *tok_val,
                      const float *S_in, void *stream);

/* qdr_decode_chunk on the state with tokens: the chunk starts from the dequantized residual
 * plus the tokens and ends with new tokens and the requantized residual (all in place).
 * T = 0 is a no-op. */
int qdr_comp_chunk(const qdr_desc *desc, const void *meta, void *packed, float *row_scale,
                   float *col_scale, int32_t m, uint16_t *tok_idx, float *tok_val, int32_t T,
                   const float *q, const float *k, const float *v, const float *a,
                   const float *b, float *o, void *stream);

/* qdr_decode_window on the state with tokens: every token call reads the stored tokens as
 * entries of the window's start state (their contributions to the prediction and the
 * readout through the gated key and query); at t = W-1 the fold adds them to the state,
 * selects new tokens and requantizes the residual (in place on all of packed, scales and
 * tokens). m and the token buffers must be the same for every call of a window; the tokens
 * change only at t = W-1. Errors: as qdr_decode_window and the token checks above. */
int qdr_comp_window(const qdr_desc *desc, const void *meta, void *packed, float *row_scale,
                    float *col_scale, int32_t m, uint16_t *tok_idx, float *tok_val,
                    void *window_buf, int32_t t, const float *q, const float *k, const float *v,
                    const float *a, const float *b, float *o, void *stream);

/* The dequantized residual plus the tokens, S_out [n_req][n_head][dv][dk] (logical). */
int qdr_comp_dequantize(const qdr_desc *desc, const void *meta, const void *packed,
                        const float *row_scale, const float *col_scale, int32_t m,
                        const uint16_t *tok_idx, const float *tok_val, float *S_out,
                        void *stream);

/* Read back the dequantized state S_hat_ij = fl(code_ij * fl(R_j*c_i)) as
 * S_out [n_req][n_head][dv][dk] (logical key order): the state the STEPQuant abstract's
 * key-row and value-column scales represent, each code times its entry's step. For
 * checking and inspection; not on the decode path. Errors: all codes. */
int qdr_dequantize_state(const qdr_desc *desc, const void *meta, const void *packed,
                         const float *row_scale, const float *col_scale, float *S_out,
                         void *stream);

/* ---- DAMP-style storage variant (freedom251 page, section "DAMP: accuracy depends on
 * the task": selected key channels kept in FP16, the others in INT8 with stochastic
 * rounding; 16 channels per head). A second state format on the same decode step:
 *   half  [n_req*n_head][128 rows][16]  binary16 values of the selected key channels
 *   codes [n_req*n_head][128 rows][112] int8 codes of the other channels
 *   R     [n_req*n_head][112]           fp32 range per INT8 key row (R_j = A_j/127)
 *   meta  [n_head][128]                 physical position -> key channel (written by init)
 * Physical positions 0..15 are the selected channels, 16..127 the others, each in
 * increasing channel order. One decode step: S'_ij = fl(f32(h) a_j) or fl(code fl(a_j R_j));
 * u_i = S' k accumulated in fp64 and rounded once to fp32 (the products are exact in fp64;
 * the order of the fp64 sum is the kernel's, so u can differ from another fp64 order in the
 * last fp32 bit on rare ties); o_i = S_new q accumulated in fp32 (within 1e-4 rel-L2); w_i = fl(b fl(v_i - u_i));
 * S_new = fma(w_i, k_j, S'_ij); then binary16 (round to nearest even) for the selected
 * channels and, for the others, A_j = max_i |S_ij| (1 if 0), R_j = fl(A_j/127),
 * y = fl(S fl(1/A_j)), code = clamp(floor(y*127 + u), +-127) evaluated in fp64 with u the
 * byte position%16 (little-endian across the four words, times 2^-8) of Philox4x32-7
 * (Salmon et al., SC11: the published round function and key schedule, seven rounds) for counter (row*8 + position/16, unit, step low, step high) and
 * key (seed low, seed high), i.e. one generator block per 16 codes of a row;
 * unit = request*n_head + head. The caller passes a fresh step per call. Errors: as for
 * the main format; QDR_EUNSUPPORTED if a head does not select exactly 16 channels. */
typedef struct qdr_damp_desc {
    int32_t n_req, n_head;  /* as in qdr_desc                                          */
    int32_t gate;           /* QDR_GATE_GDN or QDR_GATE_KDA                            */
    const uint8_t *sel;     /* HOST [n_head][128]: nonzero marks a binary16 channel     */
} qdr_damp_desc;

/* HOST: the binary16 channels as a stand-in for DAMP's calibrated ranking (which needs
 * model data): KDA, per head the 16 key channels of longest gate half-life (ties by
 * index); GDN (one half-life per head), channels 0..15. halflife: GDN [n_head], KDA
 * [n_head][128]; sel_out [n_head][128]. Errors: QDR_EINVAL. */
int qdr_damp_select(int32_t gate, int32_t n_head, const double *halflife, uint8_t *sel_out);
int qdr_damp_bytes(const qdr_damp_desc *desc, size_t *half, size_t *codes, size_t *scales,
                   size_t *meta);
/* write meta and the zero state (codes 0, binary16 zeros, R = 1/127); copies the position
 * map from the host and synchronizes `stream` once */
int qdr_damp_init(const qdr_damp_desc *desc, void *meta, void *half, void *codes, float *R,
                  void *stream);
/* quantize a caller fp32 state S [n_req][n_head][128][128] (logical key order) */
int qdr_damp_quantize(const qdr_damp_desc *desc, const void *meta, const float *S, void *half,
                      void *codes, float *R, uint64_t seed, uint64_t step, void *stream);
/* one decode step in place; q, k, a(KDA): [n_req][n_head][128]; v, o: [n_req][n_head][128];
 * a(GDN), b: [n_req][n_head] */
int qdr_damp_step(const qdr_damp_desc *desc, const void *meta, void *half, void *codes,
                  float *R, const float *q, const float *k, const float *v, const float *a,
                  const float *b, float *o, uint64_t seed, uint64_t step, void *stream);
/* readback S [n_req][n_head][128][128] (logical key order): f32(h) or fl(code R_j) */
int qdr_damp_dequantize(const qdr_damp_desc *desc, const void *meta, const void *half,
                        const void *codes, const float *R, float *S, void *stream);

/* ---- measurement helpers (not part of the decode path) -----------------------------
 * The freedom251 page's checklist under "How to decide for a deployment" asks for the
 * update kernel to be measured on the deployment's own hardware; these two kernels give
 * the reference points such a measurement is read against.
 *
 * qdr_probe_copy: a streaming copy of `bytes` bytes from src to dst (device pointers,
 * 16-byte aligned, bytes a multiple of 16, non-overlapping), 16-byte loads and stores.
 * Timed by the caller (events on `stream`), 2*bytes / time is the achievable HBM
 * read+write bandwidth. Errors: QDR_EINVAL, QDR_EHIP (text in qdr_probe_last_error).
 *
 * qdr_probe_clock: n_block work-groups of 256 threads each run `iters` iterations of a
 * dependent fp32 fma chain; thread 0 of block b writes out[4b] = shader-clock cycles and
 * out[4b+1] = ticks of the constant-rate counter elapsed over the block's run (out: device
 * [n_block][4] uint64, caller-owned). Sum(out[4b]) / Sum(out[4b+1]) * qdr_probe_wall_rate
 * is the engine clock sustained under full VALU load. Errors: QDR_EINVAL, QDR_EHIP.
 *
 * qdr_probe_clock_trace: one wave that, on `stream`, writes n_sample pairs out[2i] =
 * shader-clock counter, out[2i+1] = constant-rate counter, sample i taken at the first
 * reading at least i*period constant-rate ticks after its start (it sleeps in between, so
 * it can run on a second stream beside the kernels being timed; it holds one wave and
 * under 16 registers, and ends after n_sample*period ticks whatever else runs). The
 * difference of two samples' first words over that of their second words times
 * qdr_probe_wall_rate is the engine clock over that interval. out: device [n_sample][2]
 * uint64, caller-owned; 1 <= n_sample <= 2^20, 1 <= period <= 2^24.
 * Errors: QDR_EINVAL, QDR_EHIP.
 *
 * qdr_probe_wall_rate: HOST output, the constant-rate counter's frequency in Hz. */
int qdr_probe_copy(const void *src, void *dst, size_t bytes, void *stream);
int qdr_probe_clock(unsigned long long *out, int32_t n_block, int32_t iters, void *stream);
int qdr_probe_clock_trace(unsigned long long *out, int32_t n_sample, int32_t period,
                          void *stream);
int qdr_probe_wall_rate(double *hz);
const char *qdr_probe_last_error(void);

/* Text of the last error on the calling thread ("" if none), set by every entry point
 * that returns a negative code. Never NULL. */
const char *qdr_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* QDR_H */
