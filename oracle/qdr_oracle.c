/*
 * qdr_oracle.c -- plain scalar CPU oracle (TEST INFRASTRUCTURE; see qdr_oracle.h).
 *
 * Written for readability against the pages, not for speed: scalar loops, one IEEE
 * rounding per written operation, no blocking, no reordering. Build with
 *   gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared -lm
 */
#include "qdr_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int qmax_of(int bits) { return (1 << (bits - 1)) - 1; }
static int valid_bits(int b) { return b == 4 || b == 6 || b == 8; }

/* ------------------------------------------------------------------------------
 * S0. Lifetime-based precision map. [STEP] Fig. 1(b): longer gate half-life means
 * larger accumulated state error; Fig. 4 / Figure B1: units ordered by increasing
 * half-life, the longest-lived quarter carries most of the error. [ABS] STEPQuant
 * abstract: precision follows error magnitude and memory lifetime. Reading: shortest
 * quarter 4 bits, longest quarter 8 bits, middle half 6 bits (nominal 6.0 bits).
 * ---------------------------------------------------------------------------- */
typedef struct { double tau; int idx; } rank_item;

static int cmp_rank(const void *pa, const void *pb) {
    const rank_item *a = (const rank_item *)pa, *b = (const rank_item *)pb;
    if (a->tau < b->tau) return -1;
    if (a->tau > b->tau) return 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

static void quartile_bits(int n, const double *tau, uint8_t *out) {
    rank_item *it = (rank_item *)malloc(sizeof(rank_item) * (size_t)n);
    for (int i = 0; i < n; ++i) { it[i].tau = tau[i]; it[i].idx = i; }
    qsort(it, (size_t)n, sizeof(rank_item), cmp_rank);
    int quarter = n / 4;
    for (int r = 0; r < n; ++r) {
        uint8_t b = 6;
        if (r < quarter) b = 4;
        else if (r >= n - quarter) b = 8;
        out[it[r].idx] = b;
    }
    free(it);
}

int oref_assign_bits(int gate, int n_head, int dk, const double *halflife, uint8_t *bits_out) {
    if (n_head <= 0 || dk <= 0 || !halflife || !bits_out) return -1;
    if (gate == OREF_GDN) {
        uint8_t *hb = (uint8_t *)malloc((size_t)n_head);
        quartile_bits(n_head, halflife, hb);
        for (int h = 0; h < n_head; ++h)
            for (int j = 0; j < dk; ++j) bits_out[h * dk + j] = hb[h];
        free(hb);
        return 0;
    }
    if (gate == OREF_KDA) {
        for (int h = 0; h < n_head; ++h) quartile_bits(dk, halflife + (size_t)h * dk, bits_out + (size_t)h * dk);
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------------------------------
 * Packed tile format. [MEAS] counts packed codes, scales and precision maps as the
 * state's memory; [STEP] Key contributions: mixed widths per unit. The format itself
 * is this project's own (the pages do not print one):
 *  - physical key order = channels sorted by width 8, 6, 4, ties by channel index;
 *  - segment s = physical positions 32s..32s+31, all of one width b_s;
 *  - segment s stores dv value rows, row i = 32 codes x b_s bits = 4*b_s bytes,
 *    segments concatenated, rows in order inside a segment;
 *  - inside a row the code of position 32s+m occupies bits [m*b, m*b+b) of the row's
 *    little-endian bit stream (bit t lives in byte t/8 at bit t%8);
 *  - each field holds the offset-binary value code + 2^(b-1).
 * ---------------------------------------------------------------------------- */
long oref_layout(int dv, int dk, const uint8_t *bits, uint8_t *perm, uint8_t *seg_bits) {
    if (dv <= 0 || dk <= 0 || (dk % 32) != 0 || !bits) return -1;
    static const int widths[3] = {8, 6, 4};
    int p = 0;
    long bytes = 0;
    for (int w = 0; w < 3; ++w) {
        int count = 0;
        for (int j = 0; j < dk; ++j) {
            if (!valid_bits(bits[j])) return -1;
            if (bits[j] == widths[w]) {
                if (perm) perm[p] = (uint8_t)j;
                ++p;
                ++count;
            }
        }
        if (count % 32) return -1;
        for (int s = 0; s < count / 32; ++s) {
            if (seg_bits) seg_bits[(p - count) / 32 + s] = (uint8_t)widths[w];
        }
        bytes += (long)dv * count * widths[w] / 8;
    }
    return bytes;
}

static void put_bits(uint8_t *row, int bitpos, int nbits, unsigned value) {
    for (int t = 0; t < nbits; ++t) {
        int pos = bitpos + t;
        unsigned bit = (value >> t) & 1u;
        row[pos / 8] = (uint8_t)((row[pos / 8] & ~(1u << (pos % 8))) | (bit << (pos % 8)));
    }
}

static unsigned get_bits(const uint8_t *row, int bitpos, int nbits) {
    unsigned v = 0;
    for (int t = 0; t < nbits; ++t) {
        int pos = bitpos + t;
        v |= (unsigned)((row[pos / 8] >> (pos % 8)) & 1u) << t;
    }
    return v;
}

int oref_pack(int dv, int dk, const uint8_t *bits, const int8_t *codes, uint8_t *tile) {
    uint8_t perm[256], seg[8];
    if (dk > 256) return -1;
    long total = oref_layout(dv, dk, bits, perm, seg);
    if (total < 0) return -1;
    memset(tile, 0, (size_t)total);
    long off = 0;
    for (int s = 0; s < dk / 32; ++s) {
        int b = seg[s];
        int row_bytes = 4 * b;
        for (int i = 0; i < dv; ++i) {
            uint8_t *row = tile + off + (long)i * row_bytes;
            for (int m = 0; m < 32; ++m) {
                int j = perm[32 * s + m];
                int code = codes[(size_t)i * dk + j];
                int qm = qmax_of(b);
                if (code < -qm || code > qm) return -1;
                put_bits(row, m * b, b, (unsigned)(code + (1 << (b - 1))));
            }
        }
        off += (long)dv * row_bytes;
    }
    return 0;
}

int oref_unpack(int dv, int dk, const uint8_t *bits, const uint8_t *tile, int8_t *codes) {
    uint8_t perm[256], seg[8];
    if (dk > 256) return -1;
    if (oref_layout(dv, dk, bits, perm, seg) < 0) return -1;
    long off = 0;
    for (int s = 0; s < dk / 32; ++s) {
        int b = seg[s];
        int row_bytes = 4 * b;
        for (int i = 0; i < dv; ++i) {
            const uint8_t *row = tile + off + (long)i * row_bytes;
            for (int m = 0; m < 32; ++m) {
                int j = perm[32 * s + m];
                int field = (int)get_bits(row, m * b, b);
                codes[(size_t)i * dk + j] = (int8_t)(field - (1 << (b - 1)));
            }
        }
        off += (long)dv * row_bytes;
    }
    return 0;
}

/* ------------------------------------------------------------------------------
 * Scale refit and requantization. [ABS] STEPQuant abstract: key-row and value-column
 * scales fitted jointly to the state distribution; [STEP] Fig. 5 / Figure B2: the
 * state has outliers along both rows and columns. Reading (two-stage absmax, key axis
 * first, the key row's bit range carried by its scale):
 *   A_j = max_i |S_ij| (1 if 0),  R_j = A_j / Qmax_j,  y_ij = S_ij * (1/A_j),
 *   c_i = max_j |y_ij| (1 if 0),  code_ij = RNE(y_ij * (Qmax_j * (1/c_i))),
 * with the last product exact (fp64) before the single round-half-even.
 * ---------------------------------------------------------------------------- */
void oref_quantize_rule(int dv, int dk, const uint8_t *bits, const float *S, int8_t *codes,
                        float *R, float *c, int rule) {
    float *A = (float *)malloc(sizeof(float) * (size_t)dk);
    float *invA = (float *)malloc(sizeof(float) * (size_t)dk);
    /* key rows (columns j): absmax over the value rows */
    for (int j = 0; j < dk; ++j) {
        float m = 0.0f;
        for (int i = 0; i < dv; ++i) {
            float x = fabsf(S[(size_t)i * dk + j]);
            if (x > m) m = x;
        }
        A[j] = m;
    }
    /* per-tensor INT8 ([DEV] "Uniform per-tensor INT8"): one range for the whole state */
    if (rule == OREF_RULE_TENSOR) {
        float m = 0.0f;
        for (int j = 0; j < dk; ++j)
            if (A[j] > m) m = A[j];
        for (int j = 0; j < dk; ++j) A[j] = m;
    }
    for (int j = 0; j < dk; ++j) {
        if (A[j] == 0.0f) A[j] = 1.0f;
        R[j] = A[j] / (float)qmax_of(bits[j]);
        invA[j] = 1.0f / A[j];
    }
    for (int i = 0; i < dv; ++i) {
        /* value-column scale ([ABS] STEPQuant abstract); the INT8 baselines keep c = 1 */
        float cm = 0.0f;
        if (rule == OREF_RULE_STEP) {
            for (int j = 0; j < dk; ++j) {
                float y = S[(size_t)i * dk + j] * invA[j];
                if (fabsf(y) > cm) cm = fabsf(y);
            }
        }
        if (cm == 0.0f) cm = 1.0f;
        c[i] = cm;
        float invc = 1.0f / cm;
        for (int j = 0; j < dk; ++j) {
            int qm = qmax_of(bits[j]);
            float y = S[(size_t)i * dk + j] * invA[j];
            float M = (float)qm * invc;
            double t = rint((double)y * (double)M); /* exact product, one RNE rounding */
            if (t > qm) t = qm;
            if (t < -qm) t = -qm;
            codes[(size_t)i * dk + j] = (int8_t)t;
        }
    }
    free(A);
    free(invA);
}

void oref_quantize(int dv, int dk, const uint8_t *bits, const float *S, int8_t *codes,
                   float *R, float *c) {
    oref_quantize_rule(dv, dk, bits, S, codes, R, c, OREF_RULE_STEP);
}

void oref_dequantize(int dv, int dk, const int8_t *codes, const float *R, const float *c,
                     float *S) {
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j) {
            float step = R[j] * c[i]; /* the entry's quantization step */
            S[(size_t)i * dk + j] = (float)codes[(size_t)i * dk + j] * step;
        }
}

/* ------------------------------------------------------------------------------
 * One decode step. [DEV] running-sum section: S <- S(I - k k^T) + v k^T; with the gate
 * and the write strength (GDN scalar gate / KDA per-channel gate, [ABS] DASC abstract):
 *   S_new = S diag(a) (I - b k k^T) + b v k^T = S' + w k^T,
 *   S' = S diag(a) (KDA) or a S (GDN),  u = S' k,  w = b (v - u),  o = S_new q.
 * S' is the dequantized state with the gate folded into a scale:
 *   GDN: cf_j = R_j, rf_i = fl(a c_i);  KDA: cf_j = fl(a_j R_j), rf_i = c_i;
 *   S'_ij = fl(code_ij fl(cf_j rf_i))  (the code times its entry's gated step).
 * u_i is the exact dequantized-and-gated row times k, accumulated in fp64 and rounded
 * once: u_i = fl32(rf_i * sum_j code_ij (cf_j k_j)).
 * S_new_ij = fma(w_i, k_j, S'_ij) (one rounding); o_i = fl32(sum_j S_new_ij q_j) in fp64.
 * The new state is then refit and requantized (oref_quantize).
 * ---------------------------------------------------------------------------- */
void oref_step_rule(int dv, int dk, int gate, const uint8_t *bits, int8_t *codes, float *R,
                    float *c, const float *q, const float *k, const float *v, const float *a,
                    float b, float *o, float *S_new_out, int rule) {
    float *cf = (float *)malloc(sizeof(float) * (size_t)dk);
    float *rf = (float *)malloc(sizeof(float) * (size_t)dv);
    float *w = (float *)malloc(sizeof(float) * (size_t)dv);
    float *Sn = (float *)malloc(sizeof(float) * (size_t)dv * dk);

    for (int j = 0; j < dk; ++j) cf[j] = (gate == OREF_KDA) ? a[j] * R[j] : R[j];
    for (int i = 0; i < dv; ++i) rf[i] = (gate == OREF_GDN) ? a[0] * c[i] : c[i];

    /* u = S' k and w = b (v - u) */
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j)
            acc += (double)codes[(size_t)i * dk + j] * ((double)cf[j] * (double)k[j]);
        float u = (float)((double)rf[i] * acc);
        w[i] = b * (v[i] - u);
    }
    /* S_new = S' + w k^T */
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j) {
            float step = cf[j] * rf[i];
            float sp = (float)codes[(size_t)i * dk + j] * step;
            Sn[(size_t)i * dk + j] = fmaf(w[i], k[j], sp);
        }
    /* o = S_new q */
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += (double)Sn[(size_t)i * dk + j] * (double)q[j];
        o[i] = (float)acc;
    }
    if (S_new_out) memcpy(S_new_out, Sn, sizeof(float) * (size_t)dv * dk);
    oref_quantize_rule(dv, dk, bits, Sn, codes, R, c, rule);

    free(cf);
    free(rf);
    free(w);
    free(Sn);
}

void oref_step(int dv, int dk, int gate, const uint8_t *bits, int8_t *codes, float *R,
               float *c, const float *q, const float *k, const float *v, const float *a,
               float b, float *o, float *S_new_out) {
    oref_step_rule(dv, dk, gate, bits, codes, R, c, q, k, v, a, b, o, S_new_out, OREF_RULE_STEP);
}

/* ------------------------------------------------------------------------------
 * Unquantized recurrence, fp64 (same algebra as oref_step without quantization).
 * ---------------------------------------------------------------------------- */
void oref_recur_fp64(int dv, int dk, int gate, double *S, const float *q, const float *k,
                     const float *v, const float *a, float b, float *o) {
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j)
            S[(size_t)i * dk + j] *= (gate == OREF_KDA) ? (double)a[j] : (double)a[0];
    for (int i = 0; i < dv; ++i) {
        double u = 0.0;
        for (int j = 0; j < dk; ++j) u += S[(size_t)i * dk + j] * (double)k[j];
        double wi = (double)b * ((double)v[i] - u);
        for (int j = 0; j < dk; ++j) S[(size_t)i * dk + j] += wi * (double)k[j];
    }
    if (o) {
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * (double)q[j];
            o[i] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------------------
 * Window mode. [ABS] LeapQuant abstract: keep the state low-bit across a window of
 * tokens, compute each output from the fixed low-bit state plus high-precision
 * buffered updates, quantize once at the window end. Semantically the outputs are
 * those of the exact recurrence started from the dequantized state; this function
 * runs that recurrence directly (fp64) and requantizes at the end.
 * ---------------------------------------------------------------------------- */
void oref_window(int dv, int dk, int gate, const uint8_t *bits, int8_t *codes, float *R,
                 float *c, int W, const float *q, const float *k, const float *v,
                 const float *a, const float *b, float *o, float *S_end) {
    float *Sh = (float *)malloc(sizeof(float) * (size_t)dv * dk);
    double *S = (double *)malloc(sizeof(double) * (size_t)dv * dk);
    oref_dequantize(dv, dk, codes, R, c, Sh);
    for (size_t e = 0; e < (size_t)dv * dk; ++e) S[e] = (double)Sh[e];
    for (int t = 0; t < W; ++t) {
        const float *at = (gate == OREF_KDA) ? a + (size_t)t * dk : a + t;
        oref_recur_fp64(dv, dk, gate, S, q + (size_t)t * dk, k + (size_t)t * dk,
                        v + (size_t)t * dv, at, b[t], o + (size_t)t * dv);
    }
    for (size_t e = 0; e < (size_t)dv * dk; ++e) Sh[e] = (float)S[e];
    if (S_end) memcpy(S_end, Sh, sizeof(float) * (size_t)dv * dk);
    oref_quantize(dv, dk, bits, Sh, codes, R, c);
    free(Sh);
    free(S);
}

/* ------------------------------------------------------------------------------
 * Batched drivers over the packed pool ([MEAS] per-request packed pages).
 * ---------------------------------------------------------------------------- */
long oref_request_bytes(int n_head, int dv, int dk, const uint8_t *bits) {
    long total = 0;
    for (int h = 0; h < n_head; ++h) {
        long t = oref_layout(dv, dk, bits + (size_t)h * dk, NULL, NULL);
        if (t < 0) return -1;
        total += t;
    }
    return total;
}

typedef struct {
    long req_bytes;
    long *head_off;
    uint8_t *perm; /* [n_head][dk] */
} pool_geom;

static int geom_init(pool_geom *g, int n_head, int dv, int dk, const uint8_t *bits) {
    g->head_off = (long *)malloc(sizeof(long) * (size_t)n_head);
    g->perm = (uint8_t *)malloc((size_t)n_head * dk);
    long off = 0;
    for (int h = 0; h < n_head; ++h) {
        long t = oref_layout(dv, dk, bits + (size_t)h * dk, g->perm + (size_t)h * dk, NULL);
        if (t < 0) return -1;
        g->head_off[h] = off;
        off += t;
    }
    g->req_bytes = off;
    return 0;
}

static void geom_free(pool_geom *g) {
    free(g->head_off);
    free(g->perm);
}

/* physical-order scales <-> logical-order scales */
static void scales_to_logical(int dk, const uint8_t *perm, const float *phys, float *logical) {
    for (int p = 0; p < dk; ++p) logical[perm[p]] = phys[p];
}
static void scales_to_physical(int dk, const uint8_t *perm, const float *logical, float *phys) {
    for (int p = 0; p < dk; ++p) phys[p] = logical[perm[p]];
}

int oref_quantize_pool_rule(int n_req, int n_head, int dv, int dk, const uint8_t *bits,
                            const float *S, uint8_t *packed, float *row_scale, float *col_scale,
                            int rule) {
    pool_geom g;
    if (geom_init(&g, n_head, dv, dk, bits)) { geom_free(&g); return -1; }
    int8_t *codes = (int8_t *)malloc((size_t)dv * dk);
    float *R = (float *)malloc(sizeof(float) * (size_t)dk);
    for (int r = 0; r < n_req; ++r)
        for (int h = 0; h < n_head; ++h) {
            size_t u = (size_t)r * n_head + h;
            const uint8_t *bh = bits + (size_t)h * dk;
            oref_quantize_rule(dv, dk, bh, S + u * dv * dk, codes, R, col_scale + u * dv, rule);
            scales_to_physical(dk, g.perm + (size_t)h * dk, R, row_scale + u * dk);
            oref_pack(dv, dk, bh, codes, packed + (size_t)r * g.req_bytes + g.head_off[h]);
        }
    free(codes);
    free(R);
    geom_free(&g);
    return 0;
}

int oref_quantize_pool(int n_req, int n_head, int dv, int dk, const uint8_t *bits,
                       const float *S, uint8_t *packed, float *row_scale, float *col_scale) {
    return oref_quantize_pool_rule(n_req, n_head, dv, dk, bits, S, packed, row_scale, col_scale,
                                   OREF_RULE_STEP);
}

int oref_dequantize_pool(int n_req, int n_head, int dv, int dk, const uint8_t *bits,
                         const uint8_t *packed, const float *row_scale,
                         const float *col_scale, float *S) {
    pool_geom g;
    if (geom_init(&g, n_head, dv, dk, bits)) { geom_free(&g); return -1; }
    int8_t *codes = (int8_t *)malloc((size_t)dv * dk);
    float *R = (float *)malloc(sizeof(float) * (size_t)dk);
    for (int r = 0; r < n_req; ++r)
        for (int h = 0; h < n_head; ++h) {
            size_t u = (size_t)r * n_head + h;
            const uint8_t *bh = bits + (size_t)h * dk;
            oref_unpack(dv, dk, bh, packed + (size_t)r * g.req_bytes + g.head_off[h], codes);
            scales_to_logical(dk, g.perm + (size_t)h * dk, row_scale + u * dk, R);
            oref_dequantize(dv, dk, codes, R, col_scale + u * dv, S + u * dv * dk);
        }
    free(codes);
    free(R);
    geom_free(&g);
    return 0;
}

int oref_step_pool_rule(int n_req, int n_head, int dv, int dk, int gate, const uint8_t *bits,
                        uint8_t *packed, float *row_scale, float *col_scale, const float *q,
                        const float *k, const float *v, const float *a, const float *b, float *o,
                        long u0, long u1, int rule) {
    pool_geom g;
    if (geom_init(&g, n_head, dv, dk, bits)) { geom_free(&g); return -1; }
    int8_t *codes = (int8_t *)malloc((size_t)dv * dk);
    float *R = (float *)malloc(sizeof(float) * (size_t)dk);
    for (long u = u0; u < u1; ++u) {
        int r = (int)(u / n_head), h = (int)(u % n_head);
        const uint8_t *bh = bits + (size_t)h * dk;
        const uint8_t *perm = g.perm + (size_t)h * dk;
        uint8_t *tile = packed + (size_t)r * g.req_bytes + g.head_off[h];
        const float *au = (gate == OREF_KDA) ? a + (size_t)u * dk : a + u;
        oref_unpack(dv, dk, bh, tile, codes);
        scales_to_logical(dk, perm, row_scale + (size_t)u * dk, R);
        oref_step_rule(dv, dk, gate, bh, codes, R, col_scale + (size_t)u * dv, q + (size_t)u * dk,
                       k + (size_t)u * dk, v + (size_t)u * dv, au, b[u], o + (size_t)u * dv, NULL,
                       rule);
        scales_to_physical(dk, perm, R, row_scale + (size_t)u * dk);
        oref_pack(dv, dk, bh, codes, tile);
    }
    free(codes);
    free(R);
    geom_free(&g);
    return 0;
}

int oref_step_pool(int n_req, int n_head, int dv, int dk, int gate, const uint8_t *bits,
                   uint8_t *packed, float *row_scale, float *col_scale, const float *q,
                   const float *k, const float *v, const float *a, const float *b, float *o,
                   long u0, long u1) {
    return oref_step_pool_rule(n_req, n_head, dv, dk, gate, bits, packed, row_scale, col_scale,
                               q, k, v, a, b, o, u0, u1, OREF_RULE_STEP);
}

int oref_window_pool(int n_req, int n_head, int dv, int dk, int gate, const uint8_t *bits,
                     uint8_t *packed, float *row_scale, float *col_scale, int W,
                     const float *q, const float *k, const float *v, const float *a,
                     const float *b, float *o, long u0, long u1) {
    pool_geom g;
    if (geom_init(&g, n_head, dv, dk, bits)) { geom_free(&g); return -1; }
    size_t n_unit = (size_t)n_req * n_head;
    size_t a_len = (gate == OREF_KDA) ? (size_t)dk : 1;
    int8_t *codes = (int8_t *)malloc((size_t)dv * dk);
    float *R = (float *)malloc(sizeof(float) * (size_t)dk);
    float *tq = (float *)malloc(sizeof(float) * (size_t)W * dk);
    float *tk = (float *)malloc(sizeof(float) * (size_t)W * dk);
    float *tv = (float *)malloc(sizeof(float) * (size_t)W * dv);
    float *ta = (float *)malloc(sizeof(float) * (size_t)W * a_len);
    float *tb = (float *)malloc(sizeof(float) * (size_t)W);
    float *to = (float *)malloc(sizeof(float) * (size_t)W * dv);
    for (long u = u0; u < u1; ++u) {
        int r = (int)(u / n_head), h = (int)(u % n_head);
        const uint8_t *bh = bits + (size_t)h * dk;
        const uint8_t *perm = g.perm + (size_t)h * dk;
        uint8_t *tile = packed + (size_t)r * g.req_bytes + g.head_off[h];
        for (int t = 0; t < W; ++t) {
            size_t base = (size_t)t * n_unit + (size_t)u;
            memcpy(tq + (size_t)t * dk, q + base * dk, sizeof(float) * (size_t)dk);
            memcpy(tk + (size_t)t * dk, k + base * dk, sizeof(float) * (size_t)dk);
            memcpy(tv + (size_t)t * dv, v + base * dv, sizeof(float) * (size_t)dv);
            memcpy(ta + (size_t)t * a_len, a + base * a_len, sizeof(float) * a_len);
            tb[t] = b[base];
        }
        oref_unpack(dv, dk, bh, tile, codes);
        scales_to_logical(dk, perm, row_scale + (size_t)u * dk, R);
        oref_window(dv, dk, gate, bh, codes, R, col_scale + (size_t)u * dv, W, tq, tk, tv, ta,
                    tb, to, NULL);
        scales_to_physical(dk, perm, R, row_scale + (size_t)u * dk);
        oref_pack(dv, dk, bh, codes, tile);
        for (int t = 0; t < W; ++t)
            memcpy(o + ((size_t)t * n_unit + (size_t)u) * dv, to + (size_t)t * dv,
                   sizeof(float) * (size_t)dv);
    }
    free(codes); free(R); free(tq); free(tk); free(tv); free(ta); free(tb); free(to);
    geom_free(&g);
    return 0;
}

/* ------------------------------------------------------------------------------
 * Compensator tokens. [ABS] LeapQuant abstract: the state's largest outliers are kept
 * as a few high-precision tokens that share the update path of the real tokens, and
 * the remaining residual is quantized. Reading (the abstract gives no selection rule):
 * a token is one state entry x at (i, j) kept in fp32, i.e. the rank-one term
 * x e_i e_j^T. At a quantization the m nonzero entries of largest magnitude become the
 * tokens, listed in that order (equal magnitudes: smaller flat index i*dk + j first);
 * slots beyond the number of nonzero entries are empty. The residual, S with those
 * entries set to 0, is quantized. The next window starts from the dequantized residual
 * plus the tokens, so the tokens go through the same gated delta updates as the rest
 * of the state (the recurrence is linear in the state).
 * ---------------------------------------------------------------------------- */
typedef struct {
    float mag;
    uint32_t idx;
} tok_cand;

static int tok_order(const void *pa, const void *pb) {
    const tok_cand *a = (const tok_cand *)pa, *b = (const tok_cand *)pb;
    if (a->mag != b->mag) return a->mag > b->mag ? -1 : 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

void oref_comp_select(int dv, int dk, int m, float *S, uint16_t *tok_idx, float *tok_val) {
    const size_t n = (size_t)dv * dk;
    size_t nz = 0;
    tok_cand *c = (tok_cand *)malloc(sizeof(tok_cand) * (n ? n : 1));
    for (size_t e = 0; e < n; ++e)
        if (S[e] != 0.0f) {
            c[nz].mag = fabsf(S[e]);
            c[nz].idx = (uint32_t)e;
            ++nz;
        }
    qsort(c, nz, sizeof(tok_cand), tok_order);
    for (int t = 0; t < m; ++t) {
        if ((size_t)t < nz) {
            tok_idx[t] = (uint16_t)c[t].idx;
            tok_val[t] = S[c[t].idx];
        } else {
            tok_idx[t] = OREF_TOK_EMPTY;
            tok_val[t] = 0.0f;
        }
    }
    for (int t = 0; t < m && (size_t)t < nz; ++t) S[c[t].idx] = 0.0f;
    free(c);
}

void oref_comp_add(int m, const uint16_t *tok_idx, const float *tok_val, float *S) {
    for (int t = 0; t < m; ++t)
        if (tok_idx[t] != OREF_TOK_EMPTY) S[tok_idx[t]] += tok_val[t];
}

void oref_comp_quantize(int dv, int dk, const uint8_t *bits, const float *S, int m,
                        int8_t *codes, float *R, float *c, uint16_t *tok_idx, float *tok_val) {
    float *Sr = (float *)malloc(sizeof(float) * (size_t)dv * dk);
    memcpy(Sr, S, sizeof(float) * (size_t)dv * dk);
    oref_comp_select(dv, dk, m, Sr, tok_idx, tok_val);
    oref_quantize(dv, dk, bits, Sr, codes, R, c);
    free(Sr);
}

void oref_comp_dequantize(int dv, int dk, const int8_t *codes, const float *R, const float *c,
                          int m, const uint16_t *tok_idx, const float *tok_val, float *S) {
    oref_dequantize(dv, dk, codes, R, c, S);
    oref_comp_add(m, tok_idx, tok_val, S);
}

void oref_comp_window(int dv, int dk, int gate, const uint8_t *bits, int8_t *codes, float *R,
                      float *c, int m, uint16_t *tok_idx, float *tok_val, int W, const float *q,
                      const float *k, const float *v, const float *a, const float *b, float *o,
                      float *S_end) {
    float *Sh = (float *)malloc(sizeof(float) * (size_t)dv * dk);
    double *S = (double *)malloc(sizeof(double) * (size_t)dv * dk);
    oref_comp_dequantize(dv, dk, codes, R, c, m, tok_idx, tok_val, Sh);
    for (size_t e = 0; e < (size_t)dv * dk; ++e) S[e] = (double)Sh[e];
    for (int t = 0; t < W; ++t) {
        const float *at = (gate == OREF_KDA) ? a + (size_t)t * dk : a + t;
        oref_recur_fp64(dv, dk, gate, S, q + (size_t)t * dk, k + (size_t)t * dk,
                        v + (size_t)t * dv, at, b[t], o + (size_t)t * dv);
    }
    for (size_t e = 0; e < (size_t)dv * dk; ++e) Sh[e] = (float)S[e];
    if (S_end) memcpy(S_end, Sh, sizeof(float) * (size_t)dv * dk);
    oref_comp_select(dv, dk, m, Sh, tok_idx, tok_val);
    oref_quantize(dv, dk, bits, Sh, codes, R, c);
    free(Sh);
    free(S);
}

int oref_comp_quantize_pool(int n_req, int n_head, int dv, int dk, const uint8_t *bits,
                            const float *S, int m, uint8_t *packed, float *row_scale,
                            float *col_scale, uint16_t *tok_idx, float *tok_val) {
    pool_geom g;
    if (geom_init(&g, n_head, dv, dk, bits)) { geom_free(&g); return -1; }
    int8_t *codes = (int8_t *)malloc((size_t)dv * dk);
    float *R = (float *)malloc(sizeof(float) * (size_t)dk);
    for (int r = 0; r < n_req; ++r)
        for (int h = 0; h < n_head; ++h) {
            size_t u = (size_t)r * n_head + h;
            const uint8_t *bh = bits + (size_t)h * dk;
            oref_comp_quantize(dv, dk, bh, S + u * dv * dk, m, codes, R, col_scale + u * dv,
                               tok_idx + u * m, tok_val + u * m);
            scales_to_physical(dk, g.perm + (size_t)h * dk, R, row_scale + u * dk);
            oref_pack(dv, dk, bh, codes, packed + (size_t)r * g.req_bytes + g.head_off[h]);
        }
    free(codes);
    free(R);
    geom_free(&g);
    return 0;
}

int oref_comp_dequantize_pool(int n_req, int n_head, int dv, int dk, const uint8_t *bits,
                              const uint8_t *packed, const float *row_scale,
                              const float *col_scale, int m, const uint16_t *tok_idx,
                              const float *tok_val, float *S) {
    if (oref_dequantize_pool(n_req, n_head, dv, dk, bits, packed, row_scale, col_scale, S))
        return -1;
    for (size_t u = 0; u < (size_t)n_req * n_head; ++u)
        oref_comp_add(m, tok_idx + u * m, tok_val + u * m, S + u * dv * dk);
    return 0;
}

int oref_comp_window_pool(int n_req, int n_head, int dv, int dk, int gate, const uint8_t *bits,
                          uint8_t *packed, float *row_scale, float *col_scale, int m,
                          uint16_t *tok_idx, float *tok_val, int W, const float *q,
                          const float *k, const float *v, const float *a, const float *b,
                          float *o, long u0, long u1) {
    pool_geom g;
    if (geom_init(&g, n_head, dv, dk, bits)) { geom_free(&g); return -1; }
    size_t n_unit = (size_t)n_req * n_head;
    size_t a_len = (gate == OREF_KDA) ? (size_t)dk : 1;
    int8_t *codes = (int8_t *)malloc((size_t)dv * dk);
    float *R = (float *)malloc(sizeof(float) * (size_t)dk);
    float *tq = (float *)malloc(sizeof(float) * (size_t)W * dk);
    float *tk = (float *)malloc(sizeof(float) * (size_t)W * dk);
    float *tv = (float *)malloc(sizeof(float) * (size_t)W * dv);
    float *ta = (float *)malloc(sizeof(float) * (size_t)W * a_len);
    float *tb = (float *)malloc(sizeof(float) * (size_t)(W ? W : 1));
    float *to = (float *)malloc(sizeof(float) * (size_t)W * dv);
    for (long u = u0; u < u1; ++u) {
        int r = (int)(u / n_head), h = (int)(u % n_head);
        const uint8_t *bh = bits + (size_t)h * dk;
        const uint8_t *perm = g.perm + (size_t)h * dk;
        uint8_t *tile = packed + (size_t)r * g.req_bytes + g.head_off[h];
        for (int t = 0; t < W; ++t) {
            size_t base = (size_t)t * n_unit + (size_t)u;
            memcpy(tq + (size_t)t * dk, q + base * dk, sizeof(float) * (size_t)dk);
            memcpy(tk + (size_t)t * dk, k + base * dk, sizeof(float) * (size_t)dk);
            memcpy(tv + (size_t)t * dv, v + base * dv, sizeof(float) * (size_t)dv);
            memcpy(ta + (size_t)t * a_len, a + base * a_len, sizeof(float) * a_len);
            tb[t] = b[base];
        }
        oref_unpack(dv, dk, bh, tile, codes);
        scales_to_logical(dk, perm, row_scale + (size_t)u * dk, R);
        oref_comp_window(dv, dk, gate, bh, codes, R, col_scale + (size_t)u * dv, m,
                         tok_idx + (size_t)u * m, tok_val + (size_t)u * m, W, tq, tk, tv, ta,
                         tb, to, NULL);
        scales_to_physical(dk, perm, R, row_scale + (size_t)u * dk);
        oref_pack(dv, dk, bh, codes, tile);
        for (int t = 0; t < W; ++t)
            memcpy(o + ((size_t)t * n_unit + (size_t)u) * dv, to + (size_t)t * dv,
                   sizeof(float) * (size_t)dv);
    }
    free(codes); free(R); free(tq); free(tk); free(tv); free(ta); free(tb); free(to);
    geom_free(&g);
    return 0;
}

/* ------------------------------------------------------------------------------
 * DAMP-style storage variant ([MEAS] section "DAMP: accuracy depends on the task":
 * selected key channels kept in FP16, the rest in INT8 with stochastic rounding).
 * Written from the storage description and the arithmetic contract in the header.
 * ---------------------------------------------------------------------------- */

/* Philox4x32-R: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 * 1, 2, 3" (SC11). R rounds of two 32x32->64 multiplies on the counter, the key
 * bumped by the Weyl constants between rounds. The paper's default is R = 10; the
 * stochastic rounding below uses R = 7, the fewest rounds with which the paper reports
 * Philox4x32 passing its statistical test batteries. */
void oref_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int rounds, uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < rounds; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

void oref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    oref_philox4x32(ctr, key, 10, out);
}

/* IEEE 754 binary16 from binary32, round to nearest even (subnormals kept, overflow to
 * infinity, NaN to the quiet NaN 0x7E00), and back (exact). */
uint16_t oref_f32_to_f16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const uint32_t ex = (u >> 23) & 0xFFu;
    uint32_t man = u & 0x7FFFFFu;
    if (ex == 0xFF) return (uint16_t)(sign | (man ? 0x7E00u : 0x7C00u));
    /* value = 1.man * 2^(ex-127) (or 0.man * 2^-126 when ex == 0) */
    int e = (int)ex - 127;
    if (ex == 0) return (uint16_t)sign; /* fp32 subnormals are far below half's range */
    uint32_t sig = man | 0x800000u;     /* 24-bit significand */
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    int shift; /* bits of the 24-bit significand dropped */
    uint32_t hexp;
    if (e >= -14) {
        shift = 13;
        hexp = (uint32_t)(e + 15);
    } else {
        shift = 13 + (-14 - e); /* subnormal: 2^-24 units */
        hexp = 0;
        if (shift > 24) return (uint16_t)sign;
    }
    uint32_t q = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1;
    uint32_t h;
    if (hexp == 0) {
        h = q; /* may carry into the smallest normal, which is the right encoding */
    } else {
        /* q holds 11 bits (implicit one); a carry to 12 bits bumps the exponent */
        if (q & 0x800u) {
            q >>= 1;
            hexp += 1;
        }
        if (hexp >= 31) return (uint16_t)(sign | 0x7C00u);
        h = (hexp << 10) | (q & 0x3FFu);
    }
    return (uint16_t)(sign | h);
}

float oref_f16_to_f32(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int ex = (h >> 10) & 0x1F;
    const int man = h & 0x3FF;
    double v;
    if (ex == 0) v = ldexp((double)man, -24);
    else if (ex == 31) v = man ? NAN : INFINITY;
    else v = ldexp((double)(man | 0x400), ex - 25);
    return (float)(sign ? -v : v);
}

/* uniform in [0, 1) for state entry (i, p) of a unit at a step: byte p mod 16 (little-endian
 * across the four words) of the Philox4x32-7 block for the counter (i*8 + p/16, unit, step low,
 * step high), key = seed, times 2^-8 (one block serves sixteen consecutive positions of a
 * row) */
static double damp_uniform(uint64_t seed, uint32_t unit, uint64_t step, int i, int p) {
    const uint32_t ctr[4] = {(uint32_t)(i * 8 + p / 16), unit, (uint32_t)step,
                             (uint32_t)(step >> 32)};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oref_philox4x32(ctr, key, OREF_DAMP_PHILOX_ROUNDS, out);
    const uint32_t byte = (out[(p / 4) % 4] >> (8 * (p % 4))) & 0xFFu;
    return ldexp((double)byte, -8);
}

int oref_damp_perm(int dk, const uint8_t *sel, uint8_t *perm) {
    int n = 0;
    for (int j = 0; j < dk; ++j) n += sel[j] ? 1 : 0;
    if (dk != 128 || n != OREF_DAMP_HALF) return -1;
    int a = 0, b = OREF_DAMP_HALF;
    for (int j = 0; j < dk; ++j) {
        if (sel[j]) perm[a++] = (uint8_t)j;
        else perm[b++] = (uint8_t)j;
    }
    return 0;
}

void oref_damp_dequantize(int dv, const uint8_t *perm, const uint16_t *half, const int8_t *codes,
                          const float *R, float *S) {
    const int NI = 128 - OREF_DAMP_HALF;
    for (int i = 0; i < dv; ++i)
        for (int p = 0; p < 128; ++p) {
            const int j = perm[p];
            S[(size_t)i * 128 + j] =
                p < OREF_DAMP_HALF ? oref_f16_to_f32(half[(size_t)i * OREF_DAMP_HALF + p])
                                   : (float)codes[(size_t)i * NI + (p - OREF_DAMP_HALF)] *
                                         R[p - OREF_DAMP_HALF];
        }
}

/* requantize a physical-order fp32 state Sp[dv][128] into (half, codes, R) */
static void damp_requant(int dv, const float *Sp, uint16_t *half, int8_t *codes, float *R,
                         uint64_t seed, uint32_t unit, uint64_t step) {
    const int NI = 128 - OREF_DAMP_HALF;
    for (int i = 0; i < dv; ++i)
        for (int p = 0; p < OREF_DAMP_HALF; ++p)
            half[(size_t)i * OREF_DAMP_HALF + p] = oref_f32_to_f16(Sp[(size_t)i * 128 + p]);
    for (int c = 0; c < NI; ++c) {
        const int p = OREF_DAMP_HALF + c;
        float A = 0.0f;
        for (int i = 0; i < dv; ++i) {
            const float m = fabsf(Sp[(size_t)i * 128 + p]);
            if (m > A) A = m;
        }
        if (A == 0.0f) A = 1.0f;
        R[c] = A / 127.0f;
        const float invA = 1.0f / A;
        for (int i = 0; i < dv; ++i) {
            const float y = Sp[(size_t)i * 128 + p] * invA;
            /* stochastic rounding: floor(y*127 + u), u uniform in [0, 1); exact in fp64 */
            double t = floor((double)y * 127.0 + damp_uniform(seed, unit, step, i, p));
            if (t > 127.0) t = 127.0;
            if (t < -127.0) t = -127.0;
            codes[(size_t)i * NI + c] = (int8_t)t;
        }
    }
}

void oref_damp_quantize(int dv, const uint8_t *perm, const float *S, uint16_t *half,
                        int8_t *codes, float *R, uint64_t seed, uint32_t unit, uint64_t step) {
    float *Sp = (float *)malloc(sizeof(float) * (size_t)dv * 128);
    for (int i = 0; i < dv; ++i)
        for (int p = 0; p < 128; ++p) Sp[(size_t)i * 128 + p] = S[(size_t)i * 128 + perm[p]];
    damp_requant(dv, Sp, half, codes, R, seed, unit, step);
    free(Sp);
}

void oref_damp_step(int dv, int gate, const uint8_t *perm, uint16_t *half, int8_t *codes,
                    float *R, const float *q, const float *k, const float *v, const float *a,
                    float b, float *o, uint64_t seed, uint32_t unit, uint64_t step) {
    const int NI = 128 - OREF_DAMP_HALF;
    float *Sp = (float *)malloc(sizeof(float) * (size_t)dv * 128);
    float kp[128], gp[128];
    for (int p = 0; p < 128; ++p) {
        kp[p] = k[perm[p]];
        gp[p] = (gate == OREF_KDA) ? a[perm[p]] : a[0];
    }
    /* gated dequantization: fp16 channels fl(h * a_j); INT8 channels fl(code * fl(a_j R_j)) */
    for (int i = 0; i < dv; ++i)
        for (int p = 0; p < 128; ++p)
            Sp[(size_t)i * 128 + p] =
                p < OREF_DAMP_HALF
                    ? oref_f16_to_f32(half[(size_t)i * OREF_DAMP_HALF + p]) * gp[p]
                    : (float)codes[(size_t)i * NI + (p - OREF_DAMP_HALF)] *
                          (gp[p] * R[p - OREF_DAMP_HALF]);
    int pos[128]; /* physical position of logical key channel j */
    for (int p = 0; p < 128; ++p) pos[perm[p]] = p;
    for (int i = 0; i < dv; ++i) {
        /* u = S' k: one fp64 sum over the key channels j = 0..127 in logical order */
        double su = 0.0;
        for (int j = 0; j < 128; ++j)
            su += (double)Sp[(size_t)i * 128 + pos[j]] * (double)k[j];
        const float u = (float)su;
        const float w = b * (v[i] - u);
        for (int p = 0; p < 128; ++p)
            Sp[(size_t)i * 128 + p] = fmaf(w, kp[p], Sp[(size_t)i * 128 + p]);
        /* o = S_new q, the same way */
        double so = 0.0;
        for (int j = 0; j < 128; ++j)
            so += (double)Sp[(size_t)i * 128 + pos[j]] * (double)q[j];
        o[i] = (float)so;
    }
    damp_requant(dv, Sp, half, codes, R, seed, unit, step);
    free(Sp);
}

/* pools: half [n_unit][dv][16] (uint16), codes [n_unit][dv][112] (int8), R [n_unit][112];
 * perm [n_head][128]; unit index u = r * n_head + h */
int oref_damp_quantize_pool(int n_unit, int n_head, int dv, const uint8_t *perm, const float *S,
                            uint16_t *half, int8_t *codes, float *R, uint64_t seed,
                            uint64_t step) {
    const int NI = 128 - OREF_DAMP_HALF;
    for (long u = 0; u < n_unit; ++u) {
        const int h = (int)(u % n_head);
        oref_damp_quantize(dv, perm + (size_t)h * 128, S + (size_t)u * dv * 128,
                           half + (size_t)u * dv * OREF_DAMP_HALF, codes + (size_t)u * dv * NI,
                           R + (size_t)u * NI, seed, (uint32_t)u, step);
    }
    return 0;
}

int oref_damp_dequantize_pool(int n_unit, int n_head, int dv, const uint8_t *perm,
                              const uint16_t *half, const int8_t *codes, const float *R,
                              float *S) {
    const int NI = 128 - OREF_DAMP_HALF;
    for (long u = 0; u < n_unit; ++u) {
        const int h = (int)(u % n_head);
        oref_damp_dequantize(dv, perm + (size_t)h * 128, half + (size_t)u * dv * OREF_DAMP_HALF,
                             codes + (size_t)u * dv * NI, R + (size_t)u * NI,
                             S + (size_t)u * dv * 128);
    }
    return 0;
}

int oref_damp_step_pool(int n_unit, int n_head, int dv, int gate, const uint8_t *perm,
                        uint16_t *half, int8_t *codes, float *R, const float *q, const float *k,
                        const float *v, const float *a, const float *b, float *o, uint64_t seed,
                        uint64_t step, long u0, long u1) {
    const int NI = 128 - OREF_DAMP_HALF;
    for (long u = u0; u < u1; ++u) {
        const int h = (int)(u % n_head);
        const float *au = (gate == OREF_KDA) ? a + (size_t)u * 128 : a + u;
        oref_damp_step(dv, gate, perm + (size_t)h * 128, half + (size_t)u * dv * OREF_DAMP_HALF,
                       codes + (size_t)u * dv * NI, R + (size_t)u * NI, q + (size_t)u * 128,
                       k + (size_t)u * 128, v + (size_t)u * dv, au, b[u], o + (size_t)u * dv,
                       seed, (uint32_t)u, step);
    }
    return 0;
}
