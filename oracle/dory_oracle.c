/*
 * dory_oracle.c -- a plain, slow CPU forward of the Dory looped normalized GPT.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares nothing with the HIP path.
 *
 * Sources (pages of the cortiq-engine crate):
 *   [dory]  "dory.rs": module documentation (the seven-line summary of the
 *           model), `justnorm`, `slerp`, `silu_body`, `gate_body`, `soft_body`,
 *           `slot_loop`, `attn_layer`, `mlp_layer`, `stack`, `forward_host`,
 *           `head`, `DoryState::clear`.
 *   [kv]    "kv_cache.rs": `KV_COL_WARMUP`, `KV_K_GROUP`, `quant_row`,
 *           `freeze_cols`, `append`, `attend` / `attend_group_upto`,
 *           `truncate_last`, `clear`.
 *
 * Storage is by absolute position (row p of a slot is position p), with no
 * ring: a window is applied only as the lower bound of the keys a row reads.
 * Activations and cache rows are fp32; sums are fp64, rounded once.
 */
#include "dory_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

#define ORA_EPS 1e-6          /* [dory] `EPS`, justnorm's epsilon */
#define ORA_MAX_LOOPS 16      /* [dory] `MAX_LOOPS` */
#define ORA_WARMUP 64         /* [kv] `KV_COL_WARMUP`: rows before the field freezes */
#define ORA_KGROUP 32         /* [kv] `KV_K_GROUP`: K channels per scale */

typedef struct {
    int64_t rows;        /* rows stored: positions 0 .. rows-1 */
    float *k, *v;        /* fp32 cache: [max_ctx][nk][hd] */
    int8_t *kc, *vc;     /* q8 codes: [max_ctx][nk][hd] */
    float *ks;           /* K scales: [max_ctx][nk][ngk] */
    float *vs;           /* V scales: [max_ctx][nk] */
    float *kcol, *vcol;  /* fields [nk][hd], meaningful once frozen */
    int frozen;
} slot_t;

typedef struct {
    int64_t pos;
    float exit_rate;     /* [dory] `ExitRate`: rate of early exits (starts at 1) */
    uint32_t exit_tokens;
    uint64_t gate_tokens, gate_one;   /* gated tokens, and those that left after one pass */
    float last_top;      /* the top probability of the last read-out (-1: none yet) */
    int mode;            /* -1: not fixed yet */
    int loops;           /* per_loop: the loop count fixed at the first call; 0 unset */
    slot_t *slots;       /* [n_ord][ORA_MAX_LOOPS] */
} seq_t;

struct ora_model {
    ora_cfg c;
    char *pattern;
    ora_weights w;
    ora_layer *layers;
    int n_layers, n_ord, Q, KV, rep, ngk;
    int *ordinal;        /* per sub-layer: attention ordinal or -1 */
    int *ord_layer;      /* per attention ordinal: its sub-layer index */
    float *inv_s, *inv_f;
    seq_t *seqs;
    int prompt_loops;    /* [dory] `prompt_loops`: 0 = as many passes as any chunk */
    int gate_on;         /* [dory] `Gate::Conf(th)` for one-row calls */
    float gate_th;
};

/* ------------------------------------------------------------------ primitives */

/* [dory] `justnorm`: x * 1/sqrt(sum x^2 + eps). */
void ora_justnorm(float *x, int32_t n) {
    double s = 0.0;
    for (int i = 0; i < n; i++) s += (double)x[i] * (double)x[i];
    double r = 1.0 / sqrt(s + ORA_EPS);
    for (int i = 0; i < n; i++) x[i] = (float)((double)x[i] * r);
}

/* [dory] `slerp`, the nGPT residual: x = justnorm(x^ + alpha*(o^ - x^)). */
void ora_slerp(float *x, const float *o, const float *alpha, int32_t n) {
    float *oh = (float *)malloc(sizeof(float) * (size_t)n);
    memcpy(oh, o, sizeof(float) * (size_t)n);
    ora_justnorm(x, n);
    ora_justnorm(oh, n);
    for (int i = 0; i < n; i++)
        x[i] = (float)((double)x[i] + (double)alpha[i] * ((double)oh[i] - (double)x[i]));
    ora_justnorm(x, n);
    free(oh);
}

/* RoPE inverse frequencies theta^(-2j/hd), j < hd/2, rounded to fp32.  The page
 * calls `rope_inv_freq` without showing it; this is the standard definition. */
void ora_rope_inv(int32_t hd, double theta, float *inv) {
    for (int j = 0; j < hd / 2; j++) inv[j] = (float)pow(theta, -2.0 * j / (double)hd);
}

/* [dory] `stack` (the tables: angle p*inv[j] in f64, cos and sin rounded to f32)
 * and `attn_layer` (rotate-half pairing of channel j with j + hd/2). */
void ora_rope_rotate(float *row, int32_t hd, const float *inv, int64_t pos) {
    int half = hd / 2;
    for (int j = 0; j < half; j++) {
        double a = (double)pos * (double)inv[j];
        float cs = (float)cos(a), sn = (float)sin(a);
        double x = row[j], y = row[j + half];
        row[j] = (float)(x * cs - y * sn);
        row[j + half] = (float)(y * cs + x * sn);
    }
}

/* [dory] `silu_body`: silu(a*sg) * (b*su). */
float ora_silu_gate(float a, float sg, float b, float su) {
    double x = (double)a * (double)sg;
    return (float)(x / (1.0 + exp(-x)) * ((double)b * (double)su));
}

/* [dory] `gate_body`: y * sigmoid(g*sg), written as y / (1 + exp(-g*sg)). */
float ora_sigmoid_gate(float y, float g, float sg) {
    return (float)((double)y / (1.0 + exp(-((double)g * (double)sg))));
}

/* y[r] = W[r][:] . x, fp64 sum.  W is [rows][cols]. */
static void matvec(const float *W, const float *x, int rows, int cols, float *y) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; r++) {
        const float *wr = W + (size_t)r * cols;
        double s = 0.0;
        for (int c = 0; c < cols; c++) s += (double)wr[c] * (double)x[c];
        y[r] = (float)s;
    }
}

/* Softmax over n scores in place, max-subtracted ([dory] `soft_body`). */
static void softmax(double *s, int64_t n) {
    double top = -INFINITY;
    for (int64_t e = 0; e < n; e++) if (s[e] > top) top = s[e];
    double den = 0.0;
    for (int64_t e = 0; e < n; e++) { s[e] = exp(s[e] - top); den += s[e]; }
    for (int64_t e = 0; e < n; e++) s[e] /= den;
}

/* Attention of one row at position p over keys first ..= p, every q head h
 * reading kv head h / (nh/nk) ([dory] `attn_layer`, the exact branch).
 * q: [nh][hd]; k, v: [p+1][nk][hd] by position; y: [nh][hd];
 * probs (optional): [nh][p+1-first]. */
void ora_attend(const float *q, const float *k, const float *v, int64_t p, int64_t first,
                int32_t nh, int32_t nk, int32_t hd, float *y, float *probs) {
    int rep = nh / nk;
    int64_t n = p + 1 - first;
    double scale = 1.0 / sqrt((double)hd);
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    for (int h = 0; h < nh; h++) {
        int kh = h / rep;
        for (int64_t e = 0; e < n; e++) {
            const float *key = k + ((first + e) * nk + kh) * hd;
            double d = 0.0;
            for (int i = 0; i < hd; i++) d += (double)q[h * hd + i] * (double)key[i];
            s[e] = d * scale;
        }
        softmax(s, n);
        for (int i = 0; i < hd; i++) {
            double acc = 0.0;
            for (int64_t e = 0; e < n; e++) acc += s[e] * (double)v[((first + e) * nk + kh) * hd + i];
            y[h * hd + i] = (float)acc;
        }
        if (probs) for (int64_t e = 0; e < n; e++) probs[h * n + e] = (float)s[e];
    }
    free(s);
}

/* The same over q8_2f rows ([kv] `attend_group_upto`, quantized branches):
 * score = (sum_g ks_g * <kcode_g, (q*kcol)_g>) / sqrt(hd);
 * y = (sum_e p_e * vs_e * vcode_e) * vcol.  kcol/vcol NULL: not frozen (1). */
void ora_attend_q8(const float *q, const int8_t *kc, const float *ks, const int8_t *vc,
                   const float *vs, const float *kcol, const float *vcol, int64_t p,
                   int64_t first, int32_t nh, int32_t nk, int32_t hd, float *y, float *probs) {
    int rep = nh / nk, ngk = (hd + ORA_KGROUP - 1) / ORA_KGROUP;
    int64_t n = p + 1 - first;
    double scale = 1.0 / sqrt((double)hd);
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    float *qc = (float *)malloc(sizeof(float) * (size_t)hd);
    for (int h = 0; h < nh; h++) {
        int kh = h / rep;
        for (int i = 0; i < hd; i++) qc[i] = kcol ? q[h * hd + i] * kcol[kh * hd + i] : q[h * hd + i];
        for (int64_t e = 0; e < n; e++) {
            int64_t row = (first + e) * nk + kh;
            double d = 0.0;
            for (int g = 0; g < ngk; g++) {
                int g0 = g * ORA_KGROUP, g1 = g0 + ORA_KGROUP < hd ? g0 + ORA_KGROUP : hd;
                double dg = 0.0;
                for (int i = g0; i < g1; i++) dg += (double)kc[row * hd + i] * (double)qc[i];
                d += dg * (double)ks[row * ngk + g];
            }
            s[e] = d * scale;
        }
        softmax(s, n);
        for (int i = 0; i < hd; i++) {
            double acc = 0.0;
            for (int64_t e = 0; e < n; e++) {
                int64_t row = (first + e) * nk + kh;
                acc += s[e] * (double)vs[row] * (double)vc[row * hd + i];
            }
            y[h * hd + i] = (float)(vcol ? acc * (double)vcol[kh * hd + i] : acc);
        }
        if (probs) for (int64_t e = 0; e < n; e++) probs[h * n + e] = (float)s[e];
    }
    free(qc);
    free(s);
}

/* [kv] `quant_row`: r = x/col (x when not frozen); per group of `group`
 * channels (the last may be short) s = max(absmax/127, 1e-12) and
 * code = clamp(round(r/s), -127, 127), rounding half away from zero.  All fp32. */
void ora_q8_encode(const float *x, const float *col, int32_t n, int32_t group,
                   int8_t *codes, float *scales) {
    float *r = (float *)malloc(sizeof(float) * (size_t)n);
    for (int d = 0; d < n; d++) r[d] = col ? x[d] / col[d] : x[d];
    for (int g0 = 0, gi = 0; g0 < n; g0 += group, gi++) {
        int g1 = g0 + group < n ? g0 + group : n;
        float absmax = 0.0f;
        for (int d = g0; d < g1; d++) { float a = fabsf(r[d]); if (a > absmax) absmax = a; }
        float s = absmax / 127.0f;
        if (s < 1e-12f) s = 1e-12f;
        scales[gi] = s;
        for (int d = g0; d < g1; d++) {
            float c = roundf(r[d] / s);
            if (c < -127.0f) c = -127.0f;
            if (c > 127.0f) c = 127.0f;
            codes[d] = (int8_t)c;
        }
    }
    free(r);
}

/* [kv] `freeze_cols` for one head: dequantize every stored row (code * scale,
 * fp32), col[d] = max(sqrt(sum_p row_pd^2 / n), 1e-6) with the squares summed
 * in fp32 in row order, then re-encode every row against col.
 * codes [rows][hd], scales [rows][ceil(hd/group)]. */
void ora_q8_freeze(int8_t *codes, float *scales, int64_t rows, int32_t hd, int32_t group,
                   float *col) {
    int spp = (hd + group - 1) / group;
    float *deq = (float *)malloc(sizeof(float) * (size_t)(rows * hd));
    for (int64_t p = 0; p < rows; p++)
        for (int d = 0; d < hd; d++)
            deq[p * hd + d] = (float)codes[p * hd + d] * scales[p * spp + d / group];
    for (int d = 0; d < hd; d++) col[d] = 0.0f;
    for (int64_t p = 0; p < rows; p++)
        for (int d = 0; d < hd; d++) {
            float sq = deq[p * hd + d] * deq[p * hd + d];
            col[d] = col[d] + sq;
        }
    for (int d = 0; d < hd; d++) {
        float c = sqrtf(col[d] / (float)rows);
        col[d] = c > 1e-6f ? c : 1e-6f;
    }
    for (int64_t p = 0; p < rows; p++)
        ora_q8_encode(deq + p * hd, col, hd, group, codes + p * hd, scales + p * spp);
    free(deq);
}

/* ------------------------------------------------------------------ the cache */

static int slot_alloc(ora_model *m, slot_t *s) {
    if (s->k || s->kc) return ORA_OK;
    size_t rows = (size_t)m->c.max_ctx, row = (size_t)m->c.nk * m->c.hd;
    if (m->c.kv_q8) {
        s->kc = (int8_t *)calloc(rows * row, 1);
        s->vc = (int8_t *)calloc(rows * row, 1);
        s->ks = (float *)calloc(rows * m->c.nk * m->ngk, sizeof(float));
        s->vs = (float *)calloc(rows * m->c.nk, sizeof(float));
        s->kcol = (float *)calloc(row, sizeof(float));
        s->vcol = (float *)calloc(row, sizeof(float));
        if (!s->kc || !s->vc || !s->ks || !s->vs || !s->kcol || !s->vcol) return ORA_ENOMEM;
    } else {
        s->k = (float *)calloc(rows * row, sizeof(float));
        s->v = (float *)calloc(rows * row, sizeof(float));
        if (!s->k || !s->v) return ORA_ENOMEM;
    }
    return ORA_OK;
}

static void slot_free(slot_t *s) {
    free(s->k); free(s->v); free(s->kc); free(s->vc);
    free(s->ks); free(s->vs); free(s->kcol); free(s->vcol);
    memset(s, 0, sizeof(*s));
}

/* [kv] `freeze_cols` over a whole slot: every kv head, K (groups of 32) and V
 * (one group of hd). */
static void slot_freeze(ora_model *m, slot_t *s) {
    int nk = m->c.nk, hd = m->c.hd, ngk = m->ngk;
    int64_t n = s->rows;
    int8_t *c = (int8_t *)malloc((size_t)(n * hd));
    float *sc = (float *)malloc(sizeof(float) * (size_t)(n * ngk));
    for (int h = 0; h < nk; h++) {
        /* K of head h, gathered contiguous */
        for (int64_t p = 0; p < n; p++) {
            memcpy(c + p * hd, s->kc + (p * nk + h) * hd, (size_t)hd);
            memcpy(sc + p * ngk, s->ks + (p * nk + h) * ngk, sizeof(float) * (size_t)ngk);
        }
        ora_q8_freeze(c, sc, n, hd, ORA_KGROUP, s->kcol + h * hd);
        for (int64_t p = 0; p < n; p++) {
            memcpy(s->kc + (p * nk + h) * hd, c + p * hd, (size_t)hd);
            memcpy(s->ks + (p * nk + h) * ngk, sc + p * ngk, sizeof(float) * (size_t)ngk);
        }
        /* V of head h */
        for (int64_t p = 0; p < n; p++) {
            memcpy(c + p * hd, s->vc + (p * nk + h) * hd, (size_t)hd);
            sc[p] = s->vs[p * nk + h];
        }
        ora_q8_freeze(c, sc, n, hd, hd, s->vcol + h * hd);
        for (int64_t p = 0; p < n; p++) {
            memcpy(s->vc + (p * nk + h) * hd, c + p * hd, (size_t)hd);
            s->vs[p * nk + h] = sc[p];
        }
    }
    s->frozen = 1;
    free(c);
    free(sc);
}

/* [kv] `append`: the field freezes at the start of an append once 64 rows are
 * stored; then each kv head's K and V are stored (encoded under q8). */
static void slot_append(ora_model *m, slot_t *s, const float *k, const float *v) {
    int nk = m->c.nk, hd = m->c.hd, ngk = m->ngk;
    int64_t p = s->rows;
    if (m->c.kv_q8) {
        if (s->rows >= ORA_WARMUP && !s->frozen) slot_freeze(m, s);
        for (int h = 0; h < nk; h++) {
            ora_q8_encode(k + h * hd, s->frozen ? s->kcol + h * hd : NULL, hd, ORA_KGROUP,
                          s->kc + (p * nk + h) * hd, s->ks + (p * nk + h) * ngk);
            ora_q8_encode(v + h * hd, s->frozen ? s->vcol + h * hd : NULL, hd, hd,
                          s->vc + (p * nk + h) * hd, s->vs + (p * nk + h));
        }
    } else {
        memcpy(s->k + p * nk * hd, k, sizeof(float) * (size_t)(nk * hd));
        memcpy(s->v + p * nk * hd, v, sizeof(float) * (size_t)(nk * hd));
    }
    s->rows++;
}

/* [kv] `truncate_last`: drop the last n rows (codes and scales with them). */
static void slot_truncate(slot_t *s, int64_t n) { s->rows = n > s->rows ? 0 : s->rows - n; }

/* ------------------------------------------------------------------ the model */

int ora_create(const ora_cfg *cfg, const ora_weights *w, ora_model **out) {
    if (!cfg || !w || !out || !cfg->pattern) return ORA_EINVAL;
    const ora_cfg *c = cfg;
    int nl = (int)strlen(c->pattern);
    if (c->hidden <= 0 || c->ffn <= 0 || c->vocab <= 0 || c->nh <= 0 || c->nk <= 0 ||
        c->hd <= 0 || c->hd % 2 || c->nh % c->nk || nl != c->n_in + c->n_rec + c->n_out ||
        c->n_in < 0 || c->n_rec < 0 || c->n_out < 0 || c->window <= 0 || c->full_window < 0 ||
        c->max_ctx <= 0 || c->max_seqs <= 0)
        return ORA_EINVAL;
    ora_model *m = (ora_model *)calloc(1, sizeof(ora_model));
    m->c = *c;
    m->pattern = (char *)malloc((size_t)nl + 1);
    memcpy(m->pattern, c->pattern, (size_t)nl + 1);
    m->c.pattern = m->pattern;
    m->w = *w;
    m->n_layers = nl;
    m->layers = (ora_layer *)malloc(sizeof(ora_layer) * (size_t)nl);
    memcpy(m->layers, w->layers, sizeof(ora_layer) * (size_t)nl);
    m->w.layers = m->layers;
    m->ordinal = (int *)malloc(sizeof(int) * (size_t)nl);
    m->ord_layer = (int *)malloc(sizeof(int) * (size_t)nl);
    for (int li = 0; li < nl; li++) {
        m->ordinal[li] = c->pattern[li] == '-' ? -1 : m->n_ord;
        if (c->pattern[li] != '-') m->ord_layer[m->n_ord++] = li;
    }
    m->Q = c->nh * c->hd;
    m->KV = c->nk * c->hd;
    m->rep = c->nh / c->nk;
    m->ngk = (c->hd + ORA_KGROUP - 1) / ORA_KGROUP;
    m->inv_s = (float *)malloc(sizeof(float) * (size_t)(c->hd / 2));
    m->inv_f = (float *)malloc(sizeof(float) * (size_t)(c->hd / 2));
    ora_rope_inv(c->hd, c->theta_s, m->inv_s);
    ora_rope_inv(c->hd, c->theta_f, m->inv_f);
    m->seqs = (seq_t *)calloc((size_t)c->max_seqs, sizeof(seq_t));
    for (int s = 0; s < c->max_seqs; s++) {
        m->seqs[s].mode = -1;
        m->seqs[s].exit_rate = 1.0f;
        m->seqs[s].last_top = -1.0f;
        m->seqs[s].slots = (slot_t *)calloc((size_t)(m->n_ord * ORA_MAX_LOOPS), sizeof(slot_t));
    }
    *out = m;
    return ORA_OK;
}

void ora_destroy(ora_model *m) {
    if (!m) return;
    for (int s = 0; s < m->c.max_seqs; s++) {
        for (int i = 0; i < m->n_ord * ORA_MAX_LOOPS; i++) slot_free(&m->seqs[s].slots[i]);
        free(m->seqs[s].slots);
    }
    free(m->seqs); free(m->inv_s); free(m->inv_f); free(m->ordinal); free(m->ord_layer);
    free(m->layers); free(m->pattern); free(m);
}

/* [dory] `DoryState::clear` and [kv] `clear`: every slot empties, fields go. */
int ora_reset(ora_model *m, int32_t seq) {
    if (!m || seq < -1 || seq >= m->c.max_seqs) return ORA_EINVAL;
    for (int s = 0; s < m->c.max_seqs; s++) {
        if (seq >= 0 && s != seq) continue;
        seq_t *q = &m->seqs[s];
        for (int i = 0; i < m->n_ord * ORA_MAX_LOOPS; i++) {
            q->slots[i].rows = 0;
            q->slots[i].frozen = 0;
        }
        q->pos = 0;
        q->mode = -1;
        q->loops = 0;
        q->exit_rate = 1.0f;
        q->exit_tokens = 0;
        q->gate_tokens = q->gate_one = 0;
        q->last_top = -1.0f;
    }
    return ORA_OK;
}

/* [dory] `DoryState::rollback`: every slot forgets its rows from position n on
 * and the position becomes min(pos, n).  [kv] `truncate_last` drops rows only:
 * a frozen q8 field stays frozen (it froze once per conversation), and an
 * unfrozen one freezes at the next append with 64 or more rows stored. */
int ora_rollback(ora_model *m, int32_t seq, int64_t n) {
    if (!m || seq < 0 || seq >= m->c.max_seqs || n < 0) return ORA_EINVAL;
    seq_t *q = &m->seqs[seq];
    for (int i = 0; i < m->n_ord * ORA_MAX_LOOPS; i++)
        if (q->slots[i].rows > n) q->slots[i].rows = n;
    if (q->pos > n) q->pos = n;
    return ORA_OK;
}

int64_t ora_pos(const ora_model *m, int32_t seq) { return m->seqs[seq].pos; }

int ora_passes(const ora_model *m, int32_t loops) {
    return m->c.n_in + m->c.n_rec * loops + m->c.n_out;
}

static int is_recurrent(const ora_model *m, int li) {
    return li >= m->c.n_in && li < m->c.n_in + m->c.n_rec;
}

/* One attention sub-layer over the rows h[t][hidden] at positions pos0.. of the
 * sequence ([dory] `attn_layer`, exact branch; `stack` for the slot choice). */
static void attn_sub(ora_model *m, seq_t *sq, int li, int loop_i, float *h, int t, int64_t pos0) {
    const ora_cfg *c = &m->c;
    const ora_layer *L = &m->layers[li];
    int H = c->hidden, Q = m->Q, KV = m->KV, hd = c->hd, nh = c->nh, nk = c->nk;
    int sliding = c->pattern[li] == 'S';
    int rec = is_recurrent(m, li);
    /* [dory] `slot_loop`: per_loop keeps a slot per loop for recurrent layers. */
    int si = (sq->mode == ORA_PER_LOOP && rec) ? loop_i : 0;
    /* [dory] `stack`: under last_loop a later loop rewrites this chunk's rows
     * (in the output block, only the early exit's second read-out runs at a
     * later loop: it replaces the first read-out's rows). */
    int overwrite = sq->mode == ORA_LAST_LOOP && li >= c->n_in && loop_i > 0;
    slot_t *s = &sq->slots[m->ordinal[li] * ORA_MAX_LOOPS + si];
    const float *inv = sliding ? m->inv_s : m->inv_f;

    float *q = (float *)malloc(sizeof(float) * (size_t)t * Q);
    float *k = (float *)malloc(sizeof(float) * (size_t)t * KV);
    float *v = (float *)malloc(sizeof(float) * (size_t)t * KV);
    float *g = (float *)malloc(sizeof(float) * (size_t)t * Q);
    float *y = (float *)malloc(sizeof(float) * (size_t)t * Q);
    float *o = (float *)malloc(sizeof(float) * (size_t)t * H);
    for (int r = 0; r < t; r++) {
        matvec(L->wq, h + (size_t)r * H, Q, H, q + (size_t)r * Q);
        matvec(L->wk, h + (size_t)r * H, KV, H, k + (size_t)r * KV);
        matvec(L->wv, h + (size_t)r * H, KV, H, v + (size_t)r * KV);
        matvec(L->wg, h + (size_t)r * H, Q, H, g + (size_t)r * Q);
    }
    /* Rotate q and k, unit-normalise per head, q times sq. */
    for (int r = 0; r < t; r++) {
        for (int hh = 0; hh < nh; hh++) {
            float *row = q + (size_t)r * Q + hh * hd;
            ora_rope_rotate(row, hd, inv, pos0 + r);
            ora_justnorm(row, hd);
            for (int i = 0; i < hd; i++) row[i] *= L->sq[hh * hd + i];
        }
        for (int hh = 0; hh < nk; hh++) {
            float *row = k + (size_t)r * KV + hh * hd;
            ora_rope_rotate(row, hd, inv, pos0 + r);
            ora_justnorm(row, hd);
        }
    }
    /* The chunk's rows join the slot (after dropping them under overwrite). */
    if (overwrite) slot_truncate(s, t);
    for (int r = 0; r < t; r++) slot_append(m, s, k + (size_t)r * KV, v + (size_t)r * KV);
    /* Each row reads keys max(p+1-window, 0) ..= p. */
    int64_t win = sliding ? c->window : (c->full_window > 0 ? c->full_window : (int64_t)1 << 62);
#pragma omp parallel for schedule(dynamic)
    for (int r = 0; r < t; r++) {
        int64_t p = pos0 + r;
        int64_t first = p + 1 - win > 0 ? p + 1 - win : 0;
        if (c->kv_q8)
            ora_attend_q8(q + (size_t)r * Q, s->kc, s->ks, s->vc, s->vs,
                          s->frozen ? s->kcol : NULL, s->frozen ? s->vcol : NULL, p, first, nh, nk,
                          hd, y + (size_t)r * Q, NULL);
        else
            ora_attend(q + (size_t)r * Q, s->k, s->v, p, first, nh, nk, hd, y + (size_t)r * Q, NULL);
    }
    /* Sigmoid gate, then one justnorm over the whole Q row, then O. */
    for (int r = 0; r < t; r++) {
        float *yr = y + (size_t)r * Q;
        for (int i = 0; i < Q; i++) yr[i] = ora_sigmoid_gate(yr[i], g[(size_t)r * Q + i], L->sg[i]);
        ora_justnorm(yr, Q);
        matvec(L->wo, yr, H, Q, o + (size_t)r * H);
        ora_slerp(h + (size_t)r * H, o + (size_t)r * H, L->alpha, H);
    }
    free(q); free(k); free(v); free(g); free(y); free(o);
}

/* [dory] `mlp_layer`: silu(a*sg)*(b*su), justnorm over ffn, down, slerp. */
static void mlp_sub(ora_model *m, int li, float *h, int t) {
    const ora_cfg *c = &m->c;
    const ora_layer *L = &m->layers[li];
    int H = c->hidden, F = c->ffn;
    float *a = (float *)malloc(sizeof(float) * (size_t)F);
    float *b = (float *)malloc(sizeof(float) * (size_t)F);
    float *o = (float *)malloc(sizeof(float) * (size_t)H);
    for (int r = 0; r < t; r++) {
        float *hr = h + (size_t)r * H;
        matvec(L->wgate, hr, F, H, a);
        matvec(L->wup, hr, F, H, b);
        for (int i = 0; i < F; i++) a[i] = ora_silu_gate(a[i], L->sg[i], b[i], L->su[i]);
        ora_justnorm(a, F);
        matvec(L->wdown, a, H, F, o);
        ora_slerp(hr, o, L->alpha, H);
    }
    free(a); free(b); free(o);
}

static int check_call(ora_model *m, int32_t seq, int32_t n, int32_t loops, int32_t kv_mode) {
    if (!m || seq < 0 || seq >= m->c.max_seqs || n < 1) return ORA_EINVAL;
    if (loops < 1 || loops > ORA_MAX_LOOPS) return ORA_EINVAL;
    if (kv_mode != ORA_PER_LOOP && kv_mode != ORA_LAST_LOOP) return ORA_EINVAL;
    seq_t *q = &m->seqs[seq];
    if (q->mode >= 0 && q->mode != kv_mode) return ORA_ESTATE;
    if (kv_mode == ORA_PER_LOOP && q->loops > 0 && q->loops != loops) return ORA_ESTATE;
    if (q->pos + n > m->c.max_ctx) return ORA_ERANGE;
    return ORA_OK;
}

/* [dory] `forward_host` for one chunk, `stack` for the walk through the three
 * blocks, `head` for the logits of the last row. */
/* [dory] `top_prob`: the softmax probability of the largest logit, with the
 * terms more than 20 below it left out of the sum (f64 sum, f32 result). */
float ora_top_prob(const float *lg, int32_t n) {
    float top = -INFINITY;
    for (int32_t i = 0; i < n; i++) top = lg[i] > top ? lg[i] : top;
    double den = 0.0;
    for (int32_t i = 0; i < n; i++) {
        float t = lg[i] - top;
        if (t > -20.0f) den += exp((double)t);
    }
    return (float)(1.0 / den);
}

/* [dory] `ExitRate::probe`: is this token worth a read-out after its first
 * pass?  Always while early exits are frequent (rate >= 0.35), else one token
 * in eight. */
static int exit_probe(seq_t *q) {
    q->exit_tokens += 1u;
    return q->exit_rate >= 0.35f || q->exit_tokens % 8u == 0u;
}

/* [dory] `ExitRate::note`: a running mean of the exits, weight 0.1 (f32). */
static void exit_note(seq_t *q, int exited) {
    q->exit_rate += 0.1f * ((float)(exited ? 1 : 0) - q->exit_rate);
}

int ora_set_gate(ora_model *m, int32_t on, float th) {
    if (!m || (on && !(th >= 0.0f))) return ORA_EINVAL;
    m->gate_on = on ? 1 : 0;
    m->gate_th = th;
    return ORA_OK;
}

int ora_gate_stats(const ora_model *m, int32_t seq, int64_t *tokens, int64_t *one, float *last_top, float *rate) {
    if (!m || seq < 0 || seq >= m->c.max_seqs) return ORA_EINVAL;
    const seq_t *q = &m->seqs[seq];
    if (tokens) *tokens = (int64_t)q->gate_tokens;
    if (one) *one = (int64_t)q->gate_one;
    if (last_top) *last_top = q->last_top;
    if (rate) *rate = q->exit_rate;
    return ORA_OK;
}

/* Threads of the OpenMP loops (n <= 0: as many as the host has); the
 * arithmetic and its order do not depend on it.  Returns the count in use. */
int ora_set_threads(int32_t n) {
    omp_set_num_threads(n > 0 ? n : omp_get_num_procs());
    return omp_get_max_threads();
}

int ora_threads(void) { return omp_get_max_threads(); }

int ora_set_prompt_loops(ora_model *m, int32_t n) {
    if (!m || n < 0 || n > ORA_MAX_LOOPS) return ORA_EINVAL;
    m->prompt_loops = n;
    return ORA_OK;
}

int ora_forward(ora_model *m, int32_t seq, const int32_t *tokens, int32_t t, int32_t loops,
                int32_t kv_mode, float *logits, float *tap) {
    return ora_forward_want(m, seq, tokens, t, loops, kv_mode, logits ? ORA_WANT_LAST : ORA_WANT_NONE, logits, tap);
}

int ora_forward_want(ora_model *m, int32_t seq, const int32_t *tokens, int32_t t, int32_t loops,
                     int32_t kv_mode, int32_t want, float *logits, float *tap) {
    int rc = check_call(m, seq, t, loops, kv_mode);
    if (rc) return rc;
    if (!tokens || want < ORA_WANT_NONE || want > ORA_WANT_ALL || (want != ORA_WANT_NONE && !logits))
        return ORA_EINVAL;
    /* [dory] `stack`: under the gate a one-row call runs its first pass, and a
     * second one only if the gate asks for it, on the last-loop cache (a
     * per_loop cache would take the read-out's rows twice) */
    const int early = t == 1 && m->gate_on;
    if (early && (kv_mode != ORA_LAST_LOOP || tap)) return ORA_EINVAL;
    /* [dory] `chunk_loops`: a last_loop chunk whose logits nobody reads keeps
     * only its cache rows, and runs at most prompt_loops passes. */
    if (want == ORA_WANT_NONE && m->prompt_loops > 0 && kv_mode == ORA_LAST_LOOP && loops > m->prompt_loops)
        loops = m->prompt_loops;
    const ora_cfg *c = &m->c;
    seq_t *sq = &m->seqs[seq];
    int H = c->hidden;
    for (int i = 0; i < m->n_ord * ORA_MAX_LOOPS; i++) {
        int si = i % ORA_MAX_LOOPS;
        if (si == 0 || (kv_mode == ORA_PER_LOOP && si < loops))
            if (slot_alloc(m, &sq->slots[i])) return ORA_ENOMEM;
    }
    sq->mode = kv_mode;
    if (kv_mode == ORA_PER_LOOP) sq->loops = loops;
    int64_t pos0 = sq->pos;
    size_t rowsz = sizeof(float) * (size_t)t * H;
    float *h = (float *)calloc((size_t)t * H, sizeof(float));
    float *input = (float *)malloc(rowsz), *state = (float *)malloc(rowsz);
    /* Embedding rows; an id past the table is a zero row. */
    for (int r = 0; r < t; r++) {
        uint32_t id = (uint32_t)tokens[r];
        if (id < (uint32_t)c->vocab) memcpy(h + (size_t)r * H, m->w.embed + (size_t)id * H, sizeof(float) * H);
    }
    int pass = 0;
#define SUB(li, lp)                                                        \
    do {                                                                   \
        if (c->pattern[li] == '-') mlp_sub(m, li, h, t);                   \
        else attn_sub(m, sq, li, lp, h, t, pos0);                    \
        if (tap) memcpy(tap + (size_t)pass * t * H, h, rowsz);            \
        pass++;                                                            \
    } while (0)
    for (int li = 0; li < c->n_in; li++) SUB(li, 0);
    /* Loop: input = h; state = input; each pass h = justnorm(state + input),
     * the recurrent block, state = justnorm(h). */
    memcpy(input, h, rowsz);
    memcpy(state, input, rowsz);
    for (int i = 0; i < (early ? 1 : loops); i++) {
        for (size_t j = 0; j < (size_t)t * H; j++) h[j] = state[j] + input[j];
        for (int r = 0; r < t; r++) ora_justnorm(h + (size_t)r * H, H);
        for (int li = c->n_in; li < c->n_in + c->n_rec; li++) SUB(li, i);
        memcpy(state, h, rowsz);
        for (int r = 0; r < t; r++) ora_justnorm(state + (size_t)r * H, H);
    }
    memcpy(h, state, rowsz);
    float *exit_lg = NULL;
    if (early) {
        /* [dory] `stack`, the early exit (`Gate::Conf`): a read-out through the
         * output block and the head when the exit rate says it is worth one;
         * the token leaves if its top probability reaches the threshold.
         * Otherwise a second pass from the first one's state rewrites this
         * position (and the read-out's rows, at loop 1) and reads out again. */
        int stay = 1, readout = 0;
        if (exit_probe(sq)) {
            readout = 1;
            for (int li = c->n_in + c->n_rec; li < m->n_layers; li++) SUB(li, 0);
            exit_lg = (float *)malloc(sizeof(float) * (size_t)c->vocab);
            matvec(m->w.head, h, c->vocab, H, exit_lg);
            for (int i = 0; i < c->vocab; i++) exit_lg[i] *= m->w.logit_scale[i];
            sq->last_top = ora_top_prob(exit_lg, c->vocab);
            stay = sq->last_top < m->gate_th;
            exit_note(sq, !stay);
        }
        if (stay) {
            for (int j = 0; j < H; j++) h[j] = state[j] + input[j];
            ora_justnorm(h, H);
            for (int li = c->n_in; li < c->n_in + c->n_rec; li++) SUB(li, 1);
            ora_justnorm(h, H);
            for (int li = c->n_in + c->n_rec; li < m->n_layers; li++) SUB(li, readout);
            free(exit_lg);
            exit_lg = NULL;
        }
        sq->gate_tokens += 1;
        sq->gate_one += stay ? 0 : 1;
    } else {
        for (int li = c->n_in + c->n_rec; li < m->n_layers; li++) SUB(li, 0);
    }
#undef SUB
    if (exit_lg) {   /* the token left after one pass: the read-out's logits */
        if (want != ORA_WANT_NONE) memcpy(logits, exit_lg, sizeof(float) * (size_t)c->vocab);
        free(exit_lg);
        want = ORA_WANT_NONE;
    }
    /* [dory] `head`: the last row (`Want::Last`) or every row (`Want::All`). */
    for (int r = want == ORA_WANT_ALL ? 0 : t - 1; want != ORA_WANT_NONE && r < t; r++) {
        float *lg = logits + (want == ORA_WANT_ALL ? (size_t)r * c->vocab : 0);
        matvec(m->w.head, h + (size_t)r * H, c->vocab, H, lg);
        for (int i = 0; i < c->vocab; i++) lg[i] *= m->w.logit_scale[i];
    }
    sq->pos = pos0 + t;
    free(h); free(input); free(state);
    return ORA_OK;
}

int64_t ora_slot_rows(const ora_model *m, int32_t seq, int32_t ord, int32_t slot) {
    if (!m || seq < 0 || seq >= m->c.max_seqs || ord < 0 || ord >= m->n_ord || slot < 0 ||
        slot >= ORA_MAX_LOOPS)
        return -1;
    return m->seqs[seq].slots[ord * ORA_MAX_LOOPS + slot].rows;
}

int ora_kv_read(const ora_model *m, int32_t seq, int32_t ord, int32_t slot, int64_t pos, void *out) {
    int64_t rows = ora_slot_rows(m, seq, ord, slot);
    if (rows < 0 || pos < 0 || pos >= rows || !out) return ORA_EINVAL;
    const slot_t *s = &m->seqs[seq].slots[ord * ORA_MAX_LOOPS + slot];
    int nk = m->c.nk, hd = m->c.hd, ngk = m->ngk;
    if (!m->c.kv_q8) {
        memcpy(out, s->k + pos * nk * hd, sizeof(float) * (size_t)(nk * hd));
        memcpy((float *)out + nk * hd, s->v + pos * nk * hd, sizeof(float) * (size_t)(nk * hd));
    } else {
        char *b = (char *)out;
        memcpy(b, s->kc + pos * nk * hd, (size_t)(nk * hd)); b += nk * hd;
        memcpy(b, s->vc + pos * nk * hd, (size_t)(nk * hd)); b += nk * hd;
        memcpy(b, s->ks + pos * nk * ngk, sizeof(float) * (size_t)(nk * ngk)); b += sizeof(float) * nk * ngk;
        memcpy(b, s->vs + pos * nk, sizeof(float) * (size_t)nk);
    }
    return ORA_OK;
}

int ora_kv_field(const ora_model *m, int32_t seq, int32_t ord, int32_t slot, float *kcol, float *vcol) {
    if (ora_slot_rows(m, seq, ord, slot) < 0 || !m->c.kv_q8) return ORA_EINVAL;
    const slot_t *s = &m->seqs[seq].slots[ord * ORA_MAX_LOOPS + slot];
    int n = m->c.nk * m->c.hd;
    if (!s->kcol) return 0;
    if (kcol) memcpy(kcol, s->kcol, sizeof(float) * (size_t)n);
    if (vcol) memcpy(vcol, s->vcol, sizeof(float) * (size_t)n);
    return s->frozen;
}

int ora_kv_load(ora_model *m, int32_t seq, int32_t kv_mode, int32_t loops, int64_t npos,
                int32_t n_slot, const float *k, const float *v) {
    int rc = check_call(m, seq, 1, loops, kv_mode);
    if (rc) return rc;
    if (!k || !v || npos < 0 || npos > m->c.max_ctx || n_slot < 1 || n_slot > ORA_MAX_LOOPS) return ORA_EINVAL;
    if (n_slot < (kv_mode == ORA_PER_LOOP ? loops : 1)) return ORA_EINVAL;
    seq_t *sq = &m->seqs[seq];
    if (sq->pos != 0) return ORA_ESTATE;
    int KV = m->KV;
    for (int o = 0; o < m->n_ord; o++) {
        int ns = (kv_mode == ORA_PER_LOOP && is_recurrent(m, m->ord_layer[o])) ? loops : 1;
        for (int si = 0; si < ns; si++) {
            slot_t *s = &sq->slots[o * ORA_MAX_LOOPS + si];
            if (slot_alloc(m, s)) return ORA_ENOMEM;
            const float *kb = k + ((size_t)(o * n_slot + si) * npos) * KV;
            const float *vb = v + ((size_t)(o * n_slot + si) * npos) * KV;
            for (int64_t p = 0; p < npos; p++) slot_append(m, s, kb + p * KV, vb + p * KV);
        }
    }
    for (int i = 0; i < m->n_ord * ORA_MAX_LOOPS; i++) {
        int si = i % ORA_MAX_LOOPS;
        if (si == 0 || (kv_mode == ORA_PER_LOOP && si < loops))
            if (slot_alloc(m, &sq->slots[i])) return ORA_ENOMEM;
    }
    sq->mode = kv_mode;
    if (kv_mode == ORA_PER_LOOP) sq->loops = loops;
    sq->pos = npos;
    return ORA_OK;
}
