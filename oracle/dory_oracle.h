/*
 * dory_oracle.h -- the CPU oracle of the Dory token forward.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, constant or helper with the HIP path.
 *
 * What it computes follows three pages of the cortiq-engine crate:
 *   - "dory.rs" (the Dory module): the model, the host forward and its tests;
 *   - "kv_cache.rs" (the KV cache module): the q8_2f KV encoding;
 *   - "gpu_metal/dory.rs": the device path, used only for context.
 * Every function in dory_oracle.c names the item of those pages it follows.
 *
 * Precision: activations, weights and cache rows are stored in fp32, as the
 * pages store them; sums (dot products, norms, softmax denominators) are taken in
 * fp64 and rounded once.  The q8_2f encoder and its field freeze are the pages'
 * fp32 steps exactly, so their codes and scales are reproducible bit for bit.
 */
#ifndef DORY_ORACLE_H
#define DORY_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORA_OK = 0, ORA_EINVAL = -1, ORA_ESTATE = -2, ORA_ERANGE = -3, ORA_ENOMEM = -4 };
enum { ORA_PER_LOOP = 0, ORA_LAST_LOOP = 1 };

typedef struct {
    int32_t hidden, ffn, vocab, nh, nk, hd;
    const char *pattern;            /* one char per sub-layer: '-' MLP, 'S' sliding, other full */
    int32_t n_in, n_rec, n_out;
    int32_t window;                 /* sliding window (keys p-window+1 ..= p) */
    int32_t full_window;            /* 0: full layers read every key */
    double theta_s, theta_f;        /* RoPE bases of sliding and full layers */
    int32_t max_ctx, max_seqs;
    int32_t kv_q8;                  /* 1: q8_2f cache encoding */
} ora_cfg;

/* Per sub-layer weights, host fp32, row-major [out][in].  Attention uses
 * wq wk wv wg wo sq sg alpha; an MLP uses wgate wup wdown sg su alpha.  The
 * scale vectors are the effective (folded) ones. */
typedef struct {
    const float *wq, *wk, *wv, *wg, *wo, *sq;
    const float *wgate, *wup, *wdown, *su;
    const float *sg, *alpha;
} ora_layer;

typedef struct {
    const float *embed, *head, *logit_scale;
    const ora_layer *layers;
} ora_weights;

typedef struct ora_model ora_model;

int  ora_create(const ora_cfg *cfg, const ora_weights *w, ora_model **out);
void ora_destroy(ora_model *m);
/* One call = one chunk of n rows at the sequence's next position.
 * logits (vocab floats, row n-1) and tap ([passes][n][hidden], the residual
 * state after every sub-layer pass) may be NULL. */
int  ora_forward(ora_model *m, int32_t seq, const int32_t *tokens, int32_t n,
                 int32_t loops, int32_t kv_mode, float *logits, float *tap);
/* The same call with the rows whose logits are wanted ([dory] `Want`):
 * ORA_WANT_NONE (logits NULL), ORA_WANT_LAST (logits [vocab], row n-1) or
 * ORA_WANT_ALL (logits [n][vocab]). */
#define ORA_WANT_NONE 0
#define ORA_WANT_LAST 1
#define ORA_WANT_ALL 2
int  ora_forward_want(ora_model *m, int32_t seq, const int32_t *tokens, int32_t n,
                      int32_t loops, int32_t kv_mode, int32_t want, float *logits, float *tap);
/* [dory] `prompt_loops` (0..16, 0 = off): a last_loop call that wants no
 * logits runs min(loops, prompt_loops) passes of the recurrent block. */
int  ora_set_prompt_loops(ora_model *m, int32_t n);
int  ora_set_threads(int32_t n);   /* OpenMP threads (n <= 0: all); returns the count in use */
int  ora_threads(void);
/* [dory] `Gate::Conf(th)` (on = 0: no gate): a one-row last_loop call runs one
 * pass of the recurrent block, a read-out when the exit rate asks for one, and
 * a second pass unless the read-out's top probability reaches th.  Gated calls
 * take no tap. */
int  ora_set_gate(ora_model *m, int32_t on, float th);
/* Per sequence: gated tokens, tokens that left after one pass, the last
 * read-out's top probability (-1 before any) and the exit rate. */
int  ora_gate_stats(const ora_model *m, int32_t seq, int64_t *tokens, int64_t *one, float *last_top,
                    float *rate);
/* [dory] `top_prob`. */
float ora_top_prob(const float *lg, int32_t n);
int  ora_reset(ora_model *m, int32_t seq);
/* Forget the rows from position n on (dory.rs `DoryState::rollback`). */
int  ora_rollback(ora_model *m, int32_t seq, int64_t n);
int64_t ora_pos(const ora_model *m, int32_t seq);
int  ora_passes(const ora_model *m, int32_t loops);
/* Rows stored in a slot (attention ordinal, slot). */
int64_t ora_slot_rows(const ora_model *m, int32_t seq, int32_t ord, int32_t slot);
/* One stored row: fp32 -> K then V, each [nk][hd] floats; q8 -> K codes [nk][hd],
 * V codes [nk][hd] (int8), K scales [nk][ceil(hd/32)] f32, V scales [nk] f32. */
int  ora_kv_read(const ora_model *m, int32_t seq, int32_t ord, int32_t slot, int64_t pos, void *out);
/* The q8 per-channel fields [nk][hd] (K then V); returns 1 if frozen, 0 if not. */
int  ora_kv_field(const ora_model *m, int32_t seq, int32_t ord, int32_t slot, float *kcol, float *vcol);
/* Puts npos rows into every slot of a sequence through the append rules, as if
 * a forward had written them; k, v are [n_ord][n_slot][npos][nk][hd]. */
int  ora_kv_load(ora_model *m, int32_t seq, int32_t kv_mode, int32_t loops, int64_t npos,
                 int32_t n_slot, const float *k, const float *v);

/* Stage functions, exposed so the tests can pin them one by one. */
void ora_justnorm(float *x, int32_t n);
void ora_slerp(float *x, const float *o, const float *alpha, int32_t n);
void ora_rope_inv(int32_t hd, double theta, float *inv);
void ora_rope_rotate(float *row, int32_t hd, const float *inv, int64_t pos);
void ora_attend(const float *q, const float *k, const float *v, int64_t p, int64_t first,
                int32_t nh, int32_t nk, int32_t hd, float *y, float *probs);
void ora_attend_q8(const float *q, const int8_t *kc, const float *ks, const int8_t *vc,
                   const float *vs, const float *kcol, const float *vcol, int64_t p,
                   int64_t first, int32_t nh, int32_t nk, int32_t hd, float *y, float *probs);
void ora_q8_encode(const float *x, const float *col, int32_t n, int32_t group,
                   int8_t *codes, float *scales);
void ora_q8_freeze(int8_t *codes, float *scales, int64_t rows, int32_t hd, int32_t group,
                   float *col);
float ora_silu_gate(float a, float sg, float b, float su);
float ora_sigmoid_gate(float y, float g, float sg);

#ifdef __cplusplus
}
#endif
#endif
