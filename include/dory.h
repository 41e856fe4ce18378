/*
 * dory.h -- C ABI of libdory.so: the token forward of the Dory looped normalized
 * GPT on one AMD Instinct MI355X (gfx950).
 *
 * The method (pages of the cortiq-engine crate, "dory.rs" = the Dory module page,
 * "kv_cache.rs" = the KV cache module page):
 *   - dory.rs, module documentation and `stack`: a token passes an input block,
 *     a recurrent block run `loops` times with the input block's output re-added
 *     and renormalised before each pass, and an output block.  A sub-layer is one
 *     attention or one SwiGLU MLP; every residual state lives on the unit sphere.
 *   - dory.rs `attn_layer`: q,k,v,g projections, RoPE, per-head unit norm, q
 *     scaled by sq, k unit; grouped-query softmax over a sliding or full window;
 *     output gated by sigmoid(g*sg), renormalised over the row, projected by O.
 *   - dory.rs `mlp_layer`: silu(a*sg)*(b*su), renormalised, projected down.
 *   - dory.rs `slerp`: the residual x = norm(norm(x) + |alpha|*(norm(out) - norm(x))).
 *   - dory.rs `KvMode`, `slot_loop`, `stack`: per_loop keeps one cache per loop of
 *     each recurrent attention layer; last_loop keeps one, each loop rewriting the
 *     call's rows.
 *   - kv_cache.rs `quant_row`, `freeze_cols`, `append`, `attend_group_upto`: the
 *     optional q8_2f cache encoding (int8 codes, K scales per 32 channels, V scale
 *     per row, per-channel field frozen after 64 rows and applied retroactively).
 *
 * Conventions for every entry point:
 *   - Status codes: DORY_OK (0) or a negative DORY_E* value.  Every argument check
 *     runs before any work is enqueued; a failed check changes no state.  The
 *     message of the last failure is available from dory_last_error().
 *   - "device" pointers are HIP device memory on the current device; "host"
 *     pointers are ordinary CPU memory.
 *   - Calls on one handle must be serialised by the caller (one stream, or
 *     synchronised streams); the handle is not thread-safe.
 *   - A failed call latches (kv_cache.rs `append`: a failed transition is
 *     terminal until the sequence is cleared).  A forward or batch call that
 *     fails after its first device work was enqueued latches its sequences; a
 *     device error reported by a synchronisation inside the library latches
 *     every sequence.  A latched sequence answers DORY_ESTATE to every call
 *     (forward, batch row, rollback, taps, load) until dory_kv_reset.  Failed
 *     argument checks and failures before any device work latch nothing.
 *     A device fault that ends the process is beyond any latch.
 */
#ifndef DORY_H
#define DORY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DORY_OK 0
#define DORY_EINVAL (-1)   /* bad argument or configuration */
#define DORY_ESTATE (-2)   /* call disagrees with the sequence's state (kv mode, per_loop loop count),
                              or the sequence is latched after a failed call */
#define DORY_ERANGE (-3)   /* n > max_chunk, position past max_ctx, a row no longer held */
#define DORY_ENOMEM (-4)   /* device allocation failed */
#define DORY_EDEVICE (-5)  /* a HIP call failed */

#define DORY_PER_LOOP 0    /* dory.rs `KvMode::PerLoop` */
#define DORY_LAST_LOOP 1   /* dory.rs `KvMode::LastLoop` */
#define DORY_KV_F32 0      /* fp32 cache rows */
#define DORY_KV_Q8_2F 1    /* kv_cache.rs q8_2f encoding */
#define DORY_W_F32 0       /* fp32 weight matrices */
#define DORY_W_BF16 1      /* bf16 weight matrices (fp32 accumulation) */
#define DORY_MAX_LOOPS 16  /* dory.rs `MAX_LOOPS` */

typedef void *dory_stream_t; /* a hipStream_t; NULL is the null stream */

/* Model geometry and capacities (dory.rs `DoryCfg`, plus what a device library
 * must size up front). */
typedef struct {
    int32_t hidden, ffn, vocab;    /* H, F, V */
    int32_t nh, nk, hd;            /* q heads, kv heads (nh % nk == 0), head dim */
    const char *layer_pattern;     /* one char per sub-layer: '-' SwiGLU MLP, 'S' sliding
                                      attention, any other character full attention */
    int32_t n_in, n_rec, n_out;    /* sub-layers of the input, recurrent, output blocks */
    int32_t window;                /* sliding layers read keys p-window+1 ..= p */
    int32_t full_window;           /* full layers read at most this many keys; 0 = all */
    double rope_theta_sliding, rope_theta_full;
    int32_t max_ctx;               /* most positions a sequence may hold */
    int32_t max_chunk;             /* most rows one call may carry */
    int32_t max_seqs;              /* independent sequences (each with its own cache) */
    int32_t kv_encoding;           /* DORY_KV_F32 or DORY_KV_Q8_2F */
    int32_t weight_dtype;          /* DORY_W_F32 or DORY_W_BF16 */
} dory_config;

/* Weights of one sub-layer: device pointers, matrices row-major [out][in] in
 * weight_dtype, vectors fp32.  The vectors are the EFFECTIVE scales (the pages'
 * folded values: sq, sg, su, |alpha|).  Attention reads wq [Q][H], wk [KV][H],
 * wv [KV][H], wg [Q][H], wo [H][Q], sq [Q], sg [Q], alpha [H]; an MLP reads
 * wgate [F][H], wup [F][H], wdown [H][F], sg [F], su [F], alpha [H]
 * (Q = nh*hd, KV = nk*hd). */
typedef struct {
    const void *wq, *wk, *wv, *wg, *wo;
    const float *sq;
    const void *wgate, *wup, *wdown;
    const float *su;
    const float *sg;
    const float *alpha;
} dory_layer_weights;

typedef struct {
    const void *embed;             /* [V][H] weight_dtype */
    const void *head;              /* [V][H] weight_dtype */
    const float *logit_scale;      /* [V] */
    const dory_layer_weights *layers; /* host array, one entry per sub-layer */
} dory_weights;

typedef struct dory dory_t;

/* Builds a model over caller-owned device weights (which must outlive the handle,
 * unchanged) and allocates the caches and scratch.  Errors: DORY_EINVAL (bad
 * geometry: pattern length != n_in+n_rec+n_out, a block empty, nh % nk, hd not in
 * {8,16,32,64,128,256}, H, Q or F not a multiple of 8 or above 8192, ...),
 * DORY_ENOMEM, DORY_EDEVICE.  *out is NULL on failure. */
int dory_create(const dory_config *cfg, const dory_weights *w, dory_t **out);

void dory_destroy(dory_t *h);

/* Message of the last failed call on h (owned by h; valid until the next call).
 * With h == NULL: the last dory_create failure of this thread. */
const char *dory_last_error(const dory_t *h);

/* One forward call: n rows (tokens, host int32, copied before return) at the
 * sequence's next positions -- dory.rs `forward_host` for one chunk, `stack`
 * for the walk.  loops in 1..16.  kv_mode is fixed per sequence until
 * dory_kv_reset; under per_loop the loop count is fixed too (DORY_ESTATE).
 * Token ids outside [0, vocab) embed as zero rows.  logits: device fp32 [vocab]
 * for row n-1, scaled by logit_scale, or NULL for no head (`Want::None`).
 * Asynchronous on stream; logits are valid once the stream has reached the end
 * of this call.  Rows of one call are written to the cache at each loop before
 * any row of that loop reads it, and each row reads keys up to its own position. */
int dory_forward_chunk(dory_t *h, int32_t seq, const int32_t *tokens, int32_t n,
                       int32_t loops, int32_t kv_mode, dory_stream_t stream, float *logits);

/* dory_forward_chunk with the logits of every row (dory.rs `Want::All`):
 * logits is device fp32 [n][vocab], row r for the token at position pos + r,
 * and must not be NULL (DORY_EINVAL).  Rows of a multi-row call go through the
 * head as one GEMM (bf16 weights: bf16 operands, fp32 accumulation, as the
 * other projections of such a call); the handle allocates a [max_chunk][vocab]
 * fp32 buffer for it on the first such call.  Otherwise as dory_forward_chunk. */
int dory_forward_chunk_all(dory_t *h, int32_t seq, const int32_t *tokens, int32_t n,
                           int32_t loops, int32_t kv_mode, dory_stream_t stream, float *logits);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * dory_forward_chunk for calls of up to 8 rows that allocates nothing.  Its
 * kernels are the same; their scratch (activations, split partials, the call
 * record) is a carve-out of a static device array of 16 MiB, one per GPU,
 * held until the process ends, instead of the handle's buffers; no HIP graph
 * is captured or replayed (the kernels are enqueued on stream each call).
 * Every such call on a GPU shares that GPU's array and leaves its contents
 * there: calls that overlap on one GPU -- any handle, any stream -- race, so
 * the caller serialises them.  Besides dory_forward_chunk's checks:
 * DORY_ERANGE for n > 8 or a geometry whose scratch for 8 rows exceeds the
 * array (the message gives both sizes); DORY_EINVAL while the exit gate is on;
 * DORY_ESTATE when a per_loop slot the call needs does not exist yet (an
 * ordinary call with that loop count creates it); DORY_EDEVICE when the
 * array's address could not be had on this device.  It calls no hipMalloc,
 * hipFree or other allocating routine.  Afterwards dory_stage_bench needs an
 * ordinary call first. */
int dory_forward_chunk_noalloc(dory_t *h, int32_t seq, const int32_t *tokens, int32_t n,
                               int32_t loops, int32_t kv_mode, dory_stream_t stream, float *logits);

/* dory.rs `prompt_loops` (0..16; 0, the default, turns it off): a last_loop
 * call that wants no logits (logits NULL; a batch with logits NULL, row by row)
 * runs min(loops, n) passes of the recurrent block, since only its cache rows
 * stay (dory.rs `chunk_loops`).  per_loop calls are not affected. */
int dory_set_prompt_loops(dory_t *h, int32_t n);

/* dory.rs `Gate::Conf(threshold)`, the confidence-gated early exit (on = 0
 * turns it off; threshold >= 0, else DORY_EINVAL).  While on, every one-row
 * call (a call of one token) runs one pass of the recurrent block instead of
 * `loops`; if its sequence's exit rate asks for a read-out (dory.rs `ExitRate`:
 * while at least 0.35 of the recent read-outs exited, else one token in eight)
 * it runs the output block and the head, and the token leaves with those
 * logits when their top probability (dory.rs `top_prob`) reaches the
 * threshold.  Otherwise a second pass from the first one's state rewrites the
 * position (and the read-out's rows) and the output block and head run again.
 * A call with a read-out waits for it on the host (it synchronises its
 * stream); one without is a plain two-pass call.  Gated calls need the
 * last_loop cache and no tap (DORY_EINVAL); batches of several sequences are
 * refused while the gate is on.  The first call allocates a few buffers. */
int dory_set_gate(dory_t *h, int32_t on, float threshold);

/* The gate's counters of a sequence: gated tokens, tokens that left after one
 * pass, the last read-out's top probability (-1 before any), the exit rate
 * (any pointer may be NULL).  Cleared by dory_kv_reset. */
int dory_gate_stats(const dory_t *h, int32_t seq, int64_t *tokens, int64_t *one, float *last_top, float *rate);

/* One decode step of nseq sequences at once: row i is the next token of
 * sequence seqs[i] (distinct, 0 <= seqs[i] < max_seqs), run with loops[i] passes
 * of the recurrent block (1..16; per_loop sequences need their fixed count).
 * Rows with fewer loops leave the recurrent block early; the weights are read
 * once per pass for all rows that still run it (dory.rs `stack` for each row).
 * nseq <= max_chunk.  tokens, seqs, loops: host int32 [nseq].  logits: device
 * fp32 [nseq][vocab] (row i for seqs[i]) or NULL.  Checks as dory_forward_chunk,
 * for every row, before any work.  Asynchronous on stream. */
int dory_forward_batch(dory_t *h, int32_t nseq, const int32_t *seqs, const int32_t *tokens,
                       const int32_t *loops, int32_t kv_mode, dory_stream_t stream, float *logits);

/* A new sequence (dory.rs `DoryState::clear`, kv_cache.rs `clear`): position 0,
 * kv mode and loop count free again, q8 fields unfrozen.  seq == -1: all. */
int dory_kv_reset(dory_t *h, int32_t seq);

/* Forget the rows of a sequence from position n on (dory.rs
 * `DoryState::rollback`, e.g. a chat turn that rewrites the last answer): its
 * next call starts at position min(pos, n); kv mode, per_loop loop count and
 * frozen q8_2f fields stay as they are (kv_cache.rs `truncate_last` drops rows
 * only).  The windowed rings keep cap - W + 1 >= max_chunk rows of slack, so a
 * rollback may go back that far on them (the pages' Metal rings keep 448 rows,
 * dory.rs `REWIND`); deeper, DORY_ERANGE and nothing changes.  DORY_EINVAL for a
 * bad seq or n < 0.  Host bookkeeping only: it enqueues nothing, and the rows
 * past n are overwritten by the next call before any row reads them.  Must
 * not run while a call on the sequence is still being enqueued. */
int dory_rollback(dory_t *h, int32_t seq, int64_t n);

/* Next position of a sequence (rows held), or a negative status. */
int64_t dory_position(const dory_t *h, int32_t seq);

/* 1 if the sequence is latched after a failed call (see the conventions
 * above), 0 if not, DORY_EINVAL for a bad handle or seq. */
int dory_latched(const dory_t *h, int32_t seq);

/* Test hook for the latch: the n-th kernel or graph launch the library makes
 * from now on fails before it is launched (as if the runtime had refused it),
 * with DORY_EDEVICE; the launches before it run normally.  n == 0 turns it off.
 * Nothing faults on the device. */
int dory_debug_fail_launch(dory_t *h, int64_t n);

/* Test hook: one-row calls merge the sliding layers' attention splits inside
 * the attention kernel, per kv head within one XCD, where a check at
 * dory_create found every workgroup id of one residue mod 8 on one XCD;
 * elsewhere, and for full layers, a merge kernel of its own does it.  on = 0
 * selects the merge kernel for every layer, 1 the default, -1 leaves it as it
 * is; changing it drops the captured graphs.  Returns 1 if the in-kernel merge
 * is in use after the call, 0 if not, DORY_EINVAL for a bad handle or on. */
int dory_debug_xcd_merge(dory_t *h, int on);

/* Test tap: later calls also write the residual state after every sub-layer pass
 * to buf, device fp32 [passes][n][hidden] with passes = n_in + n_rec*loops +
 * n_out.  cap is buf's size in floats; a call that needs more fails with
 * DORY_EINVAL.  buf == NULL turns the tap off. */
int dory_debug_tap(dory_t *h, float *buf, int64_t cap);

/* Test tap: later calls also write, for every attention sub-layer pass and
 * every row, the cache row the pass appends before it is stored or encoded:
 * the rotated, unit-normed key, then the value -- device fp32
 * [attention passes][n][2][nk*hd], where the attention passes of a call are
 * those of its walk in order (n_in's, then each loop's, then n_out's).  cap is
 * buf's size in floats; a call that needs more fails with DORY_EINVAL; gated
 * calls take no tap.  buf == NULL turns it off.  (A q8_2f cache's codes and
 * scales are checked bit for bit against these rows.) */
int dory_debug_kv_tap(dory_t *h, float *buf, int64_t cap);

/* Test tap: copies one stored cache row of (sequence, attention ordinal, slot)
 * at position pos to host memory, after synchronising the device.
 * Layout -- fp32 cache: K [nk][hd] then V [nk][hd] floats (8*nk*hd bytes);
 * q8_2f: K codes [nk][hd] int8, V codes [nk][hd] int8, K scales [nk][ceil(hd/32)]
 * fp32, V scales [nk] fp32.  DORY_ERANGE if pos is not held (at or past the
 * position, or overwritten by the ring). */
int dory_kv_read(dory_t *h, int32_t seq, int32_t ord, int32_t slot, int64_t pos, void *host_out);

/* Test tap: the q8_2f fields of a slot, host fp32 [nk][hd] each (either may be
 * NULL).  Returns 1 if frozen, 0 if not, or a negative status. */
int dory_kv_field(dory_t *h, int32_t seq, int32_t ord, int32_t slot, float *kcol, float *vcol);

/* Test and benchmark set-up: fills a fresh sequence (position 0) with npos rows
 * per slot through the same append rules a forward uses (q8_2f: encoding, and
 * the freeze at the 65th row), then sets its position to npos, kv mode and (for
 * per_loop) loop count.  k, v: host fp32 [n_ord][n_slot][npos][nk][hd], stored
 * keys (already rotated and normed) and values; n_slot >= loops under per_loop,
 * >= 1 under last_loop; slots a mode does not use are skipped.  Synchronous. */
int dory_kv_load(dory_t *h, int32_t seq, int32_t kv_mode, int32_t loops, int64_t npos,
                 int32_t n_slot, const float *k, const float *v);

/* The q8_2f row encoder on its own (kv_cache.rs `quant_row`): rows rows of n
 * fp32 values (device, row-major), divided by col (device [n], or NULL = no
 * field), split in groups of `group` channels (32 or n; the last may be short),
 * scale = max(absmax/127, 1e-12), code = clamp(round-half-away(r/scale), -127,
 * 127).  codes: device int8 [rows][n]; scales: device fp32 [rows][ceil(n/group)].
 * n <= 256.  Asynchronous on stream. */
int dory_q8_encode_rows(const float *x, const float *col, int32_t rows, int32_t n, int32_t group,
                        int8_t *codes, float *scales, dory_stream_t stream);

/* Benchmark tap: launches one kernel of the forward `reps` times back to back on
 * stream, over the handle's current scratch (left by the last call) and the
 * cache rows that call read, cycling through the sub-layers that have that
 * kernel so each launch streams its own weights from HBM.  Stage:
 *   0 q|k|v|g GEMV, 1 decode attention over the last call's rows (that call a
 *   one-row or batch call), 2 O GEMV, 3 gate|up GEMV with SwiGLU, 4 down GEMV,
 *   5 head GEMV;
 *   6 q|k|v|g GEMM, 7 O GEMM, 8 gate|up GEMM, 9 down GEMM, each over max_chunk
 *   rows; 10 chunk attention over the last call's rows (that call a multi-row
 *   chunk).
 * Needs a prior forward call (DORY_ESTATE otherwise, or when the last call was
 * not of the kind stage 1 or 10 needs).  Leaves the scratch undefined; the cache
 * and positions are untouched. */
int dory_stage_bench(dory_t *h, int32_t stage, int32_t reps, dory_stream_t stream);

/* Benchmark tap: practical peaks of the GPU, for stating kernel fractions
 * against measured as well as published peaks.  kind 0: one streaming read of
 * `bytes` (a positive multiple of 16) at device buf, 16-byte nontemporal
 * loads; kind 1: `iters` (1 .. 2^24) iterations of four
 * v_mfma_f32_32x32x16_bf16 per wave on 2048 waves from registers (buf and
 * bytes unused).  sink: device memory of at least 4 bytes (a store that keeps
 * the work alive; practically never written).  *work: the bytes read or flops
 * done by the launch.  Asynchronous on stream: time it with events.
 * DORY_EINVAL for bad arguments. */
int dory_probe(int32_t kind, const void *buf, int64_t bytes, int64_t iters, void *sink,
               dory_stream_t stream, double *work);

#ifdef __cplusplus
}
#endif
#endif
