// internal.h -- types shared by the host runtime and the gfx950 kernels of
// libdory.so.  Nothing here is part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dk {

constexpr int kMaxLoops = 16;
constexpr int kWarmup = 64;     // kv_cache.rs `KV_COL_WARMUP`: rows before the q8 field freezes
constexpr int kMaxKParts = 8;  // split-K slabs of the multi-row output projections
constexpr int kKGroup = 32;     // kv_cache.rs `KV_K_GROUP`: K channels per q8 scale
constexpr float kEps = 1e-6f;   // dory.rs `EPS`: justnorm's epsilon
// dory_forward_chunk_noalloc: rows a call may carry, bytes of the static scratch
constexpr int kNoAllocRows = 8;
constexpr size_t kNoAllocBytes = (size_t)16 << 20;

// One row of a call: its position, its sequence (which selects the cache
// slots), its token, and where its logits go.
struct RowRec {
    int64_t pos;
    int32_t seq;
    int32_t token;
    int32_t out;       // logits row (rows of one sequence's chunk: only the last, at 0)
    int32_t q8f;       // 1: the sequence's q8_2f fields were frozen before this call
                       // (kv_cache.rs `append`: once frozen, they stay frozen, also
                       // across a rollback to fewer than 64 rows)
};

// The per-call record: written by the host into pinned memory and copied to the
// device ahead of the call's kernels, so a captured graph replays unchanged.
struct CallRec {
    int32_t n;         // rows
    int32_t pad;
    float *logits;     // device [.][vocab] or null
    float *tap;        // device [passes][n][hidden] or null
    // test tap: the pre-encode cache rows of every attention pass, device
    // [attention passes][n][2][nk * hd] (the rotated, normed key, then the
    // value) or null
    float *kvtap;
    RowRec rows[1];    // [max(max_chunk, max_seqs)]
};
inline size_t rec_bytes(int rows) { return sizeof(CallRec) + sizeof(RowRec) * (rows - 1); }
inline size_t rec_used(int rows) { return sizeof(CallRec) + sizeof(RowRec) * (rows - 1); }

// One cache slot (attention ordinal x loop slot) of one sequence.  Rings are
// head-major: K, V [nk][cap][hd]; position p sits at ring row p % cap.
struct SlotDesc {
    float *k, *v;          // fp32 cache
    int8_t *kc, *vc;       // q8 codes [nk][cap][hd]
    float *ks;             // q8 K scales [nk][cap][ngk]
    float *vs;             // q8 V scales [nk][cap]
    float *kcol, *vcol;    // q8 fields [nk][hd]
    int32_t cap;
    int32_t pad;
};

// Slot table on the device: [max_seqs][n_ord][kMaxLoops].
inline __host__ __device__ const SlotDesc &slot_at(const SlotDesc *tab, int seq, int n_ord, int ord, int slot) {
    return tab[(seq * n_ord + ord) * kMaxLoops + slot];
}

// How the x fed to a sub-layer is obtained from the previous sub-layer's result.
// e = slerp(h, o, alpha) (or e = h for the very first pass); then
//   kLoopNone:  x = e
//   kLoopEnter: input = e; state = e; x = norm(state + input)      (first loop)
//   kLoopNext:  state = norm(e); x = norm(state + input)           (later loops)
//   kLoopExit:  state = norm(e); x = state                          (after the loops)
enum LoopOp { kLoopNone = 0, kLoopEnter = 1, kLoopNext = 2, kLoopExit = 3 };

// Rows of a batch run different loop counts: they are sorted by loops, so the
// rows of a pass are a prefix.  n_prev rows ran the previous sub-layer, n_next
// run this one.  At a loop boundary the rows that stop keep their state in st;
// after the loops, rows that stopped early take x = st.
struct Resolve {
    const float *h;      // residual before the previous sub-layer [T][H]
    const float *o;      // previous sub-layer's output [T][H] (slerp only)
    const float *alpha;  // previous sub-layer's |alpha| [H] (slerp only)
    float *h_out;        // x for this sub-layer [T][H]
    uint16_t *hb_out;    // the same rows rounded to bf16 (the GEMMs' operand), or null
    int32_t o_parts;     // multi-row calls: o is the sum of o_parts slabs o + s * o_stride
    int64_t o_stride;
    // multi-row calls after an attention sub-layer: its output projection ran
    // on the un-normalised gated output z, so row r of o is scaled by
    // justnorm's factor of |z_r|^2 = the sum of o_ss[r*o_ss_n .. +o_ss_n); null: none
    const float *o_ss;
    int32_t o_ss_n;
    float *inp;          // the loop's input [T][H]
    float *st;           // the loop state of every row [T][H] (batches), or null
    int32_t slerp;       // 1: e = slerp(h, o, alpha); 0: e = h
    int32_t loop_op;
    int32_t tap_pass;    // pass index of e for the tap, or -1
    float *e_out;        // kLoopExit: e before its norm (the early exit's second pass starts from it), or null
    int32_t n_prev, n_next;
    int32_t pad;
};

enum WType { kF32 = 0, kBF16 = 1 };

// ---------------------------------------------------------------- launchers
// GEMV for one row (decode).  Prologue builds x in LDS, epilogue stores.
// Embed: the first pass of a one-row call, its x the embedding row of the
// record's token (dory.rs `forward_host`: an id outside the table is a zero row).
enum GemvPro { kProPlain = 0, kProNorm = 1, kProResolve = 2, kProResolveInp = 3, kProEmbed = 4 };  // Inp: the loop's next pass reads the input
enum GemvEpi { kEpiStore = 0, kEpiPair = 1, kEpiHead = 2 };

struct GemvArgs {
    // weight row pointers by segment: rows [seg_end[i-1], seg_end[i]) read w[i]
    const void *w[4];
    int32_t seg_end[4];
    int32_t nseg;
    int32_t N;           // output rows (pairs for kEpiPair)
    int32_t K;
    int32_t row;         // which row of the [T][K] source feeds x
    const float *src;    // kProPlain / kProNorm: [T][K]
    Resolve rs;          // kProResolve
    float *y;            // output [N] at row offset (kEpiStore, kEpiPair)
    const float *sg, *su;        // kEpiPair
    const float *logit_scale;    // kEpiHead
    const CallRec *rec;
    int32_t hidden;      // tap row length
    const void *embed;   // kProEmbed: the embedding table [vocab][K] (the weights' type)
    int32_t vocab;
};

hipError_t launch_gemv(int wtype, int pro, int epi, const GemvArgs &a, hipStream_t s);

// x[i] += x[i + z stride] for z = 1 .. parts-1, i < n, in slab order: the
// slabs of a K-split projection added into the first (n and stride multiples
// of 4, stride >= n).
hipError_t launch_add_slabs(float *x, size_t n, int parts, size_t stride, hipStream_t s);

// Prefill row kernels.
// The row kernels also write a bf16 copy of what they write (hb, dstb: may be
// null) for the bf16 GEMMs that read it next.
hipError_t launch_embed(int wtype, const void *embed, int V, int H, const CallRec *rec, int T,
                        float *h, uint16_t *hb, hipStream_t s);
// tap, tap_n: the record's tap buffer and row count (rec->tap, rec->n) as the
// host set them for this call: multi-row calls are never captured in a graph,
// so the kernel takes them as arguments instead of reading the record.
hipError_t launch_resolve_rows(const Resolve &rs, int H, int T, const CallRec *rec, float *tap, int tap_n,
                               hipStream_t s);
hipError_t launch_rownorm(const float *src, int ld_src, float *dst, uint16_t *dstb, int N, int T, hipStream_t s);
// a and b rows have stride ld; dst rows stride F.  dst or dstb may be null.
// With ss: the un-normalised rows are stored and ss[r] = their |z|^2 (the
// renorm is then a per-row factor its consumer applies).
hipError_t launch_swiglu_norm(const float *a, const float *b, int ld, const float *sg, const float *su,
                              float *dst, uint16_t *dstb, int F, int T, hipStream_t s, float *ss = nullptr);

// dory.rs `top_prob` of the call record's logits row (one-row calls: the
// record's logits pointer, V floats) into *out (one workgroup).
hipError_t launch_top_prob(const CallRec *rec, int V, float *out, hipStream_t s);

// Batches: logits[rows[r].out][v] = hlog[r][v] * logit_scale[v].
hipError_t launch_logits_rows(const float *hlog, const float *logit_scale, int V, int T, const CallRec *rec,
                              hipStream_t s);

// The device address of the static scratch array on the current GPU (looked up
// once per device, then cached): kNoAllocBytes bytes, 256-byte aligned.
hipError_t noalloc_scratch(void **ptr);

// Weights of a GEMM as up to 4 row segments stacked along N: output column n
// reads row n - seg_end[i-1] of w[i] for seg_end[i-1] <= n < seg_end[i].
struct GemmW {
    const void *w[4];
    int32_t seg_end[4];
    int32_t nseg;
};
inline GemmW gemm_w(const void *w, int N) { return GemmW{{w, w, w, w}, {N, N, N, N}, 1}; }

// C[T][ldc] (columns 0..N-1) = A[T][K] . W[N][K]^T, fp32 accumulation.  A is
// given in fp32 and, for bf16 weights, also rounded to bf16 (Ab, same lda):
// the bf16 MFMA kernels read Ab, the fp32 tiled kernel reads A.
// kparts > 1 (split K, only where gemm_splits_ok): part z of the sum over K goes
// to C + z * pstride, and the reader adds the kparts slabs.
hipError_t launch_gemm(int wtype, const float *A, const uint16_t *Ab, int lda, const GemmW &W, int N, int K,
                       float *C, int ldc, int T, hipStream_t s, int kparts = 1, size_t pstride = 0);
inline bool gemm_splits_ok(int wtype, bool have_bf16, int M, int K, int kparts) {
    if (wtype != kBF16 || !have_bf16 || kparts > kMaxKParts) return false;
    if (M <= 64) return K % 128 == 0 && K / 128 >= kparts;     // k_gemm_skinny: K blocks dealt out
    return K % (64 * kparts) == 0;
}
// The MLP's gate | up projection of a multi-row call with SwiGLU in its
// epilogue (bf16 weights, more than 64 rows, ffn a multiple of 64): zb [M][F]
// bf16 = silu(a sg) (b su), ssp [M][F/64] the rows' sums of z^2 per 64 indices.
inline bool gemm_swiglu_ok(int wtype, int M, int F, int K, int lda) {
    return wtype == kBF16 && M > 64 && F % 64 == 0 && K % 64 == 0 && lda % 8 == 0;
}
hipError_t launch_gemm_swiglu(const uint16_t *Ab, int lda, const void *wgate, const void *wup, int F, int K,
                              const float *sg, const float *su, uint16_t *zb, float *ssp, int M, hipStream_t s);
// Whether launch_gemm reads the fp32 A for this shape (else only the bf16 Ab).
inline bool gemm_reads_fp32_a(int wtype, bool have_bf16, int M, int K, int lda) {
    if (wtype != kBF16 || !have_bf16 || lda % 8) return true;
    return !((M <= 64 && K % 128 == 0) || (M > 64 && K % 64 == 0) || (M >= 32 && K % 8 == 0));
}
// Split-K count that fills the chip with 128 x 128 tiles (1 where it does not apply).
inline int gemm_pick_splits(int wtype, bool have_bf16, int M, int N, int K) {
    if (!gemm_splits_ok(wtype, have_bf16, M, K, 1)) return 1;
    if (M <= 64) {  // about 256 workgroups of 64 weight rows, at least 2 K blocks each
        const int tiles = (N + 63) / 64;
        int S = 1;
        while (S * 2 <= kMaxKParts && tiles * S * 2 <= 256 && K / 128 >= 2 * S * 2) S *= 2;
        return S;
    }
    const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
    int S = 1;
    while (S * 2 <= kMaxKParts && tiles * S * 2 <= 256 && K % (64 * S * 2) == 0 && K / (S * 2) >= 512) S *= 2;
    return S;
}

// Attention.
struct PrepArgs {
    const float *qkvg;   // [T][Q + 2KV + Q]
    float *qp;           // [T][Q] rotated, normed, scaled queries
    float *kstage;       // [T][KV] rotated, normed keys (q8 cache) or null (fp32 cache: ring)
    const float *rope;   // [max_ctx][hd] RoPE table of the layer's kind: cos half, sin half
    const float *sq;     // [Q]
    const SlotDesc *tab;
    int32_t n_ord, ord, slot;
    int32_t nh, nk, hd;
    const CallRec *rec;
    int32_t tap_pass;    // the call's attention pass (for the record's kvtap)
    // A chunk of one sequence is never captured in a graph, so what the kernel
    // would read from the record and the slot table (tab .. slot, rec: kept for
    // checking) comes from the host as it set them for this call:
    int64_t pos0;        // position of row 0 (rows at pos0 .. pos0+T-1)
    float *kring, *vring;  // fp32 cache: the slot's rings [nk][cap][hd] (unused with kstage)
    int32_t cap;
    float *kvtap;        // the record's kv tap, or null; rows of kvtap_n
    int32_t kvtap_n;
};
hipError_t launch_prep(const PrepArgs &a, int T, hipStream_t s);

struct AttnArgs {
    const float *qp;     // [T][Q]
    const float *qkvg;   // gate g at column Q + 2KV
    const float *sg;     // [Q]
    float *z;            // [T][Q] gated attention output (before the renorm)
    float *part;         // split partials [T][nk][max_split][rep][2 + hd]: max, sum, sum of p*v
    const SlotDesc *tab;
    int32_t n_ord, ord, slot;
    int32_t nh, nk, hd;
    int64_t window;      // keys p-window+1 ..= p (huge for full attention)
    int32_t split;       // keys per workgroup
    int32_t max_split;   // grid.x; partial stride
    int32_t q8;          // cache encoding
    int32_t field;       // q8: 1 the field is frozen (apply kcol / vcol), 0 not, -1 by
                         // each row: frozen before its call (RowRec::q8f), or frozen
                         // as its call appends position 64 or later
    const CallRec *rec;
    // one-row calls: the RoPE, norms and cache write of the new row are fused in
    const float *rope;   // [max_ctx][hd] RoPE table of the layer's kind: cos half, sin half
    const float *sq;     // [Q]
    int32_t no_write;    // benchmark only: leave the cache row of p untouched
    // multi-row calls on MFMA (k_fattn): rows per block (attn_chunk_block), and
    // then `split` keys per workgroup of the block's key range, a multiple of
    // 64; 0: one row per workgroup (k_attn), split <= 256
    int32_t blk;
    int32_t nsplit;      // k_fattn: grid.x, the most splits a block has
    // multi-row merges: z also rounded to bf16 [T][Q], and the sum of squares
    // of z over each (row, kv head) group of channels [T][nk]; null: not written
    uint16_t *zb;
    float *zss;
    // one-row calls: the row's slot table entry, read without waiting for the
    // record's sequence; null: looked up by the record
    const SlotDesc *sd1;
    int32_t dec;         // 1: the decode kernel (launch_attn_dec), whose merge reads all
                         // max_split slabs of a row; 0: the multi-row kernels
    int32_t tap_pass;    // decode kernels: the call's attention pass (for the record's kvtap)
    // Multi-row chunks of one sequence (k_fattn and its merge; never captured
    // in a graph): what these kernels would read from the record and the slot
    // table, as the host set them for this call.
    int64_t pos0;        // the chunk's first position (the record's rows[0].pos)
    int32_t nrows;       // the call's rows (the record's n)
    SlotDesc sdc;        // the sequence's slot
    // One-row calls, head dim 128, 4 q heads per kv head, at most 64 splits:
    // the splits merged inside the attention kernel, per kv head within one XCD
    // (no merge launch).  Arrival counters, (kv head kh, head h)'s at
    // xcnt[32 (4 kh + h)] (128 bytes apart), zero between launches (the kernel
    // clears them); partials then laid out per kv head on 128-byte lines
    // (attn_xm_part_floats).  Null: the merge kernel.
    uint32_t *xcnt;
    // One-row calls, head dim 128, 4 q heads per kv head, split 64: 1 lets the
    // max_split workgroups grow their splits to cover the row's keys (up to 72
    // keys each, so the keys may reach 72 max_split) instead of adding
    // workgroups; the grid then stays at max_split per kv head.
    int32_t ext;
};
// Floats of partials the in-kernel merge needs: per kv head, max_split slabs
// of rep x (2 + hd), rounded up to 32 floats.
inline size_t attn_xm_part_floats(int nk, int max_split, int rep, int hd) {
    return (size_t)nk * (((size_t)max_split * rep * (hd + 2) + 31) / 32 * 32);
}
// Writes each workgroup's XCD number to ids[0 .. G-1] (a one-off check that
// workgroup L runs on XCD L % 8, which the in-kernel merge relies on).
hipError_t launch_xcd_check(unsigned *ids, int G, hipStream_t s);
// Multi-row calls (after launch_prep): grid (max_split, nk, T), then the merge.
hipError_t launch_attn(const AttnArgs &a, int T, hipStream_t s);
// Decode rows (one new row per sequence: a one-row call, or one row of each
// sequence of a batch) from the raw projections: grid (max_split, nk, T), then
// the merge.
hipError_t launch_attn_dec(const AttnArgs &a, int T, hipStream_t s);
// Rows per block of the MFMA chunk attention for this geometry, or 0 when it
// does not serve it (head dim other than 128).
inline int attn_chunk_block(int hd, int rep) { return hd == 128 && 128 % rep == 0 ? 128 / rep : 0; }
// Keys a decode workgroup takes at most for head dim hd with `steps` load
// steps (8 or 16).
inline int attn_dec_max_split(int hd, int steps) {
    const int kb = 256 / (hd / 4);
    return steps * kb < 256 ? steps * kb : 256;
}

// q8_2f cache writes (kv_cache.rs `append` / `freeze_cols`).
struct Q8WriteArgs {
    const float *ksrc; int32_t kld;   // rotated normed keys [T][..], kv head kh at kh*hd
    const float *vsrc; int32_t vld;   // values
    const SlotDesc *tab;
    int32_t n_ord, ord, slot, nk, hd;
    int32_t r0, r1;                   // rows of the call to encode
    int32_t field;                    // encode against the frozen field
    const CallRec *rec;
};
hipError_t launch_q8_write(const Q8WriteArgs &a, hipStream_t s);
// The field freeze of the slot of call row `row`'s sequence.
hipError_t launch_q8_freeze(const SlotDesc *tab, int n_ord, int ord, int slot, int nk, int hd,
                            const CallRec *rec, int row, hipStream_t s);
hipError_t launch_q8_encode_rows(const float *x, const float *col, int rows, int n, int group,
                                 int8_t *codes, float *scales, hipStream_t s);
// fp32 rows straight into a ring (cache set-up).
hipError_t launch_kv_store(const float *k, const float *v, const SlotDesc *tab, int n_ord, int ord,
                           int slot, int nk, int hd, int T, const CallRec *rec, hipStream_t s);

}  // namespace dk
