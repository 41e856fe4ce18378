// api.hip -- the host runtime of libdory.so behind the C ABI of include/dory.h:
// configuration checks, device memory, the cache rings, the per-call record,
// the walk through the sub-layers (dory.rs `stack`) and one captured HIP graph
// per (loops, kv mode) for one-row calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "dory.h"
#include "internal.h"

using namespace dk;

namespace {

thread_local std::string g_create_error;

struct LayerInfo {
    bool attn = false, sliding = false, rec = false;
    int ord = -1;
    dory_layer_weights w{};
};

struct SeqState {
    int64_t pos = 0;
    int mode = -1;   // fixed from the first call until a reset
    int loops = 0;   // per_loop: fixed from the first call until a reset
    // q8_2f: the fields of the sequence's slots froze (a row was appended with
    // 64 rows stored; every slot of a sequence holds the same positions, so
    // they freeze in the same call).  kv_cache.rs `truncate_last` drops rows
    // only: a rollback keeps them frozen.  Cleared by a reset.
    bool q8_frozen = false;
    // dory.rs `ExitRate` and the gate's counters (the early exit)
    float exit_rate = 1.0f;
    uint32_t exit_tokens = 0;
    int64_t gate_tokens = 0, gate_one = 0;
    float last_top = -1.0f;
    // kv_cache.rs `append`: a failed transition is terminal until the sequence is
    // cleared.  Set when a call on the sequence fails after its first device
    // work was enqueued, or when a synchronisation reports a device error (which
    // no call can be blamed for alone: every sequence latches).  Every later
    // call on the sequence returns DORY_ESTATE until dory_kv_reset.
    bool latched = false;
};

constexpr int kStages = 32;
constexpr int64_t kHuge = (int64_t)1 << 62;

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Per-call device scratch of the forward: activations, split partials and the
// call record.  The ordinary entry points use the handle's own buffers (sized
// for max_chunk rows at create); dory_forward_chunk_noalloc carves one out of
// the library's static array.  A call's kernels take every pointer from here.
struct Scratch {
    float *hb[2];          // residual of pass k in hb[k % 2] [T][H]
    float *inp;            // the loop's input [T][H]
    float *o;              // output projections: kMaxKParts split-K slabs [T][H], o_stride apart
    int64_t o_stride;
    float *qkvg;           // q | k | v | g [T][2Q + 2KV]
    float *qp;             // rotated, normed, scaled queries [T][Q]
    float *z, *zn;         // gated attention output [T][Q]; its renormed copy (benchmark stage only)
    float *ga;             // gate | up [T][2F]
    float *un;             // SwiGLU output [T][F]
    float *kstage;         // rotated, normed keys before the q8 encoder [T][KV]
    float *st;             // batches: loop state of each row [T][H]
    float *hlog;           // batches: head output before the scale [min(T, seqs)][V]
    float *part;           // split-attention partials
    float *zss, *uss, *ussp;  // sums of squares: z per (row, kv head); SwiGLU rows; per 64 ffn indices
    uint16_t *xb, *znb, *unb; // bf16 copies of x, z, SwiGLU output (GEMM operands)
    CallRec *rec;          // the call record
};

}  // namespace

struct dory {
    dory_config cfg{};
    std::string pattern;
    dory_weights w{};
    std::vector<dory_layer_weights> wl;
    std::vector<LayerInfo> L;
    int n_ord = 0;
    int H = 0, F = 0, V = 0, Q = 0, KV = 0, nh = 0, nk = 0, hd = 0, ngk = 0, wt = 0, q8 = 0;
    int cap_s = 0, cap_f = 0;
    int split_pf = 256, ms_dec = 1, ms_pf = 1;
    int split_bs = 64, split_bf = 64, ms_bs = 1, ms_bf = 1;  // decode splits of batches
    int split_ds = 64, split_df = 64, ms_ds = 1, ms_df = 1;  // one-row calls: sliding, full layers
    int64_t win_s = 0, win_f = 0;
    Scratch sc{};           // the per-call scratch of the ordinary entry points (sized for max_chunk rows)
    float *rope_s = nullptr, *rope_f = nullptr, *ld_k = nullptr, *ld_v = nullptr;
    float *hlog_all = nullptr;  // every row's head output of a chunk [max_chunk][vocab] (allocated on first use)
    void *noalloc = nullptr;    // the static scratch array of this handle's device (dory_forward_chunk_noalloc)
    size_t noalloc_need = 0;    // bytes a call of kNoAllocRows rows needs of it
    std::string noalloc_err;    // why the array's address could not be had, if so
    int prompt_loops = 0;       // dory.rs `prompt_loops`: 0 = off
    // dory.rs `Gate::Conf(th)`: one-row last_loop calls leave after one pass
    // when the read-out's top probability reaches gate_th
    bool gate_on = false;
    float gate_th = 0.f;
    float *gst = nullptr;       // the first pass's e at the loop exit, before its norm [H]
    float *glog = nullptr;      // read-out logits of a call that wants none [V]
    float *gtop = nullptr;      // the read-out's top probability (device)
    float *gtop_host = nullptr; // ... copied to pinned host memory
    SlotDesc *tab = nullptr;
    std::vector<SlotDesc> tab_host;
    std::vector<void *> allocs;
    // pinned staging of call records
    char *stage = nullptr;
    size_t rec_sz = 0;
    hipEvent_t stage_ev[kStages]{};
    bool stage_used[kStages]{};
    int stage_i = 0;
    hipStream_t cap_stream = nullptr;
    std::map<std::tuple<int, int, int>, hipGraphExec_t> graphs;  // one-row calls by (loops, kv mode, sequence)
    float *tap = nullptr;
    int64_t tap_cap = 0;
    float *kvtap = nullptr;  // test tap of the pre-encode cache rows (dory_debug_kv_tap)
    // One-row calls' sliding layers merge their attention splits inside the
    // attention kernel (per kv head within one XCD): the kernel's arrival
    // counters, and whether the create-time XCD check allowed it (xm) and a
    // test has not turned it off (xm_off)
    uint32_t *xcnt = nullptr;
    bool xm = false, xm_off = false;
    // One-row calls' full layers whose window needs 65..72 splits of 64 keys:
    // 64 workgroups per kv head whose splits grow to cover the keys (one per
    // CU over the 4 kv heads, where 65+ would put two on some CUs)
    bool ext_df = false;
    int64_t kvtap_cap = 0;
    std::vector<SeqState> seqs;
    std::string err;
    int device = 0;
    // the last successful forward call (its rows are in rec): rows, kind, loops, mode, first position
    int last_T = 0, last_loops = 0, last_mode = -1;
    bool last_chunk = false;
    int64_t last_pos0 = 0;
    int last_seq0 = 0;
    // test hook (dory_debug_fail_launch): the fail_in-th launch from now fails
    // before it is launched; 0 = off
    int64_t fail_in = 0;
};

namespace {

int fail(dory_t *h, int code, const std::string &msg) {
    if (h) h->err = msg;
    else g_create_error = msg;
    return code;
}

int hip_fail(dory_t *h, hipError_t e, const char *what) {
    return fail(h, e == hipErrorOutOfMemory ? DORY_ENOMEM : DORY_EDEVICE,
                std::string(what) + ": " + hipGetErrorString(e));
}

// A device error seen at a synchronisation may come from any work enqueued
// before it: every sequence latches.
int sync_fail(dory_t *h, hipError_t e, const char *what) {
    for (SeqState &st : h->seqs) st.latched = true;
    const int rc = hip_fail(h, e, what);
    h->err += " (every sequence latched: dory_kv_reset clears it)";
    return rc;
}

#define SYNCCHECK(h, call)                                    \
    do {                                                      \
        hipError_t e_ = (call);                               \
        if (e_ != hipSuccess) return sync_fail(h, e_, #call); \
    } while (0)

// A call that failed after its first device work: its sequences latch.
int latch(dory_t *h, int rc, const int32_t *seqs, int n) {
    if (!rc) return rc;
    for (int i = 0; i < n; ++i) h->seqs[seqs[i]].latched = true;
    h->err += " (sequence latched until dory_kv_reset)";
    return rc;
}

int latched_error(dory_t *h, const char *fn, int seq) {
    return fail(h, DORY_ESTATE, std::string(fn) + ": sequence " + std::to_string(seq) +
                                    " is latched after a failed call; dory_kv_reset clears it");
}

// The test hook: true when this launch is the one to fail.
bool inject_failure(dory_t *h) { return h->fail_in > 0 && --h->fail_in == 0; }

#define HIPCHECK(h, call)                                   \
    do {                                                    \
        hipError_t e_ = (call);                             \
        if (e_ != hipSuccess) return hip_fail(h, e_, #call); \
    } while (0)

template <typename T>
hipError_t dmalloc(dory_t *h, T **p, size_t count) {
    void *q = nullptr;
    hipError_t e = hipMalloc(&q, count ? sizeof(T) * count : 16);
    if (e == hipSuccess) {
        h->allocs.push_back(q);
        *p = reinterpret_cast<T *>(q);
    }
    return e;
}

int passes(const dory_t *h, int loops) { return h->cfg.n_in + h->cfg.n_rec * loops + h->cfg.n_out; }

// Attention sub-layer passes of a call of `loops` loops.
int attn_passes(const dory_t *h, int loops) {
    int n = 0;
    for (const LayerInfo &l : h->L)
        if (l.attn) n += l.rec ? loops : 1;
    return n;
}

int check_config(const dory_config *c, const dory_weights *w) {
    auto bad = [](const std::string &m) { return fail(nullptr, DORY_EINVAL, "dory_create: " + m); };
    if (!c || !w || !c->layer_pattern || !w->layers) return bad("null argument");
    const int nl = (int)strlen(c->layer_pattern);
    if (c->n_in < 1 || c->n_rec < 1 || c->n_out < 1) return bad("every block needs at least one sub-layer");
    if (nl != c->n_in + c->n_rec + c->n_out) return bad("pattern length != n_in + n_rec + n_out");
    if (c->nh <= 0 || c->nk <= 0 || c->nh % c->nk) return bad("nh must be a positive multiple of nk");
    const int rep = c->nh / c->nk;
    if (rep != 1 && rep != 2 && rep != 4 && rep != 8) return bad("nh/nk must be 1, 2, 4 or 8");
    if (c->hd != 8 && c->hd != 16 && c->hd != 32 && c->hd != 64 && c->hd != 128 && c->hd != 256)
        return bad("hd must be 8, 16, 32, 64, 128 or 256");
    const int Q = c->nh * c->hd;
    for (int v : {c->hidden, c->ffn, Q})
        if (v <= 0 || v % 8 || v > 8192) return bad("hidden, ffn and nh*hd must be multiples of 8 up to 8192");
    if (c->vocab <= 0) return bad("vocab must be positive");
    if (c->window <= 0 || c->full_window < 0) return bad("window must be positive, full_window >= 0");
    if (c->max_chunk <= 0 || c->max_ctx < c->max_chunk || c->max_seqs <= 0)
        return bad("need 0 < max_chunk <= max_ctx and max_seqs > 0");
    if (c->kv_encoding != DORY_KV_F32 && c->kv_encoding != DORY_KV_Q8_2F) return bad("kv_encoding");
    if (c->weight_dtype != DORY_W_F32 && c->weight_dtype != DORY_W_BF16) return bad("weight_dtype");
    if (!w->embed || !w->head || !w->logit_scale) return bad("null embed, head or logit_scale");
    for (int li = 0; li < nl; ++li) {
        const dory_layer_weights &x = w->layers[li];
        if (c->layer_pattern[li] == '-') {
            if (!x.wgate || !x.wup || !x.wdown || !x.sg || !x.su || !x.alpha)
                return bad("null MLP weight at sub-layer " + std::to_string(li));
        } else if (!x.wq || !x.wk || !x.wv || !x.wg || !x.wo || !x.sq || !x.sg || !x.alpha) {
            return bad("null attention weight at sub-layer " + std::to_string(li));
        }
    }
    return DORY_OK;
}

void free_all(dory_t *h) {
    for (auto &g : h->graphs) (void)hipGraphExecDestroy(g.second);
    h->graphs.clear();
    for (void *p : h->allocs) (void)hipFree(p);
    h->allocs.clear();
    for (int i = 0; i < kStages; ++i)
        if (h->stage_ev[i]) (void)hipEventDestroy(h->stage_ev[i]);
    if (h->stage) (void)hipHostFree(h->stage);
    if (h->gtop_host) (void)hipHostFree(h->gtop_host);
    if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
}

// The slot (attention ordinal x loop) a sub-layer uses (dory.rs `slot_loop`).
int slot_of(const dory_t *h, const LayerInfo &l, int mode, int loop_i) {
    return (mode == DORY_PER_LOOP && l.rec) ? loop_i : 0;
}

int alloc_slot(dory_t *h, int seq, int ord, int slot, bool sliding) {
    SlotDesc &d = h->tab_host[(seq * h->n_ord + ord) * kMaxLoops + slot];
    if (d.k || d.kc) return DORY_OK;
    const int cap = sliding ? h->cap_s : h->cap_f;
    const size_t rows = (size_t)h->nk * cap;
    d.cap = cap;
    if (h->q8) {
        int8_t *kc, *vc;
        float *ks, *vs, *kcol, *vcol;
        HIPCHECK(h, dmalloc(h, &kc, rows * h->hd));
        HIPCHECK(h, dmalloc(h, &vc, rows * h->hd));
        HIPCHECK(h, dmalloc(h, &ks, rows * h->ngk));
        HIPCHECK(h, dmalloc(h, &vs, rows));
        HIPCHECK(h, dmalloc(h, &kcol, (size_t)h->KV));
        HIPCHECK(h, dmalloc(h, &vcol, (size_t)h->KV));
        d.kc = kc; d.vc = vc; d.ks = ks; d.vs = vs; d.kcol = kcol; d.vcol = vcol;
    } else {
        float *k, *v;
        HIPCHECK(h, dmalloc(h, &k, rows * h->hd));
        HIPCHECK(h, dmalloc(h, &v, rows * h->hd));
        d.k = k; d.v = v;
    }
    const size_t idx = (size_t)(seq * h->n_ord + ord) * kMaxLoops + slot;
    HIPCHECK(h, hipMemcpy(h->tab + idx, &d, sizeof(SlotDesc), hipMemcpyHostToDevice));
    return DORY_OK;
}

// Every slot a (mode, loops) call touches on seq.
int ensure_slots(dory_t *h, int seq, int mode, int loops) {
    for (const LayerInfo &l : h->L) {
        if (!l.attn) continue;
        const int ns = (mode == DORY_PER_LOOP && l.rec) ? loops : 1;
        for (int s = 0; s < ns; ++s) {
            int rc = alloc_slot(h, seq, l.ord, s, l.sliding);
            if (rc) return rc;
        }
    }
    return DORY_OK;
}

// The slots a (mode, loops) call touches on seq are all allocated already.
bool slots_ready(const dory_t *h, int seq, int mode, int loops) {
    for (const LayerInfo &l : h->L) {
        if (!l.attn) continue;
        const int ns = (mode == DORY_PER_LOOP && l.rec) ? loops : 1;
        for (int s = 0; s < ns; ++s) {
            const SlotDesc &d = h->tab_host[(seq * h->n_ord + l.ord) * kMaxLoops + s];
            if (!d.k && !d.kc) return false;
        }
    }
    return true;
}

// Lays out the scratch of a one-sequence call of up to `rows` rows from base
// (256-byte aligned pieces; base == nullptr only sizes it) and returns the
// bytes it takes.  The batch-only buffers (loop state, head rows) are left
// null: a one-sequence call reads neither.
size_t carve_scratch(const dory_t *h, int rows, char *base, Scratch *out) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char *p = base ? base + off : nullptr;
        off += (bytes + 255) / 256 * 256;
        return p;
    };
    const size_t T = rows, H = h->H, Q = h->Q, KV = h->KV, F = h->F, rep = h->nh / h->nk;
    Scratch sc{};
    sc.hb[0] = (float *)take(4 * T * H);
    sc.hb[1] = (float *)take(4 * T * H);
    sc.inp = (float *)take(4 * T * H);
    sc.o_stride = (int64_t)(T * H);
    sc.o = (float *)take(4 * T * H * kMaxKParts);
    sc.qkvg = (float *)take(4 * T * (2 * Q + 2 * KV));
    sc.qp = (float *)take(4 * T * Q);
    sc.z = (float *)take(4 * T * Q);
    sc.zn = (float *)take(4 * T * Q);
    sc.ga = (float *)take(4 * T * 2 * F);
    sc.un = (float *)take(4 * T * F);
    sc.kstage = (float *)take(4 * T * KV);
    sc.part = (float *)take(4 * std::max(std::max((size_t)h->ms_dec, T * h->ms_pf) * h->nk * rep * (h->hd + 2),
                                         attn_xm_part_floats(h->nk, h->ms_ds, (int)rep, h->hd)));
    sc.zss = (float *)take(4 * T * h->nk);
    sc.uss = (float *)take(4 * T);
    sc.ussp = h->F % 64 == 0 ? (float *)take(4 * T * (F / 64)) : nullptr;
    sc.xb = (uint16_t *)take(2 * T * H);
    sc.znb = (uint16_t *)take(2 * T * Q);
    sc.unb = (uint16_t *)take(2 * T * F);
    sc.rec = (CallRec *)take(rec_bytes(rows));
    if (out) *out = sc;
    return off;
}

// ------------------------------------------------------------------ enqueue

struct Enq {
    dory_t *h;
    hipStream_t s;
    const Scratch *sc;           // the call's scratch
    int T;                       // rows of the call
    int loops;                   // loops of its longest row
    int mode;
    bool batch;                  // one decode row of each of T sequences
    bool want_logits;
    std::vector<int> act;        // rows that run loop i (a prefix: rows are sorted by loops)
    std::vector<int64_t> pos;    // every row's position (host copy, for the q8 freeze)
    std::vector<int> seq;        // every row's sequence
    std::vector<uint8_t> froze;  // slots whose field this call froze: [max_seqs][n_ord][kMaxLoops]
    std::vector<uint8_t> q8f;    // per row: its sequence's fields were frozen before this call
    bool want_all = false;       // a chunk whose every row's logits are wanted (dory.rs `Want::All`)
    // the early exit: the loop exit also stores e before its norm (gate_save);
    // a second pass starts at pass k0 from e0 (one row) instead of the embedding
    bool gate_save = false;
    bool embed_pass = false;     // this pass's GEMV gathers the embedding row itself (one-row calls)
    int k0 = 0;
    const float *e0 = nullptr;
    int attn_pass = 0;           // attention passes enqueued so far (the kv tap's index)
    int o_parts = 1;             // split-K slabs of o the last output projection wrote
    const float *o_ss = nullptr; // multi-row attention: per-row partial sums of |z|^2 scaling o
    int o_ss_n = 0;
};

#define LAUNCH(call)                                                                          \
    do {                                                                                      \
        if (inject_failure(q.h)) return hip_fail(q.h, hipErrorLaunchFailure, "(injected) " #call); \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess) return hip_fail(q.h, e_, #call);                                \
    } while (0)

uint8_t &froze_at(Enq &q, int seq, int ord, int slot) {
    return q.froze[((size_t)seq * q.h->n_ord + ord) * kMaxLoops + slot];
}

// Key splits of a chunk's attention (rows pos0 .. pos0+M-1, aa.window set).
// MFMA blocks: about 512 workgroups, at least 256 keys each (a multiple of
// the 64-key tile); otherwise one row per workgroup, 256 keys each.
void chunk_split(const dory_t *h, int64_t pos0, int M, AttnArgs &aa) {
    aa.max_split = h->ms_pf;
    aa.blk = attn_chunk_block(h->hd, h->nh / h->nk);
    if (aa.blk == 0) {
        aa.split = h->split_pf;
        aa.nsplit = 0;
        return;
    }
    const int blk = aa.blk, nb = (M + blk - 1) / blk;
    int64_t len = 0;  // the longest block key range
    for (int b = 0; b < nb; ++b) {
        const int rb0 = b * blk, rb1 = std::min(M, rb0 + blk) - 1;
        const int64_t klo = std::max<int64_t>(0, pos0 + rb0 + 1 - aa.window);
        len = std::max(len, pos0 + rb1 - klo + 1);
    }
    const int64_t per = (int64_t)nb * h->nk;
    const int64_t want = std::max<int64_t>(1, (512 + per - 1) / per);
    int64_t split = std::max<int64_t>(256, ((len + want - 1) / want + 63) / 64 * 64);
    int64_t ns = (len + split - 1) / split;
    if (ns > h->ms_pf) {  // never at the sizes create() allows for; kept safe
        split = ((len + h->ms_pf - 1) / h->ms_pf + 63) / 64 * 64;
        ns = (len + split - 1) / split;
    }
    aa.split = (int)split;
    aa.nsplit = (int)ns;
}

// The fused projections of multi-row calls: q | k | v | g, and gate | up.
GemmW qkvg_w(const dory_t *h, const dory_layer_weights &w) {
    return GemmW{{w.wq, w.wk, w.wv, w.wg}, {h->Q, h->Q + h->KV, h->Q + 2 * h->KV, 2 * h->Q + 2 * h->KV}, 4};
}
GemmW gateup_w(const dory_t *h, const dory_layer_weights &w) {
    return GemmW{{w.wgate, w.wup, w.wup, w.wup}, {h->F, 2 * h->F, 2 * h->F, 2 * h->F}, 2};
}

// One attention sub-layer over the first M rows of the call.
int enq_attn(Enq &q, const LayerInfo &l, int loop_i, const Resolve &rs, const float *x, int M) {
    dory_t *h = q.h;
    const Scratch &sc = *q.sc;
    const int ld = 2 * h->Q + 2 * h->KV;
    const int slot = slot_of(h, l, q.mode, loop_i);
    const dory_layer_weights &w = l.w;
    if (q.T == 1) {
        GemvArgs a{};
        a.w[0] = w.wq; a.w[1] = w.wk; a.w[2] = w.wv; a.w[3] = w.wg;
        a.seg_end[0] = h->Q; a.seg_end[1] = h->Q + h->KV; a.seg_end[2] = h->Q + 2 * h->KV; a.seg_end[3] = ld;
        a.nseg = 4; a.N = ld; a.K = h->H; a.row = 0; a.rs = rs; a.y = sc.qkvg; a.rec = sc.rec; a.hidden = h->H;
        a.embed = h->w.embed; a.vocab = h->V;
        const int pro = q.embed_pass ? kProEmbed : rs.loop_op == kLoopNext ? kProResolveInp : kProResolve;
        LAUNCH(launch_gemv(h->wt, pro, kEpiStore, a, q.s));
    } else {
        // A batch's few-row q|k|v|g projection would leave most CUs idle: its K
        // is split into slabs (while the workgroups fit the chip in one round
        // and the slabs the buffer), added into the first before attention.
        int parts = 1;
        if (q.batch && M <= 64) {
            const int tiles = (ld + 63) / 64;
            while (parts < 4 && tiles * (parts + 1) <= 256 && h->H / 128 >= 4 * (parts + 1) &&
                   (parts + 1) * M <= h->cfg.max_chunk && gemm_splits_ok(h->wt, true, M, h->H, parts + 1))
                ++parts;
        }
        const size_t slab = (size_t)M * ld;
        LAUNCH(launch_gemm(h->wt, x, sc.xb, h->H, qkvg_w(h, w), ld, h->H, sc.qkvg, ld, M, q.s, parts, slab));
        LAUNCH(launch_add_slabs(sc.qkvg, slab, parts, slab, q.s));
    }
    AttnArgs aa{};
    aa.qp = sc.qp; aa.qkvg = sc.qkvg; aa.sg = w.sg; aa.z = sc.z; aa.part = sc.part;
    aa.tab = h->tab; aa.n_ord = h->n_ord; aa.ord = l.ord; aa.slot = slot;
    aa.nh = h->nh; aa.nk = h->nk; aa.hd = h->hd;
    aa.window = l.sliding ? h->win_s : h->win_f;
    aa.q8 = h->q8; aa.rec = sc.rec;
    aa.rope = l.sliding ? h->rope_s : h->rope_f; aa.sq = w.sq;
    aa.tap_pass = q.attn_pass++;
    if (q.T > 1) {
        aa.zb = sc.znb;
        aa.zss = sc.zss;
    }
    if (q.T == 1 || q.batch) {
        // One new row per sequence: prep and the cache write are fused into the
        // decode attention kernel.  kv_cache.rs `append`: a slot's field freezes
        // as its row of position 64 is appended, before that row is encoded.
        if (h->q8)
            for (int r = 0; r < M; ++r) {
                uint8_t &fz = froze_at(q, q.seq[r], l.ord, slot);
                if (q.pos[r] >= kWarmup && !q.q8f[r] && !fz) {
                    LAUNCH(launch_q8_freeze(h->tab, h->n_ord, l.ord, slot, h->nk, h->hd, sc.rec, r, q.s));
                    fz = 1;
                }
            }
        if (q.T == 1) {
            aa.split = l.sliding ? h->split_ds : h->split_df;
            aa.max_split = l.sliding ? h->ms_ds : h->ms_df;
            if (!l.sliding && h->ext_df) {
                aa.max_split = 64;
                aa.ext = 1;
            }
            aa.sd1 = h->tab + ((size_t)q.seq[0] * h->n_ord + l.ord) * kMaxLoops + slot;
            if (l.sliding && h->xm && !h->xm_off) aa.xcnt = h->xcnt;
        } else {
            aa.split = l.sliding ? h->split_bs : h->split_bf;
            aa.max_split = l.sliding ? h->ms_bs : h->ms_bf;
        }
        aa.field = -1;
        LAUNCH(launch_attn_dec(aa, M, q.s));
    } else {
        // A chunk of one sequence: rows pos0 .. pos0+M-1.
        const int64_t pos0 = q.pos[0];
        PrepArgs pa{};
        pa.qkvg = sc.qkvg; pa.qp = sc.qp; pa.kstage = h->q8 ? sc.kstage : nullptr;
        pa.rope = l.sliding ? h->rope_s : h->rope_f; pa.sq = w.sq; pa.tab = h->tab;
        pa.n_ord = h->n_ord; pa.ord = l.ord; pa.slot = slot; pa.nh = h->nh; pa.nk = h->nk; pa.hd = h->hd; pa.rec = sc.rec;
        pa.tap_pass = aa.tap_pass;
        pa.pos0 = pos0;
        if (!h->q8) {
            const SlotDesc &d = h->tab_host[((size_t)q.seq[0] * h->n_ord + l.ord) * kMaxLoops + slot];
            pa.kring = d.k; pa.vring = d.v; pa.cap = d.cap;
        }
        pa.kvtap = h->kvtap; pa.kvtap_n = q.T;
        LAUNCH(launch_prep(pa, M, q.s));
        bool field = false;
        if (h->q8) {
            // kv_cache.rs `append`: the field freezes when the 65th row (position 64)
            // is appended; rows before it were encoded without a field, rows after
            // against it.  A later loop's rewrite of the same rows finds it frozen.
            uint8_t &fz = froze_at(q, q.seq[0], l.ord, slot);
            const bool frozen = q.q8f[0] || fz;
            Q8WriteArgs wa{};
            wa.ksrc = sc.kstage; wa.kld = h->KV; wa.vsrc = sc.qkvg + h->Q + h->KV; wa.vld = ld;
            wa.tab = h->tab; wa.n_ord = h->n_ord; wa.ord = l.ord; wa.slot = slot; wa.nk = h->nk; wa.hd = h->hd;
            wa.rec = sc.rec;
            if (frozen) {
                wa.r0 = 0; wa.r1 = M; wa.field = 1;
                LAUNCH(launch_q8_write(wa, q.s));
            } else if (pos0 + M <= kWarmup) {
                wa.r0 = 0; wa.r1 = M; wa.field = 0;
                LAUNCH(launch_q8_write(wa, q.s));
            } else {
                const int split = (int)(kWarmup - pos0);
                wa.r0 = 0; wa.r1 = split; wa.field = 0;
                LAUNCH(launch_q8_write(wa, q.s));
                LAUNCH(launch_q8_freeze(h->tab, h->n_ord, l.ord, slot, h->nk, h->hd, sc.rec, 0, q.s));
                wa.r0 = split; wa.r1 = M; wa.field = 1;
                LAUNCH(launch_q8_write(wa, q.s));
                fz = 1;
            }
            field = q.q8f[0] || fz;
        }
        chunk_split(h, pos0, M, aa);
        aa.field = field;
        aa.pos0 = pos0;
        aa.nrows = q.T;
        aa.sdc = h->tab_host[((size_t)q.seq[0] * h->n_ord + l.ord) * kMaxLoops + slot];
        LAUNCH(launch_attn(aa, M, q.s));
    }
    if (q.T == 1) {
        GemvArgs a{};
        a.w[0] = w.wo; a.seg_end[0] = h->H; a.nseg = 1; a.N = h->H; a.K = h->Q; a.row = 0;
        a.src = sc.z; a.y = sc.o; a.rec = sc.rec; a.hidden = h->H;
        LAUNCH(launch_gemv(h->wt, kProNorm, kEpiStore, a, q.s));
    } else {
        // the projection runs on z as the merge left it (fp32 and bf16); the
        // renorm before it is a per-row factor the next residual step applies
        const int S = gemm_pick_splits(h->wt, true, M, h->H, h->Q);
        LAUNCH(launch_gemm(h->wt, sc.z, sc.znb, h->Q, gemm_w(w.wo, h->H), h->H, h->Q, sc.o, h->H, M, q.s, S,
                           sc.o_stride));
        q.o_parts = S;
        q.o_ss = sc.zss;
        q.o_ss_n = h->nk;
    }
    return DORY_OK;
}

// One MLP sub-layer over the first M rows of the call.
int enq_mlp(Enq &q, const LayerInfo &l, const Resolve &rs, const float *x, int M) {
    dory_t *h = q.h;
    const Scratch &sc = *q.sc;
    const dory_layer_weights &w = l.w;
    if (q.T == 1) {
        GemvArgs a{};
        a.w[0] = w.wgate; a.w[1] = w.wup; a.seg_end[0] = h->F; a.nseg = 1; a.N = h->F; a.K = h->H; a.row = 0;
        a.rs = rs; a.y = sc.ga; a.sg = w.sg; a.su = w.su; a.rec = sc.rec; a.hidden = h->H;
        a.embed = h->w.embed; a.vocab = h->V;
        const int pro = q.embed_pass ? kProEmbed : rs.loop_op == kLoopNext ? kProResolveInp : kProResolve;
        LAUNCH(launch_gemv(h->wt, pro, kEpiPair, a, q.s));
        GemvArgs d{};
        d.w[0] = w.wdown; d.seg_end[0] = h->H; d.nseg = 1; d.N = h->H; d.K = h->F; d.row = 0;
        d.src = sc.ga; d.y = sc.o; d.rec = sc.rec; d.hidden = h->H;
        LAUNCH(launch_gemv(h->wt, kProNorm, kEpiStore, d, q.s));
    } else {
        // the renorm before the down projection becomes a per-row factor the
        // next residual step applies (the projection is linear)
        const bool fused = sc.ussp && gemm_swiglu_ok(h->wt, M, h->F, h->H, h->H) &&
                           !gemm_reads_fp32_a(h->wt, true, M, h->F, h->F);
        if (fused) {  // SwiGLU in the GEMM's epilogue: z in bf16, sums of squares per 64 indices
            LAUNCH(launch_gemm_swiglu(sc.xb, h->H, w.wgate, w.wup, h->F, h->H, w.sg, w.su, sc.unb, sc.ussp, M, q.s));
        } else {
            LAUNCH(launch_gemm(h->wt, x, sc.xb, h->H, gateup_w(h, w), 2 * h->F, h->H, sc.ga, 2 * h->F, M, q.s));
            float *un = gemm_reads_fp32_a(h->wt, true, M, h->F, h->F) ? sc.un : nullptr;
            LAUNCH(launch_swiglu_norm(sc.ga, sc.ga + h->F, 2 * h->F, w.sg, w.su, un, sc.unb, h->F, M, q.s, sc.uss));
        }
        const int S = gemm_pick_splits(h->wt, true, M, h->H, h->F);
        LAUNCH(launch_gemm(h->wt, sc.un, sc.unb, h->F, gemm_w(w.wdown, h->H), h->H, h->F, sc.o, h->H, M, q.s, S,
                           sc.o_stride));
        q.o_parts = S;
        q.o_ss = fused ? sc.ussp : sc.uss;
        q.o_ss_n = fused ? h->F / 64 : 1;
    }
    return DORY_OK;
}

// dory.rs `stack` and `head`: embedding, input block, the recurrent block's
// loops with the loop mix, output block, head.  Sub-layer pass k reads its x
// from hb[k % 2]; the step between passes k-1 and k (slerp, loop mix) is fused
// into pass k's first kernel for one-row calls and is its own row kernel
// otherwise.  In a batch, loop i runs the first act[i] rows.
int enqueue(Enq &q) {
    dory_t *h = q.h;
    const Scratch &sc = *q.sc;
    const dory_config &c = h->cfg;
    const int T = q.T;
    // one-row calls: the first pass's GEMV gathers the embedding row itself
    if (q.k0 == 0 && T > 1)
        LAUNCH(launch_embed(h->wt, h->w.embed, h->V, h->H, sc.rec, T, sc.hb[0], sc.xb, q.s));
    const int P = passes(h, q.loops);
    auto rows_of = [&](int k) {
        if (k < c.n_in || k >= c.n_in + c.n_rec * q.loops) return T;
        return q.act[(k - c.n_in) / c.n_rec];
    };
    int prev_li = -1;
    for (int k = q.k0; k < P; ++k) {
        int li, loop_i = 0, op = kLoopNone;
        if (k < c.n_in) {
            li = k;
        } else if (k < c.n_in + c.n_rec * q.loops) {
            const int j = (k - c.n_in) % c.n_rec;
            loop_i = (k - c.n_in) / c.n_rec;
            li = c.n_in + j;
            if (j == 0) op = loop_i == 0 ? kLoopEnter : kLoopNext;
        } else {
            const int j = k - c.n_in - c.n_rec * q.loops;
            li = c.n_in + c.n_rec + j;
            if (j == 0) op = kLoopExit;
        }
        const int M = rows_of(k);
        Resolve rs{};
        rs.inp = sc.inp;
        rs.loop_op = op;
        rs.o_parts = q.o_parts;
        rs.o_stride = sc.o_stride;
        rs.o_ss = q.o_ss;
        rs.o_ss_n = q.o_ss_n;
        rs.st = q.batch ? sc.st : nullptr;
        rs.n_next = M;
        if (k == 0) {
            // the first pass takes the embedding as it is; o and alpha only need
            // to be valid addresses (the GEMV prologue loads them unconditionally).
            // One row: the GEMV gathers it and stores it as the residual.
            rs.h = sc.hb[0]; rs.o = sc.o; rs.alpha = h->L[0].w.alpha; rs.slerp = 0;
            rs.h_out = T == 1 ? sc.hb[0] : nullptr;
            rs.tap_pass = -1;
            rs.n_prev = T;
        } else if (k == q.k0) {
            // the early exit's second pass: e is the first pass's, as saved
            rs.h = q.e0; rs.o = sc.o; rs.alpha = h->L[0].w.alpha; rs.slerp = 0;
            rs.h_out = sc.hb[k % 2]; rs.hb_out = sc.xb; rs.tap_pass = -1;
            rs.n_prev = T;
        } else {
            rs.h = sc.hb[(k - 1) % 2]; rs.o = sc.o; rs.alpha = h->L[prev_li].w.alpha; rs.slerp = 1;
            rs.h_out = sc.hb[k % 2]; rs.hb_out = sc.xb; rs.tap_pass = k - 1;
            rs.n_prev = rows_of(k - 1);
            if (T > 1) LAUNCH(launch_resolve_rows(rs, h->H, op == kLoopExit ? T : rs.n_prev, sc.rec, h->tap, T, q.s));
        }
        if (op == kLoopExit && q.gate_save) rs.e_out = h->gst;
        const LayerInfo &l = h->L[li];
        const float *x = sc.hb[k % 2];
        q.embed_pass = k == 0 && T == 1;
        int rc = l.attn ? enq_attn(q, l, loop_i, rs, x, M) : enq_mlp(q, l, rs, x, M);
        q.embed_pass = false;
        if (rc) return rc;
        prev_li = li;
    }
    Resolve rf{};
    rf.o_parts = q.o_parts;
    rf.o_stride = sc.o_stride;
    rf.o_ss = q.o_ss;
    rf.o_ss_n = q.o_ss_n;
    rf.h = sc.hb[(P - 1) % 2]; rf.o = sc.o; rf.alpha = h->L[prev_li].w.alpha; rf.slerp = 1;
    rf.loop_op = kLoopNone; rf.inp = sc.inp; rf.tap_pass = P - 1; rf.n_prev = rf.n_next = T;
    GemvArgs a{};
    a.w[0] = h->w.head; a.seg_end[0] = h->V; a.nseg = 1; a.N = h->V; a.K = h->H;
    a.logit_scale = h->w.logit_scale; a.rec = sc.rec; a.hidden = h->H;
    if (T == 1) {
        rf.h_out = nullptr;
        a.row = 0; a.rs = rf;
        LAUNCH(launch_gemv(h->wt, kProResolve, kEpiHead, a, q.s));
    } else {
        rf.h_out = sc.hb[P % 2];
        rf.hb_out = sc.xb;
        LAUNCH(launch_resolve_rows(rf, h->H, T, sc.rec, h->tap, T, q.s));
        if (q.want_logits && !q.batch && !q.want_all) {
            a.row = T - 1; a.src = sc.hb[P % 2];
            LAUNCH(launch_gemv(h->wt, kProPlain, kEpiHead, a, q.s));
        } else if (q.want_logits) {
            // every row: the head as a GEMM, then the logit scale into each
            // row's logits row (the record's `out`)
            float *hl = q.want_all ? h->hlog_all : sc.hlog;
            LAUNCH(launch_gemm(h->wt, sc.hb[P % 2], sc.xb, h->H, gemm_w(h->w.head, h->V), h->V, h->H, hl, h->V, T, q.s));
            LAUNCH(launch_logits_rows(hl, h->w.logit_scale, h->V, T, sc.rec, q.s));
        }
    }
    return DORY_OK;
}

// Copies a call record to dst on the device on stream s (pinned staging ring).
int put_record(dory_t *h, CallRec *dst, const std::vector<RowRec> &rows, float *logits, hipStream_t s) {
    const int i = h->stage_i;
    h->stage_i = (i + 1) % kStages;
    if (h->stage_used[i]) SYNCCHECK(h, hipEventSynchronize(h->stage_ev[i]));
    CallRec *r = reinterpret_cast<CallRec *>(h->stage + (size_t)i * h->rec_sz);
    r->n = (int32_t)rows.size();
    r->logits = logits;
    r->tap = h->tap;
    r->kvtap = h->kvtap;
    memcpy(r->rows, rows.data(), sizeof(RowRec) * rows.size());
    HIPCHECK(h, hipMemcpyAsync(dst, r, rec_used((int)rows.size()), hipMemcpyHostToDevice, s));
    HIPCHECK(h, hipEventRecord(h->stage_ev[i], s));
    h->stage_used[i] = true;
    return DORY_OK;
}

// Rows of a chunk of one sequence: positions pos0.., logits (if any) of the last.
std::vector<RowRec> chunk_rows(int seq, int64_t pos0, int n, const int32_t *tokens, bool q8f = false,
                               bool all = false) {
    std::vector<RowRec> rows(n);
    for (int r = 0; r < n; ++r) rows[r] = RowRec{pos0 + r, seq, tokens ? tokens[r] : 0, all ? r : 0, q8f ? 1 : 0};
    return rows;
}

Enq make_enq(dory_t *h, hipStream_t s, int T, int loops, int mode, bool batch, bool want_logits,
             const std::vector<RowRec> &rows) {
    Enq q{h, s, &h->sc, T, loops, mode, batch, want_logits, {}, {}, {}, {}};
    q.act.assign(loops, T);
    for (const RowRec &r : rows) {
        q.pos.push_back(r.pos);
        q.seq.push_back(r.seq);
        q.q8f.push_back((uint8_t)r.q8f);
    }
    q.froze.assign((size_t)h->cfg.max_seqs * h->n_ord * kMaxLoops, 0);
    return q;
}

}  // namespace

// ====================================================================== ABI

extern "C" {

int dory_create(const dory_config *cfg, const dory_weights *w, dory_t **out) {
    if (out) *out = nullptr;
    int rc = check_config(cfg, w);
    if (rc) return rc;
    if (!out) return fail(nullptr, DORY_EINVAL, "dory_create: null out");
    dory_t *h = new dory();
    h->cfg = *cfg;
    h->pattern = cfg->layer_pattern;
    h->cfg.layer_pattern = h->pattern.c_str();
    const int nl = (int)h->pattern.size();
    h->wl.assign(w->layers, w->layers + nl);
    h->w = *w;
    h->w.layers = h->wl.data();
    h->H = cfg->hidden; h->F = cfg->ffn; h->V = cfg->vocab; h->nh = cfg->nh; h->nk = cfg->nk; h->hd = cfg->hd;
    h->Q = h->nh * h->hd; h->KV = h->nk * h->hd; h->ngk = (h->hd + kKGroup - 1) / kKGroup;
    h->wt = cfg->weight_dtype == DORY_W_BF16 ? kBF16 : kF32;
    h->q8 = cfg->kv_encoding == DORY_KV_Q8_2F;
    for (int li = 0; li < nl; ++li) {
        LayerInfo l;
        const char ch = h->pattern[li];
        l.attn = ch != '-';
        l.sliding = ch == 'S';
        l.rec = li >= cfg->n_in && li < cfg->n_in + cfg->n_rec;
        l.ord = l.attn ? h->n_ord++ : -1;
        l.w = h->wl[li];
        h->L.push_back(l);
    }
    // Rings: a call of up to max_chunk rows must not overwrite a key any of its
    // rows still reads, so a window of W keys needs W + max_chunk - 1 rows.
    const int chunk = cfg->max_chunk;
    h->win_s = cfg->window;
    h->win_f = cfg->full_window > 0 ? cfg->full_window : kHuge;
    h->cap_s = std::min<int64_t>(cfg->max_ctx, round_up(std::max(cfg->window + chunk - 1, 128), 64));
    h->cap_f = cfg->full_window > 0
                   ? (int)std::min<int64_t>(cfg->max_ctx, round_up(std::max(cfg->full_window + chunk - 1, 128), 64))
                   : cfg->max_ctx;
    const int64_t wmax = std::min<int64_t>(std::max<int64_t>(h->win_s, std::min<int64_t>(h->win_f, cfg->max_ctx)),
                                           cfg->max_ctx);
    // Decode splits.  One-row calls: full layers about 64 workgroups per kv
    // head at the longest window, 8 load steps each (the latency of one short
    // workgroup sets the pace); sliding layers about 16 (64 keys each, the
    // one-row kernel's full width: fewer splits to merge).  Batches: about 32 per kv head with 16 load steps (the
    // grid is large anyway, and fewer splits mean less to merge).  Each takes a
    // multiple of the keys a workgroup covers per step.
    const int kb = 256 / (h->hd / 4);
    auto pick = [&](int64_t W, int steps, int target, int lo) {
        const int dmax = attn_dec_max_split(h->hd, steps);
        int sp = (int)std::min<int64_t>(std::max<int64_t>(lo, (W + target - 1) / target), dmax);
        sp = std::max(kb, (sp + kb - 1) / kb * kb);
        return std::min(sp, dmax);
    };
    const int64_t wf = std::min<int64_t>(h->win_f, cfg->max_ctx), ws = std::min<int64_t>(h->win_s, cfg->max_ctx);
    h->split_ds = pick(ws, 8, 16, 1);
    h->split_df = pick(wf, 8, 64, 1);
    h->split_bs = pick(ws, 16, 32, 64);
    h->split_bf = pick(wf, 16, 32, 64);
    h->ms_ds = (int)((ws + h->split_ds - 1) / h->split_ds);
    h->ms_df = (int)((wf + h->split_df - 1) / h->split_df);
    h->ms_bs = (int)((ws + h->split_bs - 1) / h->split_bs);
    h->ms_bf = (int)((wf + h->split_bf - 1) / h->split_bf);
    h->ms_dec = std::max(std::max(h->ms_ds, h->ms_df), std::max(h->ms_bs, h->ms_bf));
    h->ext_df = h->hd == 128 && h->nh == 4 * h->nk && h->split_df == 64 && h->ms_df > 64 && h->ms_df <= 72;
    // multi-row calls: at least 256 keys per split over a block's key range,
    // which is at most wmax + 127 keys
    h->split_pf = 256;
    h->ms_pf = (int)((wmax + 127 + h->split_pf - 1) / h->split_pf);
    if (h->ms_dec > 1024 || h->ms_pf > 1024) {
        delete h;
        return fail(nullptr, DORY_EINVAL, "dory_create: attention window too long (more than 262144 keys)");
    }
    h->seqs.resize(cfg->max_seqs);
    h->tab_host.assign((size_t)cfg->max_seqs * std::max(h->n_ord, 1) * kMaxLoops, SlotDesc{});
    h->rec_sz = rec_bytes(std::max(chunk, cfg->max_seqs));

    auto bail = [&](int code) {
        g_create_error = h->err;
        free_all(h);
        delete h;
        return code;
    };
#define CREATE_CHECK(call)                                          \
    do {                                                            \
        hipError_t e_ = (call);                                     \
        if (e_ != hipSuccess) return bail(hip_fail(h, e_, #call));  \
    } while (0)
    CREATE_CHECK(hipGetDevice(&h->device));
    const size_t TH = (size_t)chunk * h->H;
    CREATE_CHECK(dmalloc(h, &h->sc.hb[0], TH));
    CREATE_CHECK(dmalloc(h, &h->sc.hb[1], TH));
    CREATE_CHECK(dmalloc(h, &h->sc.inp, TH));
    h->sc.o_stride = TH;
    CREATE_CHECK(dmalloc(h, &h->sc.o, TH * kMaxKParts));   // split-K slabs of the output projections
    CREATE_CHECK(dmalloc(h, &h->sc.qkvg, (size_t)chunk * (2 * h->Q + 2 * h->KV)));
    CREATE_CHECK(dmalloc(h, &h->sc.qp, (size_t)chunk * h->Q));
    CREATE_CHECK(dmalloc(h, &h->sc.z, (size_t)chunk * h->Q));
    CREATE_CHECK(dmalloc(h, &h->sc.zn, (size_t)chunk * h->Q));
    CREATE_CHECK(dmalloc(h, &h->sc.ga, (size_t)chunk * 2 * h->F));   // gate | up per row
    CREATE_CHECK(dmalloc(h, &h->sc.un, (size_t)chunk * h->F));
    CREATE_CHECK(dmalloc(h, &h->sc.xb, (size_t)chunk * h->H));
    CREATE_CHECK(dmalloc(h, &h->sc.znb, (size_t)chunk * h->Q));
    CREATE_CHECK(dmalloc(h, &h->sc.zss, (size_t)chunk * h->nk));
    CREATE_CHECK(dmalloc(h, &h->sc.uss, (size_t)chunk));
    if (h->F % 64 == 0) CREATE_CHECK(dmalloc(h, &h->sc.ussp, (size_t)chunk * (h->F / 64)));
    CREATE_CHECK(dmalloc(h, &h->sc.unb, (size_t)chunk * h->F));
    CREATE_CHECK(dmalloc(h, &h->sc.kstage, (size_t)chunk * h->KV));
    CREATE_CHECK(dmalloc(h, &h->ld_k, (size_t)chunk * h->KV));
    CREATE_CHECK(dmalloc(h, &h->ld_v, (size_t)chunk * h->KV));
    CREATE_CHECK(dmalloc(h, &h->sc.st, TH));
    CREATE_CHECK(dmalloc(h, &h->sc.hlog, (size_t)std::min(chunk, cfg->max_seqs) * h->V));
    const size_t rep = h->nh / h->nk;
    // decode rows (one per sequence of a batch) or the rows of a chunk
    const size_t dec_rows = std::min(chunk, cfg->max_seqs);
    const size_t part = std::max(std::max(dec_rows * h->ms_dec, (size_t)chunk * h->ms_pf) * h->nk * rep * (h->hd + 2),
                                 attn_xm_part_floats(h->nk, h->ms_ds, (int)rep, h->hd));
    CREATE_CHECK(dmalloc(h, &h->sc.part, part));
    CREATE_CHECK(dmalloc(h, &h->tab, h->tab_host.size()));
    CREATE_CHECK(hipMemset(h->tab, 0, sizeof(SlotDesc) * h->tab_host.size()));
    char *recp = nullptr;
    CREATE_CHECK(dmalloc(h, &recp, h->rec_sz));
    h->sc.rec = reinterpret_cast<CallRec *>(recp);
    // RoPE tables for every position (dory.rs `stack`): inverse frequencies
    // theta^(-2j/hd) rounded to fp32, angle p * inv in f64, cos and sin rounded
    // to fp32; row p is [cos half | sin half].
    {
        const int hd = h->hd, half = hd / 2;
        std::vector<float> tab((size_t)cfg->max_ctx * hd), inv(half);
        for (int kind = 0; kind < 2; ++kind) {
            const double theta = kind == 0 ? cfg->rope_theta_sliding : cfg->rope_theta_full;
            for (int j = 0; j < half; ++j) inv[j] = (float)std::pow(theta, -2.0 * j / hd);
            for (int64_t p = 0; p < cfg->max_ctx; ++p)
                for (int j = 0; j < half; ++j) {
                    const double ang = (double)p * (double)inv[j];
                    tab[p * hd + j] = (float)std::cos(ang);
                    tab[p * hd + half + j] = (float)std::sin(ang);
                }
            float *&dst = kind == 0 ? h->rope_s : h->rope_f;
            CREATE_CHECK(dmalloc(h, &dst, tab.size()));
            CREATE_CHECK(hipMemcpy(dst, tab.data(), sizeof(float) * tab.size(), hipMemcpyHostToDevice));
        }
    }
    // The in-kernel merge of the sliding layers' one-row attention (head dim
    // 128, 4 q heads per kv head, at most 64 splits) needs every workgroup id of one residue mod 8 on
    // one XCD: checked once on this device over the grid it launches (else the
    // merge kernel serves, as for the full layers).
    if (h->hd == 128 && h->nh == 4 * h->nk && h->ms_ds <= 64 && h->split_ds <= 64) {
        const int G = 8 * h->ms_ds * ((h->nk + 7) / 8);
        unsigned *ids = nullptr;
        CREATE_CHECK(dmalloc(h, &ids, (size_t)G));
        CREATE_CHECK(launch_xcd_check(ids, G, nullptr));
        std::vector<unsigned> got(G);
        CREATE_CHECK(hipMemcpy(got.data(), ids, sizeof(unsigned) * G, hipMemcpyDeviceToHost));
        bool same = true;
        for (int i = 8; i < G; ++i) same = same && got[i] == got[i % 8];
        if (same) {
            CREATE_CHECK(dmalloc(h, &h->xcnt, (size_t)32 * h->nh));
            CREATE_CHECK(hipMemset(h->xcnt, 0, sizeof(uint32_t) * 32 * h->nh));
            CREATE_CHECK(hipDeviceSynchronize());
            h->xm = true;
        }
    }
    CREATE_CHECK(hipHostMalloc((void **)&h->stage, h->rec_sz * kStages, hipHostMallocDefault));
    for (int i = 0; i < kStages; ++i) CREATE_CHECK(hipEventCreateWithFlags(&h->stage_ev[i], hipEventDisableTiming));
    CREATE_CHECK(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking));
    // the static scratch of dory_forward_chunk_noalloc: its address on this
    // device (looked up once per device and kept); a failure only disables
    // that entry point
    {
        void *p = nullptr;
        const hipError_t e = noalloc_scratch(&p);
        if (e == hipSuccess) h->noalloc = p;
        else h->noalloc_err = std::string("the static scratch's address: ") + hipGetErrorString(e);
        h->noalloc_need = carve_scratch(h, kNoAllocRows, nullptr, nullptr);
    }
    // Every sequence's slot 0 of every attention layer; per_loop's further
    // slots come on the first per_loop call that needs them.
    for (int s = 0; s < cfg->max_seqs; ++s)
        for (const LayerInfo &l : h->L)
            if (l.attn && alloc_slot(h, s, l.ord, 0, l.sliding)) return bail(DORY_ENOMEM);
#undef CREATE_CHECK
    *out = h;
    return DORY_OK;
}

void dory_destroy(dory_t *h) {
    if (!h) return;
    (void)hipSetDevice(h->device);
    (void)hipDeviceSynchronize();
    free_all(h);
    delete h;
}

const char *dory_last_error(const dory_t *h) { return h ? h->err.c_str() : g_create_error.c_str(); }

namespace {

// dory.rs `ExitRate::probe`: a read-out after the first pass while early exits
// are frequent (rate >= 0.35), else for one token in eight.
bool exit_probe(SeqState &st) {
    st.exit_tokens += 1u;
    return st.exit_rate >= 0.35f || st.exit_tokens % 8u == 0u;
}

// dory.rs `ExitRate::note`: running mean of the exits, weight 0.1.
void exit_note(SeqState &st, bool exited) { st.exit_rate += 0.1f * ((exited ? 1.0f : 0.0f) - st.exit_rate); }

// Replays the captured graph of key (capturing it first) with the work of q
// (and the read-out's top probability when top): every pointer a replay needs
// per call comes from the device record, so one graph serves every call.
int replay(dory_t *h, std::tuple<int, int, int> key, const Enq &q, bool top, hipStream_t s) {
    auto it = h->graphs.find(key);
    if (it == h->graphs.end()) {
        Enq cq = q;
        cq.s = h->cap_stream;
        HIPCHECK(h, hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
        int rc = enqueue(cq);
        hipError_t e0 = hipSuccess;
        if (!rc && top) e0 = launch_top_prob(q.sc->rec, h->V, h->gtop, h->cap_stream);
        hipGraph_t g = nullptr;
        hipError_t e = hipStreamEndCapture(h->cap_stream, &g);
        if (rc || e0 != hipSuccess) {
            if (g) (void)hipGraphDestroy(g);
            return rc ? rc : hip_fail(h, e0, "launch_top_prob");
        }
        if (e != hipSuccess) return hip_fail(h, e, "hipStreamEndCapture");
        hipGraphExec_t ex = nullptr;
        e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
        (void)hipGraphDestroy(g);
        if (e != hipSuccess) return hip_fail(h, e, "hipGraphInstantiate");
        it = h->graphs.emplace(key, ex).first;
    }
    if (inject_failure(h)) return hip_fail(h, hipErrorLaunchFailure, "(injected) hipGraphLaunch");
    HIPCHECK(h, hipGraphLaunch(it->second, s));
    return DORY_OK;
}

// Graph keys of the early exit's two phases: (kKeyGateFirst / kKeyGateSecond,
// kv mode, sequence), apart from the (loops 1..16, mode, sequence) of plain
// one-row calls.
constexpr int kKeyGateFirst = 101, kKeyGateSecond = 102;

// A gated one-row call whose token reads out after its first pass (dory.rs
// `stack`, `Gate::Conf`): the first pass, the output block and the head
// (saving the loop exit's e), the top probability back on the host; then,
// unless it reaches the threshold, a second pass from the saved e that
// rewrites this position (the read-out's rows too: one-row writes go to the
// position's ring row) and reads out again.  Synchronous: it waits for the
// read-out.
int gated_readout(dory_t *h, int32_t seq, const int32_t *tokens, hipStream_t s, float *logits) {
    const dory_config &c = h->cfg;
    SeqState &st = h->seqs[seq];
    const std::vector<RowRec> rows = chunk_rows(seq, st.pos, 1, tokens, st.q8_frozen);
    float *lg = logits ? logits : h->glog;
    int rc = put_record(h, h->sc.rec, rows, lg, s);
    if (rc) return rc;
    Enq q = make_enq(h, s, 1, 1, DORY_LAST_LOOP, false, true, rows);
    q.gate_save = true;
    // (q8_2f: graphs once the fields froze, when no phase launches a freeze)
    const bool graphs = !h->q8 || st.q8_frozen;
    if (graphs) {
        rc = replay(h, std::make_tuple(kKeyGateFirst, (int)DORY_LAST_LOOP, seq), q, true, s);
        if (rc) return rc;
    } else {
        rc = enqueue(q);
        if (rc) return rc;
        HIPCHECK(h, launch_top_prob(h->sc.rec, h->V, h->gtop, s));
    }
    HIPCHECK(h, hipMemcpyAsync(h->gtop_host, h->gtop, sizeof(float), hipMemcpyDeviceToHost, s));
    SYNCCHECK(h, hipStreamSynchronize(s));
    const float tp = *h->gtop_host;
    const bool stay = tp < h->gate_th;
    st.last_top = tp;
    exit_note(st, !stay);
    if (stay) {
        Enq q2 = q;  // the same record and the freezes the first pass made
        q2.loops = 2;
        q2.act.assign(2, 1);
        q2.gate_save = false;
        q2.k0 = c.n_in + c.n_rec;
        q2.e0 = h->gst;
        rc = graphs ? replay(h, std::make_tuple(kKeyGateSecond, (int)DORY_LAST_LOOP, seq), q2, false, s) : enqueue(q2);
        if (rc) return rc;
    }
    st.gate_tokens += 1;
    st.gate_one += stay ? 0 : 1;
    h->last_T = 1;
    h->last_chunk = false;
    h->last_loops = stay ? 2 : 1;
    h->last_mode = DORY_LAST_LOOP;
    h->last_pos0 = st.pos;
    h->last_seq0 = seq;
    if (h->q8 && st.pos + 1 > kWarmup) st.q8_frozen = true;
    st.pos += 1;
    st.mode = DORY_LAST_LOOP;
    return DORY_OK;
}

// dory_forward_chunk (all = false: logits of the last row, or none) and
// dory_forward_chunk_all (every row's logits).
int forward_chunk(dory_t *h, int32_t seq, const int32_t *tokens, int32_t n, int32_t loops, int32_t kv_mode,
                  dory_stream_t stream, float *logits, bool all, bool noalloc = false) {
    if (!h) return DORY_EINVAL;
    const dory_config &c = h->cfg;
    if (seq < 0 || seq >= c.max_seqs) return fail(h, DORY_EINVAL, "dory_forward_chunk: seq out of range");
    if (!tokens || n < 1) return fail(h, DORY_EINVAL, "dory_forward_chunk: need n >= 1 tokens");
    if (n > c.max_chunk) return fail(h, DORY_ERANGE, "dory_forward_chunk: n > max_chunk");
    if (loops < 1 || loops > DORY_MAX_LOOPS)
        return fail(h, DORY_EINVAL, "dory_forward_chunk: loops must be in 1..16, got " + std::to_string(loops));
    if (kv_mode != DORY_PER_LOOP && kv_mode != DORY_LAST_LOOP)
        return fail(h, DORY_EINVAL, "dory_forward_chunk: kv_mode must be per_loop or last_loop");
    SeqState &st = h->seqs[seq];
    if (st.latched) return latched_error(h, "dory_forward_chunk", seq);
    if (st.mode >= 0 && st.mode != kv_mode)
        return fail(h, DORY_ESTATE, "dory_forward_chunk: kv mode changed without dory_kv_reset");
    if (kv_mode == DORY_PER_LOOP && st.loops > 0 && st.loops != loops)
        return fail(h, DORY_ESTATE, "dory_forward_chunk: per_loop needs the same loop count on every call");
    if (st.pos + n > c.max_ctx) return fail(h, DORY_ERANGE, "dory_forward_chunk: position past max_ctx");
    if (all && !logits) return fail(h, DORY_EINVAL, "dory_forward_chunk_all: logits must not be null");
    if (noalloc) {
        if (n > kNoAllocRows)
            return fail(h, DORY_ERANGE, "dory_forward_chunk_noalloc: n > " + std::to_string(kNoAllocRows));
        if (h->gate_on) return fail(h, DORY_EINVAL, "dory_forward_chunk_noalloc: takes no exit gate");
        if (!h->noalloc) return fail(h, DORY_EDEVICE, "dory_forward_chunk_noalloc: " + h->noalloc_err);
        if (h->noalloc_need > kNoAllocBytes)
            return fail(h, DORY_ERANGE, "dory_forward_chunk_noalloc: this geometry needs " +
                                            std::to_string(h->noalloc_need) + " bytes of scratch, the static array holds " +
                                            std::to_string(kNoAllocBytes));
    }
    // dory.rs `stack`: under the gate a one-row call runs one pass, a read-out
    // when the exit rate asks for one, and a second pass unless it exits
    const bool gated = n == 1 && h->gate_on;
    if (gated && kv_mode != DORY_LAST_LOOP)
        return fail(h, DORY_EINVAL, "dory_forward_chunk: the exit gate works on the last_loop cache");
    if (gated && (h->tap || h->kvtap)) return fail(h, DORY_EINVAL, "dory_forward_chunk: gated calls take no tap");
    // dory.rs `chunk_loops`: a last_loop call whose logits nobody reads keeps
    // only its cache rows and runs at most prompt_loops passes
    if (!logits && kv_mode == DORY_LAST_LOOP && h->prompt_loops > 0) loops = std::min(loops, h->prompt_loops);
    if (h->tap && (int64_t)passes(h, loops) * n * h->H > h->tap_cap)
        return fail(h, DORY_EINVAL, "dory_forward_chunk: the tap buffer is too small for this call");
    if (h->kvtap && (int64_t)attn_passes(h, loops) * n * 2 * h->KV > h->kvtap_cap)
        return fail(h, DORY_EINVAL, "dory_forward_chunk: the kv tap buffer is too small for this call");
    HIPCHECK(h, hipSetDevice(h->device));
    if (gated) {
        int rc0 = ensure_slots(h, seq, kv_mode, 2);
        if (rc0) return rc0;
        if (exit_probe(st))
            return latch(h, gated_readout(h, seq, tokens, reinterpret_cast<hipStream_t>(stream), logits), &seq, 1);
        loops = 2;  // no read-out: both passes, then the output block once
    }
    all = all && n > 1;  // one row: its logits are the last row's
    if (all && !h->hlog_all) HIPCHECK(h, dmalloc(h, &h->hlog_all, (size_t)c.max_chunk * h->V));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (noalloc) {
        // no allocation, no graph: the slots must exist, the kernels run over a
        // carve-out of the static array, the record goes there too
        if (!slots_ready(h, seq, kv_mode, loops))
            return fail(h, DORY_ESTATE, "dory_forward_chunk_noalloc: a per_loop slot this call needs is not "
                                        "allocated yet (an ordinary call with this loop count allocates it)");
        Scratch sc{};
        carve_scratch(h, kNoAllocRows, reinterpret_cast<char *>(h->noalloc), &sc);
        const std::vector<RowRec> rows = chunk_rows(seq, st.pos, n, tokens, st.q8_frozen);
        int rc = put_record(h, sc.rec, rows, logits, s);
        if (rc) return latch(h, rc, &seq, 1);
        Enq q = make_enq(h, s, n, loops, kv_mode, false, logits != nullptr, rows);
        q.sc = &sc;
        rc = enqueue(q);
        if (rc) return latch(h, rc, &seq, 1);
        h->last_T = 0;  // the stage benchmark reads the handle's scratch: not this call's
        if (h->q8 && st.pos + n > kWarmup) st.q8_frozen = true;
        st.pos += n;
        st.mode = kv_mode;
        if (kv_mode == DORY_PER_LOOP) st.loops = loops;
        return DORY_OK;
    }
    int rc = ensure_slots(h, seq, kv_mode, loops);
    if (rc) return rc;
    const std::vector<RowRec> rows = chunk_rows(seq, st.pos, n, tokens, st.q8_frozen, all);
    rc = put_record(h, h->sc.rec, rows, logits, s);
    if (rc) return latch(h, rc, &seq, 1);
    Enq q = make_enq(h, s, n, loops, kv_mode, false, logits != nullptr, rows);
    q.want_all = all;
    // (q8_2f: once the fields froze, a one-row call launches no freeze)
    const bool graphable = n == 1 && (!h->q8 || st.q8_frozen);
    rc = graphable ? replay(h, std::make_tuple(loops, kv_mode, seq), q, false, s) : enqueue(q);
    if (rc) return latch(h, rc, &seq, 1);
    h->last_T = n;
    h->last_chunk = n > 1;
    h->last_loops = loops;
    h->last_mode = kv_mode;
    h->last_pos0 = st.pos;
    h->last_seq0 = seq;
    if (h->q8 && st.pos + n > kWarmup) st.q8_frozen = true;
    if (gated) st.gate_tokens += 1;
    st.pos += n;
    st.mode = kv_mode;
    if (kv_mode == DORY_PER_LOOP) st.loops = loops;
    return DORY_OK;
}

}  // namespace

int dory_forward_chunk(dory_t *h, int32_t seq, const int32_t *tokens, int32_t n, int32_t loops, int32_t kv_mode,
                       dory_stream_t stream, float *logits) {
    return forward_chunk(h, seq, tokens, n, loops, kv_mode, stream, logits, false);
}

int dory_forward_chunk_all(dory_t *h, int32_t seq, const int32_t *tokens, int32_t n, int32_t loops, int32_t kv_mode,
                           dory_stream_t stream, float *logits) {
    return forward_chunk(h, seq, tokens, n, loops, kv_mode, stream, logits, true);
}

int dory_forward_chunk_noalloc(dory_t *h, int32_t seq, const int32_t *tokens, int32_t n, int32_t loops,
                               int32_t kv_mode, dory_stream_t stream, float *logits) {
    return forward_chunk(h, seq, tokens, n, loops, kv_mode, stream, logits, false, true);
}

int dory_set_gate(dory_t *h, int32_t on, float threshold) {
    if (!h) return DORY_EINVAL;
    if (on && !(threshold >= 0.0f)) return fail(h, DORY_EINVAL, "dory_set_gate: the threshold must be >= 0");
    if (on && !h->gst) {
        HIPCHECK(h, hipSetDevice(h->device));
        HIPCHECK(h, dmalloc(h, &h->gst, (size_t)h->H));
        HIPCHECK(h, dmalloc(h, &h->glog, (size_t)h->V));
        HIPCHECK(h, dmalloc(h, &h->gtop, (size_t)1));
        HIPCHECK(h, hipHostMalloc((void **)&h->gtop_host, sizeof(float), hipHostMallocDefault));
    }
    h->gate_on = on != 0;
    h->gate_th = on ? threshold : 0.f;
    return DORY_OK;
}

int dory_gate_stats(const dory_t *h, int32_t seq, int64_t *tokens, int64_t *one, float *last_top, float *rate) {
    if (!h || seq < 0 || seq >= h->cfg.max_seqs) return DORY_EINVAL;
    const SeqState &st = h->seqs[seq];
    if (tokens) *tokens = st.gate_tokens;
    if (one) *one = st.gate_one;
    if (last_top) *last_top = st.last_top;
    if (rate) *rate = st.exit_rate;
    return DORY_OK;
}

int dory_set_prompt_loops(dory_t *h, int32_t n) {
    if (!h) return DORY_EINVAL;
    if (n < 0 || n > DORY_MAX_LOOPS) return fail(h, DORY_EINVAL, "dory_set_prompt_loops: n must be in 0..16");
    h->prompt_loops = n;
    return DORY_OK;
}

int dory_forward_batch(dory_t *h, int32_t nseq, const int32_t *seqs, const int32_t *tokens, const int32_t *loops,
                       int32_t kv_mode, dory_stream_t stream, float *logits) {
    if (!h) return DORY_EINVAL;
    const dory_config &c = h->cfg;
    if (!seqs || !tokens || !loops || nseq < 1) return fail(h, DORY_EINVAL, "dory_forward_batch: need nseq >= 1 rows");
    if (nseq > c.max_chunk || nseq > c.max_seqs) return fail(h, DORY_ERANGE, "dory_forward_batch: nseq > max_chunk or max_seqs");
    if (kv_mode != DORY_PER_LOOP && kv_mode != DORY_LAST_LOOP)
        return fail(h, DORY_EINVAL, "dory_forward_batch: kv_mode must be per_loop or last_loop");
    if (h->gate_on && nseq > 1) return fail(h, DORY_EINVAL, "dory_forward_batch: the exit gate takes one-row calls");
    std::vector<uint8_t> seen(c.max_seqs, 0);
    for (int i = 0; i < nseq; ++i) {
        const int sq = seqs[i];
        if (sq < 0 || sq >= c.max_seqs) return fail(h, DORY_EINVAL, "dory_forward_batch: seq out of range");
        if (seen[sq]) return fail(h, DORY_EINVAL, "dory_forward_batch: a sequence appears twice");
        seen[sq] = 1;
        if (loops[i] < 1 || loops[i] > DORY_MAX_LOOPS) return fail(h, DORY_EINVAL, "dory_forward_batch: loops must be in 1..16");
        const SeqState &st = h->seqs[sq];
        if (st.latched) return latched_error(h, "dory_forward_batch", sq);
        if (st.mode >= 0 && st.mode != kv_mode)
            return fail(h, DORY_ESTATE, "dory_forward_batch: kv mode changed without dory_kv_reset");
        if (kv_mode == DORY_PER_LOOP && st.loops > 0 && st.loops != loops[i])
            return fail(h, DORY_ESTATE, "dory_forward_batch: per_loop needs the same loop count on every call");
        if (st.pos + 1 > c.max_ctx) return fail(h, DORY_ERANGE, "dory_forward_batch: position past max_ctx");
    }
    // dory.rs `chunk_loops` for rows whose logits nobody reads (each row is a
    // one-row call of its sequence)
    std::vector<int32_t> lp(loops, loops + nseq);
    if (!logits && kv_mode == DORY_LAST_LOOP && h->prompt_loops > 0)
        for (int32_t &x : lp) x = std::min(x, (int32_t)h->prompt_loops);
    loops = lp.data();
    if (h->tap) {
        int lmax = 0;
        for (int i = 0; i < nseq; ++i) lmax = std::max(lmax, (int)loops[i]);
        if ((int64_t)passes(h, lmax) * nseq * h->H > h->tap_cap)
            return fail(h, DORY_EINVAL, "dory_forward_batch: the tap buffer is too small for this call");
    }
    if (h->kvtap) {
        int lmax = 0;
        for (int i = 0; i < nseq; ++i) lmax = std::max(lmax, (int)loops[i]);
        if ((int64_t)attn_passes(h, lmax) * nseq * 2 * h->KV > h->kvtap_cap)
            return fail(h, DORY_EINVAL, "dory_forward_batch: the kv tap buffer is too small for this call");
    }
    if (nseq == 1) return dory_forward_chunk(h, seqs[0], tokens, 1, loops[0], kv_mode, stream, logits);
    HIPCHECK(h, hipSetDevice(h->device));
    for (int i = 0; i < nseq; ++i) {
        int rc = ensure_slots(h, seqs[i], kv_mode, loops[i]);
        if (rc) return rc;
    }
    // rows sorted by loops, longest first: the rows of loop i are a prefix
    std::vector<int> order(nseq);
    for (int i = 0; i < nseq; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return loops[a] > loops[b]; });
    std::vector<RowRec> rows(nseq);
    for (int r = 0; r < nseq; ++r) {
        const int i = order[r];
        rows[r] = RowRec{h->seqs[seqs[i]].pos, seqs[i], tokens[i], i, h->seqs[seqs[i]].q8_frozen ? 1 : 0};
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int rc = put_record(h, h->sc.rec, rows, logits, s);
    if (rc) return latch(h, rc, seqs, nseq);
    const int lmax = loops[order[0]];
    Enq q = make_enq(h, s, nseq, lmax, kv_mode, true, logits != nullptr, rows);
    for (int i = 0; i < lmax; ++i) {
        int a = 0;
        while (a < nseq && loops[order[a]] > i) ++a;
        q.act[i] = a;
    }
    rc = enqueue(q);
    if (rc) return latch(h, rc, seqs, nseq);
    h->last_T = nseq;
    h->last_seq0 = seqs[0];
    h->last_chunk = false;
    h->last_loops = lmax;
    h->last_mode = kv_mode;
    for (int i = 0; i < nseq; ++i) {
        SeqState &st = h->seqs[seqs[i]];
        if (h->q8 && st.pos >= kWarmup) st.q8_frozen = true;
        st.pos += 1;
        st.mode = kv_mode;
        if (kv_mode == DORY_PER_LOOP) st.loops = loops[i];
    }
    return DORY_OK;
}

int dory_kv_reset(dory_t *h, int32_t seq) {
    if (!h) return DORY_EINVAL;
    if (seq < -1 || seq >= h->cfg.max_seqs) return fail(h, DORY_EINVAL, "dory_kv_reset: seq out of range");
    for (int s = 0; s < h->cfg.max_seqs; ++s)
        if (seq < 0 || s == seq) h->seqs[s] = SeqState{};
    return DORY_OK;
}

int dory_rollback(dory_t *h, int32_t seq, int64_t n) {
    if (!h) return DORY_EINVAL;
    if (seq < 0 || seq >= h->cfg.max_seqs) return fail(h, DORY_EINVAL, "dory_rollback: seq out of range");
    if (n < 0) return fail(h, DORY_EINVAL, "dory_rollback: n must be >= 0");
    SeqState &st = h->seqs[seq];
    if (st.latched) return latched_error(h, "dory_rollback", seq);
    if (n >= st.pos) return DORY_OK;
    // The next row, at position n, reads keys max(0, n - W + 1) .. n - 1; a
    // ring of cap rows still holds positions pos - cap .. pos - 1.
    auto keeps = [&](int64_t W, int64_t cap) {
        return cap >= h->cfg.max_ctx || std::max<int64_t>(0, n - W + 1) >= st.pos - cap;
    };
    if (!keeps(h->win_s, h->cap_s) || !keeps(h->win_f, h->cap_f))
        return fail(h, DORY_ERANGE, "dory_rollback: from position " + std::to_string(st.pos) + " to " +
                                        std::to_string(n) + " is deeper than the windowed rings keep");
    st.pos = n;
    return DORY_OK;
}

int64_t dory_position(const dory_t *h, int32_t seq) {
    if (!h || seq < 0 || seq >= h->cfg.max_seqs) return DORY_EINVAL;
    return h->seqs[seq].pos;
}

int dory_debug_fail_launch(dory_t *h, int64_t n) {
    if (!h) return DORY_EINVAL;
    if (n < 0) return fail(h, DORY_EINVAL, "dory_debug_fail_launch: n must be >= 0");
    h->fail_in = n;
    return DORY_OK;
}

int dory_debug_xcd_merge(dory_t *h, int on) {
    if (!h) return DORY_EINVAL;
    if (on == 0 || on == 1) {
        if (h->xm_off != (on == 0)) {
            // captured graphs hold the other path's launches
            (void)hipDeviceSynchronize();
            for (auto &g : h->graphs) (void)hipGraphExecDestroy(g.second);
            h->graphs.clear();
        }
        h->xm_off = on == 0;
    } else if (on != -1) {
        return fail(h, DORY_EINVAL, "dory_debug_xcd_merge: on must be 0, 1 or -1");
    }
    return h->xm && !h->xm_off ? 1 : 0;
}

int dory_latched(const dory_t *h, int32_t seq) {
    if (!h || seq < 0 || seq >= h->cfg.max_seqs) return DORY_EINVAL;
    return h->seqs[seq].latched ? 1 : 0;
}

int dory_debug_kv_tap(dory_t *h, float *buf, int64_t cap) {
    if (!h) return DORY_EINVAL;
    if (buf && cap <= 0) return fail(h, DORY_EINVAL, "dory_debug_kv_tap: cap must be positive");
    h->kvtap = buf;
    h->kvtap_cap = buf ? cap : 0;
    return DORY_OK;
}

int dory_debug_tap(dory_t *h, float *buf, int64_t cap) {
    if (!h) return DORY_EINVAL;
    if (buf && cap <= 0) return fail(h, DORY_EINVAL, "dory_debug_tap: cap must be positive");
    h->tap = buf;
    h->tap_cap = buf ? cap : 0;
    return DORY_OK;
}

static int slot_check(dory_t *h, int32_t seq, int32_t ord, int32_t slot, const SlotDesc **out) {
    if (!h) return DORY_EINVAL;
    if (seq < 0 || seq >= h->cfg.max_seqs || ord < 0 || ord >= h->n_ord || slot < 0 || slot >= kMaxLoops)
        return fail(h, DORY_EINVAL, "kv tap: seq, ordinal or slot out of range");
    if (h->seqs[seq].latched) return latched_error(h, "kv tap", seq);
    const SlotDesc &d = h->tab_host[(seq * h->n_ord + ord) * kMaxLoops + slot];
    if (!d.k && !d.kc) return fail(h, DORY_EINVAL, "kv tap: slot not in use");
    *out = &d;
    return DORY_OK;
}

int dory_kv_read(dory_t *h, int32_t seq, int32_t ord, int32_t slot, int64_t pos, void *host_out) {
    const SlotDesc *d = nullptr;
    int rc = slot_check(h, seq, ord, slot, &d);
    if (rc) return rc;
    if (!host_out) return fail(h, DORY_EINVAL, "dory_kv_read: null output");
    const int64_t held = h->seqs[seq].pos;
    if (pos < 0 || pos >= held || pos < held - d->cap) return fail(h, DORY_ERANGE, "dory_kv_read: row not held");
    HIPCHECK(h, hipSetDevice(h->device));
    SYNCCHECK(h, hipDeviceSynchronize());
    const size_t row = (size_t)(pos % d->cap);
    char *b = reinterpret_cast<char *>(host_out);
    const int hd = h->hd, nk = h->nk, ngk = h->ngk;
    for (int kh = 0; kh < nk; ++kh) {
        const size_t r = (size_t)kh * d->cap + row;
        if (!h->q8) {
            HIPCHECK(h, hipMemcpy(b + sizeof(float) * kh * hd, d->k + r * hd, sizeof(float) * hd, hipMemcpyDeviceToHost));
            HIPCHECK(h, hipMemcpy(b + sizeof(float) * (nk + kh) * hd, d->v + r * hd, sizeof(float) * hd,
                                  hipMemcpyDeviceToHost));
        } else {
            HIPCHECK(h, hipMemcpy(b + kh * hd, d->kc + r * hd, hd, hipMemcpyDeviceToHost));
            HIPCHECK(h, hipMemcpy(b + (nk + kh) * hd, d->vc + r * hd, hd, hipMemcpyDeviceToHost));
            HIPCHECK(h, hipMemcpy(b + 2 * nk * hd + sizeof(float) * kh * ngk, d->ks + r * ngk, sizeof(float) * ngk,
                                  hipMemcpyDeviceToHost));
            HIPCHECK(h, hipMemcpy(b + 2 * nk * hd + sizeof(float) * (nk * ngk + kh), d->vs + r, sizeof(float),
                                  hipMemcpyDeviceToHost));
        }
    }
    return DORY_OK;
}

int dory_kv_field(dory_t *h, int32_t seq, int32_t ord, int32_t slot, float *kcol, float *vcol) {
    const SlotDesc *d = nullptr;
    int rc = slot_check(h, seq, ord, slot, &d);
    if (rc) return rc;
    if (!h->q8) return fail(h, DORY_EINVAL, "dory_kv_field: the cache is not q8_2f");
    if (!h->seqs[seq].q8_frozen) return 0;
    HIPCHECK(h, hipSetDevice(h->device));
    SYNCCHECK(h, hipDeviceSynchronize());
    if (kcol) HIPCHECK(h, hipMemcpy(kcol, d->kcol, sizeof(float) * h->KV, hipMemcpyDeviceToHost));
    if (vcol) HIPCHECK(h, hipMemcpy(vcol, d->vcol, sizeof(float) * h->KV, hipMemcpyDeviceToHost));
    return 1;
}

int dory_kv_load(dory_t *h, int32_t seq, int32_t kv_mode, int32_t loops, int64_t npos, int32_t n_slot,
                 const float *k, const float *v) {
    if (!h) return DORY_EINVAL;
    if (seq < 0 || seq >= h->cfg.max_seqs) return fail(h, DORY_EINVAL, "dory_kv_load: seq out of range");
    if (kv_mode != DORY_PER_LOOP && kv_mode != DORY_LAST_LOOP) return fail(h, DORY_EINVAL, "dory_kv_load: kv_mode");
    if (loops < 1 || loops > DORY_MAX_LOOPS) return fail(h, DORY_EINVAL, "dory_kv_load: loops must be in 1..16");
    if (!k || !v || npos < 0 || npos > h->cfg.max_ctx || n_slot < 1 || n_slot > kMaxLoops)
        return fail(h, DORY_EINVAL, "dory_kv_load: bad rows");
    if (n_slot < (kv_mode == DORY_PER_LOOP ? loops : 1))
        return fail(h, DORY_EINVAL, "dory_kv_load: n_slot below the slots the mode uses");
    if (h->seqs[seq].latched) return latched_error(h, "dory_kv_load", seq);
    if (h->seqs[seq].pos != 0) return fail(h, DORY_ESTATE, "dory_kv_load: the sequence is not fresh");
    HIPCHECK(h, hipSetDevice(h->device));
    int rc = ensure_slots(h, seq, kv_mode, loops);
    if (rc) return rc;
    SYNCCHECK(h, hipDeviceSynchronize());
    const int chunk = std::min(h->cfg.max_chunk, std::min(h->cap_s, h->cap_f));
    const size_t row = h->KV;
    for (const LayerInfo &l : h->L) {
        if (!l.attn) continue;
        const int ns = (kv_mode == DORY_PER_LOOP && l.rec) ? loops : 1;
        for (int s = 0; s < ns; ++s) {
            const float *kb = k + ((size_t)(l.ord * n_slot + s) * npos) * row;
            const float *vb = v + ((size_t)(l.ord * n_slot + s) * npos) * row;
            bool froze = false;
            for (int64_t p0 = 0; p0 < npos; p0 += chunk) {
                const int T = (int)std::min<int64_t>(chunk, npos - p0);
                rc = put_record(h, h->sc.rec, chunk_rows(seq, p0, T, nullptr), nullptr, nullptr);
                if (rc) return rc;
                HIPCHECK(h, hipMemcpy(h->ld_k, kb + p0 * row, sizeof(float) * T * row, hipMemcpyHostToDevice));
                HIPCHECK(h, hipMemcpy(h->ld_v, vb + p0 * row, sizeof(float) * T * row, hipMemcpyHostToDevice));
                if (!h->q8) {
                    HIPCHECK(h, launch_kv_store(h->ld_k, h->ld_v, h->tab, h->n_ord, l.ord, s, h->nk, h->hd, T,
                                                h->sc.rec, nullptr));
                } else {
                    Q8WriteArgs wa{};
                    wa.ksrc = h->ld_k; wa.kld = h->KV; wa.vsrc = h->ld_v; wa.vld = h->KV;
                    wa.tab = h->tab; wa.n_ord = h->n_ord; wa.ord = l.ord; wa.slot = s; wa.nk = h->nk; wa.hd = h->hd;
                    wa.rec = h->sc.rec;
                    const bool frozen = froze || p0 >= kWarmup + 1;
                    if (frozen || p0 + T <= kWarmup) {
                        wa.r0 = 0; wa.r1 = T; wa.field = frozen;
                        HIPCHECK(h, launch_q8_write(wa, nullptr));
                    } else {
                        const int split = (int)(kWarmup - p0);
                        wa.r0 = 0; wa.r1 = split; wa.field = 0;
                        HIPCHECK(h, launch_q8_write(wa, nullptr));
                        HIPCHECK(h, launch_q8_freeze(h->tab, h->n_ord, l.ord, s, h->nk, h->hd, h->sc.rec, 0, nullptr));
                        wa.r0 = split; wa.r1 = T; wa.field = 1;
                        HIPCHECK(h, launch_q8_write(wa, nullptr));
                        froze = true;
                    }
                }
                SYNCCHECK(h, hipDeviceSynchronize());
            }
        }
    }
    SeqState &st = h->seqs[seq];
    st.pos = npos;
    st.mode = kv_mode;
    st.loops = kv_mode == DORY_PER_LOOP ? loops : 0;
    st.q8_frozen = h->q8 && npos > kWarmup;
    return DORY_OK;
}

int dory_stage_bench(dory_t *h, int32_t stage, int32_t reps, dory_stream_t stream) {
    if (!h) return DORY_EINVAL;
    if (stage < 0 || stage > 10 || reps < 1) return fail(h, DORY_EINVAL, "dory_stage_bench: stage 0..10, reps >= 1");
    if (h->last_T == 0) return fail(h, DORY_ESTATE, "dory_stage_bench: needs a forward call first");
    if (stage == 1 && h->last_chunk)
        return fail(h, DORY_ESTATE, "dory_stage_bench: decode attention needs a one-row or batch call last");
    if (stage == 10 && !h->last_chunk)
        return fail(h, DORY_ESTATE, "dory_stage_bench: chunk attention needs a multi-row call last");
    HIPCHECK(h, hipSetDevice(h->device));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool attn_stage = stage <= 2 || stage == 6 || stage == 7 || stage == 10;
    std::vector<const LayerInfo *> ls;
    for (const LayerInfo &l : h->L)
        if (attn_stage == l.attn) ls.push_back(&l);
    if (stage == 5) ls.assign(1, nullptr);
    if (ls.empty()) return fail(h, DORY_EINVAL, "dory_stage_bench: no sub-layer has this stage");
    const int ld = 2 * h->Q + 2 * h->KV;
    const int MC = h->cfg.max_chunk;
    for (int i = 0; i < reps; ++i) {
        const LayerInfo *l = ls[i % ls.size()];
        Resolve rs{};
        rs.h = h->sc.hb[0]; rs.o = h->sc.o; rs.alpha = h->L[0].w.alpha; rs.slerp = 1; rs.loop_op = kLoopNone;
        rs.inp = h->sc.inp; rs.h_out = nullptr; rs.tap_pass = -1;
        GemvArgs a{};
        a.rec = h->sc.rec; a.hidden = h->H; a.row = 0; a.rs = rs;
        AttnArgs aa{};
        if (stage == 1 || stage == 10) {
            aa.qp = h->sc.qp; aa.qkvg = h->sc.qkvg; aa.sg = l->w.sg; aa.z = h->sc.z; aa.part = h->sc.part;
            aa.tab = h->tab; aa.n_ord = h->n_ord; aa.ord = l->ord;
            aa.slot = slot_of(h, *l, h->last_mode, 0);
            aa.nh = h->nh; aa.nk = h->nk; aa.hd = h->hd;
            aa.window = l->sliding ? h->win_s : h->win_f;
            aa.rope = l->sliding ? h->rope_s : h->rope_f; aa.sq = l->w.sq; aa.no_write = 1;
            aa.q8 = h->q8; aa.rec = h->sc.rec;
        }
        hipError_t e = hipSuccess;
        switch (stage) {
        case 0:
            a.w[0] = l->w.wq; a.w[1] = l->w.wk; a.w[2] = l->w.wv; a.w[3] = l->w.wg;
            a.seg_end[0] = h->Q; a.seg_end[1] = h->Q + h->KV; a.seg_end[2] = h->Q + 2 * h->KV; a.seg_end[3] = ld;
            a.nseg = 4; a.N = ld; a.K = h->H; a.y = h->sc.qkvg;
            e = launch_gemv(h->wt, kProResolve, kEpiStore, a, s);
            break;
        case 1:
            aa.split = h->last_T == 1 ? (l->sliding ? h->split_ds : h->split_df) : (l->sliding ? h->split_bs : h->split_bf);
            aa.max_split = h->last_T == 1 ? (l->sliding ? h->ms_ds : h->ms_df) : (l->sliding ? h->ms_bs : h->ms_bf);
            if (h->last_T == 1) aa.sd1 = h->tab + ((size_t)h->last_seq0 * h->n_ord + l->ord) * kMaxLoops + aa.slot;
            if (h->last_T == 1 && l->sliding && h->xm && !h->xm_off) aa.xcnt = h->xcnt;
            if (h->last_T == 1 && !l->sliding && h->ext_df) {
                aa.max_split = 64;
                aa.ext = 1;
            }
            aa.field = -1;
            e = launch_attn_dec(aa, h->last_T, s);
            break;
        case 2:
            a.w[0] = l->w.wo; a.seg_end[0] = h->H; a.nseg = 1; a.N = h->H; a.K = h->Q; a.src = h->sc.z; a.y = h->sc.o;
            e = launch_gemv(h->wt, kProNorm, kEpiStore, a, s);
            break;
        case 3:
            a.w[0] = l->w.wgate; a.w[1] = l->w.wup; a.seg_end[0] = h->F; a.nseg = 1; a.N = h->F; a.K = h->H;
            a.y = h->sc.ga; a.sg = l->w.sg; a.su = l->w.su;
            e = launch_gemv(h->wt, kProResolve, kEpiPair, a, s);
            break;
        case 4:
            a.w[0] = l->w.wdown; a.seg_end[0] = h->H; a.nseg = 1; a.N = h->H; a.K = h->F; a.src = h->sc.ga; a.y = h->sc.o;
            e = launch_gemv(h->wt, kProNorm, kEpiStore, a, s);
            break;
        case 5:
            a.w[0] = h->w.head; a.seg_end[0] = h->V; a.nseg = 1; a.N = h->V; a.K = h->H;
            a.logit_scale = h->w.logit_scale;
            e = launch_gemv(h->wt, kProResolve, kEpiHead, a, s);
            break;
        case 6:
            e = launch_gemm(h->wt, h->sc.hb[0], h->sc.xb, h->H, qkvg_w(h, l->w), ld, h->H, h->sc.qkvg, ld, MC, s);
            break;
        case 7:
            e = launch_gemm(h->wt, h->sc.zn, h->sc.znb, h->Q, gemm_w(l->w.wo, h->H), h->H, h->Q, h->sc.o, h->H, MC, s,
                            gemm_pick_splits(h->wt, true, MC, h->H, h->Q), h->sc.o_stride);
            break;
        case 8:
            if (h->sc.ussp && gemm_swiglu_ok(h->wt, MC, h->F, h->H, h->H))
                e = launch_gemm_swiglu(h->sc.xb, h->H, l->w.wgate, l->w.wup, h->F, h->H, l->w.sg, l->w.su, h->sc.unb,
                                       h->sc.ussp, MC, s);
            else
                e = launch_gemm(h->wt, h->sc.hb[0], h->sc.xb, h->H, gateup_w(h, l->w), 2 * h->F, h->H, h->sc.ga, 2 * h->F, MC, s);
            break;
        case 9:
            e = launch_gemm(h->wt, h->sc.un, h->sc.unb, h->F, gemm_w(l->w.wdown, h->H), h->H, h->F, h->sc.o, h->H, MC, s,
                            gemm_pick_splits(h->wt, true, MC, h->H, h->F), h->sc.o_stride);
            break;
        default:
            chunk_split(h, h->last_pos0, h->last_T, aa);
            aa.field = h->q8 && h->last_pos0 >= kWarmup + 1;
            aa.pos0 = h->last_pos0;
            aa.nrows = h->last_T;
            aa.sdc = h->tab_host[((size_t)h->last_seq0 * h->n_ord + l->ord) * kMaxLoops + aa.slot];
            e = launch_attn(aa, h->last_T, s);
            break;
        }
        if (e != hipSuccess) return hip_fail(h, e, "dory_stage_bench");
    }
    return DORY_OK;
}

int dory_q8_encode_rows(const float *x, const float *col, int32_t rows, int32_t n, int32_t group, int8_t *codes,
                        float *scales, dory_stream_t stream) {
    if (!x || !codes || !scales || rows < 0 || n <= 0 || n > 256 || !(group == kKGroup || group >= n))
        return fail(nullptr, DORY_EINVAL, "dory_q8_encode_rows: bad arguments (n <= 256, group 32 or >= n)");
    hipError_t e = launch_q8_encode_rows(x, col, rows, n, group, codes, scales, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(nullptr, e, "dory_q8_encode_rows");
    return DORY_OK;
}

}  // extern "C"
