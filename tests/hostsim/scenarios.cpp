// scenarios.cpp -- drives the library's host runtime (api.hip, built for the
// CPU against fake_hip.cpp) through the call sequences of the benchmark
// workloads and of the error paths, at their real geometries and sizes.
// Every kernel launch is checked by the fake launchers (extents and the
// kernels' invariants); this program adds the checks of return codes and
// state.  Usage: hostsim <scenario>; prints one summary line and exits 0 when
// there is no violation and every expectation holds.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "dory.h"
#include "internal.h"

extern "C" {
void *fake_alloc(size_t bytes, const char *tag);
void fake_fail_launch_at(long n);
void fake_fail_sync_at(long n);
long fake_violations();
long fake_launches();
long fake_checks();
void fake_print_violations(FILE *f);
}

namespace {

int g_fail = 0;

void expect(bool ok, const char *what, dory_t *h = nullptr) {
    if (ok) return;
    ++g_fail;
    if (g_fail <= 20) fprintf(stderr, "  expectation failed: %s%s%s\n", what, h ? " -- " : "", h ? dory_last_error(h) : "");
}

struct Geo {
    int H, F, V, nh, nk, hd;
    std::string pattern;
    int n_in, n_rec, n_out, window, full_window;
    int wt, kv;
};

Geo g2b(bool q8 = false, int full_window = 0) {
    return Geo{2048, 5632, 32000, 16, 4, 128, "S-*-S-*-S-*-S-*-", 4, 8, 4, 1024, full_window, DORY_W_BF16,
               q8 ? DORY_KV_Q8_2F : DORY_KV_F32};
}
Geo gtiny(bool q8 = false) {
    return Geo{256, 688, 512, 16, 4, 16, "S-*-S-", 2, 2, 2, 64, 0, DORY_W_F32, q8 ? DORY_KV_Q8_2F : DORY_KV_F32};
}
Geo gpages() { return Geo{16, 16, 11, 4, 2, 8, "S-*-S-*-S-*-", 4, 4, 4, 5, 0, DORY_W_F32, DORY_KV_F32}; }

// A model over fake device weights, each matrix and vector its own allocation
// (so a read past one is caught).
struct Model {
    Geo g;
    dory_config cfg{};
    dory_weights w{};
    std::vector<dory_layer_weights> layers;
    dory_t *h = nullptr;
    float *logits = nullptr;   // [max(max_chunk, max_seqs)][V]
    int rows_cap = 0;

    Model(const Geo &geo, int max_ctx, int max_chunk, int max_seqs) : g(geo) {
        const size_t es = g.wt == DORY_W_BF16 ? 2 : 4;
        const int Q = g.nh * g.hd, KV = g.nk * g.hd;
        auto mat = [&](size_t r, size_t c, const char *t) { return fake_alloc(r * c * es, t); };
        auto vec = [&](size_t n, const char *t) { return (const float *)fake_alloc(n * 4, t); };
        for (size_t i = 0; i < g.pattern.size(); ++i) {
            dory_layer_weights l{};
            if (g.pattern[i] == '-') {
                l.wgate = mat(g.F, g.H, "wgate");
                l.wup = mat(g.F, g.H, "wup");
                l.wdown = mat(g.H, g.F, "wdown");
                l.sg = vec(g.F, "mlp sg");
                l.su = vec(g.F, "mlp su");
            } else {
                l.wq = mat(Q, g.H, "wq");
                l.wk = mat(KV, g.H, "wk");
                l.wv = mat(KV, g.H, "wv");
                l.wg = mat(Q, g.H, "wg");
                l.wo = mat(g.H, Q, "wo");
                l.sq = vec(Q, "sq");
                l.sg = vec(Q, "attn sg");
            }
            l.alpha = vec(g.H, "alpha");
            layers.push_back(l);
        }
        w.embed = mat(g.V, g.H, "embed");
        w.head = mat(g.V, g.H, "head");
        w.logit_scale = vec(g.V, "logit_scale");
        w.layers = layers.data();
        cfg = dory_config{g.H, g.F, g.V, g.nh, g.nk, g.hd, g.pattern.c_str(), g.n_in, g.n_rec, g.n_out, g.window,
                          g.full_window, 1e4, 1e7, max_ctx, max_chunk, max_seqs, g.kv, g.wt};
        const int rc = dory_create(&cfg, &w, &h);
        if (rc) {
            fprintf(stderr, "dory_create: %d %s\n", rc, dory_last_error(nullptr));
            exit(2);
        }
        rows_cap = max_chunk > max_seqs ? max_chunk : max_seqs;
        logits = (float *)fake_alloc((size_t)rows_cap * g.V * 4, "logits");
    }
    ~Model() { dory_destroy(h); }

    int chunk(int seq, int n, int loops, int mode, bool want, int tok0 = 0) {
        std::vector<int32_t> t(n);
        for (int i = 0; i < n; ++i) t[i] = (tok0 + 7 * i) % (g.V + 3);  // a few ids past the table
        return dory_forward_chunk(h, seq, t.data(), n, loops, mode, nullptr, want ? logits : nullptr);
    }
    int batch(const std::vector<int32_t> &seqs, const std::vector<int32_t> &loops, int mode, bool want) {
        std::vector<int32_t> t(seqs.size());
        for (size_t i = 0; i < t.size(); ++i) t[i] = (int32_t)(i * 13 % g.V);
        return dory_forward_batch(h, (int)seqs.size(), seqs.data(), t.data(), loops.data(), mode, nullptr,
                                  want ? logits : nullptr);
    }
};

uint32_t g_lcg = 12345;
int draw_loops() {
    g_lcg = g_lcg * 1664525u + 1013904223u;
    return 1 + (int)((g_lcg >> 16) % 16);
}

void stage_all(Model &m, std::initializer_list<int> stages) {
    for (int st : stages) expect(dory_stage_bench(m.h, st, 24, nullptr) == DORY_OK, "stage bench", m.h);
}

// ---- the benchmark workloads, at their sizes

void decode2b() {
    const int ctx = 4096, W = 16, K = 256;
    Model m(g2b(), ctx + W + K + 8, 512, 1);
    expect(dory_debug_xcd_merge(m.h, -1) == 1, "sliding layers merge their splits in the attention kernel", m.h);
    for (int c = 0; c < ctx; c += 512) expect(m.chunk(0, 512, 4, DORY_LAST_LOOP, c + 512 >= ctx, c) == 0, "prompt", m.h);
    for (int i = 0; i < W + K; ++i) expect(m.chunk(0, 1, 4, DORY_LAST_LOOP, true, i) == 0, "decode", m.h);
    stage_all(m, {0, 1, 2, 3, 4, 5});
    // the merge kernel for every layer, then back
    expect(dory_debug_xcd_merge(m.h, 0) == 0, "merge kernel selected", m.h);
    for (int i = 0; i < 4; ++i) expect(m.chunk(0, 1, 4, DORY_LAST_LOOP, true, i) == 0, "decode, merge kernel", m.h);
    stage_all(m, {1});
    expect(dory_debug_xcd_merge(m.h, 1) == 1, "in-kernel merge selected again", m.h);
    for (int i = 0; i < 4; ++i) expect(m.chunk(0, 1, 4, DORY_LAST_LOOP, true, i) == 0, "decode, in-kernel merge", m.h);
    expect(dory_debug_xcd_merge(m.h, 2) == DORY_EINVAL, "bad switch value", m.h);
}

void q8_2b() {
    const int ctx = 32768, W = 16, K = 64;
    Model m(g2b(true, 8192), ctx + W + K + 8, 512, 1);
    for (int c = 0; c < ctx; c += 512) expect(m.chunk(0, 512, 4, DORY_LAST_LOOP, c + 512 >= ctx, c) == 0, "prompt", m.h);
    for (int i = 0; i < W + K; ++i) expect(m.chunk(0, 1, 4, DORY_LAST_LOOP, true, i) == 0, "decode", m.h);
    stage_all(m, {0, 1, 2, 3, 4, 5});
}

void prefill2b() {
    const int n = 8192;
    Model m(g2b(), n + 8, 512, 1);
    for (int rep = 0; rep < 2; ++rep) {
        expect(dory_kv_reset(m.h, -1) == 0, "reset");
        for (int c = 0; c < n; c += 512) expect(m.chunk(0, 512, 8, DORY_PER_LOOP, c + 512 >= n, c) == 0, "prompt", m.h);
    }
    stage_all(m, {6, 7, 8, 9, 10});
}

// The batched workload: 64 sequences prefilled to 8192 in calls of 512 rows
// (the set-up whose counter run aborted in the runtime), then batched steps
// with a loop count per (sequence, step) in 1..16.
void batch2b() {
    const int nseq = 64, ctx = 8192, W = 4, K = 128;
    Model m(g2b(), ctx + W + K + 8, 512, nseq);
    for (int s = 0; s < nseq; ++s)
        for (int c = 0; c < ctx; c += 512) expect(m.chunk(s, 512, 4, DORY_LAST_LOOP, false, c + s) == 0, "prompt", m.h);
    std::vector<int32_t> seqs(nseq);
    for (int i = 0; i < nseq; ++i) seqs[i] = i;
    for (int step = 0; step < W + K; ++step) {
        std::vector<int32_t> loops(nseq);
        for (int &l : loops) l = draw_loops();
        expect(m.batch(seqs, loops, DORY_LAST_LOOP, true) == 0, "batch step", m.h);
    }
    stage_all(m, {1});
}

void gate2b() {
    const int ctx = 1024;
    Model m(g2b(), ctx + 200, 512, 1);
    for (int c = 0; c < ctx; c += 512) expect(m.chunk(0, 512, 4, DORY_LAST_LOOP, false, c) == 0, "prompt", m.h);
    expect(dory_set_gate(m.h, 1, 0.7f) == 0, "gate on", m.h);
    for (int i = 0; i < 80; ++i) expect(m.chunk(0, 1, 4, DORY_LAST_LOOP, true, i) == 0, "gated decode", m.h);
    expect(dory_set_gate(m.h, 0, 0.f) == 0, "gate off", m.h);
}

// ---- call shapes around the dispatch edges, both modes, every entry point

void shapes(const Geo &g, int max_ctx, int max_chunk, int max_seqs) {
    Model m(g, max_ctx, max_chunk, max_seqs);
    const int sizes[] = {1, 16, 17, 33, 64, 65, 100, 128, max_chunk};
    for (int mode : {DORY_LAST_LOOP, DORY_PER_LOOP}) {
        for (int loops : {1, 3, 16}) {
            expect(dory_kv_reset(m.h, -1) == 0, "reset");
            int64_t pos = 0;
            for (int n : sizes) {
                if (n > max_chunk || pos + n > max_ctx) continue;
                expect(m.chunk(0, n, loops, mode, true, (int)pos) == 0, "chunk", m.h);
                pos += n;
            }
            for (int i = 0; i < 3 && pos < max_ctx; ++i, ++pos) expect(m.chunk(0, 1, loops, mode, true) == 0, "one row", m.h);
            if (pos + 40 <= max_ctx) {
                expect(dory_forward_chunk_all(m.h, 0, std::vector<int32_t>(40, 3).data(), 40, loops, mode, nullptr,
                                              m.logits) == 0, "want all", m.h);
                pos += 40;
            }
            if (mode == DORY_LAST_LOOP) {
                expect(dory_rollback(m.h, 0, pos - 20) == 0, "rollback", m.h);
                expect(m.chunk(0, 20, loops, mode, false) == 0, "after rollback", m.h);
            }
        }
    }
    // batches: every sequence a few rows in, then steps over subsets
    if (max_seqs > 1) {
        for (int mode : {DORY_LAST_LOOP, DORY_PER_LOOP}) {
            expect(dory_kv_reset(m.h, -1) == 0, "reset");
            std::vector<int32_t> seqs, loops;
            for (int s = 0; s < max_seqs; ++s) {
                const int L = mode == DORY_PER_LOOP ? 2 : 1 + s % 16;
                expect(m.chunk(s, 1 + s % 5, L, mode, false) == 0, "batch set-up", m.h);
                seqs.push_back(s);
                loops.push_back(mode == DORY_PER_LOOP ? 2 : draw_loops());
            }
            for (int step = 0; step < 6; ++step) {
                expect(m.batch(seqs, loops, mode, step % 2 == 0) == 0, "batch", m.h);
                if (mode == DORY_LAST_LOOP)
                    for (int32_t &l : loops) l = draw_loops();
            }
            std::vector<int32_t> sub(seqs.rbegin(), seqs.rend()), sl(loops.rbegin(), loops.rend());
            sub.resize(sub.size() / 2 + 1);
            sl.resize(sub.size());
            expect(m.batch(sub, sl, mode, true) == 0, "batch subset", m.h);
        }
        expect(dory_set_prompt_loops(m.h, 1) == 0, "prompt loops");
        expect(dory_kv_reset(m.h, -1) == 0, "reset");
        expect(m.chunk(0, 30, 5, DORY_LAST_LOOP, false) == 0, "prompt loops chunk", m.h);
        expect(dory_set_prompt_loops(m.h, 0) == 0, "prompt loops off");
    }
}

void tiny() { shapes(gtiny(), 512, 128, 8); }
void tiny_q8() { shapes(gtiny(true), 512, 128, 8); }
void pages() { shapes(gpages(), 200, 64, 4); }
void shapes2b() { shapes(g2b(), 3000, 512, 4); }
void shapes2b_q8() { shapes(g2b(true, 1500), 3000, 512, 4); }

// ---- the latch

// A sequence latches when a call on it fails after its first device work;
// others do not.  Then every call on it is DORY_ESTATE until it is reset.
void latch_case(Model &m, int fail_at, bool hook, int kind) {
    expect(dory_kv_reset(m.h, -1) == 0, "reset");
    expect(m.chunk(0, 20, 2, DORY_LAST_LOOP, false) == 0, "set-up 0", m.h);
    expect(m.chunk(1, 20, 2, DORY_LAST_LOOP, false) == 0, "set-up 1", m.h);
    expect(m.chunk(0, 1, 2, DORY_LAST_LOOP, true) == 0, "a one-row call (its graph captured)", m.h);
    const int64_t p0 = dory_position(m.h, 0), p1 = dory_position(m.h, 1);
    if (hook) expect(dory_debug_fail_launch(m.h, fail_at) == 0, "hook");
    else fake_fail_launch_at(fail_at);
    int rc;
    if (kind == 0) rc = m.chunk(0, 9, 2, DORY_LAST_LOOP, true);                  // multi-row, no graph
    else if (kind == 1) rc = m.chunk(0, 1, 2, DORY_LAST_LOOP, true);             // graph replay
    else if (kind == 2) rc = m.chunk(0, 1, 5, DORY_LAST_LOOP, true);             // graph capture
    else rc = m.batch({0, 1}, {2, 3}, DORY_LAST_LOOP, true);                      // batch
    dory_debug_fail_launch(m.h, 0);
    fake_fail_launch_at(0);
    expect(rc == DORY_EDEVICE, "the failed call reports DORY_EDEVICE", m.h);
    expect(dory_latched(m.h, 0) == 1, "its sequence latched");
    expect(dory_latched(m.h, 1) == (kind == 3 ? 1 : 0), "the other sequence latched only if in the batch");
    expect(dory_position(m.h, 0) == p0 && dory_position(m.h, 1) == p1, "positions unchanged");
    expect(m.chunk(0, 1, 2, DORY_LAST_LOOP, true) == DORY_ESTATE, "a later call is DORY_ESTATE", m.h);
    expect(m.batch({1, 0}, {1, 1}, DORY_LAST_LOOP, false) == DORY_ESTATE, "a batch with it is DORY_ESTATE", m.h);
    expect(dory_rollback(m.h, 0, 3) == DORY_ESTATE, "rollback is DORY_ESTATE", m.h);
    if (kind != 3) expect(m.chunk(1, 2, 2, DORY_LAST_LOOP, true) == 0, "the other sequence goes on", m.h);
    expect(dory_kv_reset(m.h, 0) == 0, "reset clears");
    expect(dory_latched(m.h, 0) == 0, "not latched after reset");
    expect(m.chunk(0, 5, 2, DORY_LAST_LOOP, true) == 0, "a call after the reset", m.h);
}

void latch() {
    Model m(gtiny(), 256, 32, 2);
    // (a graph replay is one launch)
    for (int kind = 0; kind < 4; ++kind)
        for (int at : {1, 2, 5, 17})
            for (bool hook : {true, false})
                if (kind != 1 || at == 1) latch_case(m, at, hook, kind);
    // a device error seen at a synchronisation: every sequence latches
    expect(dory_kv_reset(m.h, -1) == 0, "reset");
    expect(m.chunk(0, 3, 2, DORY_LAST_LOOP, false) == 0, "set-up", m.h);
    fake_fail_sync_at(1);
    const std::vector<float> buf(2 * 4 * 16);
    const int rc = dory_kv_read(m.h, 0, 0, 0, 1, (void *)buf.data());
    fake_fail_sync_at(0);
    expect(rc == DORY_EDEVICE, "the synchronisation's error is reported", m.h);
    expect(dory_latched(m.h, 0) == 1 && dory_latched(m.h, 1) == 1, "every sequence latched");
    expect(dory_kv_reset(m.h, -1) == 0 && dory_latched(m.h, 1) == 0, "reset of all clears");
    // failed argument checks and failures before device work latch nothing
    expect(m.chunk(0, 1, 17, DORY_LAST_LOOP, true) == DORY_EINVAL, "bad loops");
    expect(m.chunk(0, 40, 2, DORY_LAST_LOOP, true) == DORY_ERANGE, "too many rows");
    expect(dory_latched(m.h, 0) == 0, "no latch after argument errors");
    // the q8 cache: a failure after the freeze was enqueued latches, and the
    // reset starts the sequence over (the freeze runs again at position 64)
    Model q(gtiny(true), 256, 128, 1);
    expect(q.chunk(0, 60, 2, DORY_LAST_LOOP, false) == 0, "q8 set-up", q.h);
    expect(dory_debug_fail_launch(q.h, 12) == 0, "hook");
    expect(q.chunk(0, 10, 2, DORY_LAST_LOOP, true) == DORY_EDEVICE, "q8 call across the freeze fails", q.h);
    expect(dory_latched(q.h, 0) == 1, "q8 sequence latched");
    expect(dory_kv_reset(q.h, 0) == 0, "q8 reset");
    expect(q.chunk(0, 70, 2, DORY_LAST_LOOP, true) == 0, "q8 after the reset", q.h);
}

// The checker itself: launches whose extents run past their buffers, and a
// chunk attention whose ring cannot hold its window, must be reported.
void selftest() {
    float *a = (float *)fake_alloc(4 * 100 * 4, "a"), *b = (float *)fake_alloc(4 * 100 * 4, "b");
    float *vec = (float *)fake_alloc(100 * 4, "vec");
    uint16_t *zb = (uint16_t *)fake_alloc(4 * 100 * 2, "zb");
    long v0 = fake_violations();
    dk::launch_swiglu_norm(a, b, 100, vec, vec, nullptr, zb, 100, 4, nullptr, nullptr);
    expect(fake_violations() == v0, "a launch inside its buffers passes");
    dk::launch_swiglu_norm(a, b, 100, vec, vec, nullptr, zb, 100, 5, nullptr, nullptr);
    expect(fake_violations() > v0, "five rows over buffers of four are caught");
    v0 = fake_violations();
    dk::launch_swiglu_norm(a, b, 100, vec, vec, nullptr, zb, 100, 4, nullptr, vec + 98);
    expect(fake_violations() > v0, "sums of squares past their buffer are caught");
    v0 = fake_violations();
    float *c = (float *)fake_alloc(4 * 65 * 4, "c"), *w = (float *)fake_alloc(64 * 100 * 4, "w");
    dk::launch_gemm(dk::kF32, a, nullptr, 100, dk::gemm_w(w, 64), 64, 100, c, 64, 4, nullptr);
    expect(fake_violations() == v0, "a GEMM inside its buffers passes");
    dk::launch_gemm(dk::kF32, a, nullptr, 100, dk::gemm_w(w, 65), 65, 100, c, 65, 4, nullptr);
    expect(fake_violations() > v0, "a GEMM reading a weight row too many is caught");
    // the in-kernel merge's partials: its layout needs more than the plain one
    {
        dk::AttnArgs aa{};
        // (15 splits: 15 slabs of 520 floats end off a 32-float line)
        aa.nh = 16; aa.nk = 4; aa.hd = 128; aa.split = 64; aa.max_split = 15; aa.window = 960;
        const size_t Q = 16 * 128, KV = 4 * 128, plain = (size_t)4 * 15 * 4 * 130;
        aa.sg = (float *)fake_alloc(Q * 4, "sg"); aa.z = (float *)fake_alloc(Q * 4, "z");
        aa.sq = (float *)fake_alloc(Q * 4, "sq");
        aa.qkvg = (float *)fake_alloc((2 * Q + 2 * KV) * 4, "qkvg");
        aa.xcnt = (uint32_t *)fake_alloc(32 * 16 * 4, "xcnt");
        aa.rec = (dk::CallRec *)fake_alloc(dk::rec_bytes(1), "rec");
        // the same launch over a buffer of the in-kernel layout's size, then a
        // plain-sized one: only the second adds a violation
        aa.part = (float *)fake_alloc(dk::attn_xm_part_floats(4, 15, 4, 128) * 4, "part");
        v0 = fake_violations();
        dk::launch_attn_dec(aa, 1, nullptr);
        const long d1 = fake_violations() - v0;
        aa.part = (float *)fake_alloc(plain * 4, "part (plain size)");
        v0 = fake_violations();
        dk::launch_attn_dec(aa, 1, nullptr);
        expect(fake_violations() - v0 > d1, "in-kernel merge partials past a plain-sized buffer are caught");
    }
    printf("selftest: %ld violations reported, as planted\n", fake_violations());
}

// The no-allocation variant: short calls of both modes over the static array,
// interleaved with ordinary calls on another sequence, every extent inside it.
void noalloc_case(const Geo &g, int max_ctx) {
    Model m(g, max_ctx, 64, 2);
    std::vector<int32_t> t(8, 5);
    for (int mode : {DORY_LAST_LOOP, DORY_PER_LOOP}) {
        expect(dory_kv_reset(m.h, -1) == 0, "reset");
        expect(m.chunk(0, 8, 3, mode, true) == 0, "an ordinary call creates the slots", m.h);
        for (int n : {8, 3, 1, 1, 7}) {
            expect(dory_forward_chunk_noalloc(m.h, 0, t.data(), n, 3, mode, nullptr, m.logits) == 0, "noalloc", m.h);
            expect(m.chunk(1, n, 3, mode, true) == 0, "ordinary call between", m.h);
        }
        expect(dory_forward_chunk_noalloc(m.h, 0, t.data(), 9, 3, mode, nullptr, m.logits) == DORY_ERANGE, "9 rows");
        expect(dory_forward_chunk_noalloc(m.h, 0, t.data(), 2, 3, mode, nullptr, m.logits) == 0, "noalloc", m.h);
        expect(dory_stage_bench(m.h, 0, 2, nullptr) == DORY_ESTATE, "the stage benchmark needs an ordinary call");
    }
    expect(dory_kv_reset(m.h, -1) == 0, "reset");
    expect(m.chunk(0, 4, 2, DORY_PER_LOOP, true) == 0, "per_loop at loops 2", m.h);
    expect(dory_kv_reset(m.h, 0) == 0, "reset");
    expect(dory_forward_chunk_noalloc(m.h, 0, t.data(), 2, 5, DORY_PER_LOOP, nullptr, m.logits) == DORY_ESTATE,
           "per_loop slots that do not exist yet", m.h);
}
// The kv tap, sized exactly for each call: every writer stays inside it.
void kvtap_case(const Geo &g) {
    Model m(g, 600, 128, 3);
    const int KV = g.nk * g.hd;
    auto attn_passes = [&](int loops) {
        int n = 0;
        for (int i = 0; i < (int)g.pattern.size(); ++i)
            if (g.pattern[i] != '-') n += (i >= g.n_in && i < g.n_in + g.n_rec) ? loops : 1;
        return n;
    };
    for (int mode : {DORY_LAST_LOOP, DORY_PER_LOOP}) {
        expect(dory_kv_reset(m.h, -1) == 0, "reset");
        for (int n : {100, 1, 1, 33}) {
            const size_t cap = (size_t)attn_passes(3) * n * 2 * KV;
            float *buf = (float *)fake_alloc(cap * 4, "kv tap");
            expect(dory_debug_kv_tap(m.h, buf, (int64_t)cap) == 0, "kv tap", m.h);
            expect(m.chunk(0, n, 3, mode, true) == 0, "tapped call", m.h);
            expect(dory_debug_kv_tap(m.h, buf, (int64_t)cap - 1) == 0, "kv tap", m.h);
            expect(m.chunk(0, n, 3, mode, true) == DORY_EINVAL, "a tap one float short", m.h);
        }
        for (int s = 1; s < 3; ++s) expect(m.chunk(s, 5, 3, mode, false) == 0, "set-up", m.h);
        const size_t cap = (size_t)attn_passes(3) * 3 * 2 * KV;
        float *buf = (float *)fake_alloc(cap * 4, "kv tap");
        expect(dory_debug_kv_tap(m.h, buf, (int64_t)cap) == 0, "kv tap", m.h);
        expect(m.batch({0, 1, 2}, {3, 3, 3}, mode, true) == 0, "tapped batch", m.h);
        if (mode == DORY_LAST_LOOP) expect(m.batch({2, 0, 1}, {1, 3, 2}, mode, true) == 0, "tapped batch", m.h);
        expect(dory_debug_kv_tap(m.h, nullptr, 0) == 0, "kv tap off", m.h);
    }
}
void kvtap() {
    kvtap_case(gtiny());
    kvtap_case(gtiny(true));
    kvtap_case(g2b(true, 300));
}

void noalloc() {
    noalloc_case(gtiny(), 512);
    noalloc_case(gtiny(true), 512);
    noalloc_case(g2b(), 4400);
    noalloc_case(g2b(true, 8192), 40000);
}

struct Entry {
    const char *name;
    void (*fn)();
};
const Entry kScenarios[] = {
    {"decode2b", decode2b}, {"q8_2b", q8_2b}, {"prefill2b", prefill2b}, {"batch2b", batch2b},
    {"gate2b", gate2b},     {"tiny", tiny},   {"tiny_q8", tiny_q8},     {"pages", pages},
    {"shapes2b", shapes2b}, {"shapes2b_q8", shapes2b_q8}, {"latch", latch}, {"noalloc", noalloc}, {"kvtap", kvtap},
};

}  // namespace

int main(int argc, char **argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: hostsim <scenario>\n");
        return 2;
    }
    if (!strcmp(argv[1], "selftest")) {
        selftest();
        return g_fail ? 1 : 0;
    }
    for (const Entry &e : kScenarios) {
        if (strcmp(e.name, argv[1])) continue;
        e.fn();
        const long v = fake_violations();
        printf("scenario %s: launches %ld, checks %ld, violations %ld, failed expectations %d\n", e.name,
               fake_launches(), fake_checks(), v, g_fail);
        fake_print_violations(stdout);
        return v || g_fail ? 1 : 0;
    }
    fprintf(stderr, "unknown scenario %s\n", argv[1]);
    return 2;
}
