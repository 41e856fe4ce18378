// fake_hip.cpp -- a CPU stand-in for the HIP runtime and for the kernel
// launchers of libdory.so, so that the library's host runtime (api.hip, built
// with g++ and the sanitizers) runs without a GPU.
//
// "Device" memory is anonymous mmap (untouched pages cost nothing, so the
// Dory-2B geometry fits), kept in a registry of allocations.  No kernel runs:
// each launcher instead checks the extents its kernel reads and writes, as the
// kernel's indexing defines them, against the registry -- every range must lie
// inside one allocation -- plus the invariants the kernels rely on (a ring
// holds every key a row reads, the split grid covers every key, a captured
// graph's slot belongs to the record's sequence).  Checks that depend on the
// per-call record (positions, sequences, logits rows) are kept with a captured
// graph and run again on every replay.  Violations are counted and the first
// few are kept as messages.
//
// Test infrastructure only: nothing in the library links this file.
#include <hip/hip_runtime_api.h>
#include <sys/mman.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <string>
#include <vector>

#include "internal.h"

using namespace dk;

namespace fake {

struct Alloc {
    size_t bytes;
    std::string tag;
    bool mapped;  // mmap (device and pinned host memory); false: registered only
};
std::map<uintptr_t, Alloc> allocs;
std::vector<std::string> msgs;
long violations = 0, launches = 0, syncs = 0, checks = 0;
long fail_launch_at = 0, fail_sync_at = 0;
const char *cur = "";

struct Graph {
    std::vector<std::function<void()>> dyn;  // record-dependent checks, rerun per replay
};
Graph *capturing = nullptr;

void violation(const std::string &m) {
    ++violations;
    if (msgs.size() < 20) msgs.push_back(std::string(cur) + ": " + m);
}

const Alloc *find(const void *p, uintptr_t *base) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    auto it = allocs.upper_bound(a);
    if (it == allocs.begin()) return nullptr;
    --it;
    if (a >= it->first + it->second.bytes) return nullptr;
    *base = it->first;
    return &it->second;
}

// [p, p + n) must lie inside one allocation.
void need(const char *what, const void *p, size_t n) {
    ++checks;
    if (n == 0) return;
    if (!p) {
        violation(std::string(what) + ": null pointer for " + std::to_string(n) + " bytes");
        return;
    }
    uintptr_t base = 0;
    const Alloc *a = find(p, &base);
    if (!a) {
        char b[160];
        snprintf(b, sizeof b, "%s: %p (+%zu bytes) is in no allocation", what, p, n);
        violation(b);
        return;
    }
    const size_t off = reinterpret_cast<uintptr_t>(p) - base;
    if (off + n > a->bytes) {
        char b[200];
        snprintf(b, sizeof b, "%s: bytes [%zu, %zu) of '%s' (%zu bytes)", what, off, off + n, a->tag.c_str(),
                 a->bytes);
        violation(b);
    }
}

void *map_bytes(size_t bytes) {
    const size_t len = (bytes + 4095) / 4096 * 4096;
    void *p = mmap(nullptr, len ? len : 4096, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE,
                   -1, 0);
    return p == MAP_FAILED ? nullptr : p;
}

void *alloc(size_t bytes, const char *tag) {
    void *p = map_bytes(bytes);
    if (p) allocs[reinterpret_cast<uintptr_t>(p)] = Alloc{bytes ? bytes : 1, tag, true};
    return p;
}

bool release(void *p) {
    auto it = allocs.find(reinterpret_cast<uintptr_t>(p));
    if (it == allocs.end()) return false;
    if (it->second.mapped) munmap(p, (it->second.bytes + 4095) / 4096 * 4096);
    allocs.erase(it);
    return true;
}

// A launch: args-only checks now; record-dependent checks now and, inside a
// capture, again at every replay of the graph.
hipError_t launch(const char *name, const std::function<void()> &stat, const std::function<void()> &dyn) {
    ++launches;
    if (fail_launch_at && launches == fail_launch_at) return hipErrorLaunchFailure;
    cur = name;
    stat();
    if (dyn) {
        dyn();
        if (capturing)
            capturing->dyn.push_back([name, dyn]() {
                cur = name;
                dyn();
            });
    }
    return hipSuccess;
}

hipError_t sync_point() {
    ++syncs;
    if (fail_sync_at && syncs == fail_sync_at) return hipErrorIllegalAddress;
    return hipSuccess;
}

// ---- the record and the slot table, as the kernels read them

void need_record(const CallRec *rec, int rows) {
    need("call record", rec, sizeof(CallRec));
    if (!rec) return;
    need("call record rows", rec, rec_bytes(rows < 1 ? 1 : rows));
    if (rec->n < rows) violation("the record holds " + std::to_string(rec->n) + " rows, the kernel reads " +
                                 std::to_string(rows));
}

// The slot of (seq, ord, slot), checked: in the table, in use, its rings whole.
const SlotDesc *slot(const SlotDesc *tab, int seq, int n_ord, int ord, int sl, int nk, int hd, bool q8) {
    if (seq < 0 || ord < 0 || ord >= n_ord || sl < 0 || sl >= kMaxLoops) {
        violation("slot index out of range: seq " + std::to_string(seq) + " ord " + std::to_string(ord) + " slot " +
                  std::to_string(sl));
        return nullptr;
    }
    const SlotDesc *d = &slot_at(tab, seq, n_ord, ord, sl);
    need("slot table entry", d, sizeof(SlotDesc));
    if (!q8 && !d->k) {
        violation("fp32 slot not allocated: seq " + std::to_string(seq) + " ord " + std::to_string(ord) + " slot " +
                  std::to_string(sl));
        return nullptr;
    }
    if (q8 && !d->kc) {
        violation("q8 slot not allocated: seq " + std::to_string(seq) + " ord " + std::to_string(ord));
        return nullptr;
    }
    const size_t rows = (size_t)nk * d->cap, ngk = (hd + kKGroup - 1) / kKGroup;
    if (d->cap <= 0) violation("slot with capacity " + std::to_string(d->cap));
    if (q8) {
        need("ring K codes", d->kc, rows * hd);
        need("ring V codes", d->vc, rows * hd);
        need("ring K scales", d->ks, rows * ngk * 4);
        need("ring V scales", d->vs, rows * 4);
        need("K field", d->kcol, (size_t)nk * hd * 4);
        need("V field", d->vcol, (size_t)nk * hd * 4);
    } else {
        need("ring K", d->k, rows * hd * 4);
        need("ring V", d->v, rows * hd * 4);
    }
    return d;
}

// A row reading keys lo ..= p after the call wrote positions up to hi into the
// ring: the oldest key must not have been overwritten.
void keys_held(const SlotDesc *d, int64_t lo, int64_t p, int64_t hi) {
    if (!d) return;
    if (lo < 0 || lo > p) violation("key range [" + std::to_string(lo) + ", " + std::to_string(p) + "]");
    if (hi - lo >= d->cap)
        violation("ring of " + std::to_string(d->cap) + " rows cannot hold keys from " + std::to_string(lo) +
                  " while position " + std::to_string(hi) + " is written");
}

size_t esz(int wt) { return wt == kBF16 ? 2 : 4; }

// Weight rows of a stacked GEMM operand: rows [0, seg rows) of each segment.
void need_segments(const char *what, const void *const w[4], const int32_t seg_end[4], int nseg, int K, int wt) {
    int start = 0;
    for (int i = 0; i < nseg; ++i) {
        need(what, w[i], (size_t)(seg_end[i] - start) * K * esz(wt));
        start = seg_end[i];
    }
}

// The writes and reads of resolve_regs / resolve_row for row r of width H (the
// writer's stores; inputs are checked by the caller).
void resolve_writes(const Resolve &rs, int r, int H, const CallRec *rec, bool regs) {
    const size_t row = (size_t)r * H;
    if (rs.loop_op == kLoopExit && r >= rs.n_prev) {
        if (rs.h_out) need("h_out", rs.h_out + row, H * 4);
        if (rs.hb_out) need("hb_out", rs.hb_out + row, H * 2);
        return;
    }
    if (rec && rec->tap && rs.tap_pass >= 0) need("tap", rec->tap + ((size_t)rs.tap_pass * rec->n + r) * H, H * 4);
    if (rs.loop_op == kLoopEnter) need("loop input (written)", rs.inp + row, H * 4);
    if (rs.loop_op == kLoopExit && rs.e_out && regs) need("e_out", rs.e_out + row, H * 4);
    if (rs.loop_op == kLoopNext) {
        if (rs.st) need("loop state", rs.st + row, H * 4);
        if (r >= rs.n_next) return;
        need("loop input (read)", rs.inp + row, H * 4);
    }
    if (rs.h_out) need("h_out", rs.h_out + row, H * 4);
    if (rs.hb_out) need("hb_out", rs.hb_out + row, H * 2);
}

}  // namespace fake

using fake::esz;
using fake::need;

// ====================================================================== HIP API

extern "C" {

hipError_t hipMalloc(void **ptr, size_t size) {
    *ptr = fake::alloc(size, "device");
    return *ptr ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void *ptr) {
    if (!ptr) return hipSuccess;
    return fake::release(ptr) ? hipSuccess : hipErrorInvalidValue;
}
hipError_t hipHostMalloc(void **ptr, size_t size, unsigned int flags) {
    *ptr = fake::alloc(size, "pinned host");
    return *ptr ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipHostFree(void *ptr) { return fake::release(ptr) ? hipSuccess : hipErrorInvalidValue; }

static hipError_t copy(void *dst, const void *src, size_t n, hipMemcpyKind kind) {
    fake::cur = "hipMemcpy";
    // device sides must be allocations; host sides are the caller's memory
    if (kind == hipMemcpyHostToDevice || kind == hipMemcpyDeviceToDevice) need("copy destination", dst, n);
    if (kind == hipMemcpyDeviceToHost || kind == hipMemcpyDeviceToDevice) need("copy source", src, n);
    if (n) memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipMemcpy(void *dst, const void *src, size_t sizeBytes, hipMemcpyKind kind) {
    return copy(dst, src, sizeBytes, kind);
}
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t sizeBytes, hipMemcpyKind kind, hipStream_t stream) {
    return copy(dst, src, sizeBytes, kind);
}
hipError_t hipMemset(void *dst, int value, size_t sizeBytes) {
    fake::cur = "hipMemset";
    need("memset", dst, sizeBytes);
    memset(dst, value, sizeBytes);
    return hipSuccess;
}

hipError_t hipEventCreateWithFlags(hipEvent_t *event, unsigned flags) {
    *event = reinterpret_cast<hipEvent_t>(new char[8]);
    return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t event) {
    delete[] reinterpret_cast<char *>(event);
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t event) { return fake::sync_point(); }
hipError_t hipStreamCreateWithFlags(hipStream_t *stream, unsigned int flags) {
    *stream = reinterpret_cast<hipStream_t>(new char[8]);
    return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t stream) {
    delete[] reinterpret_cast<char *>(stream);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t stream) { return fake::sync_point(); }
hipError_t hipDeviceSynchronize(void) { return fake::sync_point(); }
hipError_t hipGetDevice(int *deviceId) {
    *deviceId = 0;
    return hipSuccess;
}
hipError_t hipSetDevice(int deviceId) { return deviceId == 0 ? hipSuccess : hipErrorInvalidDevice; }
const char *hipGetErrorString(hipError_t e) {
    switch (e) {
        case hipSuccess: return "no error";
        case hipErrorOutOfMemory: return "out of memory";
        case hipErrorInvalidValue: return "invalid argument";
        case hipErrorLaunchFailure: return "unspecified launch failure";
        case hipErrorIllegalAddress: return "an illegal memory access was encountered";
        default: return "hip error";
    }
}

hipError_t hipStreamBeginCapture(hipStream_t stream, hipStreamCaptureMode mode) {
    if (fake::capturing) return hipErrorIllegalState;
    fake::capturing = new fake::Graph();
    return hipSuccess;
}
hipError_t hipStreamEndCapture(hipStream_t stream, hipGraph_t *pGraph) {
    if (!fake::capturing) return hipErrorIllegalState;
    *pGraph = reinterpret_cast<hipGraph_t>(fake::capturing);
    fake::capturing = nullptr;
    return hipSuccess;
}
hipError_t hipGraphInstantiate(hipGraphExec_t *pGraphExec, hipGraph_t graph, hipGraphNode_t *pErrorNode,
                               char *pLogBuffer, size_t bufferSize) {
    *pGraphExec = reinterpret_cast<hipGraphExec_t>(new fake::Graph(*reinterpret_cast<fake::Graph *>(graph)));
    return hipSuccess;
}
hipError_t hipGraphDestroy(hipGraph_t graph) {
    delete reinterpret_cast<fake::Graph *>(graph);
    return hipSuccess;
}
hipError_t hipGraphExecDestroy(hipGraphExec_t graphExec) {
    delete reinterpret_cast<fake::Graph *>(graphExec);
    return hipSuccess;
}
hipError_t hipGraphLaunch(hipGraphExec_t graphExec, hipStream_t stream) {
    ++fake::launches;
    if (fake::fail_launch_at && fake::launches == fake::fail_launch_at) return hipErrorLaunchFailure;
    for (auto &f : reinterpret_cast<fake::Graph *>(graphExec)->dyn) f();
    return hipSuccess;
}

// ---- controls for the scenario driver
void *fake_alloc(size_t bytes, const char *tag) { return fake::alloc(bytes, tag); }
void fake_fail_launch_at(long n) { fake::fail_launch_at = n ? fake::launches + n : 0; }
void fake_fail_sync_at(long n) { fake::fail_sync_at = n ? fake::syncs + n : 0; }
long fake_violations() { return fake::violations; }
long fake_launches() { return fake::launches; }
long fake_checks() { return fake::checks; }
void fake_print_violations(FILE *f) {
    for (const std::string &m : fake::msgs) fprintf(f, "  violation: %s\n", m.c_str());
}

}  // extern "C"

// ====================================================================== launchers

namespace dk {

hipError_t noalloc_scratch(void **ptr) {
    static void *p = fake::alloc(kNoAllocBytes, "static scratch");
    *ptr = p;
    return p ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t launch_gemv(int wt, int pro, int epi, const GemvArgs &a, hipStream_t s) {
    if (a.K <= 0 || a.K > 8192 || a.K % 8 || a.N <= 0) return hipErrorInvalidValue;
    if (pro == kProEmbed && (!a.embed || a.vocab <= 0)) return hipErrorInvalidValue;
    const bool res = pro == kProResolve || pro == kProResolveInp || pro == kProEmbed;
    const bool ok = (res && (epi == kEpiStore || epi == kEpiPair || (epi == kEpiHead && pro == kProResolve))) ||
                    (pro == kProNorm && epi == kEpiStore) || (pro == kProPlain && epi == kEpiHead);
    if (!ok) return hipErrorInvalidValue;
    const int K = a.K, N = a.N;
    const int ROWS = N >= 16 * 1024 ? 16 : N >= 8 * 512 ? 8 : 4;
    auto stat = [=]() {
        // every workgroup of ROWS rows reads them from the segment its first row
        // lies in: a workgroup across a segment boundary reads past that segment
        if (epi == kEpiPair) {
            need("gemv gate rows", a.w[0], (size_t)N * K * esz(wt));
            need("gemv up rows", a.w[1], (size_t)N * K * esz(wt));
            need("gemv sg", a.sg, (size_t)N * 4);
            need("gemv su", a.su, (size_t)N * 4);
            need("gemv y", a.y, (size_t)N * 4);
        } else {
            int maxrow[4] = {-1, -1, -1, -1};
            for (int row0 = 0; row0 < N; row0 += ROWS) {
                int seg = 0;
                while (seg + 1 < a.nseg && row0 >= a.seg_end[seg]) ++seg;
                const int seg0 = seg ? a.seg_end[seg - 1] : 0;
                const int last = (row0 + ROWS < N ? row0 + ROWS : N) - 1;
                if (last - seg0 > maxrow[seg]) maxrow[seg] = last - seg0;
            }
            for (int i = 0; i < a.nseg; ++i)
                if (maxrow[i] >= 0) need("gemv weight rows", a.w[i], (size_t)(maxrow[i] + 1) * K * esz(wt));
            if (a.seg_end[a.nseg - 1] != N) fake::violation("gemv segments end at " + std::to_string(a.seg_end[a.nseg - 1]));
            if (epi == kEpiStore) need("gemv y", a.y, (size_t)N * 4);
            if (epi == kEpiHead) need("gemv logit_scale", a.logit_scale, (size_t)N * 4);
        }
        if (res) {
            if (pro != kProEmbed) need("gemv prologue h", a.rs.h + (size_t)a.row * K, (size_t)K * 4);
            need("gemv prologue o", a.rs.o + (size_t)a.row * K, (size_t)K * 4);
            need("gemv prologue alpha", a.rs.alpha, (size_t)K * 4);
            if (pro == kProResolveInp) need("gemv prologue loop input", a.rs.inp + (size_t)a.row * K, (size_t)K * 4);
            if (pro == kProEmbed) need("gemv embedding table", a.embed, (size_t)a.vocab * K * esz(wt));
            if (a.rs.slerp && a.rs.o_parts > 1) fake::violation("the GEMV prologue reads one slab of a split-K o");
        } else {
            need("gemv source row", a.src + (size_t)a.row * K, (size_t)K * 4);
        }
        if (K > 8192 || sizeof(float) * (K + 16 + 8 * ROWS) > 160 * 1024) fake::violation("gemv LDS");
    };
    auto dyn = [=]() {
        fake::need_record(a.rec, a.row + 1);
        const CallRec *rec = a.rec;
        if (epi == kEpiHead) {
            if (rec->logits) need("logits row", rec->logits + (size_t)rec->rows[a.row].out * N, (size_t)N * 4);
            else if (!res || !rec->tap) return;
        }
        if (res) fake::resolve_writes(a.rs, a.row, K, rec, true);
    };
    return fake::launch("launch_gemv", stat, dyn);
}

hipError_t launch_add_slabs(float *x, size_t n, int parts, size_t stride, hipStream_t s) {
    if (!x || parts < 1) return hipErrorInvalidValue;
    if (parts == 1 || n == 0) return hipSuccess;
    if (n % 4 || stride % 4 || stride < n) return hipErrorInvalidValue;
    return fake::launch("launch_add_slabs", [=]() { need("slabs", x, ((size_t)(parts - 1) * stride + n) * 4); },
                        nullptr);
}

hipError_t launch_embed(int wt, const void *E, int V, int H, const CallRec *rec, int T, float *h, uint16_t *hb,
                        hipStream_t s) {
    auto stat = [=]() {
        need("embedding table", E, (size_t)V * H * esz(wt));
        need("embed h", h, (size_t)T * H * 4);
        if (hb) need("embed hb", hb, (size_t)T * H * 2);
    };
    return fake::launch("launch_embed", stat, [=]() { fake::need_record(rec, T); });
}

hipError_t launch_resolve_rows(const Resolve &rs, int H, int T, const CallRec *rec, float *tap, int tap_n,
                               hipStream_t s) {
    if (H > 8192) return hipErrorInvalidValue;
    if (rs.slerp && rs.o_parts > kMaxKParts) return hipErrorInvalidValue;
    if (rs.slerp && rs.o_ss && (rs.o_ss_n < 1 || rs.o_ss_n > 128)) return hipErrorInvalidValue;
    if (tap && tap_n < T) return hipErrorInvalidValue;
    if (fake::capturing) fake::violation("a multi-row residual step in a graph: its tap arguments would go stale");
    auto stat = [=]() {
        // rows past n_prev leave the loops early: after them (kLoopExit) their
        // state comes from st
        const int srows = rs.loop_op == kLoopExit ? (rs.n_prev < T ? rs.n_prev : T) : T;
        if (srows > 0) need("resolve h", rs.h, (size_t)srows * H * 4);
        if (srows < T) need("resolve loop state", rs.st, (size_t)T * H * 4);
        if (rs.slerp && srows > 0) {
            const int parts = rs.o_parts > 1 ? rs.o_parts : 1;
            for (int p = 0; p < parts; ++p) need("resolve o slab", rs.o + (size_t)p * rs.o_stride, (size_t)srows * H * 4);
            if (parts > 1 && rs.o_stride < (int64_t)T * H) fake::violation("o slabs overlap");
            need("resolve alpha", rs.alpha, (size_t)H * 4);
            if (rs.o_ss) need("resolve o sums of squares", rs.o_ss, (size_t)srows * rs.o_ss_n * 4);
        }
        if (rs.loop_op == kLoopNext) need("resolve loop input", rs.inp, (size_t)T * H * 4);
    };
    auto dyn = [=]() {
        fake::need_record(rec, T);
        if (tap != rec->tap || (tap && tap_n != rec->n))
            fake::violation("the residual step's tap arguments differ from the record's");
        for (int r = 0; r < T; ++r) fake::resolve_writes(rs, r, H, rec, true);
    };
    return fake::launch("launch_resolve_rows", stat, dyn);
}

hipError_t launch_rownorm(const float *src, int ld, float *dst, uint16_t *dstb, int N, int T, hipStream_t s) {
    auto stat = [=]() {
        need("rownorm src", src, ((size_t)(T - 1) * ld + N) * 4);
        need("rownorm dst", dst, (size_t)T * N * 4);
        if (dstb) need("rownorm dstb", dstb, (size_t)T * N * 2);
    };
    return fake::launch("launch_rownorm", stat, nullptr);
}

hipError_t launch_swiglu_norm(const float *a, const float *b, int ld, const float *sg, const float *su, float *dst,
                              uint16_t *dstb, int F, int T, hipStream_t s, float *ss) {
    auto stat = [=]() {
        need("swiglu a", a, ((size_t)(T - 1) * ld + F) * 4);
        need("swiglu b", b, ((size_t)(T - 1) * ld + F) * 4);
        need("swiglu sg", sg, (size_t)F * 4);
        need("swiglu su", su, (size_t)F * 4);
        if (dst) need("swiglu dst", dst, (size_t)T * F * 4);
        if (dstb) need("swiglu dstb", dstb, (size_t)T * F * 2);
        if (ss) need("swiglu sums of squares", ss, (size_t)T * 4);
        if (T < 1 || T > 65535) fake::violation("swiglu grid of " + std::to_string(T) + " rows");
    };
    return fake::launch("launch_swiglu_norm", stat, nullptr);
}

hipError_t launch_top_prob(const CallRec *rec, int V, float *out, hipStream_t s) {
    if (V <= 0) return hipErrorInvalidValue;
    auto dyn = [=]() {
        fake::need_record(rec, 1);
        need("top_prob logits", rec->logits, (size_t)V * 4);
    };
    return fake::launch("launch_top_prob", [=]() { need("top_prob out", out, 4); }, dyn);
}

hipError_t launch_logits_rows(const float *hlog, const float *ls, int V, int T, const CallRec *rec, hipStream_t s) {
    auto stat = [=]() {
        need("head output rows", hlog, (size_t)T * V * 4);
        need("logit_scale", ls, (size_t)V * 4);
    };
    auto dyn = [=]() {
        fake::need_record(rec, T);
        if (rec->logits)
            for (int r = 0; r < T; ++r) need("logits row", rec->logits + (size_t)rec->rows[r].out * V, (size_t)V * 4);
    };
    return fake::launch("launch_logits_rows", stat, dyn);
}

hipError_t launch_gemm(int wt, const float *A, const uint16_t *Ab, int lda, const GemmW &W, int N, int K, float *C,
                       int ldc, int M, hipStream_t s, int kparts, size_t pstride) {
    if (kparts < 1 || (kparts > 1 && !gemm_splits_ok(wt, Ab != nullptr, M, K, kparts))) return hipErrorInvalidValue;
    if (K % 4 || lda % 4 || W.nseg < 1 || W.nseg > 4 || W.seg_end[W.nseg - 1] != N) return hipErrorInvalidValue;
    auto stat = [=]() {
        if (M < 1) fake::violation("GEMM with " + std::to_string(M) + " rows");
        if (K > lda) fake::violation("GEMM K " + std::to_string(K) + " > lda " + std::to_string(lda));
        if (N > ldc) fake::violation("GEMM N " + std::to_string(N) + " > ldc " + std::to_string(ldc));
        if (gemm_reads_fp32_a(wt, Ab != nullptr, M, K, lda)) need("GEMM A (fp32)", A, ((size_t)(M - 1) * lda + K) * 4);
        else need("GEMM A (bf16)", Ab, ((size_t)(M - 1) * lda + K) * 2);
        fake::need_segments("GEMM weight rows", W.w, W.seg_end, W.nseg, K, wt);
        for (int z = 0; z < kparts; ++z) need("GEMM C slab", C + (size_t)z * pstride, ((size_t)(M - 1) * ldc + N) * 4);
        if (kparts > 1 && pstride < (size_t)(M - 1) * ldc + N) fake::violation("GEMM C slabs overlap");
    };
    return fake::launch("launch_gemm", stat, nullptr);
}

hipError_t launch_gemm_swiglu(const uint16_t *Ab, int lda, const void *wgate, const void *wup, int F, int K,
                              const float *sg, const float *su, uint16_t *zb, float *ssp, int M, hipStream_t s) {
    if (!gemm_swiglu_ok(kBF16, M, F, K, lda) || !Ab || !zb || !ssp) return hipErrorInvalidValue;
    auto stat = [=]() {
        need("GEMM A (bf16)", Ab, ((size_t)(M - 1) * lda + K) * 2);
        need("gate rows", wgate, (size_t)F * K * 2);
        need("up rows", wup, (size_t)F * K * 2);
        need("swiglu sg", sg, (size_t)F * 4);
        need("swiglu su", su, (size_t)F * 4);
        need("swiglu z (bf16)", zb, (size_t)M * F * 2);
        need("swiglu partial sums", ssp, (size_t)M * (F / 64) * 4);
    };
    return fake::launch("launch_gemm_swiglu", stat, nullptr);
}

hipError_t launch_prep(const PrepArgs &a, int T, hipStream_t s) {
    const int Q = a.nh * a.hd, KV = a.nk * a.hd, ld = 2 * Q + 2 * KV;
    if (a.hd > 256 || a.hd % 2 || (!a.kstage && (!a.kring || !a.vring || a.cap < 1)) || (a.kvtap && a.kvtap_n < T))
        return hipErrorInvalidValue;
    if (fake::capturing) fake::violation("a chunk's prep in a graph: its position and ring arguments would go stale");
    auto stat = [=]() {
        need("prep projections", a.qkvg, (size_t)T * ld * 4);
        need("prep queries", a.qp, (size_t)T * Q * 4);
        if (a.kstage) need("prep key stage", a.kstage, (size_t)T * KV * 4);
        need("prep sq", a.sq, (size_t)Q * 4);
    };
    auto dyn = [=]() {
        fake::need_record(a.rec, T);
        if (a.kvtap != a.rec->kvtap || (a.kvtap && a.kvtap_n != a.rec->n))
            fake::violation("the prep's kv tap arguments differ from the record's");
        for (int r = 0; r < T; ++r) {
            const RowRec &row = a.rec->rows[r];
            if (row.pos != a.pos0 + r) fake::violation("prep row " + std::to_string(r) + " is not at pos0 + r");
            need("RoPE row", a.rope + (size_t)row.pos * a.hd, (size_t)a.hd * 4);
            if (!a.kstage) {
                const SlotDesc *d = fake::slot(a.tab, row.seq, a.n_ord, a.ord, a.slot, a.nk, a.hd, false);
                if (d && (d->k != a.kring || d->v != a.vring || d->cap != a.cap))
                    fake::violation("the prep's ring arguments differ from the row's slot");
                const size_t ring = (size_t)(a.nk - 1) * a.cap + (size_t)(row.pos % a.cap);
                need("prep key ring row", a.kring, (ring + 1) * a.hd * 4);
                need("prep value ring row", a.vring, (ring + 1) * a.hd * 4);
            }
            if (a.kvtap) need("kv tap", a.kvtap + ((size_t)a.tap_pass * a.kvtap_n + r) * 2 * KV, (size_t)2 * KV * 4);
        }
    };
    return fake::launch("launch_prep", stat, dyn);
}

// Both attention launchers: T rows (decode: each its own sequence and
// position; chunk: consecutive positions of one sequence).
static hipError_t attn_common(const char *name, const AttnArgs &a, int T, bool dec) {
    const int Q = a.nh * a.hd, KV = a.nk * a.hd, ld = 2 * Q + 2 * KV, rep = a.nh / a.nk;
    if (!dec && a.blk > 0 && fake::capturing)
        fake::violation("a chunk's attention in a graph: its position, row and slot arguments would go stale");
    auto stat = [=]() {
        need("attention sg", a.sg, (size_t)Q * 4);
        need("attention z", a.z, (size_t)T * Q * 4);
        if (a.zb) need("attention z (bf16)", a.zb, (size_t)T * Q * 2);
        if (a.zss) need("attention z sums of squares", a.zss, (size_t)T * a.nk * 4);
        if (a.xcnt) {
            // one row, the splits merged in the kernel: per-kv-head counters and
            // the line-aligned partial layout
            if (!dec || T != 1 || a.hd != 128 || rep != 4 || a.split > 64 || a.max_split > 64)
                fake::violation("in-kernel merge counters passed where that merge does not apply");
            need("in-kernel merge counters", a.xcnt, (size_t)32 * a.nh * 4);
            need("attention partials (in-kernel merge)", a.part, attn_xm_part_floats(a.nk, a.max_split, rep, a.hd) * 4);
        } else {
            need("attention partials", a.part, (size_t)T * a.nk * a.max_split * rep * (a.hd + 2) * 4);
        }
        need("attention projections", a.qkvg, (size_t)T * ld * 4);
        if (dec) {
            need("attention sq", a.sq, (size_t)Q * 4);
        } else {
            need("attention queries", a.qp, (size_t)T * Q * 4);
        }
    };
    auto dyn = [=]() {
        fake::need_record(a.rec, T);
        const CallRec *rec = a.rec;
        const int64_t pos0 = rec->rows[0].pos;
        for (int r = 0; r < T; ++r) {
            const RowRec &row = rec->rows[r];
            const int64_t p = row.pos;
            if (!dec && p != pos0 + r) fake::violation("chunk rows at non-consecutive positions");
            const SlotDesc *d = fake::slot(a.tab, row.seq, a.n_ord, a.ord, a.slot, a.nk, a.hd, a.q8);
            if (dec && a.sd1) {
                need("the graph's slot entry", a.sd1, sizeof(SlotDesc));
                if (a.sd1 != &slot_at(a.tab, row.seq, a.n_ord, a.ord, a.slot))
                    fake::violation("the graph's slot belongs to another sequence than the record's row");
            }
            if (dec) need("RoPE row", a.rope + (size_t)p * a.hd, (size_t)a.hd * 4);
            if (dec && rec->kvtap)
                need("kv tap", rec->kvtap + ((size_t)a.tap_pass * rec->n + r) * 2 * KV, (size_t)2 * KV * 4);
            const int64_t lo = p + 1 - a.window > 0 ? p + 1 - a.window : 0;
            const int64_t nkeys = p - lo + 1;
            if (a.ext) {
                // the grown split: max_split workgroups of up to 72 keys
                if (!dec || T != 1 || a.hd != 128 || rep != 4 || a.split != 64)
                    fake::violation("a grown split where the one-row kernel does not take it");
                const int64_t S = std::max<int64_t>(a.split, (nkeys + a.max_split - 1) / a.max_split);
                if (S > a.split * 9 / 8)
                    fake::violation("row at " + std::to_string(p) + " needs splits of " + std::to_string(S) +
                                    " keys, more than the grown split's 72");
            } else if (dec || a.blk == 0) {
                const int64_t ns = (nkeys + a.split - 1) / a.split;
                if (ns > a.max_split)
                    fake::violation("row at " + std::to_string(p) + " needs " + std::to_string(ns) +
                                    " key splits, the grid has " + std::to_string(a.max_split));
            }
            fake::keys_held(d, lo, p, dec ? p : pos0 + T - 1);
        }
        if (!dec && a.blk > 0) {
            // the chunk kernels take these from the arguments, not the record
            if (a.pos0 != pos0 || a.nrows != rec->n)
                fake::violation("the chunk attention's position or row arguments differ from the record's");
            const SlotDesc &e = slot_at(a.tab, rec->rows[0].seq, a.n_ord, a.ord, a.slot);
            const SlotDesc &c = a.sdc;
            if (c.k != e.k || c.v != e.v || c.kc != e.kc || c.vc != e.vc || c.ks != e.ks || c.vs != e.vs ||
                c.kcol != e.kcol || c.vcol != e.vcol || c.cap != e.cap)
                fake::violation("the chunk attention's slot argument differs from the table's entry");
            const int nb = (T + a.blk - 1) / a.blk;
            for (int b = 0; b < nb; ++b) {
                const int rb0 = b * a.blk, rb1 = (rb0 + a.blk < T ? rb0 + a.blk : T) - 1;
                const int64_t klo = pos0 + rb0 + 1 - a.window > 0 ? pos0 + rb0 + 1 - a.window : 0;
                const int64_t ns = (pos0 + rb1 - klo + a.split) / a.split;
                if (ns > a.nsplit)
                    fake::violation("block " + std::to_string(b) + " needs " + std::to_string(ns) +
                                    " splits, the grid has " + std::to_string(a.nsplit));
            }
        }
    };
    return fake::launch(name, stat, dyn);
}

// The XCD check at create: reports workgroup L on XCD L % 8 (the in-kernel
// merge's paths then run here too).
hipError_t launch_xcd_check(unsigned *ids, int G, hipStream_t s) {
    if (!ids || G < 1) return hipErrorInvalidValue;
    auto stat = [=]() {
        need("XCD ids", ids, (size_t)G * 4);
        uintptr_t base = 0;
        const fake::Alloc *al = fake::find(ids, &base);
        if (al && al->mapped && reinterpret_cast<uintptr_t>(ids) + (size_t)G * 4 <= base + al->bytes)
            for (int i = 0; i < G; ++i) ids[i] = (unsigned)(i % 8);
    };
    return fake::launch("launch_xcd_check", stat, [] {});
}

hipError_t launch_attn(const AttnArgs &a, int T, hipStream_t s) {
    if (a.split <= 0 || T <= 0 || (a.blk == 0 && a.split > 256) || (a.blk > 0 && a.split % 64))
        return hipErrorInvalidValue;
    if (a.blk > 0 && (a.blk != attn_chunk_block(a.hd, a.nh / a.nk) || a.nsplit < 1 || a.nsplit > a.max_split))
        return hipErrorInvalidValue;
    return attn_common("launch_attn", a, T, false);
}

hipError_t launch_attn_dec(const AttnArgs &a, int T, hipStream_t s) {
    if (a.split <= 0 || a.split > attn_dec_max_split(a.hd, 16) || T <= 0) return hipErrorInvalidValue;
    return attn_common("launch_attn_dec", a, T, true);
}

hipError_t launch_q8_write(const Q8WriteArgs &a, hipStream_t s) {
    if (a.r1 <= a.r0) return hipSuccess;
    const int KV = a.nk * a.hd;
    auto stat = [=]() {
        need("q8 write keys", a.ksrc + (size_t)a.r0 * a.kld, ((size_t)(a.r1 - 1 - a.r0) * a.kld + KV) * 4);
        need("q8 write values", a.vsrc + (size_t)a.r0 * a.vld, ((size_t)(a.r1 - 1 - a.r0) * a.vld + KV) * 4);
    };
    auto dyn = [=]() {
        fake::need_record(a.rec, a.r1);
        for (int r = a.r0; r < a.r1; ++r) fake::slot(a.tab, a.rec->rows[r].seq, a.n_ord, a.ord, a.slot, a.nk, a.hd, true);
    };
    return fake::launch("launch_q8_write", stat, dyn);
}

hipError_t launch_q8_freeze(const SlotDesc *tab, int n_ord, int ord, int slot, int nk, int hd, const CallRec *rec,
                            int row, hipStream_t s) {
    auto dyn = [=]() {
        fake::need_record(rec, row + 1);
        const SlotDesc *d = fake::slot(tab, rec->rows[row].seq, n_ord, ord, slot, nk, hd, true);
        if (d && d->cap < kWarmup) fake::violation("a ring too short for the 64 rows the freeze re-encodes");
    };
    return fake::launch("launch_q8_freeze", []() {}, dyn);
}

hipError_t launch_q8_encode_rows(const float *x, const float *col, int rows, int n, int group, int8_t *codes,
                                 float *scales, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    auto stat = [=]() {
        need("encoder input", x, (size_t)rows * n * 4);
        if (col) need("encoder field", col, (size_t)n * 4);
        need("encoder codes", codes, (size_t)rows * n);
        need("encoder scales", scales, (size_t)rows * ((n + group - 1) / group) * 4);
    };
    return fake::launch("launch_q8_encode_rows", stat, nullptr);
}

hipError_t launch_kv_store(const float *k, const float *v, const SlotDesc *tab, int n_ord, int ord, int slot, int nk,
                           int hd, int T, const CallRec *rec, hipStream_t s) {
    auto stat = [=]() {
        need("stored keys", k, (size_t)T * nk * hd * 4);
        need("stored values", v, (size_t)T * nk * hd * 4);
    };
    auto dyn = [=]() {
        fake::need_record(rec, T);
        for (int r = 0; r < T; ++r) fake::slot(tab, rec->rows[r].seq, n_ord, ord, slot, nk, hd, false);
    };
    return fake::launch("launch_kv_store", stat, dyn);
}

}  // namespace dk
