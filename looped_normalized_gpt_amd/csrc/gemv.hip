// gemv.hip -- weight-streaming matrix-vector products for one-row calls (decode).
//
// y = W x with W [N][K] row-major in bf16 or fp32 and x, y fp32 (dory.rs
// `attn_layer` / `mlp_layer` / `head`, the one-row matvec branches).  The work is
// HBM-bound: every weight byte is read once, so the kernel keeps many 16-byte
// loads in flight and hides the prologue behind them.
//
// Workgroup: 256 threads = 4 waves, ROWS output rows (4, 8 or 16: more rows per
// workgroup for the larger matrices, so fewer workgroups repeat the prologue).  The K axis is cut in
// 512-element chunks (64 lanes x 8 elements = one 16-byte bf16 load per lane),
// dealt round-robin to the 4 waves; a wave issues the loads of all its chunks
// for all its rows before the prologue runs.  Each lane's prologue inputs are
// the 8 elements of each of its chunks that its dot products take, so x stays
// in registers; a reduce-scatter leaves each row's sum over a half wave in one
// lane, and the 8 half-wave partials of a row are added through LDS.
//
// Prologues build x (in registers):
//   kProResolve: the previous sub-layer's slerp and the loop mix (Resolve);
//                workgroup 0 also stores the new residual, loop input and tap.
//   kProEmbed:   kProResolve for the very first pass of a one-row call, its
//                h the embedding row of the record's token (zero for an id
//                outside the table); workgroup 0 stores it as the residual.
//   kProNorm:    x = justnorm(src row) (the renorm over Q before O and over F
//                before down, dory.rs `attn_layer` / `mlp_layer`).
// Epilogues:
//   kEpiStore:   y[n] = acc.
//   kEpiPair:    rows n of Wgate and Wup together: y[n] = silu(a*sg)*(b*su)
//                (dory.rs `silu_body`).
//   kEpiHead:    logits[n] = acc * logit_scale[n] into the call record's
//                pointer (dory.rs `head`); nothing when it is null.
#include "device.h"

namespace dk {

namespace {

template <int WT>
struct W8;

// Weights are read once per token: streaming (nontemporal) loads keep them from
// displacing what the caches hold for the next kernels.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <>
struct W8<kBF16> {
    uint4 v;
    __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void load(const void *base, size_t elem) {
        const u32x4 t = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(base) + elem));
        v = make_uint4(t.x, t.y, t.z, t.w);
    }
    __device__ __forceinline__ float dot(const float4 &a, const float4 &b) const {
        float s = bf16lo(v.x) * a.x;
        s = fmaf(bf16hi(v.x), a.y, s);
        s = fmaf(bf16lo(v.y), a.z, s);
        s = fmaf(bf16hi(v.y), a.w, s);
        s = fmaf(bf16lo(v.z), b.x, s);
        s = fmaf(bf16hi(v.z), b.y, s);
        s = fmaf(bf16lo(v.w), b.z, s);
        s = fmaf(bf16hi(v.w), b.w, s);
        return s;
    }
};

template <>
struct W8<kF32> {
    float4 a, b;
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void load(const void *base, size_t elem) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(base) + elem);
        const f32x4 x = __builtin_nontemporal_load(p), y = __builtin_nontemporal_load(p + 1);
        a = make_float4(x.x, x.y, x.z, x.w);
        b = make_float4(y.x, y.y, y.z, y.w);
    }
    __device__ __forceinline__ float dot(const float4 &x, const float4 &y) const {
        float s = a.x * x.x;
        s = fmaf(a.y, x.y, s);
        s = fmaf(a.z, x.z, s);
        s = fmaf(a.w, x.w, s);
        s = fmaf(b.x, y.x, s);
        s = fmaf(b.y, y.y, s);
        s = fmaf(b.z, y.z, s);
        s = fmaf(b.w, y.w, s);
        return s;
    }
};

template <int WT, int PRO, int EPI, int MAXC, int ROWS>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
    constexpr bool RES = PRO == kProResolve || PRO == kProResolveInp || PRO == kProEmbed;
    extern __shared__ float smem[];
    constexpr int WR = EPI == kEpiPair ? 2 * ROWS : ROWS;
    constexpr int EPT = 8 * MAXC;  // prologue elements per thread: K <= 2048 * MAXC
    static_assert(ROWS >= 1 && ROWS <= 64 && (ROWS & (ROWS - 1)) == 0, "ROWS: a power of two");
    float *xs = smem;              // [K] (the logits-free head path)
    float *red = smem + a.K;       // [16]: two reduction slots
    float *part = red + 16;        // [8][WR]: half-wave partials
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row0 = blockIdx.x * ROWS;
    const int K = a.K, N = a.N;
    const CallRec *rec = a.rec;
    const Resolve &rs = a.rs;

    if (EPI == kEpiHead && rec->logits == nullptr) {
        // No logits wanted: only the tap of the last pass, if any.
        if (!RES || blockIdx.x != 0 || rec->tap == nullptr) return;
        resolve_row(rs, a.row, K, xs, red, true, rec);
        return;
    }

    // 1. The prologue's inputs, the float4 groups of this lane's dot elements
    // (elem_index<1>).  Every load is unconditional (out-of-range groups re-read
    // group 0 and are zeroed), so the compiler can count them and wait for
    // exactly these below.
    float ph[EPT], po[EPT], pa[EPT], pi[EPT];
    {
        const float *src = (RES ? rs.h : a.src) + (size_t)a.row * K;
        uint32_t tok = 0;
        bool tok_ok = false;
        if (PRO == kProEmbed) {
            tok = (uint32_t)rec->rows[a.row].token;
            tok_ok = tok < (uint32_t)a.vocab;
            tok = tok_ok ? tok : 0u;
        }
#pragma unroll
        for (int jj = 0; jj < EPT / 4; ++jj) {
            const int i = elem_index<1>(4 * jj);
            const int ic = i < K ? i : 0;
            float4 v;
            if (PRO == kProEmbed) {
                if (WT == kBF16) {
                    const uint2 u = *reinterpret_cast<const uint2 *>(
                        reinterpret_cast<const uint16_t *>(a.embed) + (size_t)tok * K + ic);
                    v = make_float4(bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y));
                } else {
                    v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.embed) + (size_t)tok * K + ic);
                }
                if (!tok_ok) v = make_float4(0.f, 0.f, 0.f, 0.f);
            } else {
                v = *reinterpret_cast<const float4 *>(src + ic);
            }
            ph[4 * jj] = v.x; ph[4 * jj + 1] = v.y; ph[4 * jj + 2] = v.z; ph[4 * jj + 3] = v.w;
            if (RES) {
                const float4 vo = *reinterpret_cast<const float4 *>(rs.o + (size_t)a.row * K + ic);
                const float4 va = *reinterpret_cast<const float4 *>(rs.alpha + ic);
                po[4 * jj] = vo.x; po[4 * jj + 1] = vo.y; po[4 * jj + 2] = vo.z; po[4 * jj + 3] = vo.w;
                pa[4 * jj] = va.x; pa[4 * jj + 1] = va.y; pa[4 * jj + 2] = va.z; pa[4 * jj + 3] = va.w;
            }
            if (PRO == kProResolveInp) {
                const float4 vi = *reinterpret_cast<const float4 *>(rs.inp + (size_t)a.row * K + ic);
                pi[4 * jj] = vi.x; pi[4 * jj + 1] = vi.y; pi[4 * jj + 2] = vi.z; pi[4 * jj + 3] = vi.w;
            } else {
                pi[4 * jj] = pi[4 * jj + 1] = pi[4 * jj + 2] = pi[4 * jj + 3] = 0.f;
            }
        }
    }

    // The epilogue's per-row scalars, the head's output row and the record's tap
    // pointer, read now with the prologue's inputs: read where they are used,
    // each would add a round trip to the workgroup (the tap's after the whole
    // weight stream).  Every lane reads (the row of lane tid % ROWS, clamped).
    float e0 = 0.f, e1 = 0.f;
    int32_t out_row = 0;
    float *tap = nullptr;
    {
        const int en = row0 + (tid & (ROWS - 1));
        const int enc = en < N ? en : row0;
        if (EPI == kEpiPair) {
            e0 = a.sg[enc];
            e1 = a.su[enc];
        } else if (EPI == kEpiHead) {
            e0 = a.logit_scale[enc];
            out_row = rec->rows[a.row].out;
        }
        if (RES) {
            float *t = rec->tap;
            const int tn = rec->n;
            tap = blockIdx.x == 0 && rs.tap_pass >= 0 && t ? t + ((size_t)rs.tap_pass * tn + a.row) * K : nullptr;
        }
    }

    // 2. Weight rows of this workgroup, every load issued now (the prologue runs
    // while they fly).  Rows past N and chunks past K re-read a valid address
    // and are masked at use.
    const void *base[WR];
    size_t roff[WR];
    bool valid[WR];
    int seg = 0;
    while (seg + 1 < a.nseg && row0 >= a.seg_end[seg]) ++seg;
    const int seg0 = seg ? a.seg_end[seg - 1] : 0;
#pragma unroll
    for (int j = 0; j < WR; ++j) {
        const int n = row0 + (j % ROWS);
        valid[j] = n < N;
        const int nn = valid[j] ? n : row0;
        if (EPI == kEpiPair) {
            base[j] = a.w[j < ROWS ? 0 : 1];
            roff[j] = (size_t)nn * K;
        } else {
            base[j] = a.w[seg];
            roff[j] = (size_t)(nn - seg0) * K;
        }
    }
    W8<WT> wv[WR][MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int k0 = (wave + 4 * c) * 512 + lane * 8;
        const int kc = k0 < K ? k0 : 0;
#pragma unroll
        for (int j = 0; j < WR; ++j) wv[j][c].load(base[j], roff[j] + kc);
    }
    // Nothing below moves above this point: the weight loads stay ahead of the
    // prologue's waits.
    __builtin_amdgcn_sched_barrier(0);
    // Pin the prologue's inputs here: otherwise the compiler sinks their loads
    // into the branches of the prologue that use them, behind the weight loads,
    // and the prologue then waits for every weight load.
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        asm volatile("" ::"v"(ph[j]));
        if (RES) asm volatile("" ::"v"(po[j]), "v"(pa[j]));
        if (PRO == kProResolveInp) asm volatile("" ::"v"(pi[j]));
    }
    asm volatile("" ::"v"(e0), "v"(e1), "v"(out_row), "v"(tap));

    // 3. x in registers, slot for slot with the dot elements.
    float xr[EPT];
    if (RES) {
#pragma unroll
        for (int jj = 0; jj < EPT / 4; ++jj)
            if (elem_index<1>(4 * jj) >= K)
#pragma unroll
                for (int c = 0; c < 4; ++c) ph[4 * jj + c] = po[4 * jj + c] = pa[4 * jj + c] = pi[4 * jj + c] = 0.f;
#pragma unroll
        for (int j = 0; j < EPT; ++j) xr[j] = 0.f;
        resolve_regs<EPT, 1>(rs, a.row, K, ph, po, pa, pi, nullptr, red, blockIdx.x == 0, tap, xr);
    } else {
        float f = 1.f;
        if (PRO == kProNorm) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < EPT; ++j)
                if (elem_index<1>(j) < K) s += ph[j] * ph[j];
            f = norm_factor(block_sum(s, red, 0));
        }
#pragma unroll
        for (int j = 0; j < EPT; ++j) xr[j] = ph[j] * f;
    }

    // 4. Dot products; each row's sum over a half wave by the reduce-scatter,
    // the 8 half-wave partials of a row through LDS.
    float acc[WR];
#pragma unroll
    for (int j = 0; j < WR; ++j) acc[j] = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int k0 = (wave + 4 * c) * 512 + lane * 8;
        if (k0 < K) {
            const float4 x0 = make_float4(xr[8 * c], xr[8 * c + 1], xr[8 * c + 2], xr[8 * c + 3]);
            const float4 x1 = make_float4(xr[8 * c + 4], xr[8 * c + 5], xr[8 * c + 6], xr[8 * c + 7]);
#pragma unroll
            for (int j = 0; j < WR; ++j) acc[j] += wv[j][c].dot(x0, x1);
        }
    }
    {
        const float v = row_sums_rs<WR>(acc, lane);
        if ((lane & 31) < WR) part[(2 * wave + (lane >> 5)) * WR + (lane & 31)] = v;
    }
    __syncthreads();
    if (tid < ROWS) {
        const int n = row0 + tid;
        if (n < N) {
            float v = 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) v += part[q * WR + tid];
            if (EPI == kEpiStore) {
                a.y[n] = v;
            } else if (EPI == kEpiPair) {
                const int j = ROWS + tid;
                float b = 0.f;
#pragma unroll
                for (int q = 0; q < 8; ++q) b += part[q * WR + j];
                float g = v * e0;
                a.y[n] = g / (1.0f + expf(-g)) * (b * e1);
            } else {
                rec->logits[(size_t)out_row * N + n] = v * e0;
            }
        }
    }
}

template <int WT, int PRO, int EPI, int ROWS>
hipError_t launch_r(const GemvArgs &a, hipStream_t s) {
    const int nch = (a.K + 511) / 512;
    const int maxc = (nch + 3) / 4;
    dim3 grid((a.N + ROWS - 1) / ROWS), block(256);
    const size_t lds = sizeof(float) * (a.K + 16 + 8 * 2 * ROWS);
    switch (maxc) {
        case 1: hipLaunchKernelGGL((k_gemv<WT, PRO, EPI, 1, ROWS>), grid, block, lds, s, a); break;
        case 2: hipLaunchKernelGGL((k_gemv<WT, PRO, EPI, 2, ROWS>), grid, block, lds, s, a); break;
        case 3: hipLaunchKernelGGL((k_gemv<WT, PRO, EPI, 3, ROWS>), grid, block, lds, s, a); break;
        case 4: hipLaunchKernelGGL((k_gemv<WT, PRO, EPI, 4, ROWS>), grid, block, lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Rows per workgroup: enough workgroups to cover the chip twice, no more.
template <int WT, int PRO, int EPI>
hipError_t launch_c(const GemvArgs &a, hipStream_t s) {
    if (a.N >= 16 * 1024) return launch_r<WT, PRO, EPI, 16>(a, s);
    if (a.N >= 8 * 512) return launch_r<WT, PRO, EPI, 8>(a, s);
    return launch_r<WT, PRO, EPI, 4>(a, s);
}

template <int WT>
hipError_t launch_w(int pro, int epi, const GemvArgs &a, hipStream_t s) {
    if (pro == kProResolve && epi == kEpiStore) return launch_c<WT, kProResolve, kEpiStore>(a, s);
    if (pro == kProEmbed && epi == kEpiStore) return launch_c<WT, kProEmbed, kEpiStore>(a, s);
    if (pro == kProEmbed && epi == kEpiPair) return launch_c<WT, kProEmbed, kEpiPair>(a, s);
    if (pro == kProResolveInp && epi == kEpiStore) return launch_c<WT, kProResolveInp, kEpiStore>(a, s);
    if (pro == kProNorm && epi == kEpiStore) return launch_c<WT, kProNorm, kEpiStore>(a, s);
    if (pro == kProResolve && epi == kEpiPair) return launch_c<WT, kProResolve, kEpiPair>(a, s);
    if (pro == kProResolveInp && epi == kEpiPair) return launch_c<WT, kProResolveInp, kEpiPair>(a, s);
    if (pro == kProResolve && epi == kEpiHead) return launch_c<WT, kProResolve, kEpiHead>(a, s);
    if (pro == kProPlain && epi == kEpiHead) return launch_c<WT, kProPlain, kEpiHead>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemv(int wtype, int pro, int epi, const GemvArgs &a, hipStream_t s) {
    if (a.K <= 0 || a.K > 8192 || a.K % 8 || a.N <= 0) return hipErrorInvalidValue;
    if (pro == kProEmbed && (!a.embed || a.vocab <= 0)) return hipErrorInvalidValue;
    return wtype == kBF16 ? launch_w<kBF16>(pro, epi, a, s) : launch_w<kF32>(pro, epi, a, s);
}

}  // namespace dk
