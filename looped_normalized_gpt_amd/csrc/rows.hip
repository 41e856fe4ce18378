// rows.hip -- per-row kernels of multi-row calls (prefill chunks): embedding
// gather, the residual step between sub-layers, and the renorms before O and
// down.  One 256-thread workgroup per row; these are launch-latency work.
#include "device.h"

namespace dk {

namespace {

// dory.rs `forward_host`: h[r] = E[token r]; an id past the table is a zero row.
template <int WT>
__global__ __launch_bounds__(256) void k_embed(const void *E, int V, int H, const CallRec *rec, float *h,
                                               uint16_t *hb) {
    const int r = blockIdx.x;
    const uint32_t id = (uint32_t)rec->rows[r].token;
    float *out = h + (size_t)r * H;
    uint16_t *outb = hb ? hb + (size_t)r * H : nullptr;
    for (int i = threadIdx.x; i < H; i += 256) {
        float x = 0.f;
        if (id < (uint32_t)V)
            x = WT == kBF16 ? bf16f(reinterpret_cast<const uint16_t *>(E)[(size_t)id * H + i])
                            : reinterpret_cast<const float *>(E)[(size_t)id * H + i];
        out[i] = x;
        if (outb) outb[i] = f2bf(x);
    }
}

// One row per workgroup; thread t holds the float4 groups at 4t + 1024 jj of
// the row in registers (EPT / 4 groups).  Every load is issued before any
// arithmetic, unconditionally where its count varies (P slabs of o, the
// renorm's partial sums: clamped addresses, masked values), so none waits
// for another: the renorm partials, h, o, alpha, the loop input.  The tap
// pointer and row count come as arguments: a read of the record here cost a
// round trip before or after the loads.  (A loop over the slabs waited for each slab in turn, and the
// renorm's sum and the record's tap pointer each took a round trip of their
// own before and after the loads.)
template <int EPT, int P>
__global__ __launch_bounds__(256) void k_resolve_rows(Resolve rs, int H, float *tap_base, int tap_n) {
    __shared__ float red[16];  // resolve_regs' two reduction slots
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const bool from_st = rs.loop_op == kLoopExit && r >= rs.n_prev;  // a batch row whose loops ended early
    const bool slerp = rs.slerp && !from_st;
    const float *hs = (from_st ? rs.st : rs.h) + (size_t)r * H;
    // the renorm of the attention output before its projection, applied here
    // (the projection is linear): o times justnorm's factor of |z|^2, the sum
    // of up to 128 partials (one per kv head, or per 64 ffn indices), two a lane
    const bool ren = slerp && rs.o_ss;
    const int nss = rs.o_ss_n;
    float s0 = 0.f, s1 = 0.f;
    if (ren) {
        const float *ps = rs.o_ss + (size_t)r * nss;
        s0 = ps[lane < nss ? lane : 0];
        s1 = ps[lane + 64 < nss ? lane + 64 : 0];
    }
    const int parts = rs.o_parts > 1 ? rs.o_parts : 1;
    float4 vh[EPT / 4], vo[EPT / 4][P], va[EPT / 4], vi[EPT / 4];
#pragma unroll
    for (int jj = 0; jj < EPT / 4; ++jj) {
        const int i = 4 * tid + 1024 * jj, ic = i < H ? i : 0;
        vh[jj] = *reinterpret_cast<const float4 *>(hs + ic);
        vo[jj][0] = va[jj] = vi[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (slerp) {
            // o: the sum of the output projection's split-K slabs
#pragma unroll
            for (int p = 0; p < P; ++p)
                vo[jj][p] = *reinterpret_cast<const float4 *>(rs.o + (size_t)(p < parts ? p : 0) * rs.o_stride +
                                                              (size_t)r * H + ic);
            va[jj] = *reinterpret_cast<const float4 *>(rs.alpha + ic);
        }
        if (rs.loop_op == kLoopNext) vi[jj] = *reinterpret_cast<const float4 *>(rs.inp + (size_t)r * H + ic);
    }
    // every load above is in flight before the first use of any of them
    asm volatile("" ::"v"(s0), "v"(s1));
#pragma unroll
    for (int jj = 0; jj < EPT / 4; ++jj) {
        asm volatile("" ::"v"(vh[jj].x), "v"(vh[jj].w), "v"(va[jj].x), "v"(va[jj].w), "v"(vi[jj].x), "v"(vi[jj].w));
#pragma unroll
        for (int p = 0; p < P; ++p) asm volatile("" ::"v"(vo[jj][p].x), "v"(vo[jj][p].w));
    }
    float *tap = !from_st && rs.tap_pass >= 0 && tap_base ? tap_base + ((size_t)rs.tap_pass * tap_n + r) * H : nullptr;
    const float oc = ren ? norm_factor(wave_sum((lane < nss ? s0 : 0.f) + (lane + 64 < nss ? s1 : 0.f))) : 1.f;
    float h[EPT], o[EPT], al[EPT], in[EPT];
#pragma unroll
    for (int jj = 0; jj < EPT / 4; ++jj) {
        const bool ok = 4 * tid + 1024 * jj < H;
        float4 so = vo[jj][0];
#pragma unroll
        for (int p = 1; p < P; ++p)
            if (p < parts) {
                so.x += vo[jj][p].x; so.y += vo[jj][p].y; so.z += vo[jj][p].z; so.w += vo[jj][p].w;
            }
        const float4 vhh = vh[jj], vaa = va[jj], vii = vi[jj];
        h[4 * jj] = ok ? vhh.x : 0.f; h[4 * jj + 1] = ok ? vhh.y : 0.f; h[4 * jj + 2] = ok ? vhh.z : 0.f; h[4 * jj + 3] = ok ? vhh.w : 0.f;
        o[4 * jj] = ok ? so.x * oc : 0.f; o[4 * jj + 1] = ok ? so.y * oc : 0.f;
        o[4 * jj + 2] = ok ? so.z * oc : 0.f; o[4 * jj + 3] = ok ? so.w * oc : 0.f;
        al[4 * jj] = vaa.x; al[4 * jj + 1] = vaa.y; al[4 * jj + 2] = vaa.z; al[4 * jj + 3] = vaa.w;
        in[4 * jj] = ok ? vii.x : 0.f; in[4 * jj + 1] = ok ? vii.y : 0.f; in[4 * jj + 2] = ok ? vii.z : 0.f; in[4 * jj + 3] = ok ? vii.w : 0.f;
    }
    if (from_st) {
#pragma unroll
        for (int jj = 0; jj < EPT / 4; ++jj) {
            const int i = 4 * tid + 1024 * jj;
            if (i >= H) continue;
            const float4 v = make_float4(h[4 * jj], h[4 * jj + 1], h[4 * jj + 2], h[4 * jj + 3]);
            if (rs.h_out) *reinterpret_cast<float4 *>(rs.h_out + (size_t)r * H + i) = v;
            if (rs.hb_out) {
                uint16_t *hb = rs.hb_out + (size_t)r * H + i;
                hb[0] = f2bf(v.x); hb[1] = f2bf(v.y); hb[2] = f2bf(v.z); hb[3] = f2bf(v.w);
            }
        }
        return;
    }
    Resolve rr = rs;
    rr.slerp = slerp;
    resolve_regs<EPT>(rr, r, H, h, o, al, in, nullptr, red, true, tap);
}

// dst[r] = justnorm(src[r]) over N values.
__global__ __launch_bounds__(256) void k_rownorm(const float *src, int ld, float *dst, uint16_t *dstb, int N) {
    __shared__ float red[8];
    const float *x = src + (size_t)blockIdx.x * ld;
    float *y = dst + (size_t)blockIdx.x * N;
    float s = 0.f;
    for (int i = threadIdx.x; i < N; i += 256) s += x[i] * x[i];
    const float f = norm_factor(block_sum(s, red));
    for (int i = threadIdx.x; i < N; i += 256) {
        const float v = x[i] * f;
        y[i] = v;
        if (dstb) dstb[(size_t)blockIdx.x * N + i] = f2bf(v);
    }
}

// dory.rs `mlp_layer`: z = silu(a*sg) * (b*su), then justnorm over F.  With
// ss: z itself is stored and ss[row] = |z|^2 (the consumer of the projection
// applies the renorm's factor).  dst (fp32) or dstb (bf16) may be null.
__global__ __launch_bounds__(256) void k_swiglu_norm(const float *a, const float *b, int ld, const float *sg,
                                                     const float *su, float *dst, uint16_t *dstb, int F, float *ss) {
    extern __shared__ float smem[];
    float *red = smem, *z = smem + 8;
    const size_t off = (size_t)blockIdx.x * F, offi = (size_t)blockIdx.x * ld;
    float s = 0.f;
    for (int i = threadIdx.x; i < F; i += 256) {
        float g = a[offi + i] * sg[i];
        float v = g / (1.0f + expf(-g)) * (b[offi + i] * su[i]);
        z[i] = v;
        s += v * v;
    }
    s = block_sum(s, red);
    const float f = ss ? 1.f : norm_factor(s);
    if (ss && threadIdx.x == 0) ss[blockIdx.x] = s;
    for (int i = threadIdx.x; i < F; i += 256) {
        const float v = z[i] * f;
        if (dst) dst[off + i] = v;
        if (dstb) dstb[off + i] = f2bf(v);
    }
}

// Register versions of the two renorms for rows of 4-aligned length: thread t
// holds the float4 groups t + 256 j (j < G) of its row, all loads issued first.
template <int G>
__global__ __launch_bounds__(256) void k_rownorm_v(const float *src, int ld, float *dst, uint16_t *dstb, int N) {
    __shared__ float red[8];
    const float *x = src + (size_t)blockIdx.x * ld;
    float4 v[G];
    float s = 0.f;
    // every load before any use (computing each group as it arrived waited
    // for the groups one at a time)
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int i = 4 * (threadIdx.x + 256 * j);
        v[j] = *reinterpret_cast<const float4 *>(x + (i < N ? i : 0));
    }
#pragma unroll
    for (int j = 0; j < G; ++j) asm volatile("" ::"v"(v[j].x), "v"(v[j].w));
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int i = 4 * (threadIdx.x + 256 * j);
        if (i >= N) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        s += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    }
    const float f = norm_factor(block_sum(s, red));
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int i = 4 * (threadIdx.x + 256 * j);
        if (i >= N) continue;
        const float4 y = make_float4(v[j].x * f, v[j].y * f, v[j].z * f, v[j].w * f);
        *reinterpret_cast<float4 *>(dst + (size_t)blockIdx.x * N + i) = y;
        if (dstb) {
            uint16_t *b = dstb + (size_t)blockIdx.x * N + i;
            b[0] = f2bf(y.x); b[1] = f2bf(y.y); b[2] = f2bf(y.z); b[3] = f2bf(y.w);
        }
    }
}

template <int G>
__global__ __launch_bounds__(256) void k_swiglu_norm_v(const float *a, const float *b, int ld, const float *sg,
                                                       const float *su, float *dst, uint16_t *dstb, int F, float *ss) {
    __shared__ float red[8];
    const size_t offi = (size_t)blockIdx.x * ld, off = (size_t)blockIdx.x * F;
    float4 z[G];
    float s = 0.f;
    // every load before any use (computing each group as it arrived waited
    // for the groups one at a time)
    float4 la[G], lb[G], lg[G], lu[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int i = 4 * (threadIdx.x + 256 * j), ic = i < F ? i : 0;
        la[j] = *reinterpret_cast<const float4 *>(a + offi + ic);
        lb[j] = *reinterpret_cast<const float4 *>(b + offi + ic);
        lg[j] = *reinterpret_cast<const float4 *>(sg + ic);
        lu[j] = *reinterpret_cast<const float4 *>(su + ic);
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
        asm volatile("" ::"v"(la[j].x), "v"(la[j].w), "v"(lb[j].x), "v"(lb[j].w), "v"(lg[j].x), "v"(lg[j].w),
                     "v"(lu[j].x), "v"(lu[j].w));
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int i = 4 * (threadIdx.x + 256 * j);
        const float4 va = la[j], vb = lb[j], vg = lg[j], vu = lu[j];
        const float ga[4] = {va.x * vg.x, va.y * vg.y, va.z * vg.z, va.w * vg.w};
        const float ub[4] = {vb.x * vu.x, vb.y * vu.y, vb.z * vu.z, vb.w * vu.w};
        float zz[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) zz[c] = i < F ? ga[c] / (1.0f + expf(-ga[c])) * ub[c] : 0.f;
        z[j] = make_float4(zz[0], zz[1], zz[2], zz[3]);
        s += zz[0] * zz[0] + zz[1] * zz[1] + zz[2] * zz[2] + zz[3] * zz[3];
    }
    // with ss the stores need not wait for the row's sum
    float f = 1.f;
    if (!ss) f = norm_factor(block_sum(s, red));
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int i = 4 * (threadIdx.x + 256 * j);
        if (i >= F) continue;
        const float4 y = make_float4(z[j].x * f, z[j].y * f, z[j].z * f, z[j].w * f);
        if (dst) *reinterpret_cast<float4 *>(dst + off + i) = y;
        if (dstb) {
            const uint32_t lo = (uint32_t)f2bf(y.x) | ((uint32_t)f2bf(y.y) << 16);
            const uint32_t hi = (uint32_t)f2bf(y.z) | ((uint32_t)f2bf(y.w) << 16);
            *reinterpret_cast<uint2 *>(dstb + off + i) = make_uint2(lo, hi);
        }
    }
    if (ss) {
        s = block_sum(s, red);
        if (threadIdx.x == 0) ss[blockIdx.x] = s;
    }
}

// dory.rs `head` for every row of a batch: the logit scale, and each row's
// logits to its place in the caller's array.
__global__ __launch_bounds__(256) void k_logits_rows(const float *hlog, const float *ls, int V, const CallRec *rec) {
    const int r = blockIdx.y;
    const int v = blockIdx.x * 256 + threadIdx.x;
    if (v >= V || rec->logits == nullptr) return;
    rec->logits[(size_t)rec->rows[r].out * V + v] = hlog[(size_t)r * V + v] * ls[v];
}

// dory.rs `top_prob`: the softmax probability of the largest logit, the terms
// more than 20 below it left out, the sum in f64.  One workgroup of 1024
// threads: the maximum, then the sum, each reduced through LDS.
__global__ __launch_bounds__(1024) void k_top_prob(const CallRec *rec, int V, float *__restrict__ out) {
    __shared__ float mx[16];
    const float *lg = rec->logits;  // the call's logits row (one-row calls: row 0)
    __shared__ double sm[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float m = -INFINITY;
    for (int i = tid; i < V; i += 1024) m = fmaxf(m, lg[i]);
    m = wave_max(m);
    if (lane == 0) mx[wave] = m;
    __syncthreads();
    float top = mx[0];
#pragma unroll
    for (int w = 1; w < 16; ++w) top = fmaxf(top, mx[w]);
    double d = 0.0;
    for (int i = tid; i < V; i += 1024) {
        const float t = lg[i] - top;
        if (t > -20.0f) d += exp((double)t);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) d += __shfl_xor(d, off);
    if (lane == 0) sm[wave] = d;
    __syncthreads();
    if (tid == 0) {
        double den = 0.0;
#pragma unroll
        for (int w = 0; w < 16; ++w) den += sm[w];
        *out = (float)(1.0 / den);
    }
}

__global__ __launch_bounds__(256) void k_add_slabs(float *x, size_t n4, int parts, size_t stride4) {
    float4 *x4 = reinterpret_cast<float4 *>(x);
    for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
        float4 v = x4[i];
        for (int z = 1; z < parts; ++z) {
            const float4 u = x4[i + z * stride4];
            v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
        }
        x4[i] = v;
    }
}

}  // namespace

hipError_t launch_top_prob(const CallRec *rec, int V, float *out, hipStream_t s) {
    if (V <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_top_prob, dim3(1), dim3(1024), 0, s, rec, V, out);
    return hipGetLastError();
}

hipError_t launch_logits_rows(const float *hlog, const float *ls, int V, int T, const CallRec *rec, hipStream_t s) {
    hipLaunchKernelGGL(k_logits_rows, dim3((V + 255) / 256, T), dim3(256), 0, s, hlog, ls, V, rec);
    return hipGetLastError();
}

hipError_t launch_embed(int wtype, const void *E, int V, int H, const CallRec *rec, int T, float *h,
                        uint16_t *hb, hipStream_t s) {
    if (wtype == kBF16) hipLaunchKernelGGL((k_embed<kBF16>), dim3(T), dim3(256), 0, s, E, V, H, rec, h, hb);
    else hipLaunchKernelGGL((k_embed<kF32>), dim3(T), dim3(256), 0, s, E, V, H, rec, h, hb);
    return hipGetLastError();
}

template <int EPT>
hipError_t launch_resolve_p(const Resolve &rs, int H, int T, float *tap, int tap_n, hipStream_t s) {
    const int parts = rs.slerp && rs.o_parts > 1 ? rs.o_parts : 1;
    if (parts == 1) hipLaunchKernelGGL((k_resolve_rows<EPT, 1>), dim3(T), dim3(256), 0, s, rs, H, tap, tap_n);
    else if (parts == 2) hipLaunchKernelGGL((k_resolve_rows<EPT, 2>), dim3(T), dim3(256), 0, s, rs, H, tap, tap_n);
    else if (parts <= 4) hipLaunchKernelGGL((k_resolve_rows<EPT, 4>), dim3(T), dim3(256), 0, s, rs, H, tap, tap_n);
    else hipLaunchKernelGGL((k_resolve_rows<EPT, 8>), dim3(T), dim3(256), 0, s, rs, H, tap, tap_n);
    return hipGetLastError();
}

hipError_t launch_resolve_rows(const Resolve &rs, int H, int T, const CallRec *rec, float *tap, int tap_n,
                               hipStream_t s) {
    (void)rec;  // what the kernel would read from it comes as tap, tap_n
    if (rs.slerp && rs.o_parts > kMaxKParts) return hipErrorInvalidValue;
    if (rs.slerp && rs.o_ss && (rs.o_ss_n < 1 || rs.o_ss_n > 128)) return hipErrorInvalidValue;
    if (tap && tap_n < T) return hipErrorInvalidValue;
    if (H <= 2048) return launch_resolve_p<8>(rs, H, T, tap, tap_n, s);
    if (H <= 4096) return launch_resolve_p<16>(rs, H, T, tap, tap_n, s);
    if (H <= 8192) return launch_resolve_p<32>(rs, H, T, tap, tap_n, s);
    return hipErrorInvalidValue;
}

#define DK_G_SWITCH(G, KERNEL, ...)                                                          \
    switch (G) {                                                                              \
        case 1: hipLaunchKernelGGL((KERNEL<1>), __VA_ARGS__); break;                          \
        case 2: hipLaunchKernelGGL((KERNEL<2>), __VA_ARGS__); break;                          \
        case 3: hipLaunchKernelGGL((KERNEL<3>), __VA_ARGS__); break;                          \
        case 4: hipLaunchKernelGGL((KERNEL<4>), __VA_ARGS__); break;                          \
        case 5: case 6: hipLaunchKernelGGL((KERNEL<6>), __VA_ARGS__); break;                  \
        default: hipLaunchKernelGGL((KERNEL<8>), __VA_ARGS__); break;                         \
    }

hipError_t launch_rownorm(const float *src, int ld, float *dst, uint16_t *dstb, int N, int T, hipStream_t s) {
    const int G = (N / 4 + 255) / 256;
    if (N % 4 == 0 && ld % 4 == 0 && G <= 8) {
        DK_G_SWITCH(G, k_rownorm_v, dim3(T), dim3(256), 0, s, src, ld, dst, dstb, N)
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_rownorm, dim3(T), dim3(256), 0, s, src, ld, dst, dstb, N);
    return hipGetLastError();
}

hipError_t launch_add_slabs(float *x, size_t n, int parts, size_t stride, hipStream_t s) {
    if (!x || parts < 1) return hipErrorInvalidValue;
    if (parts == 1 || n == 0) return hipSuccess;
    if (n % 4 || stride % 4 || stride < n) return hipErrorInvalidValue;
    const size_t n4 = n / 4;
    const unsigned blocks = (unsigned)((n4 + 255) / 256 < 1024 ? (n4 + 255) / 256 : 1024);
    hipLaunchKernelGGL(k_add_slabs, dim3(blocks), dim3(256), 0, s, x, n4, parts, stride / 4);
    return hipGetLastError();
}

hipError_t launch_swiglu_norm(const float *a, const float *b, int ld, const float *sg, const float *su, float *dst,
                              uint16_t *dstb, int F, int T, hipStream_t s, float *ss) {
    const int G = (F / 4 + 255) / 256;
    if (F % 4 == 0 && ld % 4 == 0 && G <= 8) {
        DK_G_SWITCH(G, k_swiglu_norm_v, dim3(T), dim3(256), 0, s, a, b, ld, sg, su, dst, dstb, F, ss)
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_swiglu_norm, dim3(T), dim3(256), sizeof(float) * (F + 8), s, a, b, ld, sg, su, dst, dstb, F,
                       ss);
    return hipGetLastError();
}

}  // namespace dk
