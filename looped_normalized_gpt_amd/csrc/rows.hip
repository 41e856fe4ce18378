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

__global__ __launch_bounds__(256) void k_resolve_rows(Resolve rs, int H, const CallRec *rec) {
    extern __shared__ float smem[];
    resolve_row(rs, blockIdx.x, H, smem + 8, smem, true, rec);
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

// dory.rs `mlp_layer`: z = silu(a*sg) * (b*su), then justnorm over F.
__global__ __launch_bounds__(256) void k_swiglu_norm(const float *a, const float *b, int ld, const float *sg,
                                                     const float *su, float *dst, uint16_t *dstb, int F) {
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
    const float f = norm_factor(block_sum(s, red));
    for (int i = threadIdx.x; i < F; i += 256) {
        const float v = z[i] * f;
        dst[off + i] = v;
        if (dstb) dstb[off + i] = f2bf(v);
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

}  // namespace

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

hipError_t launch_resolve_rows(const Resolve &rs, int H, int T, const CallRec *rec, hipStream_t s) {
    hipLaunchKernelGGL(k_resolve_rows, dim3(T), dim3(256), sizeof(float) * (H + 8), s, rs, H, rec);
    return hipGetLastError();
}

hipError_t launch_rownorm(const float *src, int ld, float *dst, uint16_t *dstb, int N, int T, hipStream_t s) {
    hipLaunchKernelGGL(k_rownorm, dim3(T), dim3(256), 0, s, src, ld, dst, dstb, N);
    return hipGetLastError();
}

hipError_t launch_swiglu_norm(const float *a, const float *b, int ld, const float *sg, const float *su, float *dst,
                              uint16_t *dstb, int F, int T, hipStream_t s) {
    hipLaunchKernelGGL(k_swiglu_norm, dim3(T), dim3(256), sizeof(float) * (F + 8), s, a, b, ld, sg, su, dst, dstb, F);
    return hipGetLastError();
}

}  // namespace dk
