// attn.hip -- the attention sub-layer between its projections: RoPE and unit
// norms with the cache write (prep), and grouped-query attention over the ring
// with the sigmoid gate (attn).
#include "device.h"

namespace dk {

namespace {

// dory.rs `attn_layer` (rotate, justnorm per head, q times sq) and `stack` (the
// RoPE tables: angle = position * inverse frequency in f64, cos/sin rounded to
// f32).  One wave per (row, head); lane j owns the pairs (j, j + hd/2),
// (j + 64, j + 64 + hd/2), ...
__global__ __launch_bounds__(64) void k_prep(PrepArgs a) {
    const int r = blockIdx.x, hh = blockIdx.y, lane = threadIdx.x;
    const int hd = a.hd, half = hd / 2, Q = a.nh * hd, KV = a.nk * hd;
    const int ld = Q + 2 * KV + Q;
    const int64_t p = a.rec->pos0 + r;
    const bool isq = hh < a.nh;
    const int kh = hh - a.nh;
    const float *src = a.qkvg + (size_t)r * ld + (isq ? hh * hd : Q + kh * hd);
    float nx[2], ny[2];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = lane + 64 * i;
        nx[i] = ny[i] = 0.f;
        if (j < half) {
            const double ang = (double)p * (double)a.inv[j];
            const float cs = (float)cos(ang), sn = (float)sin(ang);
            const float x = src[j], y = src[j + half];
            nx[i] = x * cs - y * sn;
            ny[i] = y * cs + x * sn;
            s += nx[i] * nx[i] + ny[i] * ny[i];
        }
    }
    const float f = norm_factor(wave_sum(s));
    if (isq) {
        float *dst = a.qp + (size_t)r * Q + hh * hd;
        const float *sq = a.sq + hh * hd;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int j = lane + 64 * i;
            if (j < half) {
                dst[j] = nx[i] * f * sq[j];
                dst[j + half] = ny[i] * f * sq[j + half];
            }
        }
        return;
    }
    if (a.kstage) {  // q8 cache: the encoder reads the keys from here
        float *dst = a.kstage + (size_t)r * KV + kh * hd;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int j = lane + 64 * i;
            if (j < half) {
                dst[j] = nx[i] * f;
                dst[j + half] = ny[i] * f;
            }
        }
        return;
    }
    const SlotDesc &sd = slot_at(a.tab, a.rec->seq, a.n_ord, a.ord, a.slot);
    const size_t row = (size_t)kh * sd.cap + (size_t)(p % sd.cap);
    float *kd = sd.k + row * hd;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = lane + 64 * i;
        if (j < half) {
            kd[j] = nx[i] * f;
            kd[j + half] = ny[i] * f;
        }
    }
    const float *v = a.qkvg + (size_t)r * ld + Q + KV + kh * hd;
    float *vd = sd.v + row * hd;
    for (int j = lane; j < hd; j += 64) vd[j] = v[j];
}

__device__ __forceinline__ float load_agent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grouped-query attention of one row over keys max(p+1-window, 0) ..= p for the
// REP q heads of one kv head (dory.rs `attn_layer`, the per-(row, kv head)
// task; kv_cache.rs `attend_group_upto` for the q8_2f rows).
//
// Grid (splits, nk, T): workgroup (s, kh, r) takes keys [lo + s*split, ...) of
// row r.  It reads each K row once for its REP heads (HD/4 lanes per key, one
// 16-byte load each), keeps the scores in LDS, takes per-head maxima and sums,
// then reads each V row once.  It leaves (max, sum, unnormalised sum of
// p*v) per head; the last workgroup of (r, kh) to arrive merges the splits in
// log-sum-exp form and applies the sigmoid gate (dory.rs `gate_body`).
template <int HD, int REP, int Q8>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
    constexpr int LPK = HD / 4;       // lanes per key
    constexpr int KPW = 64 / LPK;     // keys per wave step
    constexpr int G = 256 / LPK;      // key groups in the value pass
    constexpr int SLMAX = 256;
    constexpr int NGK = (HD + kKGroup - 1) / kKGroup;
    __shared__ float sc[REP][SLMAX];
    __shared__ float red[G * REP * HD];
    __shared__ float stat[2][REP];
    __shared__ int last;
    const int s = blockIdx.x, kh = blockIdx.y, r = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const CallRec *rec = a.rec;
    const int64_t p = rec->pos0 + r;
    const int64_t lo = p + 1 - a.window > 0 ? p + 1 - a.window : 0;
    const int64_t nkeys = p - lo + 1;
    const int nsplit = (int)((nkeys + a.split - 1) / a.split);
    if (s >= nsplit) return;
    const int64_t e0 = lo + (int64_t)s * a.split;
    const int len = (int)(nkeys - (int64_t)s * a.split < a.split ? nkeys - (int64_t)s * a.split : a.split);
    const SlotDesc &sd = slot_at(a.tab, rec->seq, a.n_ord, a.ord, a.slot);
    const int cap = sd.cap;
    const int Q = a.nh * HD;
    const float scale = 1.0f / sqrtf((float)HD);

    // ---- scores: s_e = q . k_e / sqrt(hd) for each head of the group
    {
        const int g = lane / LPK, dq = lane % LPK;
        float4 q[REP];
        const float *qrow = a.qp + (size_t)r * Q + (size_t)kh * REP * HD + dq * 4;
#pragma unroll
        for (int h = 0; h < REP; ++h) q[h] = *reinterpret_cast<const float4 *>(qrow + h * HD);
        if (Q8 && a.field) {
            const float4 c = *reinterpret_cast<const float4 *>(sd.kcol + kh * HD + dq * 4);
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                q[h].x *= c.x; q[h].y *= c.y; q[h].z *= c.z; q[h].w *= c.w;
            }
        }
        for (int base = 0; base < len; base += 4 * KPW) {
            const int e = base + wave * KPW + g;
            const bool ok = e < len;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
            float ks = 0.f;
            if (ok) {
                const size_t row = (size_t)kh * cap + (size_t)((e0 + e) % cap);
                if (Q8) {
                    const char4 c = *reinterpret_cast<const char4 *>(sd.kc + row * HD + dq * 4);
                    kv = make_float4((float)c.x, (float)c.y, (float)c.z, (float)c.w);
                    ks = sd.ks[row * NGK + (dq * 4) / kKGroup];
                } else {
                    kv = *reinterpret_cast<const float4 *>(sd.k + row * HD + dq * 4);
                }
            }
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                float d = q[h].x * kv.x + q[h].y * kv.y + q[h].z * kv.z + q[h].w * kv.w;
                if (Q8) d *= ks;
                d = group_sum<LPK>(d);
                if (ok && dq == 0) sc[h][e] = d * scale;
            }
        }
    }
    __syncthreads();

    // ---- per-head max and sum of exp (dory.rs `soft_body`)
    for (int h = wave; h < REP; h += 4) {
        float m = -INFINITY;
        for (int e = lane; e < len; e += 64) m = fmaxf(m, sc[h][e]);
        m = wave_max(m);
        float l = 0.f;
        for (int e = lane; e < len; e += 64) {
            const float pv = expf(sc[h][e] - m);
            sc[h][e] = pv;
            l += pv;
        }
        l = wave_sum(l);
        if (lane == 0) {
            stat[0][h] = m;
            stat[1][h] = l;
        }
    }
    __syncthreads();

    // ---- values: acc_h = sum_e p_e v_e
    {
        const int dq = tid % LPK, grp = tid / LPK;
        float4 acc[REP];
#pragma unroll
        for (int h = 0; h < REP; ++h) acc[h] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int e = grp; e < len; e += G) {
            const size_t row = (size_t)kh * cap + (size_t)((e0 + e) % cap);
            float4 vv;
            float vs = 1.f;
            if (Q8) {
                const char4 c = *reinterpret_cast<const char4 *>(sd.vc + row * HD + dq * 4);
                vv = make_float4((float)c.x, (float)c.y, (float)c.z, (float)c.w);
                vs = sd.vs[row];
            } else {
                vv = *reinterpret_cast<const float4 *>(sd.v + row * HD + dq * 4);
            }
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                const float w = Q8 ? sc[h][e] * vs : sc[h][e];
                acc[h].x += w * vv.x;
                acc[h].y += w * vv.y;
                acc[h].z += w * vv.z;
                acc[h].w += w * vv.w;
            }
        }
#pragma unroll
        for (int h = 0; h < REP; ++h)
            *reinterpret_cast<float4 *>(&red[(grp * REP + h) * HD + dq * 4]) = acc[h];
    }
    __syncthreads();
    const size_t pstride = (size_t)REP * (HD + 2);
    float *mine = a.part + (((size_t)r * a.nk + kh) * a.max_split + s) * pstride;
    for (int idx = tid; idx < REP * HD; idx += 256) {
        const int h = idx / HD, d = idx % HD;
        float v = 0.f;
        for (int grp = 0; grp < G; ++grp) v += red[(grp * REP + h) * HD + d];
        mine[h * (HD + 2) + 2 + d] = v;
    }
    if (tid < REP) {
        mine[tid * (HD + 2)] = stat[0][tid];
        mine[tid * (HD + 2) + 1] = stat[1][tid];
    }

    // ---- the last workgroup of (r, kh) merges the splits
    __threadfence();
    __syncthreads();
    if (tid == 0) last = atomicAdd(&a.cnt[r * a.nk + kh], 1) == nsplit - 1;
    __syncthreads();
    if (!last) return;
    __threadfence();
    const float *all = a.part + ((size_t)r * a.nk + kh) * a.max_split * pstride;
    float *wts = red;  // [nsplit][REP]
    if (tid < REP) {
        float M = -INFINITY;
        for (int j = 0; j < nsplit; ++j) M = fmaxf(M, load_agent(all + j * pstride + tid * (HD + 2)));
        float L = 0.f;
        for (int j = 0; j < nsplit; ++j) {
            const float w = expf(load_agent(all + j * pstride + tid * (HD + 2)) - M);
            wts[j * REP + tid] = w;
            L += w * load_agent(all + j * pstride + tid * (HD + 2) + 1);
        }
        const float inv = 1.0f / L;
        for (int j = 0; j < nsplit; ++j) wts[j * REP + tid] *= inv;
    }
    __syncthreads();
    const int ld = Q + 2 * a.nk * HD + Q;
    for (int idx = tid; idx < REP * HD; idx += 256) {
        const int h = idx / HD, d = idx % HD;
        float y = 0.f;
        for (int j = 0; j < nsplit; ++j) y += wts[j * REP + h] * load_agent(all + j * pstride + h * (HD + 2) + 2 + d);
        if (Q8 && a.field) y *= sd.vcol[kh * HD + d];
        const int hq = kh * REP + h;
        const float g = a.qkvg[(size_t)r * ld + Q + 2 * a.nk * HD + hq * HD + d];
        y = y / (1.0f + expf(-(g * a.sg[hq * HD + d])));
        a.z[(size_t)r * Q + hq * HD + d] = y;
    }
    if (tid == 0) a.cnt[r * a.nk + kh] = 0;
}

template <int HD, int REP>
hipError_t launch_hr(const AttnArgs &a, int T, hipStream_t s) {
    dim3 grid(a.max_split, a.nk, T), block(256);
    if (a.q8) hipLaunchKernelGGL((k_attn<HD, REP, 1>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_attn<HD, REP, 0>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int HD>
hipError_t launch_h(const AttnArgs &a, int T, hipStream_t s) {
    switch (a.nh / a.nk) {
        case 1: return launch_hr<HD, 1>(a, T, s);
        case 2: return launch_hr<HD, 2>(a, T, s);
        case 4: return launch_hr<HD, 4>(a, T, s);
        case 8: return launch_hr<HD, 8>(a, T, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prep(const PrepArgs &a, int T, hipStream_t s) {
    hipLaunchKernelGGL(k_prep, dim3(T, a.nh + a.nk), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a, int T, hipStream_t s) {
    if (a.split <= 0 || a.split > 256) return hipErrorInvalidValue;
    switch (a.hd) {
        case 8: return launch_h<8>(a, T, s);
        case 16: return launch_h<16>(a, T, s);
        case 32: return launch_h<32>(a, T, s);
        case 64: return launch_h<64>(a, T, s);
        case 128: return launch_h<128>(a, T, s);
        case 256: return launch_h<256>(a, T, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dk
