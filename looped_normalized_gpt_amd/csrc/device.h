// device.h -- wavefront and workgroup helpers for the gfx950 kernels (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace dk {

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Sum over aligned groups of G lanes (G a power of two, <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sums of two values over a 256-thread workgroup; red holds >= 8 floats.
// Every thread gets both results.
__device__ __forceinline__ void block_sum2(float &a, float &b, float *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    a = wave_sum(a);
    b = wave_sum(b);
    __syncthreads();  // red may still be read by a previous reduction
    if (lane == 0) {
        red[wave] = a;
        red[4 + wave] = b;
    }
    __syncthreads();
    a = red[0] + red[1] + red[2] + red[3];
    b = red[4] + red[5] + red[6] + red[7];
}

__device__ __forceinline__ float block_sum(float a, float *red) {
    float b = 0.f;
    block_sum2(a, b, red);
    return a;
}

// 1/sqrt(s + eps): justnorm's factor (dory.rs `justnorm`).
__device__ __forceinline__ float norm_factor(float s) { return 1.0f / sqrtf(s + kEps); }

// Builds in xs[0..H) the x fed to a sub-layer from the previous one's result
// (see Resolve).  Workgroup of 256 threads; each thread touches only indices
// tid, tid+256, ...  The writer stores h_out / inp / tap for row r.
__device__ inline void resolve_row(const Resolve &rs, int r, int H, float *xs, float *red, bool writer,
                                   const CallRec *rec) {
    const int tid = threadIdx.x;
    const float *h = rs.h + (size_t)r * H;
    if (!rs.slerp) {
        for (int i = tid; i < H; i += 256) xs[i] = h[i];
    } else {
        // dory.rs `slerp`: x^ = norm(h), o^ = norm(o), e = norm(x^ + alpha*(o^ - x^))
        const float *o = rs.o + (size_t)r * H;
        float sx = 0.f, so = 0.f;
        for (int i = tid; i < H; i += 256) {
            float a = h[i], b = o[i];
            xs[i] = a;
            sx += a * a;
            so += b * b;
        }
        block_sum2(sx, so, red);
        const float rx = norm_factor(sx), ro = norm_factor(so);
        float se = 0.f;
        for (int i = tid; i < H; i += 256) {
            float xh = xs[i] * rx, oh = o[i] * ro;
            float e = xh + rs.alpha[i] * (oh - xh);
            xs[i] = e;
            se += e * e;
        }
        const float re = norm_factor(block_sum(se, red));
        for (int i = tid; i < H; i += 256) xs[i] *= re;
    }
    if (writer && rec->tap && rs.tap_pass >= 0) {
        float *t = rec->tap + ((size_t)rs.tap_pass * rec->n + r) * H;
        for (int i = tid; i < H; i += 256) t[i] = xs[i];
    }
    // dory.rs `stack`: the loop's mix of state and input.
    if (rs.loop_op != kLoopNone) {
        float *inp = rs.inp + (size_t)r * H;
        if (rs.loop_op == kLoopEnter) {
            float s = 0.f;
            for (int i = tid; i < H; i += 256) {
                float e = xs[i];
                if (writer) inp[i] = e;
                float x = e + e;
                xs[i] = x;
                s += x * x;
            }
            const float f = norm_factor(block_sum(s, red));
            for (int i = tid; i < H; i += 256) xs[i] *= f;
        } else {
            float s = 0.f;
            for (int i = tid; i < H; i += 256) s += xs[i] * xs[i];
            const float fs = norm_factor(block_sum(s, red));
            if (rs.loop_op == kLoopExit) {
                for (int i = tid; i < H; i += 256) xs[i] *= fs;
            } else {
                float s2 = 0.f;
                for (int i = tid; i < H; i += 256) {
                    float x = xs[i] * fs + inp[i];
                    xs[i] = x;
                    s2 += x * x;
                }
                const float f = norm_factor(block_sum(s2, red));
                for (int i = tid; i < H; i += 256) xs[i] *= f;
            }
        }
    }
    if (writer && rs.h_out) {
        float *ho = rs.h_out + (size_t)r * H;
        for (int i = tid; i < H; i += 256) ho[i] = xs[i];
    }
}

}  // namespace dk
