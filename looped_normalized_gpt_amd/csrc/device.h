// device.h -- wavefront and workgroup helpers for the gfx950 kernels (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace dk {

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// A load through a global-address-space pointer.  Pointers fetched from memory
// (the slot table) are generic to the compiler, which then emits flat loads;
// those also count against the LDS wait counter, so an LDS wait would wait for
// them too.
typedef float gf32x4_t __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ T gld(const void *p) {  // scalars
    return *(const __attribute__((address_space(1))) T *)(p);
}
__device__ __forceinline__ float4 gld4(const float *p) {
    const gf32x4_t v = *(const __attribute__((address_space(1))) gf32x4_t *)(p);
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 gld_codes4(const int8_t *p) {  // 4 int8 codes as floats
    const int u = *(const __attribute__((address_space(1))) int *)(p);
    return make_float4((float)(int8_t)(u & 0xff), (float)(int8_t)((u >> 8) & 0xff), (float)(int8_t)((u >> 16) & 0xff),
                       (float)(int8_t)((u >> 24) & 0xff));
}

// e^x on the hardware exp2 (about 1 ulp of exp2, plus the rounding of
// x*log2(e)): for softmax weights, where the libm expf's range reduction costs
// a long dependent chain.  e^-inf = 0.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// fp32 -> bf16 bits, round to nearest even
__device__ __forceinline__ uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Cross-lane steps on wave64 without LDS traffic: DPP quad permutes and row
// mirrors inside 16-lane rows, a swizzle across the two rows of a 32-lane half,
// and a bpermute across the halves.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float swap16(float v) {  // lane i <-> lane i ^ 16 (within 32)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
__device__ __forceinline__ float swap32(float v) { return __shfl_xor(v, 32, 64); }

// Sum over aligned groups of G lanes (G a power of two, <= 64); every lane of
// a group gets the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if (G >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if (G >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if (G >= 8) v += dpp<0x141>(v);   // row_half_mirror: the other quad of 8
    if (G >= 16) v += dpp<0x140>(v);  // row_mirror: the other 8 of 16
    if (G >= 32) v += swap16(v);
    if (G >= 64) v += swap32(v);
    return v;
}

template <int G>
__device__ __forceinline__ float group_max(float v) {
    if (G >= 2) v = fmaxf(v, dpp<0xB1>(v));
    if (G >= 4) v = fmaxf(v, dpp<0x4E>(v));
    if (G >= 8) v = fmaxf(v, dpp<0x141>(v));
    if (G >= 16) v = fmaxf(v, dpp<0x140>(v));
    if (G >= 32) v = fmaxf(v, swap16(v));
    if (G >= 64) v = fmaxf(v, swap32(v));
    return v;
}


// The sum over the wave, complete in lane 63 only (the other lanes hold
// partial sums): DPP row reductions, then the row broadcasts of lanes 15 and
// 31; no LDS permutes, so it costs no LDS round trip.
__device__ __forceinline__ float wave_sum63(float v) {
    v = group_sum<16>(v);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
    return v;
}
__device__ __forceinline__ float wave_max63(float v) {
    v = group_max<16>(v);
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x142, 0xA, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x143, 0xC, 0xF, false)));
    return v;
}
// Every lane gets the wave's sum / maximum (lane 63's, read into a scalar).
__device__ __forceinline__ float wave_sum(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum63(v)), 63));
}
__device__ __forceinline__ float wave_max(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_max63(v)), 63));
}

// Sums of two values over a 256-thread workgroup; every thread gets both
// results.  slot < 0: red[0..8), after a barrier (red may still be read by a
// previous reduction).  slot 0 or 1: red[8*slot..8*slot+8) and no leading
// barrier; the caller alternates the slots, so a reduction never overwrites
// values another thread may still be reading.
__device__ __forceinline__ void block_sum2(float &a, float &b, float *red, int slot = -1) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    a = wave_sum63(a);
    b = wave_sum63(b);
    float *r = red;
    if (slot < 0) __syncthreads();
    else r = red + 8 * slot;
    if (lane == 63) {
        r[wave] = a;
        r[4 + wave] = b;
    }
    __syncthreads();
    a = r[0] + r[1] + r[2] + r[3];
    b = r[4] + r[5] + r[6] + r[7];
}

__device__ __forceinline__ float block_sum(float a, float *red, int slot = -1) {
    float b = 0.f;
    block_sum2(a, b, red, slot);
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
    if (rs.loop_op == kLoopExit && r >= rs.n_prev) {
        // a batch row that stopped looping early: its state is kept in st
        for (int i = tid; i < H; i += 256) xs[i] = rs.st[(size_t)r * H + i];
        if (writer && rs.h_out)
            for (int i = tid; i < H; i += 256) rs.h_out[(size_t)r * H + i] = xs[i];
        if (writer && rs.hb_out)
            for (int i = tid; i < H; i += 256) rs.hb_out[(size_t)r * H + i] = f2bf(xs[i]);
        return;
    }
    const float *h = rs.h + (size_t)r * H;
    if (!rs.slerp) {
        for (int i = tid; i < H; i += 256) xs[i] = h[i];
    } else {
        // dory.rs `slerp`: x^ = norm(h), o^ = norm(o), e = norm(x^ + alpha*(o^ - x^))
        // o: the sum of the split-K slabs of the sub-layer's output projection
        const float *o = rs.o + (size_t)r * H;
        auto oval = [&](int i) {
            float v = o[i];
            for (int p = 1; p < rs.o_parts; ++p) v += o[(size_t)p * rs.o_stride + i];
            return v;
        };
        float sx = 0.f, so = 0.f;
        for (int i = tid; i < H; i += 256) {
            float a = h[i], b = oval(i);
            xs[i] = a;
            sx += a * a;
            so += b * b;
        }
        block_sum2(sx, so, red);
        const float rx = norm_factor(sx), ro = norm_factor(so);
        float se = 0.f;
        for (int i = tid; i < H; i += 256) {
            float xh = xs[i] * rx, oh = oval(i) * ro;
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
                for (int i = tid; i < H; i += 256) xs[i] *= fs;
                if (writer && rs.st)
                    for (int i = tid; i < H; i += 256) rs.st[(size_t)r * H + i] = xs[i];
                if (r >= rs.n_next) return;  // this row's loops are over
                float s2 = 0.f;
                for (int i = tid; i < H; i += 256) {
                    float x = xs[i] + inp[i];
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
    if (writer && rs.hb_out) {
        uint16_t *hb = rs.hb_out + (size_t)r * H;
        for (int i = tid; i < H; i += 256) hb[i] = f2bf(xs[i]);
    }
}

// The same step with the inputs already in registers.  Thread tid holds the
// row's elements elem_index<MAP>(j) in slots j < EPT (zeros past H): MAP 0, the
// float4 groups at 4*tid + 1024*jj; MAP 1, the GEMV's dot layout, 8
// consecutive elements of each 512-wide chunk (wave + 4c) at lane*8 (slots
// 8c .. 8c+7).  h, o, al, in: the residual, the sub-layer output, |alpha| and
// the loop input.  No global loads, so it can run while a caller's earlier
// loads are still in flight.
template <int MAP>
__device__ __forceinline__ int elem_index(int j) {
    if (MAP == 0) return 4 * (int)threadIdx.x + 1024 * (j >> 2) + (j & 3);
    return (((int)threadIdx.x >> 6) + 4 * (j >> 3)) * 512 + ((int)threadIdx.x & 63) * 8 + (j & 7);
}
__device__ __forceinline__ int reg_index(int j) { return elem_index<0>(j); }

// Row sums of R = 4, 8, 16 or 32 values a lane, by a reduce-scatter: each
// step pairs lanes that differ in one bit (the swap of 16 lanes, row mirror,
// half-row mirror, the two quad permutes) and halves what a lane holds, so
// lane i ends with value i % R summed over its R-lane group; rotations inside
// the 16-lane row and the swap of 16 lanes then add the groups of its 32-lane
// half.  Lanes whose lane % 32 < R return row lane % 32 summed over their half
// of the wave.
template <int BIT, int R>
__device__ __forceinline__ void rs_step(const float (&v)[R], float (&out)[R / 2], int lane) {
    const bool hi = (lane >> BIT) & 1;
#pragma unroll
    for (int k = 0; k < R / 2; ++k) {
        const float send = hi ? v[k] : v[R / 2 + k], keep = hi ? v[R / 2 + k] : v[k];
        const float got = BIT == 4   ? swap16(send)
                          : BIT == 3 ? dpp<0x140>(send)
                          : BIT == 2 ? dpp<0x141>(send)
                          : BIT == 1 ? dpp<0x4E>(send)
                                     : dpp<0xB1>(send);
        out[k] = keep + got;
    }
}
template <int R>
__device__ __forceinline__ float row_sums_rs(const float (&v)[R], int lane) {
    static_assert(R == 4 || R == 8 || R == 16 || R == 32, "rows a lane");
    float r;
    if constexpr (R == 32) {
        float t16[16], t8[8], t4[4], t2[2], t1[1];
        rs_step<4, 32>(v, t16, lane);
        rs_step<3, 16>(t16, t8, lane);
        rs_step<2, 8>(t8, t4, lane);
        rs_step<1, 4>(t4, t2, lane);
        rs_step<0, 2>(t2, t1, lane);
        return t1[0];
    } else if constexpr (R == 16) {
        float t8[8], t4[4], t2[2], t1[1];
        rs_step<3, 16>(v, t8, lane);
        rs_step<2, 8>(t8, t4, lane);
        rs_step<1, 4>(t4, t2, lane);
        rs_step<0, 2>(t2, t1, lane);
        r = t1[0];
    } else if constexpr (R == 8) {
        float t4[4], t2[2], t1[1];
        rs_step<2, 8>(v, t4, lane);
        rs_step<1, 4>(t4, t2, lane);
        rs_step<0, 2>(t2, t1, lane);
        r = t1[0];
        r += dpp<0x128>(r);  // row_ror:8
    } else {
        float t2[2], t1[1];
        rs_step<1, 4>(v, t2, lane);
        rs_step<0, 2>(t2, t1, lane);
        r = t1[0];
        r += dpp<0x128>(r);  // row_ror:8
        r += dpp<0x124>(r);  // row_ror:4
    }
    return r + swap16(r);
}

// The record's tap row of pass `pass`, row r, rows of n floats (null: no tap).
__device__ __forceinline__ float *tap_row(const CallRec *rec, int pass, int r, int n) {
    if (pass < 0) return nullptr;
    float *t = rec->tap;
    return t ? t + ((size_t)pass * rec->n + r) * n : nullptr;
}

// tap: where the writer stores e for the record's tap (row r of pass
// rs.tap_pass), or null; callers read the record's pointer ahead, with their
// other loads.
// xo: if not null, the resulting x, slot for slot (the GEMV's dots read it from
// registers).
template <int EPT, int MAP = 0>
__device__ inline void resolve_regs(const Resolve &rs, int r, int H, const float (&h)[EPT], const float (&o)[EPT],
                                    const float (&al)[EPT], const float (&in)[EPT], float *xs, float *red,
                                    bool writer, float *tap, float *xo = nullptr) {
    float e[EPT];
    if (!rs.slerp) {
#pragma unroll
        for (int j = 0; j < EPT; ++j) e[j] = h[j];
    } else {
        float sx = 0.f, so = 0.f;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            sx += h[j] * h[j];
            so += o[j] * o[j];
        }
        block_sum2(sx, so, red, 0);
        const float rx = norm_factor(sx), ro = norm_factor(so);
        float se = 0.f;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const float xh = h[j] * rx, oh = o[j] * ro;
            e[j] = xh + al[j] * (oh - xh);
            se += e[j] * e[j];
        }
        const float re = norm_factor(block_sum(se, red, 1));
#pragma unroll
        for (int j = 0; j < EPT; ++j) e[j] *= re;
    }
    if (writer && tap) {
#pragma unroll
        for (int j = 0; j < EPT; j += 4)
            if (elem_index<MAP>(j) < H) *reinterpret_cast<float4 *>(tap + elem_index<MAP>(j)) = make_float4(e[j], e[j + 1], e[j + 2], e[j + 3]);
    }
    if (rs.loop_op == kLoopEnter) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < EPT; j += 4) {
            if (writer && elem_index<MAP>(j) < H)
                *reinterpret_cast<float4 *>(rs.inp + (size_t)r * H + elem_index<MAP>(j)) =
                    make_float4(e[j], e[j + 1], e[j + 2], e[j + 3]);
        }
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            e[j] = e[j] + e[j];
            s += e[j] * e[j];
        }
        const float f = norm_factor(block_sum(s, red, 0));
#pragma unroll
        for (int j = 0; j < EPT; ++j) e[j] *= f;
    } else if (rs.loop_op != kLoopNone) {
        if (rs.loop_op == kLoopExit && writer && rs.e_out)
#pragma unroll
            for (int j = 0; j < EPT; j += 4)
                if (elem_index<MAP>(j) < H)
                    *reinterpret_cast<float4 *>(rs.e_out + (size_t)r * H + elem_index<MAP>(j)) =
                        make_float4(e[j], e[j + 1], e[j + 2], e[j + 3]);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < EPT; ++j) s += e[j] * e[j];
        const float fs = norm_factor(block_sum(s, red, 0));
#pragma unroll
        for (int j = 0; j < EPT; ++j) e[j] *= fs;
        if (rs.loop_op == kLoopNext) {
            if (writer && rs.st)  // batches: every row's loop state
#pragma unroll
                for (int j = 0; j < EPT; j += 4)
                    if (elem_index<MAP>(j) < H)
                        *reinterpret_cast<float4 *>(rs.st + (size_t)r * H + elem_index<MAP>(j)) =
                            make_float4(e[j], e[j + 1], e[j + 2], e[j + 3]);
            if (r >= rs.n_next) return;  // this row's loops are over (uniform over the workgroup)
            float s2 = 0.f;
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                e[j] = e[j] + in[j];
                s2 += e[j] * e[j];
            }
            const float f = norm_factor(block_sum(s2, red, 1));
#pragma unroll
            for (int j = 0; j < EPT; ++j) e[j] *= f;
        }
    }
    if (xo)
#pragma unroll
        for (int j = 0; j < EPT; ++j) xo[j] = e[j];
#pragma unroll
    for (int j = 0; j < EPT; j += 4) {
        const int i = elem_index<MAP>(j);
        if (i < H) {
            const float4 v = make_float4(e[j], e[j + 1], e[j + 2], e[j + 3]);
            if (xs) *reinterpret_cast<float4 *>(xs + i) = v;
            if (writer && rs.h_out) *reinterpret_cast<float4 *>(rs.h_out + (size_t)r * H + i) = v;
            if (writer && rs.hb_out) {
                uint16_t *hb = rs.hb_out + (size_t)r * H + i;
                hb[0] = f2bf(v.x); hb[1] = f2bf(v.y); hb[2] = f2bf(v.z); hb[3] = f2bf(v.w);
            }
        }
    }
}

// kv_cache.rs `quant_row` for one row of n <= 256 values, one wave: r = x/col
// (x when col is null); per group of `group` channels (32, or one group when
// group >= n) scale = max(absmax/127, 1e-12) and code = clamp(round(r/scale),
// -127, 127), rounding half away from zero.  Only IEEE correctly rounded
// divisions and exact max/abs/round: no step a compiler could contract, so the
// codes and scales equal the fp32 definition bit for bit.
__device__ inline void encode_row(const float *x, const float *col, int n, int group, int8_t *codes,
                                  float *scales) {
    const int lane = threadIdx.x & 63;
    float r[4];
    float m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        r[i] = 0.f;
        if (d < n) r[i] = col ? __fdiv_rn(x[d], col[d]) : x[d];
        m[i] = fabsf(r[i]);
    }
    if (group >= n) {
        float mm = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
        mm = wave_max(mm);
#pragma unroll
        for (int i = 0; i < 4; ++i) m[i] = mm;
    } else {
        // group == 32: channel lane + 64i is in group (lane >> 5) + 2i, one half-wave
#pragma unroll
        for (int i = 0; i < 4; ++i) m[i] = group_max<32>(m[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d >= n) continue;
        const float s = fmaxf(__fdiv_rn(m[i], 127.0f), 1e-12f);
        float c = roundf(__fdiv_rn(r[i], s));
        c = fminf(fmaxf(c, -127.0f), 127.0f);
        codes[d] = (int8_t)c;
        if (group >= n) {
            if (d == 0) scales[0] = s;
        } else if (d % group == 0) {
            scales[d / group] = s;
        }
    }
}

}  // namespace dk
