// q8.hip -- the q8_2f cache encoding (kv_cache.rs `quant_row`, `freeze_cols`,
// `append`), and fp32 cache rows written from outside a forward.
//
// The codes, scales and fields must equal, bit for bit, what the page's fp32
// steps give for the same fp32 rows.  So this file is built with fp contraction
// off, and every step that rounds is an IEEE correctly rounded operation: the
// divisions (x/col, absmax/127, r/scale, sum/n), the square root (the compiler's
// default correctly rounded sqrt; HIP's __fsqrt_rn is the approximate native
// one unless the OCML rounded operations are enabled), and the product and sum
// of the field's sum of squares, taken in row order.
#include "device.h"

namespace dk {

namespace {

// One wave per (row of the call, kv head): the row's K (groups of 32) and V (one
// group of hd) into ring row p % cap, against the field when it is frozen.
__global__ __launch_bounds__(64) void k_q8_write(Q8WriteArgs a) {
    const int r = a.r0 + blockIdx.x, kh = blockIdx.y;
    const int hd = a.hd, ngk = (hd + kKGroup - 1) / kKGroup;
    const CallRec *rec = a.rec;
    const SlotDesc &sd = slot_at(a.tab, rec->rows[r].seq, a.n_ord, a.ord, a.slot);
    const int64_t p = rec->rows[r].pos;
    const size_t row = (size_t)kh * sd.cap + (size_t)(p % sd.cap);
    encode_row(a.ksrc + (size_t)r * a.kld + kh * hd, a.field ? sd.kcol + kh * hd : nullptr, hd, kKGroup,
               sd.kc + row * hd, sd.ks + row * ngk);
    encode_row(a.vsrc + (size_t)r * a.vld + kh * hd, a.field ? sd.vcol + kh * hd : nullptr, hd, hd,
               sd.vc + row * hd, sd.vs + row);
}

// kv_cache.rs `freeze_cols` at the 65th append: for each kv head, the field is
// col[d] = max(sqrt(sum_p deq[p][d]^2 / 64), 1e-6) over the 64 stored rows
// (positions 0..63, ring rows 0..63), then every stored row is re-encoded from
// its dequantised values against the field.  One workgroup per kv head.
__global__ __launch_bounds__(256) void k_q8_freeze(const SlotDesc *tab, int n_ord, int ord, int slot,
                                                   int hd, const CallRec *rec, int crow) {
    __shared__ float kcol[256], vcol[256];
    __shared__ float deq[4][2][256];
    const int kh = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ngk = (hd + kKGroup - 1) / kKGroup;
    const SlotDesc &sd = slot_at(tab, rec->rows[crow].seq, n_ord, ord, slot);
    const size_t base = (size_t)kh * sd.cap;
    const int n = kWarmup;
    if (tid < hd) {
        const int d = tid;
        float ck = 0.f, cv = 0.f;
        for (int p = 0; p < n; ++p) {
            const size_t row = base + p;
            const float dk = __fmul_rn((float)sd.kc[row * hd + d], sd.ks[row * ngk + d / kKGroup]);
            const float dv = __fmul_rn((float)sd.vc[row * hd + d], sd.vs[row]);
            ck = __fadd_rn(ck, __fmul_rn(dk, dk));
            cv = __fadd_rn(cv, __fmul_rn(dv, dv));
        }
        ck = fmaxf(__builtin_sqrtf(__fdiv_rn(ck, (float)n)), 1e-6f);
        cv = fmaxf(__builtin_sqrtf(__fdiv_rn(cv, (float)n)), 1e-6f);
        kcol[d] = ck;
        vcol[d] = cv;
        sd.kcol[kh * hd + d] = ck;
        sd.vcol[kh * hd + d] = cv;
    }
    __syncthreads();
    for (int p = wave; p < n; p += 4) {
        const size_t row = base + p;
        for (int d = lane; d < hd; d += 64) {
            deq[wave][0][d] = __fmul_rn((float)sd.kc[row * hd + d], sd.ks[row * ngk + d / kKGroup]);
            deq[wave][1][d] = __fmul_rn((float)sd.vc[row * hd + d], sd.vs[row]);
        }
        __syncthreads();
        encode_row(deq[wave][0], kcol, hd, kKGroup, sd.kc + row * hd, sd.ks + row * ngk);
        encode_row(deq[wave][1], vcol, hd, hd, sd.vc + row * hd, sd.vs + row);
        __syncthreads();
    }
}

__global__ __launch_bounds__(64) void k_q8_encode_rows(const float *x, const float *col, int n, int group,
                                                       int8_t *codes, float *scales) {
    const int r = blockIdx.x, ng = group >= n ? 1 : (n + group - 1) / group;
    encode_row(x + (size_t)r * n, col, n, group, codes + (size_t)r * n, scales + (size_t)r * ng);
}

__global__ __launch_bounds__(64) void k_kv_store(const float *k, const float *v, const SlotDesc *tab, int n_ord,
                                                 int ord, int slot, int nk, int hd, const CallRec *rec) {
    const int r = blockIdx.x, kh = blockIdx.y;
    const SlotDesc &sd = slot_at(tab, rec->rows[r].seq, n_ord, ord, slot);
    const int64_t p = rec->rows[r].pos;
    const size_t row = (size_t)kh * sd.cap + (size_t)(p % sd.cap);
    const size_t src = ((size_t)r * nk + kh) * hd;
    for (int d = threadIdx.x; d < hd; d += 64) {
        sd.k[row * hd + d] = k[src + d];
        sd.v[row * hd + d] = v[src + d];
    }
}

}  // namespace

hipError_t launch_q8_write(const Q8WriteArgs &a, hipStream_t s) {
    if (a.r1 <= a.r0) return hipSuccess;
    hipLaunchKernelGGL(k_q8_write, dim3(a.r1 - a.r0, a.nk), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_q8_freeze(const SlotDesc *tab, int n_ord, int ord, int slot, int nk, int hd, const CallRec *rec,
                            int row, hipStream_t s) {
    hipLaunchKernelGGL(k_q8_freeze, dim3(nk), dim3(256), 0, s, tab, n_ord, ord, slot, hd, rec, row);
    return hipGetLastError();
}

hipError_t launch_q8_encode_rows(const float *x, const float *col, int rows, int n, int group, int8_t *codes,
                                 float *scales, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_q8_encode_rows, dim3(rows), dim3(64), 0, s, x, col, n, group, codes, scales);
    return hipGetLastError();
}

hipError_t launch_kv_store(const float *k, const float *v, const SlotDesc *tab, int n_ord, int ord, int slot,
                           int nk, int hd, int T, const CallRec *rec, hipStream_t s) {
    hipLaunchKernelGGL(k_kv_store, dim3(T, nk), dim3(64), 0, s, k, v, tab, n_ord, ord, slot, nk, hd, rec);
    return hipGetLastError();
}

}  // namespace dk
