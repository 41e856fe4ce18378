// attn.hip -- the attention sub-layer between its projections: RoPE and unit
// norms with the cache write (prep), and grouped-query attention over the ring
// with the sigmoid gate (attn).
#include "device.h"

namespace dk {

namespace {

// Whether the cache rows of call row `row` use the frozen q8_2f field (see
// AttnArgs::field): kv_cache.rs `append` freezes the field at the first append
// with 64 rows stored, and it stays frozen from then on.
__device__ __forceinline__ bool field_on(const AttnArgs &a, const RowRec &row) {
    return a.field > 0 || (a.field < 0 && (row.pos >= kWarmup || row.q8f));
}

// dory.rs `attn_layer` (rotate, justnorm per head, q times sq), with the RoPE
// table row of the position (dory.rs `stack`: cos half, sin half).  One wave
// per (row, head); lane j owns the pairs (j, j + hd/2), (j + 64, j + 64 + hd/2).
// Every load is issued first and unconditionally (clamped, masked at use), and
// nothing is read from the record or the slot table (the host passes the
// chunk's first position and the slot's rings): one round trip a wave, where
// the record, slot and value-row reads had made six.
__global__ __launch_bounds__(64) void k_prep(PrepArgs a) {
    const int r = blockIdx.x, hh = blockIdx.y, lane = threadIdx.x;
    const int hd = a.hd, half = hd / 2, Q = a.nh * hd, KV = a.nk * hd;
    const int ld = Q + 2 * KV + Q;
    const int64_t p = a.pos0 + r;
    const bool isq = hh < a.nh;
    const int kh = hh - a.nh;
    const float *src = a.qkvg + (size_t)r * ld + (isq ? hh * hd : Q + kh * hd);
    const float *vsrc = a.qkvg + (size_t)r * ld + Q + KV + (isq ? 0 : kh) * hd;  // the value row
    const float *rp = a.rope + (size_t)p * hd;
    const float *sqh = a.sq + (size_t)(isq ? hh : 0) * hd;
    float x[2], y[2], cs[2], sn[2], q0[2], q1[2], vv[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = lane + 64 * i, jc = j < half ? j : 0;
        x[i] = src[jc];
        y[i] = src[jc + half];
        cs[i] = rp[jc];
        sn[i] = rp[half + jc];
        q0[i] = sqh[jc];
        q1[i] = sqh[jc + half];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        vv[i] = vsrc[j < hd ? j : 0];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) asm volatile("" ::"v"(x[i]), "v"(y[i]), "v"(cs[i]), "v"(sn[i]), "v"(q0[i]), "v"(q1[i]));
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(vv[i]));
    float nx[2], ny[2];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = lane + 64 * i;
        nx[i] = ny[i] = 0.f;
        if (j < half) {
            nx[i] = x[i] * cs[i] - y[i] * sn[i];
            ny[i] = y[i] * cs[i] + x[i] * sn[i];
            s += nx[i] * nx[i] + ny[i] * ny[i];
        }
    }
    const float f = norm_factor(wave_sum(s));
    if (!isq && a.kvtap) {  // test tap: the row's key and value before the cache write
        float *t = a.kvtap + ((size_t)a.tap_pass * a.kvtap_n + r) * 2 * KV + kh * hd;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int j = lane + 64 * i;
            if (j < half) {
                t[j] = nx[i] * f;
                t[j + half] = ny[i] * f;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i < hd) t[KV + lane + 64 * i] = vv[i];
    }
    if (isq) {
        float *dst = a.qp + (size_t)r * Q + hh * hd;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int j = lane + 64 * i;
            if (j < half) {
                dst[j] = nx[i] * f * q0[i];
                dst[j + half] = ny[i] * f * q1[i];
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
    const size_t row = (size_t)kh * a.cap + (size_t)(p % a.cap);
    float *kd = a.kring + row * hd;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = lane + 64 * i;
        if (j < half) {
            kd[j] = nx[i] * f;
            kd[j + half] = ny[i] * f;
        }
    }
    float *vd = a.vring + row * hd;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < hd) vd[lane + 64 * i] = vv[i];
}


// Merges the split partials of (row r, q head h) in log-sum-exp form, scales by
// the V field (q8), applies the sigmoid gate (dory.rs `gate_body`) and writes z.
// Grid (T, nh, ceil(hd/64)), 4 waves; lane d owns one channel, wave w takes
// splits w, w+4, .. with all U of its loads in flight before the running
// (max, sum, acc) merge, then wave 0 merges the 4 waves' results.  A kernel of
// its own: the partials come from workgroups on other XCDs, whose L2s are only
// coherent with this one at kernel boundaries.
template <int Q8, int U>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
    __shared__ float sm[4][66];
    const int r = blockIdx.x, hq = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = blockIdx.z * 64 + lane;
    const int hd = a.hd, rep = a.nh / a.nk, kh = hq / rep, h = hq % rep;
    const int Q = a.nh * hd, ld = 2 * Q + 2 * a.nk * hd;
    const int dc = d < hd ? d : 0;
    // what does not depend on the partials first
    const float gate = a.qkvg[(size_t)r * ld + Q + 2 * a.nk * hd + hq * hd + dc];
    const float sgv = a.sg[hq * hd + dc];
    int nsplit;
    if (a.dec) {  // decode kernel: every slab of the grid, those past the row's keys hold max -inf
        nsplit = a.max_split;
    } else if (a.blk > 0) {  // k_fattn: the splits of the row's block of a.blk rows
        const int rb0 = r / a.blk * a.blk, rb1 = (rb0 + a.blk < a.rec->n ? rb0 + a.blk : a.rec->n) - 1;
        const int64_t pos0 = a.rec->rows[0].pos;
        const int64_t klo = pos0 + rb0 + 1 - a.window > 0 ? pos0 + rb0 + 1 - a.window : 0;
        nsplit = (int)((pos0 + rb1 - klo + a.split) / a.split);
    } else {
        const int64_t p = a.rec->rows[r].pos;
        const int64_t lo = p + 1 - a.window > 0 ? p + 1 - a.window : 0;
        nsplit = (int)((p - lo + 1 + a.split - 1) / a.split);
    }
    const size_t pstride = (size_t)rep * (hd + 2);
    const float *all = a.part + ((size_t)r * a.nk + kh) * a.max_split * pstride + (size_t)h * (hd + 2);
    float M = -INFINITY, L = 0.f, acc = 0.f;
    for (int base = wave; base < nsplit; base += 4 * U) {
        float m[U], l[U], v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + 4 * u;
            const float *pj = all + (size_t)(j < nsplit ? j : base) * pstride;
            m[u] = pj[0];
            l[u] = pj[1];
            v[u] = pj[2 + dc];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) asm volatile("" ::"v"(m[u]), "v"(l[u]), "v"(v[u]));
        // the group's maximum first, then independent weights; a split past
        // the end or with no key (max -inf: its sums are stale) adds nothing
        float Mn = M;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + 4 * u < nsplit) Mn = fmaxf(Mn, m[u]);
        if (Mn != -INFINITY) {
            const float c0 = fexp(M - Mn);
            L *= c0;
            acc *= c0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool ok = base + 4 * u < nsplit && m[u] != -INFINITY;
                const float c = fexp((ok ? m[u] : Mn) - Mn);
                L += ok ? l[u] * c : 0.f;
                acc += ok ? v[u] * c : 0.f;
            }
            M = Mn;
        }
    }
    sm[wave][2 + lane] = acc;
    if (lane == 0) {
        sm[wave][0] = M;
        sm[wave][1] = L;
    }
    float vcol = 1.f;
    if (Q8 && wave == 0) {
        if (field_on(a, a.rec->rows[r]))
            vcol = (a.sd1 ? *a.sd1 : slot_at(a.tab, a.rec->rows[r].seq, a.n_ord, a.ord, a.slot)).vcol[kh * hd + dc];
    }
    __syncthreads();
    if (wave != 0 || d >= hd) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mt = fmaxf(Mt, sm[w][0]);
    float Lt = 0.f, y = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float mw = sm[w][0];
        const float c = mw == -INFINITY ? 0.f : fexp(mw - Mt);  // a wave with no split adds nothing
        Lt += sm[w][1] * c;
        y += sm[w][2 + lane] * c;
    }
    y = y / Lt * vcol;
    a.z[(size_t)r * Q + hq * hd + d] = y / (1.0f + expf(-(gate * sgv)));
}


// The merge of multi-row calls: workgroup per (row r, kv head kh), k_attn_merge's
// arithmetic.  Wave w takes splits w, w+4, ... (4 at a time in flight), lane l
// the CPL channels l*CPL .. of the group's REP*HD (one head); the 4 waves'
// running (max, sum, acc) are then combined through LDS.
// MODE: 0 the decode kernel's partials (a.dec), 1 a chunk's (a.blk > 0), 2 the
// one-row-per-workgroup kernel's: a compile-time choice, so no path loads what
// only another needs (a hoisted read of the record cost a round trip).
template <int Q8, int HD, int REP, int MODE>
__global__ __launch_bounds__(256) void k_attn_merge_rows(AttnArgs a) {
    constexpr int CH = REP * HD, CPL = CH >= 64 ? CH / 64 : 1;
    static_assert(CH % 64 == 0 || CH < 64, "channels split evenly over the lanes");
    static_assert(HD % CPL == 0, "a lane's channels lie in one head");
    __shared__ float wm[4][64], wl[4][64], wacc[4][CH], red[8];
    const int r = blockIdx.x, kh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Q = a.nh * HD, ld = 2 * Q + 2 * a.nk * HD;
    // the gate and its scale of this thread's channels, loaded first (after
    // the barrier below they took a round trip of their own)
    float gpre[(CH + 255) / 256], spre[(CH + 255) / 256];
#pragma unroll
    for (int k = 0; k < (CH + 255) / 256; ++k) {
        const int c = tid + 256 * k < CH ? tid + 256 * k : 0, hq = kh * REP + c / HD, d = c % HD;
        gpre[k] = a.qkvg[(size_t)r * ld + Q + 2 * a.nk * HD + hq * HD + d];
        spre[k] = a.sg[hq * HD + d];
    }
    int nsplit;
    if constexpr (MODE == 0) {  // decode kernel: every slab of the grid, those past the row's keys hold max -inf
        nsplit = a.max_split;
    } else if constexpr (MODE == 1) {  // a chunk: its first position and rows come from the host
        const int rb0 = r / a.blk * a.blk, rb1 = (rb0 + a.blk < a.nrows ? rb0 + a.blk : a.nrows) - 1;
        const int64_t pos0 = a.pos0;
        const int64_t klo = pos0 + rb0 + 1 - a.window > 0 ? pos0 + rb0 + 1 - a.window : 0;
        nsplit = (int)((pos0 + rb1 - klo + a.split) / a.split);
    } else {
        const int64_t p = a.rec->rows[r].pos;
        const int64_t lo = p + 1 - a.window > 0 ? p + 1 - a.window : 0;
        nsplit = (int)((p - lo + 1 + a.split - 1) / a.split);
    }
    const size_t pstride = (size_t)REP * (HD + 2);
    const int c0 = lane * CPL < CH ? lane * CPL : 0, h = c0 / HD, d0 = c0 % HD;  // lanes past CH: a copy, unused
    const float *ph = a.part + ((size_t)r * a.nk + kh) * a.max_split * pstride + (size_t)h * (HD + 2);
    float M = -INFINITY, L = 0.f, acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
    for (int j0 = wave; j0 < nsplit; j0 += 16) {
        float m[4], l[4], v[4][CPL];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + 4 * u < nsplit ? j0 + 4 * u : j0;
            const float *pj = ph + (size_t)j * pstride;
            m[u] = pj[0];
            l[u] = pj[1];
#pragma unroll
            for (int i = 0; i < CPL; ++i) v[u][i] = pj[2 + d0 + i];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            asm volatile("" ::"v"(m[u]), "v"(l[u]));
#pragma unroll
            for (int i = 0; i < CPL; ++i) asm volatile("" ::"v"(v[u][i]));
        }
        // the group's maximum first, then independent weights; a split past
        // the end or with no key (max -inf: its sums are stale) adds nothing
        float Mn = M;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (j0 + 4 * u < nsplit) Mn = fmaxf(Mn, m[u]);
        if (Mn != -INFINITY) {
            const float e0 = fexp(M - Mn);
            L *= e0;
#pragma unroll
            for (int i = 0; i < CPL; ++i) acc[i] *= e0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = j0 + 4 * u < nsplit && m[u] != -INFINITY;
                const float e1 = fexp((ok ? m[u] : Mn) - Mn);
                L += ok ? l[u] * e1 : 0.f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) acc[i] += ok ? v[u][i] * e1 : 0.f;
            }
            M = Mn;
        }
    }
    wm[wave][lane] = M;
    wl[wave][lane] = L;
    if (lane * CPL < CH)
#pragma unroll
        for (int i = 0; i < CPL; ++i) wacc[wave][c0 + i] = acc[i];
    __syncthreads();
    const bool field = Q8 && field_on(a, a.rec->rows[r]);
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < (CH + 255) / 256; ++k) {
        const int c = tid + 256 * k;
        if (c >= CH) break;
        const int ln = c / CPL, hh = c / HD, d = c % HD, hq = kh * REP + hh;
        float Mt = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) Mt = fmaxf(Mt, wm[w][ln]);
        float Lt = 0.f, y = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (wm[w][ln] == -INFINITY) continue;  // a wave with no split
            const float e = fexp(wm[w][ln] - Mt);
            Lt += wl[w][ln] * e;
            y += wacc[w][c] * e;
        }
        const float vcol =
            field ? (MODE == 1 ? a.sdc : slot_at(a.tab, a.rec->rows[r].seq, a.n_ord, a.ord, a.slot)).vcol[kh * HD + d]
                  : 1.f;
        y = y / Lt * vcol;
        const float zv = y / (1.0f + expf(-(gpre[k] * spre[k])));
        a.z[(size_t)r * Q + hq * HD + d] = zv;
        if (a.zb) a.zb[(size_t)r * Q + hq * HD + d] = f2bf(zv);
        ss += zv * zv;
    }
    if (a.zss) {
        ss = block_sum(ss, red);
        if (tid == 0) a.zss[(size_t)r * a.nk + kh] = ss;
    }
}

// Grouped-query attention of one row over keys max(p+1-window, 0) ..= p for the
// REP q heads of one kv head (dory.rs `attn_layer`, the per-(row, kv head)
// task; kv_cache.rs `attend_group_upto` for the q8_2f rows).
//
// Grid (splits, nk, T): workgroup (s, kh, r) takes keys [lo + s*split, ...) of
// row r.  It reads each K row once for its REP heads (HD/4 lanes per key, one
// 16-byte load each), keeps the scores in LDS, takes per-head maxima and sums,
// then reads each V row once.  It leaves (max, sum, unnormalised sum of
// p*v) per head for k_attn_merge.
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
    const int s = blockIdx.x, kh = blockIdx.y, r = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const CallRec *rec = a.rec;
    const int64_t p = rec->rows[r].pos;
    const int64_t lo = p + 1 - a.window > 0 ? p + 1 - a.window : 0;
    const int64_t nkeys = p - lo + 1;
    const int nsplit = (int)((nkeys + a.split - 1) / a.split);
    if (s >= nsplit) return;
    const int64_t e0 = lo + (int64_t)s * a.split;
    const int len = (int)(nkeys - (int64_t)s * a.split < a.split ? nkeys - (int64_t)s * a.split : a.split);
    const SlotDesc &sd = slot_at(a.tab, rec->rows[r].seq, a.n_ord, a.ord, a.slot);
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

}


// Decode attention: one row at position p (the call's only row), kv head kh,
// keys max(p+1-window, 0) ..= p split across workgroups (dory.rs
// `attn_layer`; kv_cache.rs `attend_group_upto` for q8_2f rows).  The
// projections arrive raw: every workgroup rotates and normalises its group's
// REP query heads itself (cheap, and it saves a kernel per sub-layer), and the
// workgroup whose split ends at p also rotates and normalises the new key,
// writes the new row to the cache (encoding it under q8_2f) and uses it from
// LDS in place of the ring row it prefetched.
//
// Each thread owns key slot g = tid / (HD/4) and the 4 channels dq*4.. of it;
// the workgroup takes KB = 256/(HD/4) keys per step and IT steps.  Load
// order: the projections, sq and the RoPE row first, then every K and V load
// of the split; the prep waits only for the first group while the cache rows
// are in flight.
template <int HD, int REP, int Q8, int IT>
__global__ __launch_bounds__(256) void k_attn_dec(AttnArgs a) {
    constexpr int LPK = HD / 4, KB = 256 / LPK;
    constexpr int SMAX = IT * KB < 256 ? IT * KB : 256;
    constexpr int NGK = (HD + kKGroup - 1) / kKGroup;
    constexpr int HALF = HD / 2;
    constexpr int QPT = (REP * HD + 255) / 256;  // query values per thread
    __shared__ float sc[REP][SMAX];
    __shared__ float red[KB * REP * HD];
    __shared__ float qs[REP + 1][HD];  // the group's query heads, then the new key
    __shared__ float sqs[REP][HD];
    __shared__ float vn[HD];
    __shared__ float rot[HD];          // cos half, sin half
    __shared__ int8_t kcn[HD], vcn[HD];
    __shared__ float ksn[NGK], vsn[1];
    __shared__ float stat[2][REP];
    const int s = blockIdx.x, kh = blockIdx.y, r = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const CallRec *rec = a.rec;
    // the slot's descriptor and the row's position, fetched together when the
    // caller names the slot (pinned: else the compiler sinks the descriptor's
    // load below the early exit, behind the position)
    SlotDesc sd;
    if (a.sd1) sd = *a.sd1;
    else sd = slot_at(a.tab, rec->rows[r].seq, a.n_ord, a.ord, a.slot);
    const int64_t p = rec->rows[r].pos;
    if (Q8) asm volatile("" ::"s"(sd.cap), "s"(sd.kc), "s"(sd.vc), "s"(sd.ks), "s"(sd.vs));
    else asm volatile("" ::"s"(sd.cap), "s"(sd.k), "s"(sd.v));
    const int64_t lo = p + 1 - a.window > 0 ? p + 1 - a.window : 0;
    const int64_t nkeys = p - lo + 1;
    const int nsplit = (int)((nkeys + a.split - 1) / a.split);
    if (s >= nsplit) {  // no key here: the merge skips a slab whose max is -inf
        if (tid < REP)
            a.part[(((size_t)r * a.nk + kh) * a.max_split + s) * REP * (HD + 2) + (size_t)tid * (HD + 2)] = -INFINITY;
        return;
    }
    const int64_t e0 = lo + (int64_t)s * a.split;
    const int len = (int)(nkeys - (int64_t)s * a.split < a.split ? nkeys - (int64_t)s * a.split : a.split);
    const bool tail = s == nsplit - 1;
    const bool field = Q8 && field_on(a, a.rec->rows[r]);
    const int cap = sd.cap;
    const int Q = a.nh * HD, KV = a.nk * HD;
    const int g = tid / LPK, dq = tid % LPK;
    const float scale = 1.0f / sqrtf((float)HD);

    // ---- 0. the prep's inputs (unconditional loads at clamped indices)
    const float *qrow = a.qkvg + (size_t)r * (2 * Q + 2 * KV);
    float qv[QPT], sv[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int idx = tid + 256 * i < REP * HD ? tid + 256 * i : 0;
        qv[i] = qrow[(size_t)kh * REP * HD + idx];
        sv[i] = a.sq[(size_t)kh * REP * HD + idx];
    }
    const int td = tid < HD ? tid : 0;
    const float kraw = qrow[Q + (size_t)kh * HD + td];
    const float vraw = qrow[Q + KV + (size_t)kh * HD + td];
    const float rv = a.rope[(size_t)p * HD + td];

    // ---- 1. every K and V row of the split, in flight at once
    const int rbase = (int)(e0 % cap);
    float4 kr[IT], vr[IT];
    float ksr[IT], vsr[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int e = g + KB * it;
        int rr = rbase + (e < len ? e : 0);
        if (rr >= cap) rr -= cap;
        const size_t row = (size_t)kh * cap + rr;
        if (Q8) {
            const char4 kc = *reinterpret_cast<const char4 *>(sd.kc + row * HD + dq * 4);
            const char4 vc = *reinterpret_cast<const char4 *>(sd.vc + row * HD + dq * 4);
            kr[it] = make_float4((float)kc.x, (float)kc.y, (float)kc.z, (float)kc.w);
            vr[it] = make_float4((float)vc.x, (float)vc.y, (float)vc.z, (float)vc.w);
            ksr[it] = sd.ks[row * NGK + (dq * 4) / kKGroup];
            vsr[it] = sd.vs[row];
        } else {
            kr[it] = *reinterpret_cast<const float4 *>(sd.k + row * HD + dq * 4);
            vr[it] = *reinterpret_cast<const float4 *>(sd.v + row * HD + dq * 4);
        }
    }

    // ---- 2. RoPE, unit norms, q times sq
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int idx = tid + 256 * i;
        if (idx < REP * HD) {
            qs[idx / HD][idx % HD] = qv[i];
            sqs[idx / HD][idx % HD] = sv[i];
        }
    }
    if (tid < HD) {
        qs[REP][tid] = kraw;
        vn[tid] = vraw;
        rot[tid] = rv;
    }
    __syncthreads();
    const int nvec = REP + (tail ? 1 : 0);
    for (int idx = tid; idx < nvec * HALF; idx += 256) {
        const int v = idx / HALF, j = idx % HALF;
        const float x = qs[v][j], y = qs[v][j + HALF], cs = rot[j], sn = rot[HALF + j];
        qs[v][j] = x * cs - y * sn;
        qs[v][j + HALF] = y * cs + x * sn;
    }
    __syncthreads();
    for (int v = wave; v < nvec; v += 4) {
        float ss = 0.f;
        for (int d = lane; d < HD; d += 64) ss += qs[v][d] * qs[v][d];
        const float f = norm_factor(wave_sum(ss));
        for (int d = lane; d < HD; d += 64) qs[v][d] *= v < REP ? f * sqs[v][d] : f;
    }
    __syncthreads();
    // ---- 3. the new row: into the cache, and in place of its prefetched copy
    if (tail) {
        const size_t row = (size_t)kh * cap + (size_t)(p % cap);
        if (Q8) {
            if (wave == 0) encode_row(qs[REP], field ? sd.kcol + kh * HD : nullptr, HD, kKGroup, kcn, ksn);
            if (wave == 1) encode_row(vn, field ? sd.vcol + kh * HD : nullptr, HD, HD, vcn, vsn);
            __syncthreads();
            if (!a.no_write) {
            for (int d = tid; d < HD; d += 256) {
                sd.kc[row * HD + d] = kcn[d];
                sd.vc[row * HD + d] = vcn[d];
            }
            if (tid < NGK) sd.ks[row * NGK + tid] = ksn[tid];
            if (tid == 0) sd.vs[row] = vsn[0];
            }
        } else if (!a.no_write) {
            for (int d = tid; d < HD; d += 256) {
                sd.k[row * HD + d] = qs[REP][d];
                sd.v[row * HD + d] = vn[d];
            }
        }
        if (rec->kvtap) {  // test tap: the new row's key and value before the cache write
            float *t = rec->kvtap + ((size_t)a.tap_pass * rec->n + r) * 2 * KV + (size_t)kh * HD;
            for (int d = tid; d < HD; d += 256) {
                t[d] = qs[REP][d];
                t[KV + d] = vn[d];
            }
        }
        const int el = len - 1;
        if (g == el % KB) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                if (it != el / KB) continue;
                if (Q8) {
                    const char4 kc = *reinterpret_cast<const char4 *>(kcn + dq * 4);
                    const char4 vc = *reinterpret_cast<const char4 *>(vcn + dq * 4);
                    kr[it] = make_float4((float)kc.x, (float)kc.y, (float)kc.z, (float)kc.w);
                    vr[it] = make_float4((float)vc.x, (float)vc.y, (float)vc.z, (float)vc.w);
                    ksr[it] = ksn[(dq * 4) / kKGroup];
                    vsr[it] = vsn[0];
                } else {
                    kr[it] = *reinterpret_cast<const float4 *>(&qs[REP][dq * 4]);
                    vr[it] = *reinterpret_cast<const float4 *>(&vn[dq * 4]);
                }
            }
        }
    }

    // ---- 4. scores s_e = q . k_e / sqrt(hd)
    {
        float4 q[REP];
#pragma unroll
        for (int h = 0; h < REP; ++h) q[h] = *reinterpret_cast<const float4 *>(&qs[h][dq * 4]);
        if (field) {
            const float4 c = *reinterpret_cast<const float4 *>(sd.kcol + kh * HD + dq * 4);
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                q[h].x *= c.x; q[h].y *= c.y; q[h].z *= c.z; q[h].w *= c.w;
            }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int e = g + KB * it;
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                float d = q[h].x * kr[it].x + q[h].y * kr[it].y + q[h].z * kr[it].z + q[h].w * kr[it].w;
                if (Q8) d *= ksr[it];
                d = group_sum<LPK>(d);
                if (e < len && dq == 0) sc[h][e] = d * scale;
            }
        }
    }
    __syncthreads();

    // ---- 5. per-head max and sum of exp (dory.rs `soft_body`)
    for (int h = wave; h < REP; h += 4) {
        float m = -INFINITY;
        for (int e = lane; e < len; e += 64) m = fmaxf(m, sc[h][e]);
        m = wave_max(m);
        float l = 0.f;
        for (int e = lane; e < len; e += 64) {
            const float pv = fexp(sc[h][e] - m);
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

    // ---- 6. values: acc_h = sum_e p_e v_e
    {
        float4 acc[REP];
#pragma unroll
        for (int h = 0; h < REP; ++h) acc[h] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int e = g + KB * it;
            if (e < len) {
#pragma unroll
                for (int h = 0; h < REP; ++h) {
                    const float w = Q8 ? sc[h][e] * vsr[it] : sc[h][e];
                    acc[h].x += w * vr[it].x;
                    acc[h].y += w * vr[it].y;
                    acc[h].z += w * vr[it].z;
                    acc[h].w += w * vr[it].w;
                }
            }
        }
#pragma unroll
        for (int h = 0; h < REP; ++h) *reinterpret_cast<float4 *>(&red[(g * REP + h) * HD + dq * 4]) = acc[h];
    }
    __syncthreads();
    const size_t pstride = (size_t)REP * (HD + 2);
    float *mine = a.part + (((size_t)r * a.nk + kh) * a.max_split + s) * pstride;
    for (int idx = tid; idx < REP * HD; idx += 256) {
        const int h = idx / HD, d = idx % HD;
        float v = 0.f;
#pragma unroll 8
        for (int gg = 0; gg < KB; ++gg) v += red[(gg * REP + h) * HD + d];
        mine[h * (HD + 2) + 2 + d] = v;
    }
    if (tid < REP) {
        mine[tid * (HD + 2)] = stat[0][tid];
        mine[tid * (HD + 2) + 1] = stat[1][tid];
    }
}

// Decode attention of one row for head dim 128, 64 keys per workgroup: the
// arithmetic of k_attn_dec with its steps laid out for short latency.
//   0. Wave w loads vectors w, w+4, .. of the group's REP query heads and, as
//      vector REP, the new key: lane j holds elements j and j+64, which are
//      exactly the pairs RoPE rotates, so RoPE, the unit norm and the sq scale
//      run in registers and one sync publishes them.  Every K and V load of the
//      split is issued behind these loads, 16 bytes per lane, 8 keys a step
//      (the key field and 1/sqrt(hd) are folded into the queries).
// REP = 4 (one q head a wave): the scores come from the registers that hold
// the keys, summed over the half wave by a reduce-scatter (described where it
// runs); the softmax of head w runs in wave w; the values accumulate in
// registers and the 8 key groups' sums meet in LDS.  Other REP:
//   1. The split's K and V rows go to LDS in fp32 (q8_2f: codes times their
//      scales).
//   2. Wave w takes heads w, w+4, ..: lane e scores key e against the head's
//      query from LDS, and the softmax of the head's 64 keys stays in the wave.
//   3. Lane l accumulates channels 2l, 2l+1 over the 64 keys, taking each
//      key's weight from its lane (readlane), and stores the partial.
// EXT = 1 (REP = 4, merge kernel): the split grows past 64 keys (a ninth load
// step, up to 72) so max_split workgroups cover the row's keys.
// XM = 1 (one row, a.xcnt set): the splits are merged in the kernel, inside
// one XCD.  A 1-D grid whose workgroup L runs on XCD L % 8 (the dispatcher
// deals workgroups to the XCDs in turn; launch_xcd_check confirms it at
// create) gives kv head kh the ids L = kh (mod 8), so the group's partials
// meet in that XCD's L2, which every CU of the XCD shares.  Each workgroup
// wave (one q head each: REP = 4) writes its head's partial, waits until the
// L2 has acknowledged the stores, and takes a ticket from the (kv head, head)
// counter (an L2 atomic); the wave with the last one reads the head's partials
// past its L1 (sc0), merges them as k_attn_merge does, applies the gate,
// writes z and clears the counter for the next launch.
template <int REP, int Q8, int XM, int EXT = 0>
__global__ __launch_bounds__(256) void k_attn_dec1(AttnArgs a) {
    static_assert(!EXT || (REP == 4 && !XM), "the extended split takes the register path, merge kernel");
    constexpr int HD = 128, HALF = 64, NK = 64, KP = HD + 4;
    constexpr int IT = EXT ? 9 : NK / 8;  // load steps: keys g + 8 it
    constexpr int NKX = 8 * IT;           // keys a workgroup can take
    constexpr int NGK = HD / kKGroup;
    constexpr int VPW = (REP + 1 + 3) / 4;  // vectors a wave prepares
    constexpr int HPW = (REP + 3) / 4;      // heads a wave merges (XM)
    __shared__ float qs[REP + 1][HD];  // queries (times the key field and 1/sqrt(hd)), then the new key
    __shared__ float vn[HD];
    __shared__ int8_t kcn[HD], vcn[HD];
    __shared__ float ksn[NGK], vsn[1];
    int s, kh;
    if (XM) {
        const int L = blockIdx.x, j = L >> 3;
        kh = (L & 7) + 8 * (j / a.max_split);
        s = j % a.max_split;
        if (kh >= a.nk) return;
    } else {
        s = blockIdx.x;
        kh = blockIdx.y;
    }
    const int r = XM ? 0 : blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Q = a.nh * HD, KV = a.nk * HD;
    // ---- 0. the prologue's inputs (which do not depend on the row's position:
    // issued before the record's read), then every cache row of the split
    const float *qrow = a.qkvg + (size_t)r * (2 * Q + 2 * KV);
    float x0[VPW], x1[VPW], s0[VPW], s1[VPW];
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
        const int v = wave + 4 * i < REP + 1 ? wave + 4 * i : REP;
        const float *src = v < REP ? qrow + (size_t)(kh * REP + v) * HD : qrow + Q + (size_t)kh * HD;
        x0[i] = src[lane];
        x1[i] = src[lane + HALF];
        const int vq = v < REP ? v : 0;
        s0[i] = a.sq[(size_t)(kh * REP + vq) * HD + lane];
        s1[i] = a.sq[(size_t)(kh * REP + vq) * HD + lane + HALF];
    }
    const float vr0 = qrow[Q + KV + (size_t)kh * HD + lane], vr1 = qrow[Q + KV + (size_t)kh * HD + lane + HALF];
    // XM: what the merge applies to lane l's channels 2l, 2l+1 of head wave + 4i
    // (the gate and its scale), read now in case this workgroup merges
    float2 xg[HPW], xs[HPW];
    if (XM) {
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int hq = kh * REP + (wave + 4 * i < REP ? wave + 4 * i : 0);
            xg[i] = *reinterpret_cast<const float2 *>(qrow + Q + 2 * KV + (size_t)hq * HD + 2 * lane);
            xs[i] = *reinterpret_cast<const float2 *>(a.sg + (size_t)hq * HD + 2 * lane);
        }
    }
    const CallRec *rec = a.rec;
    SlotDesc sd;
    if (a.sd1) sd = *a.sd1;
    else sd = slot_at(a.tab, rec->rows[r].seq, a.n_ord, a.ord, a.slot);
    const int64_t p = rec->rows[r].pos;
    if (Q8) asm volatile("" ::"s"(sd.cap), "s"(sd.kc), "s"(sd.vc), "s"(sd.ks), "s"(sd.vs));
    else asm volatile("" ::"s"(sd.cap), "s"(sd.k), "s"(sd.v));
    const int64_t lo = p + 1 - a.window > 0 ? p + 1 - a.window : 0;
    const int64_t nkeys = p - lo + 1;
    // EXT: the max_split workgroups cover the row's keys, each taking more
    // than `split` (at most 9/8 of it) once the keys outgrow split x max_split
    int S = a.split;
    if (EXT) {
        const int need = (int)((nkeys + a.max_split - 1) / a.max_split);
        S = need > S ? need : S;
    }
    const int nsplit = (int)((nkeys + S - 1) / S);
    if (s >= nsplit) {  // no key here: the merge skips a slab whose max is -inf (XM: not in the group)
        if (!XM && tid < REP)
            a.part[(((size_t)r * a.nk + kh) * a.max_split + s) * REP * (HD + 2) + (size_t)tid * (HD + 2)] = -INFINITY;
        return;
    }
    const int64_t e0 = lo + (int64_t)s * S;
    const int len = (int)(nkeys - (int64_t)s * S < S ? nkeys - (int64_t)s * S : S);
    const bool tail = s == nsplit - 1;
    const bool field = Q8 && field_on(a, a.rec->rows[r]);
    const int cap = sd.cap;
    const int g = tid >> 5, dq = tid & 31;
    const float cs = a.rope[(size_t)p * HD + lane], sn = a.rope[(size_t)p * HD + HALF + lane];
    float2 xv = make_float2(1.f, 1.f);  // XM: q8's V field of lane l's channels 2l, 2l+1
    if (XM && Q8 && field) xv = *reinterpret_cast<const float2 *>(sd.vcol + (size_t)kh * HD + 2 * lane);
    const int rbase = (int)(e0 % cap);
    float4 kr[IT], vr[IT];
    float ksr[IT], vsr[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int e = g + 8 * it;
        int rr = rbase + (e < len ? e : 0);
        if (rr >= cap) rr -= cap;
        const size_t row = (size_t)kh * cap + rr;
        if (Q8) {
            kr[it] = gld_codes4(sd.kc + row * HD + dq * 4);
            vr[it] = gld_codes4(sd.vc + row * HD + dq * 4);
            ksr[it] = gld<float>(sd.ks + row * NGK + (dq * 4) / kKGroup);
            vsr[it] = gld<float>(sd.vs + row);
        } else {
            kr[it] = gld4(sd.k + row * HD + dq * 4);
            vr[it] = gld4(sd.v + row * HD + dq * 4);
        }
    }
    // the prologue waits only for its own loads (issued first)
#pragma unroll
    for (int i = 0; i < VPW; ++i) asm volatile("" ::"v"(x0[i]), "v"(x1[i]), "v"(s0[i]), "v"(s1[i]));
    asm volatile("" ::"v"(vr0), "v"(vr1), "v"(cs), "v"(sn));

    // ---- RoPE, unit norm, sq (queries) in registers
    float kc0 = 1.f, kc1 = 1.f;
    if (field) {
        kc0 = gld<float>(sd.kcol + kh * HD + lane);
        kc1 = gld<float>(sd.kcol + kh * HD + lane + HALF);
    }
    const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
        const int v = wave + 4 * i;
        if (v > REP) break;
        const float y0 = x0[i] * cs - x1[i] * sn, y1 = x1[i] * cs + x0[i] * sn;
        const float f = norm_factor(wave_sum(y0 * y0 + y1 * y1));
        if (v < REP) {
            qs[v][lane] = y0 * f * s0[i] * kc0 * scale;
            qs[v][lane + HALF] = y1 * f * s1[i] * kc1 * scale;
        } else {
            qs[REP][lane] = y0 * f;
            qs[REP][lane + HALF] = y1 * f;
            vn[lane] = vr0;
            vn[lane + HALF] = vr1;
        }
    }
    __syncthreads();

    // ---- the new row: into the cache, and in place of its prefetched copy
    if (tail) {
        const size_t row = (size_t)kh * cap + (size_t)(p % cap);
        if (Q8) {
            if (wave == 0) encode_row(qs[REP], field ? sd.kcol + kh * HD : nullptr, HD, kKGroup, kcn, ksn);
            if (wave == 1) encode_row(vn, field ? sd.vcol + kh * HD : nullptr, HD, HD, vcn, vsn);
            __syncthreads();
            if (!a.no_write) {
                if (tid < HD) {
                    sd.kc[row * HD + tid] = kcn[tid];
                    sd.vc[row * HD + tid] = vcn[tid];
                }
                if (tid < NGK) sd.ks[row * NGK + tid] = ksn[tid];
                if (tid == 0) sd.vs[row] = vsn[0];
            }
        } else if (!a.no_write && tid < HD) {
            sd.k[row * HD + tid] = qs[REP][tid];
            sd.v[row * HD + tid] = vn[tid];
        }
        if (rec->kvtap && tid < HD) {  // test tap: the new row's key and value before the cache write
            float *t = rec->kvtap + ((size_t)a.tap_pass * rec->n + r) * 2 * KV + (size_t)kh * HD;
            t[tid] = qs[REP][tid];
            t[KV + tid] = vn[tid];
        }
        const int el = len - 1;
        if (g == el % 8) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                if (it != el / 8) continue;
                if (Q8) {
                    const char4 kc = *reinterpret_cast<const char4 *>(kcn + dq * 4);
                    const char4 vc = *reinterpret_cast<const char4 *>(vcn + dq * 4);
                    kr[it] = make_float4((float)kc.x, (float)kc.y, (float)kc.z, (float)kc.w);
                    vr[it] = make_float4((float)vc.x, (float)vc.y, (float)vc.z, (float)vc.w);
                    ksr[it] = ksn[(dq * 4) / kKGroup];
                    vsr[it] = vsn[0];
                } else {
                    kr[it] = *reinterpret_cast<const float4 *>(&qs[REP][dq * 4]);
                    vr[it] = *reinterpret_cast<const float4 *>(&vn[dq * 4]);
                }
            }
        }
    }

    const size_t pstride = (size_t)REP * (HD + 2);
    // XM: a group's slabs start on a 128-byte line of their own (no line is
    // shared with another XCD's group)
    const size_t gstride = ((size_t)a.max_split * pstride + 31) & ~(size_t)31;
    float *mine = XM ? a.part + (size_t)kh * gstride + (size_t)s * pstride
                     : a.part + (((size_t)r * a.nk + kh) * a.max_split + s) * pstride;
    if constexpr (REP == 4) {
        // ---- 1. scores from registers.  Lane (g, dq) holds channels 4dq..4dq+3
        // of keys g + 8 it; its 32 partial products (value v = 4 it + h) are
        // summed over the 32 lanes of its half wave by a reduce-scatter: each
        // step pairs lanes that differ in one bit of dq (a DPP mirror, quad
        // permute or the swizzle across rows), and each lane keeps the half of
        // its values whose matching bit of v equals its own, adding its
        // partner's copy.  After the five steps lane dq holds value v = dq: the
        // score of key g + 8 (dq >> 2) for head dq & 3.
        __shared__ float scs[REP][NKX + 1];     // scores by head (padded row)
        __shared__ float4 pw[NKX];              // softmax weights by key, the 4 heads
        __shared__ float red[8][REP][HD];       // per key group g: its sums of p * v
        float4 q4[REP];
#pragma unroll
        for (int h = 0; h < REP; ++h) q4[h] = *reinterpret_cast<const float4 *>(&qs[h][dq * 4]);
        float cur[32];
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                float d = q4[h].x * kr[it].x + q4[h].y * kr[it].y + q4[h].z * kr[it].z + q4[h].w * kr[it].w;
                if (Q8) d *= ksr[it];
                cur[4 * it + h] = d;
            }
#define DK_RS_STEP(BIT, DONE, STEP)                                           \
    do {                                                                      \
        const bool hi_ = (dq >> (BIT)) & 1;                                   \
        _Pragma("unroll") for (int v = 0; v < 32; ++v) {                      \
            if ((v & (DONE)) || (v & (1 << (BIT)))) continue;                 \
            const float lo = cur[v], hv = cur[v | (1 << (BIT))];              \
            cur[v] = (hi_ ? hv : lo) + STEP(hi_ ? lo : hv);                   \
        }                                                                     \
    } while (0)
        DK_RS_STEP(3, 0, dpp<0x140>);   // row_mirror: lane i <-> 15 - i (flips bits 0-3; every lane holds all values)
        DK_RS_STEP(2, 8, dpp<0x141>);   // row_half_mirror: i <-> 7 - i (bit 3 equal)
        DK_RS_STEP(0, 12, dpp<0xB1>);   // quad_perm [1,0,3,2]: i ^ 1
        DK_RS_STEP(1, 13, dpp<0x4E>);   // quad_perm [2,3,0,1]: i ^ 2
        DK_RS_STEP(4, 15, swap16);      // swizzle: i ^ 16 within the half wave
#undef DK_RS_STEP
        {
            const int e = g + 8 * (dq >> 2);
            scs[dq & 3][e] = e < len ? cur[0] : -INFINITY;
        }
        if (EXT) {
            // the ninth step's key 64 + g: its 4 heads' dot products summed over
            // the half wave; lane dq < 4 writes head dq's
            float x[REP];
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                float d = q4[h].x * kr[IT - 1].x + q4[h].y * kr[IT - 1].y + q4[h].z * kr[IT - 1].z +
                          q4[h].w * kr[IT - 1].w;
                if (Q8) d *= ksr[IT - 1];
                x[h] = group_sum<32>(d);
            }
            const float xe = dq == 0 ? x[0] : dq == 1 ? x[1] : dq == 2 ? x[2] : x[3];
            if (dq < REP) scs[dq][NK + g] = NK + g < len ? xe : -INFINITY;
        }
        __syncthreads();
        // ---- 2. softmax of head `wave` over the split's keys (lane = key)
        {
            const int h = wave;
            const float sv = scs[h][lane];
            const float sv2 = EXT && lane < NKX - NK ? scs[h][NK + lane] : -INFINITY;  // keys 64..
            const float m = wave_max(fmaxf(sv, sv2));
            const float pe = fexp(sv - m), pe2 = fexp(sv2 - m);  // 0 past len
            const float l = wave_sum(pe + pe2);
            reinterpret_cast<float *>(&pw[lane])[h] = pe;
            if (EXT && lane < NKX - NK) reinterpret_cast<float *>(&pw[NK + lane])[h] = pe2;
            if (lane == 0) {
                mine[(size_t)h * (HD + 2)] = m;
                mine[(size_t)h * (HD + 2) + 1] = l;
            }
        }
        __syncthreads();
        // ---- 3. values: lane (g, dq) adds p v over its 8 keys for the 4 heads;
        // the 8 key groups' sums meet in LDS
        float4 acc[REP];
#pragma unroll
        for (int h = 0; h < REP; ++h) acc[h] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            float4 pv = pw[g + 8 * it];
            if (Q8) {
                pv.x *= vsr[it]; pv.y *= vsr[it]; pv.z *= vsr[it]; pv.w *= vsr[it];
            }
            const float pa[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                acc[h].x += pa[h] * vr[it].x;
                acc[h].y += pa[h] * vr[it].y;
                acc[h].z += pa[h] * vr[it].z;
                acc[h].w += pa[h] * vr[it].w;
            }
        }
#pragma unroll
        for (int h = 0; h < REP; ++h) *reinterpret_cast<float4 *>(&red[g][h][dq * 4]) = acc[h];
        __syncthreads();
        {
            // wave h writes head h's channels (as it wrote its max and sum)
            const int h = wave;
            float2 v = make_float2(0.f, 0.f);
#pragma unroll
            for (int gg = 0; gg < 8; ++gg) {
                const float2 t = *reinterpret_cast<const float2 *>(&red[gg][h][2 * lane]);
                v.x += t.x;
                v.y += t.y;
            }
            *reinterpret_cast<float2 *>(mine + (size_t)h * (HD + 2) + 2 + 2 * lane) = v;
        }
    } else {
        __shared__ float Ks[NK][KP], Vs[NK][KP];
        // ---- 1. the split's rows to LDS
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int e = g + 8 * it;
            float4 k = kr[it], v = vr[it];
            if (Q8) {
                k.x *= ksr[it]; k.y *= ksr[it]; k.z *= ksr[it]; k.w *= ksr[it];
                v.x *= vsr[it]; v.y *= vsr[it]; v.z *= vsr[it]; v.w *= vsr[it];
            }
            *reinterpret_cast<float4 *>(&Ks[e][dq * 4]) = k;
            *reinterpret_cast<float4 *>(&Vs[e][dq * 4]) = v;
        }
        __syncthreads();

        // ---- 2, 3. per head: scores of lane e's key, softmax, values
        for (int h = wave; h < REP; h += 4) {
            // LDS reads in batches, all issued before their first use (else the
            // compiler keeps two in flight and waits on each pair)
            float d = 0.f;
#pragma unroll
            for (int c0 = 0; c0 < HD; c0 += 32) {
                float4 k[8], q[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    k[i] = *reinterpret_cast<const float4 *>(&Ks[lane][c0 + 4 * i]);
                    q[i] = *reinterpret_cast<const float4 *>(&qs[h][c0 + 4 * i]);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(k[i].x), "v"(k[i].w), "v"(q[i].x), "v"(q[i].w));
#pragma unroll
                for (int i = 0; i < 8; ++i) d += k[i].x * q[i].x + k[i].y * q[i].y + k[i].z * q[i].z + k[i].w * q[i].w;
            }
            const float sc = lane < len ? d : -INFINITY;
            const float m = wave_max(sc);
            const float pe = fexp(sc - m);  // 0 past len
            const float l = wave_sum(pe);
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int e0 = 0; e0 < NK; e0 += 16) {
                float2 v[16];
                float w[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const float2 *>(&Vs[e0 + i][2 * lane]);
#pragma unroll
                for (int i = 0; i < 16; ++i) w[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pe), e0 + i));
#pragma unroll
                for (int i = 0; i < 16; ++i) asm volatile("" ::"v"(v[i].x), "v"(v[i].y));
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    acc0 += w[i] * v[i].x;
                    acc1 += w[i] * v[i].y;
                }
            }
            float *dst = mine + (size_t)h * (HD + 2);
            *reinterpret_cast<float2 *>(dst + 2 + 2 * lane) = make_float2(acc0, acc1);
            if (lane == 0) {
                dst[0] = m;
                dst[1] = l;
            }
        }
    }
    if constexpr (XM) {
        static_assert(REP == 4, "the in-kernel merge takes one head a wave");
        // ---- XM: head h = wave's ticket; the wave that takes the last one
        // merges head h (each wave wrote all of its head's partial)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores acknowledged (by the L2)
        const int h = wave;
        uint32_t *cnt = a.xcnt + 32 * (kh * REP + h);
        unsigned t = 0;
        if (lane == 0) t = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readlane(t, 0) != (unsigned)(nsplit - 1)) return;
        const float *gp = a.part + (size_t)kh * gstride;
        // the group's slabs, read with sc0 (past this CU's L1); offsets past the
        // nsplit slabs read 0
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(gp), (short)0, (int)(nsplit * pstride * 4), 0x00020000);
        const int hoff = h * (HD + 2);
        // lane j: split j's (max, sum); the channels of splits 16 at a time
        const float2 ml = __builtin_bit_cast(
            float2, __builtin_amdgcn_raw_buffer_load_b64(rs, (lane * (int)pstride + hoff) * 4, 0, 1));
        float2 v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            v[j] = __builtin_bit_cast(
                float2, __builtin_amdgcn_raw_buffer_load_b64(rs, (j * (int)pstride + hoff + 2 + 2 * lane) * 4, 0, 1));
        // all 17 loads in flight before the first use (else the channel loads
        // wait for the reductions)
        asm volatile("" ::"v"(ml.x), "v"(ml.y));
#pragma unroll
        for (int j = 0; j < 16; ++j) asm volatile("" ::"v"(v[j].x), "v"(v[j].y));
        const float mj = lane < nsplit ? ml.x : -INFINITY;
        const float M = wave_max(mj);
        const float c = lane < nsplit ? fexp(mj - M) : 0.f;
        const float Lt = wave_sum(ml.y * c);
        float y0 = 0.f, y1 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float cj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), j));
            y0 += cj * v[j].x;
            y1 += cj * v[j].y;
        }
        for (int j0 = 16; j0 < nsplit; j0 += 16) {  // more than 16 splits
#pragma unroll
            for (int j = 0; j < 16; ++j)
                v[j] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(
                                                      rs, ((j0 + j) * (int)pstride + hoff + 2 + 2 * lane) * 4, 0, 1));
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float cj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), j0 + j));
                y0 += cj * v[j].x;
                y1 += cj * v[j].y;
            }
        }
        const int hq = kh * REP + h;
        y0 = y0 / Lt * xv.x;
        y1 = y1 / Lt * xv.y;
        *reinterpret_cast<float2 *>(a.z + (size_t)hq * HD + 2 * lane) =
            make_float2(y0 / (1.0f + expf(-(xg[0].x * xs[0].x))), y1 / (1.0f + expf(-(xg[0].y * xs[0].y))));
        if (lane == 0) *cnt = 0u;
    }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Grouped-query attention of a chunk of one sequence on bf16 MFMA (the
// pages' attend_chunk: a panel of queries per kv head against the cache), for
// rows at consecutive positions pos0 .. pos0+T-1 after launch_prep has written
// their keys and values.
//
// Workgroup (s, kh, b): kv head kh, rows b*BQ .. b*BQ+BQ-1 with their REP q
// heads (128 query vectors, qv = h*BQ + row), and split s of the keys the block
// sees: [klo + s*split, ..) with klo = max(0, pos0 + b*BQ + 1 - window).  Wave w
// owns query vectors 32w .. 32w+31.  Per tile of 64 keys, staged in LDS as
// bf16 (K as [key][d]; V transposed as [d][slot]):
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16: A = K rows, B = Q from registers):
//                 lane l then holds query vector l%32 and 16 keys of each
//                 32-key block, keys 8(j/4) + 4(l/32) + j%4 in element j;
//   online softmax per lane (the partner lane l^32 holds the other 16 keys);
//   O^T += V^T P^T (A = V^T from LDS, B = P^T straight from the registers):
//                 the key slots of V^T are laid out in the order the P^T
//                 registers hold them, so no shuffle is needed.
// O^T leaves lane l with 16 channels of query vector l%32 per 32-channel tile,
// so the softmax rescale is one multiplier per lane.  Each workgroup writes
// (max, sum, unnormalised sum of p*v) per (row, head) for k_attn_merge.
template <int HD, int REP, int Q8>
__global__ __launch_bounds__(256, Q8 ? 1 : 2) void k_fattn(AttnArgs a) {
    static_assert(HD == 128, "the loaders assume 32 lanes per 128-channel row");
    constexpr int BQ = 128 / REP;        // rows per workgroup
    constexpr int KT = 64;               // keys per tile
    constexpr int KP = HD + 8, VP = KT + 8;
    constexpr int NGK = (HD + kKGroup - 1) / kKGroup;
    constexpr int DT = HD / 32;          // output tiles of 32 channels
    constexpr int KS = HD / 16;          // k-steps of the score MFMA
    constexpr int KL = 256 / (HD / 4);   // keys a pass of the K loader covers
    __shared__ __bf16 Ks[2][KT][KP];
    __shared__ __bf16 Vt[2][HD][VP];
    const int s = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    const int T = a.nrows;
    const int r0 = b * BQ, r1 = (r0 + BQ < T ? r0 + BQ : T) - 1;
    const int64_t pos0 = a.pos0;
    const int64_t klo = pos0 + r0 + 1 - a.window > 0 ? pos0 + r0 + 1 - a.window : 0;
    const int64_t khi = pos0 + r1;
    const int64_t eb = klo + (int64_t)s * a.split;
    if (eb > khi) return;
    const int64_t ee = eb + a.split - 1 < khi ? eb + a.split - 1 : khi;  // last key of the split
    const int ntiles = (int)((ee - eb + KT) / KT);
    const SlotDesc &sd = a.sdc;
    const int cap = sd.cap;
    const int Q = a.nh * HD;

    // ---- this lane's query vector
    const int qv = wave * 32 + (lane & 31), h = qv / BQ, r = r0 + qv % BQ;
    const bool rok = r < T;
    const int64_t p = pos0 + (rok ? r : r1);
    const int64_t lo_r = p + 1 - a.window > 0 ? p + 1 - a.window : 0;
    const int lo_i = (int)lo_r, p_i = (int)p, ee_i = (int)ee;
    bf16x8_t qb[KS];
    {
        const float *qrow = a.qp + (size_t)(rok ? r : r1) * Q + (size_t)(kh * REP + h) * HD;
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            const int d = 16 * t + 8 * g;
            float4 x0 = gld4(qrow + d);
            float4 x1 = gld4(qrow + d + 4);
            if (Q8 && a.field) {
                const float4 c0 = gld4(sd.kcol + kh * HD + d);
                const float4 c1 = gld4(sd.kcol + kh * HD + d + 4);
                x0.x *= c0.x; x0.y *= c0.y; x0.z *= c0.z; x0.w *= c0.w;
                x1.x *= c1.x; x1.y *= c1.y; x1.z *= c1.z; x1.w *= c1.w;
            }
            qb[t][0] = (__bf16)x0.x; qb[t][1] = (__bf16)x0.y; qb[t][2] = (__bf16)x0.z; qb[t][3] = (__bf16)x0.w;
            qb[t][4] = (__bf16)x1.x; qb[t][5] = (__bf16)x1.y; qb[t][6] = (__bf16)x1.z; qb[t][7] = (__bf16)x1.w;
        }
    }

    // ---- loaders.  K: thread (key tid/(HD/4) + KL*i, channels 4*(tid%(HD/4))).
    // V: thread (slot chunk ci = tid % 8, channels 4*(tid/8)); chunk ci holds
    // keys 16(ci/2) + 4(ci%2) + {0..3} and 16(ci/2) + 8 + 4(ci%2) + {0..3} in
    // slots 8ci .. 8ci+7, so 8 consecutive lanes store one 128-byte run of a
    // V^T row (and read 128-byte runs of 8 key rows).
    constexpr int KPASS = KT / KL;           // K rows per thread
    constexpr int VPASS = 1;                 // V slot chunks per thread (8 chunks x HD/4 channel groups = 256)
    const int lc = tid % (HD / 4), lk = tid / (HD / 4);
    const int vci = tid & 7, vlc = tid >> 3;
    float4 kr[KPASS], vr[VPASS][8];
    float ksr[KPASS], vsr[VPASS][8];
    // Ring rows of a tile: one wave-uniform remainder per tile, then a wrap
    // check per key (positions fit in 32 bits: they are below max_ctx); keys
    // past the split's last re-read its row and are masked.
    auto gload = [&](int tile) {
        const int t0 = (int)eb + tile * KT;
        const int rb = (int)((unsigned)t0 % (unsigned)cap);
        const int last = (int)ee - t0;
        if (!Q8 && rb + KT <= cap && last >= KT - 1) {
            // the common tile (no ring wrap, every key inside the split): key k
            // sits at row rb + k, so one 32-bit offset for the tile and a fixed
            // one per key (the per-key wrap and 64-bit row arithmetic below were
            // ~20% of the kernel's VALU work)
            // (byte offsets in 32 bits: the loads then take the ring's base as a
            // scalar and the offset as a 32-bit register, no 64-bit adds)
            const uint32_t tb = ((uint32_t)kh * (uint32_t)cap + (uint32_t)rb) * (HD * 4);
            const char *kb = reinterpret_cast<const char *>(sd.k), *vb = reinterpret_cast<const char *>(sd.v);
#pragma unroll
            for (int i = 0; i < KPASS; ++i)
                kr[i] = gld4(reinterpret_cast<const float *>(kb + (tb + (uint32_t)(((lk + KL * i) * HD + 4 * lc) * 4))));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kk = 16 * (vci >> 1) + 8 * (j >> 2) + 4 * (vci & 1) + (j & 3);
                vr[0][j] = gld4(reinterpret_cast<const float *>(vb + (tb + (uint32_t)((kk * HD + 4 * vlc) * 4))));
            }
            return;
        }
        auto key_row = [&](int k) -> size_t {
            int rr = rb + (k < last ? k : last);
            rr = rr >= cap ? rr - cap : rr;
            return (size_t)kh * cap + rr;
        };
#pragma unroll
        for (int i = 0; i < KPASS; ++i) {
            const size_t row = key_row(lk + KL * i);
            if (Q8) {
                kr[i] = gld_codes4(sd.kc + row * HD + 4 * lc);
                ksr[i] = gld<float>(sd.ks + row * NGK + (4 * lc) / kKGroup);
            } else {
                kr[i] = gld4(sd.k + row * HD + 4 * lc);
            }
        }
#pragma unroll
        for (int i = 0; i < VPASS; ++i) {
            const int ci = vci;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kk = 16 * (ci >> 1) + 8 * (j >> 2) + 4 * (ci & 1) + (j & 3);
                const size_t row = key_row(kk);
                if (Q8) {
                    vr[i][j] = gld_codes4(sd.vc + row * HD + 4 * vlc);
                    vsr[i][j] = gld<float>(sd.vs + row);
                } else {
                    vr[i][j] = gld4(sd.v + row * HD + 4 * vlc);
                }
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KPASS; ++i) {
            float4 x = kr[i];
            if (Q8) { x.x *= ksr[i]; x.y *= ksr[i]; x.z *= ksr[i]; x.w *= ksr[i]; }
            __bf16 *dst = &Ks[buf][lk + KL * i][4 * lc];
            dst[0] = (__bf16)x.x; dst[1] = (__bf16)x.y; dst[2] = (__bf16)x.z; dst[3] = (__bf16)x.w;
        }
#pragma unroll
        for (int i = 0; i < VPASS; ++i) {
            const int ci = vci;
            bf16x8_t col[4];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float4 x = vr[i][j];
                if (Q8) { x.x *= vsr[i][j]; x.y *= vsr[i][j]; x.z *= vsr[i][j]; x.w *= vsr[i][j]; }
                col[0][j] = (__bf16)x.x; col[1][j] = (__bf16)x.y; col[2][j] = (__bf16)x.z; col[3][j] = (__bf16)x.w;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) *reinterpret_cast<bf16x8_t *>(&Vt[buf][4 * vlc + c][8 * ci]) = col[c];
        }
    };

    f32x16_t o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[t][e] = 0.f;
    float m = -INFINITY, l = 0.f;  // running maximum (log2 units) and sum
    const float scale2 = 1.4426950408889634f / sqrtf((float)HD);
    // keys every row of this wave sees (rows rlo .. rhi, consecutive positions):
    // [wlo, whi]; empty when the wave has a row past T
    const int rlo = r0 + (BQ >= 32 ? (wave * 32) % BQ : 0), rhi = rlo + (BQ >= 32 ? 32 : BQ) - 1;
    const int wlo = rhi < T ? (int)(pos0 + rhi + 1 - a.window > 0 ? pos0 + rhi + 1 - a.window : 0) : 1 << 30;
    const int whi = (int)(pos0 + rlo) < ee_i ? (int)(pos0 + rlo) : ee_i;

    gload(0);
    sstore(0);
    __syncthreads();
    int buf = 0;
    for (int tile = 0; tile < ntiles; ++tile) {
        const bool more = tile + 1 < ntiles;
        if (more) gload(tile + 1);
        const int t0 = (int)eb + tile * KT;
        // scores of the two 32-key blocks
        f32x16_t sc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                const bf16x8_t kv = *reinterpret_cast<const bf16x8_t *>(&Ks[buf][32 * kb + (lane & 31)][16 * t + 8 * g]);
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qb[t], sc[kb], 0, 0, 0);
            }
        }
        // mask (only on tiles some row of this wave does not see whole) and
        // tile maximum; scores in log2 units (scale * log2 e folded in)
        float mx = -INFINITY;
        if (t0 >= wlo && t0 + KT - 1 <= whi) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    sc[kb][e] *= scale2;
                    mx = fmaxf(mx, sc[kb][e]);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = t0 + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
                    const bool vis = rok && key >= lo_i && key <= p_i && key <= ee_i;
                    const float v = vis ? sc[kb][e] * scale2 : -INFINITY;
                    sc[kb][e] = v;
                    mx = fmaxf(mx, v);
                }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m, mx);
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        bf16x8_t pb[2][2];
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float pv = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[kb][e] - mn);
                ls += pv;
                pb[kb][e >> 3][e & 7] = (__bf16)pv;
            }
        l = l * alpha + ls;
        if (__ballot(alpha != 1.f) != 0)  // some lane's maximum moved
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[t][e] *= alpha;
        // O^T += V^T P^T over the 64 keys (4 MFMA k-steps of 16 slots)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const bf16x8_t vv = *reinterpret_cast<const bf16x8_t *>(
                        &Vt[buf][32 * t + (lane & 31)][32 * kb + 16 * mm + 8 * g]);
                    o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[kb][mm], o[t], 0, 0, 0);
                }
        if (more) {
            sstore(buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }
    l += __shfl_xor(l, 32);
    if (!rok) return;
    const size_t pstride = (size_t)REP * (HD + 2);
    float *mine = a.part + (((size_t)r * a.nk + kh) * a.max_split + s) * pstride + (size_t)h * (HD + 2);
    if (g == 0) {
        mine[0] = m * 0.6931471805599453f;  // log2 units -> natural units for the merge
        mine[1] = l;
    }
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            float *dst = mine + 2 + 32 * t + 8 * q4 + 4 * g;
            dst[0] = o[t][4 * q4 + 0];
            dst[1] = o[t][4 * q4 + 1];
            dst[2] = o[t][4 * q4 + 2];
            dst[3] = o[t][4 * q4 + 3];
        }
}

template <int HD, int REP>
hipError_t launch_hr(const AttnArgs &a, int T, hipStream_t s) {
    if (T < 0) {  // decode kernel: -T rows, each of its own sequence and position
        if (!a.dec) return hipErrorInvalidValue;
        dim3 grid(a.max_split, a.nk, -T), block(256);
        // one row, head dim 128, up to 64 keys a workgroup: the short-latency
        // kernel; else 8 load steps per workgroup, or 16 when the split needs them
        if constexpr (HD == 128 && REP == 4) {
            if (T == -1 && a.split <= 64 && a.xcnt) {
                // the splits merged in the kernel: no merge launch follows
                if (a.max_split > 64) return hipErrorInvalidValue;
                const dim3 xgrid(8 * a.max_split * ((a.nk + 7) / 8));
                if (a.q8) hipLaunchKernelGGL((k_attn_dec1<REP, 1, 1>), xgrid, block, 0, s, a);
                else hipLaunchKernelGGL((k_attn_dec1<REP, 0, 1>), xgrid, block, 0, s, a);
                return hipGetLastError();
            }
        }
        bool ext = false;
        if constexpr (HD == 128 && REP == 4) {
            if (T == -1 && a.split == 64 && a.ext) {
                // 64-key splits grown to cover the row's keys with max_split workgroups
                if (a.q8) hipLaunchKernelGGL((k_attn_dec1<REP, 1, 0, 1>), grid, block, 0, s, a);
                else hipLaunchKernelGGL((k_attn_dec1<REP, 0, 0, 1>), grid, block, 0, s, a);
                ext = true;
            }
        }
        if (ext) {
        } else if (HD == 128 && T == -1 && a.split <= 64) {
            if (a.q8) hipLaunchKernelGGL((k_attn_dec1<REP, 1, 0>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_attn_dec1<REP, 0, 0>), grid, block, 0, s, a);
        } else if (a.split <= 8 * (256 / (HD / 4))) {
            if (a.q8) hipLaunchKernelGGL((k_attn_dec<HD, REP, 1, 8>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_attn_dec<HD, REP, 0, 8>), grid, block, 0, s, a);
        } else {
            if (a.q8) hipLaunchKernelGGL((k_attn_dec<HD, REP, 1, 16>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_attn_dec<HD, REP, 0, 16>), grid, block, 0, s, a);
        }
    } else if (a.blk > 0) {
        if constexpr (HD == 128 && 128 % REP == 0) {
            if (a.blk != 128 / REP) return hipErrorInvalidValue;
            if (a.nsplit < 1 || a.nsplit > a.max_split) return hipErrorInvalidValue;
            dim3 grid(a.nsplit, a.nk, (T + a.blk - 1) / a.blk), block(256);
            if (a.q8) hipLaunchKernelGGL((k_fattn<HD, REP, 1>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_fattn<HD, REP, 0>), grid, block, 0, s, a);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        dim3 grid(a.max_split, a.nk, T), block(256);
        if (a.q8) hipLaunchKernelGGL((k_attn<HD, REP, 1>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_attn<HD, REP, 0>), grid, block, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one row: 4 waves per head channel block walk the splits in parallel;
    // several rows: a workgroup per (row, kv head)
    const int rows = T < 0 ? -T : T;
    if (rows == 1 && !a.zss) {  // (a row of a multi-row call needs zb and zss: the merge below)
        // each wave holds its splits' loads in flight at once (up to 68 splits)
        dim3 mgrid(1, a.nh, (HD + 63) / 64), mblock(256);
        const int per_wave = (a.max_split + 3) / 4;
        if (per_wave <= 4) {
            if (a.q8) hipLaunchKernelGGL((k_attn_merge<1, 4>), mgrid, mblock, 0, s, a);
            else hipLaunchKernelGGL((k_attn_merge<0, 4>), mgrid, mblock, 0, s, a);
        } else if (per_wave <= 8) {
            if (a.q8) hipLaunchKernelGGL((k_attn_merge<1, 8>), mgrid, mblock, 0, s, a);
            else hipLaunchKernelGGL((k_attn_merge<0, 8>), mgrid, mblock, 0, s, a);
        } else {
            if (a.q8) hipLaunchKernelGGL((k_attn_merge<1, 17>), mgrid, mblock, 0, s, a);
            else hipLaunchKernelGGL((k_attn_merge<0, 17>), mgrid, mblock, 0, s, a);
        }
    } else {
        dim3 mgrid(rows, a.nk);
#define DK_MERGE_ROWS(MODE)                                                                          \
    do {                                                                                             \
        if (a.q8) hipLaunchKernelGGL((k_attn_merge_rows<1, HD, REP, MODE>), mgrid, dim3(256), 0, s, a); \
        else hipLaunchKernelGGL((k_attn_merge_rows<0, HD, REP, MODE>), mgrid, dim3(256), 0, s, a);      \
    } while (0)
        if (a.dec) DK_MERGE_ROWS(0);
        else if (a.blk > 0) DK_MERGE_ROWS(1);
        else DK_MERGE_ROWS(2);
#undef DK_MERGE_ROWS
    }
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

hipError_t launch_hd(const AttnArgs &a, int T, hipStream_t s) {
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

// Each workgroup's XCD (hardware register XCC_ID, bits 3:0) into ids[blockIdx.x].
__global__ void k_xcd_ids(unsigned *ids) {
    if (threadIdx.x == 0) ids[blockIdx.x] = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));
}

}  // namespace

hipError_t launch_xcd_check(unsigned *ids, int G, hipStream_t s) {
    if (!ids || G < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_xcd_ids, dim3(G), dim3(64), 0, s, ids);
    return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs &a, int T, hipStream_t s) {
    if (a.hd > 256 || a.hd % 2 || (!a.kstage && (!a.kring || !a.vring || a.cap < 1)) || (a.kvtap && a.kvtap_n < T))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_prep, dim3(T, a.nh + a.nk), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a, int T, hipStream_t s) {
    if (a.split <= 0 || T <= 0 || (a.blk == 0 && a.split > 256) || (a.blk > 0 && a.split % 64))
        return hipErrorInvalidValue;
    AttnArgs b = a;
    b.dec = 0;
    return launch_hd(b, T, s);
}

hipError_t launch_attn_dec(const AttnArgs &a, int T, hipStream_t s) {
    if (a.split <= 0 || a.split > attn_dec_max_split(a.hd, 16) || T <= 0) return hipErrorInvalidValue;
    AttnArgs b = a;
    b.dec = 1;
    return launch_hd(b, -T, s);
}

}  // namespace dk
