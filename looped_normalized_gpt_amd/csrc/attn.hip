// attn.hip -- the attention sub-layer between its projections: RoPE and unit
// norms with the cache write (prep), and grouped-query attention over the ring
// with the sigmoid gate (attn).
#include "device.h"

namespace dk {

namespace {

// dory.rs `attn_layer` (rotate, justnorm per head, q times sq), with the RoPE
// table row of the position (dory.rs `stack`: cos half, sin half).  One wave
// per (row, head); lane j owns the pairs (j, j + hd/2), (j + 64, j + 64 + hd/2).
__global__ __launch_bounds__(64) void k_prep(PrepArgs a) {
    const int r = blockIdx.x, hh = blockIdx.y, lane = threadIdx.x;
    const int hd = a.hd, half = hd / 2, Q = a.nh * hd, KV = a.nk * hd;
    const int ld = Q + 2 * KV + Q;
    const int64_t p = a.rec->rows[r].pos;
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
            const float cs = a.rope[(size_t)p * hd + j], sn = a.rope[(size_t)p * hd + half + j];
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
    const SlotDesc &sd = slot_at(a.tab, a.rec->rows[r].seq, a.n_ord, a.ord, a.slot);
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


// Merges the split partials of (row r, q head h) in log-sum-exp form, scales by
// the V field (q8), applies the sigmoid gate (dory.rs `gate_body`) and writes z.
// Grid (T, nh, ceil(hd/64)); lane d of every wave owns one channel, wave w takes
// splits w, w + waves, ... with a running (max, sum, acc) merge, then wave 0
// merges the waves' results.  A kernel of its own: the partials come from
// workgroups on other XCDs, whose L2s are only coherent with this one at kernel
// boundaries.
template <int Q8>
__global__ __launch_bounds__(1024) void k_attn_merge(AttnArgs a) {
    constexpr int U = 8;  // splits a wave holds in flight
    __shared__ float sm[16][66];
    const int r = blockIdx.x, hq = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int d = blockIdx.z * 64 + lane;
    const int hd = a.hd, rep = a.nh / a.nk, kh = hq / rep, h = hq % rep;
    const int Q = a.nh * hd, ld = 2 * Q + 2 * a.nk * hd;
    const int dc = d < hd ? d : 0;
    // what does not depend on the partials first
    const float gate = a.qkvg[(size_t)r * ld + Q + 2 * a.nk * hd + hq * hd + dc];
    const float sgv = a.sg[hq * hd + dc];
    const int64_t p = a.rec->rows[r].pos;
    float vcol = 1.f;
    if (Q8 && (a.field > 0 || (a.field < 0 && p >= kWarmup)))
        vcol = slot_at(a.tab, a.rec->rows[r].seq, a.n_ord, a.ord, a.slot).vcol[kh * hd + dc];
    const int64_t lo = p + 1 - a.window > 0 ? p + 1 - a.window : 0;
    const int nsplit = (int)((p - lo + 1 + a.split - 1) / a.split);
    const size_t pstride = (size_t)rep * (hd + 2);
    const float *all = a.part + ((size_t)r * a.nk + kh) * a.max_split * pstride + (size_t)h * (hd + 2);
    float M = -INFINITY, L = 0.f, acc = 0.f;
    for (int base = wave; base < nsplit; base += nw * U) {
        float m[U], l[U], v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + nw * u;
            const float *pj = all + (size_t)(j < nsplit ? j : base) * pstride;
            m[u] = pj[0];
            l[u] = pj[1];
            v[u] = pj[2 + dc];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (base + nw * u >= nsplit) break;
            const float Mn = fmaxf(M, m[u]);
            const float c0 = expf(M - Mn), c1 = expf(m[u] - Mn);
            L = L * c0 + l[u] * c1;
            acc = acc * c0 + v[u] * c1;
            M = Mn;
        }
    }
    sm[wave][2 + lane] = acc;
    if (lane == 0) {
        sm[wave][0] = M;
        sm[wave][1] = L;
    }
    __syncthreads();
    if (wave != 0 || d >= hd) return;
    float Mt = -INFINITY;
    for (int w = 0; w < nw; ++w) Mt = fmaxf(Mt, sm[w][0]);
    float Lt = 0.f, y = 0.f;
    for (int w = 0; w < nw; ++w) {
        if (sm[w][0] == -INFINITY) continue;  // a wave with no split
        const float c = expf(sm[w][0] - Mt);
        Lt += sm[w][1] * c;
        y += sm[w][2 + lane] * c;
    }
    y = y / Lt * vcol;
    a.z[(size_t)r * Q + hq * hd + d] = y / (1.0f + expf(-(gate * sgv)));
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
// the workgroup takes KB = 256/(HD/4) keys per step and IT = 8 steps.  Load
// order: the projections, sq and the RoPE row first, then every K and V load
// of the split; the prep waits only for the first group while the cache rows
// are in flight.
template <int HD, int REP, int Q8>
__global__ __launch_bounds__(256) void k_attn_dec(AttnArgs a) {
    constexpr int LPK = HD / 4, KB = 256 / LPK, IT = 8;
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
    const int64_t p = rec->rows[r].pos;
    const int64_t lo = p + 1 - a.window > 0 ? p + 1 - a.window : 0;
    const int64_t nkeys = p - lo + 1;
    const int nsplit = (int)((nkeys + a.split - 1) / a.split);
    if (s >= nsplit) return;
    const int64_t e0 = lo + (int64_t)s * a.split;
    const int len = (int)(nkeys - (int64_t)s * a.split < a.split ? nkeys - (int64_t)s * a.split : a.split);
    const bool tail = s == nsplit - 1;
    const bool field = Q8 && (a.field > 0 || (a.field < 0 && p >= kWarmup));
    const SlotDesc &sd = slot_at(a.tab, rec->rows[r].seq, a.n_ord, a.ord, a.slot);
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

template <int HD, int REP>
hipError_t launch_hr(const AttnArgs &a, int T, hipStream_t s) {
    if (T < 0) {  // decode kernel: -T rows, each of its own sequence and position
        dim3 grid(a.max_split, a.nk, -T), block(256);
        if (a.q8) hipLaunchKernelGGL((k_attn_dec<HD, REP, 1>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_attn_dec<HD, REP, 0>), grid, block, 0, s, a);
    } else {
        dim3 grid(a.max_split, a.nk, T), block(256);
        if (a.q8) hipLaunchKernelGGL((k_attn<HD, REP, 1>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_attn<HD, REP, 0>), grid, block, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one-row calls: 16 waves per head channel block; multi-row calls have
    // fewer, longer splits and many more rows, so 4
    dim3 mgrid(T < 0 ? -T : T, a.nh, (HD + 63) / 64);
    const int waves = T > 1 ? 4 : 16;
    if (a.q8) hipLaunchKernelGGL((k_attn_merge<1>), mgrid, dim3(64 * waves), 0, s, a);
    else hipLaunchKernelGGL((k_attn_merge<0>), mgrid, dim3(64 * waves), 0, s, a);
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

}  // namespace

hipError_t launch_prep(const PrepArgs &a, int T, hipStream_t s) {
    hipLaunchKernelGGL(k_prep, dim3(T, a.nh + a.nk), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a, int T, hipStream_t s) {
    if (a.split <= 0 || a.split > 256 || T <= 0) return hipErrorInvalidValue;
    return launch_hd(a, T, s);
}

int attn_dec_max_split(int hd) {
    const int kb = 256 / (hd / 4);
    return 8 * kb < 256 ? 8 * kb : 256;
}

hipError_t launch_attn_dec(const AttnArgs &a, int T, hipStream_t s) {
    if (a.split <= 0 || a.split > attn_dec_max_split(a.hd) || T <= 0) return hipErrorInvalidValue;
    return launch_hd(a, -T, s);
}

}  // namespace dk
