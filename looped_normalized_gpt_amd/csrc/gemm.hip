// gemm.hip -- projections of multi-row calls: C[m][n] = sum_k A[m][k] W[n][k]
// (dory.rs `attn_layer` / `mlp_layer`, the matmat branches), A fp32 [T][K]
// activations, W [N][K] weights in bf16 or fp32, fp32 accumulation.
//
// Two forms:
//  * k_gemm_mfma (bf16 weights): v_mfma_f32_32x32x16_bf16 on 128 x BN tiles,
//    K in steps of 32 through double-buffered LDS; activations are rounded to
//    bf16 as they are staged (the prefill chunks are dense contractions).
//  * k_gemm_tiled: 64x64 fp32 FMA tiles that keep fp32 activations; it serves
//    the fp32-weight geometries exactly, and short chunks.
#include "device.h"

namespace dk {

namespace {

constexpr int BM = 64, BN = 64, BK = 16;

// Row n of the stacked weight segments.
template <typename T>
__device__ inline const T *seg_row(const GemmW &g, int n, int K) {
    const void *b = g.w[0];
    int start = 0;
#pragma unroll
    for (int i = 1; i < 4; ++i)
        if (i < g.nseg && n >= g.seg_end[i - 1]) {
            b = g.w[i];
            start = g.seg_end[i - 1];
        }
    return reinterpret_cast<const T *>(b) + (size_t)(n - start) * K;
}

template <int WT>
__global__ __launch_bounds__(256) void k_gemm_tiled(const float *__restrict__ A, int lda,
                                                    const GemmW Wv, int N, int K,
                                                    float *__restrict__ C, int ldc, int M) {
    __shared__ float As[BK][BM + 4];
    __shared__ float Ws[BK][BN + 4];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row lr, k lk..lk+3
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
        {
            const int m = m0 + lr, k = k0 + lk;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m < M && k < K) v = *reinterpret_cast<const float4 *>(A + (size_t)m * lda + k);
            As[lk + 0][lr] = v.x;
            As[lk + 1][lr] = v.y;
            As[lk + 2][lr] = v.z;
            As[lk + 3][lr] = v.w;
        }
        {
            const int n = n0 + lr, k = k0 + lk;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (n < N && k < K) {
                if (WT == kBF16) {
                    const uint2 u = *reinterpret_cast<const uint2 *>(seg_row<uint16_t>(Wv, n, K) + k);
                    v = make_float4(bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y));
                } else {
                    v = *reinterpret_cast<const float4 *>(seg_row<float>(Wv, n, K) + k);
                }
            }
            Ws[lk + 0][lr] = v.x;
            Ws[lk + 1][lr] = v.y;
            Ws[lk + 2][lr] = v.z;
            Ws[lk + 3][lr] = v.w;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const float4 a = *reinterpret_cast<const float4 *>(&As[k][ty * 4]);
            const float4 w = *reinterpret_cast<const float4 *>(&Ws[k][tx * 4]);
            const float av[4] = {a.x, a.y, a.z, a.w}, wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], wv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n < N) C[(size_t)m * ldc + n] = acc[i][j];
        }
    }
}


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 256 threads = 4 waves in a 2 x 2 arrangement; a wave owns a (BM/2) x (BN/2)
// block of C as 32x32 MFMA tiles.  Operand layout of the 32x32x16 bf16 MFMA:
// lane l supplies row (l % 32) and k = 8 (l / 32) .. +7 of A (and of B); it
// receives C[8 (j/4) + 4 (l/32) + j%4][l % 32] in accumulator j.
template <int BN>
__global__ __launch_bounds__(256) void k_gemm_mfma(const uint16_t *__restrict__ A, int lda,
                                                   const GemmW W, int N, int K,
                                                   float *__restrict__ C, int ldc, int M) {
    constexpr int BM = 128, BK = 32, LDK = BK + 8;  // padded LDS rows (bf16)
    constexpr int TM = BM / 2 / 32, TN = BN / 2 / 32; // MFMA tiles per wave
    __shared__ __bf16 As[2][BM][LDK];
    __shared__ __bf16 Bs[2][BN][LDK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    // loaders: A rows tid/2 (128 rows), 16 bf16 each; B rows tid/2 (< BN), 16 bf16 each
    const int lr = tid >> 1, lc = (tid & 1) * 16;
    uint4 ra[2];
    uint4 rb[2];
    auto gload = [&](int k0) {
        const int m = m0 + lr, k = k0 + lc;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const bool ok = m < M && k + 8 * i < K;
            ra[i] = ok ? *reinterpret_cast<const uint4 *>(A + (size_t)m * lda + k + 8 * i) : make_uint4(0, 0, 0, 0);
        }
        const int n = n0 + lr;
        const uint16_t *wr = seg_row<uint16_t>(W, n < N ? n : 0, K);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const bool ok = lr < BN && n < N && k + 8 * i < K;
            rb[i] = ok ? *reinterpret_cast<const uint4 *>(wr + k + 8 * i) : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
        *reinterpret_cast<uint4 *>(&As[buf][lr][lc]) = ra[0];
        *reinterpret_cast<uint4 *>(&As[buf][lr][lc + 8]) = ra[1];
        if (lr < BN) {
            *reinterpret_cast<uint4 *>(&Bs[buf][lr][lc]) = rb[0];
            *reinterpret_cast<uint4 *>(&Bs[buf][lr][lc + 8]) = rb[1];
        }
    };
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    gload(0);
    sstore(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < K; k0 += BK) {
        const bool more = k0 + BK < K;
        if (more) gload(k0 + BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = *reinterpret_cast<const bf16x8 *>(&As[buf][wm * (BM / 2) + i * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[buf][wn * (BN / 2) + j * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            sstore(buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * (BM / 2) + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (row < M) C[(size_t)row * ldc + col] = acc[i][j][e];
            }
        }
}



// Multi-row projections (prefill chunks): 128 x 128 tiles of C, K in steps of
// 64 through double-buffered LDS (rows padded to 72 bf16), with the global
// loads of the next two K steps in flight in registers.  256 threads = 4 waves
// in a 2 x 2 arrangement, each owning a 64 x 64 block as 2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 (lane l supplies row l % 32 and k = 8 (l/32) .. +7
// of A and of B, and receives C[8 (j/4) + 4 (l/32) + j%4][l % 32] in
// accumulator j).  73.7 KB of LDS: two workgroups per CU.
// Split K: workgroup z takes K range [z K/S, (z+1) K/S) and writes its partial
// C to C + z * pstride; the caller's consumer adds the S slabs.
// SWIGLU (the MLP's gate | up projection, dory.rs `mlp_layer`): tile x pairs
// gate rows 64x .. 64x+63 (columns 0..63, W.w[0]) with the same up rows
// (columns 64..127, W.w[1]); the waves holding the up half hand their
// accumulators to the gate waves through LDS (same lane layout, so the same
// element is the same (row, ffn index)), which store z = silu(a sg) (b su)
// rounded to bf16 at zb[row][64x + c] (row stride N/2 = ffn) and the row's sum
// of z^2 over the tile's 64 indices at ssp[row][x] (the renorm before the down
// projection is then a per-row factor its consumer applies).  No C is written.
template <bool SWIGLU>
__global__ __launch_bounds__(256, 2) void k_gemm_mfma2(const uint16_t *__restrict__ A, int lda, const GemmW W, int N,
                                                       int K, float *__restrict__ C, int ldc, int M, int S,
                                                       size_t pstride, const float *__restrict__ sg,
                                                       const float *__restrict__ su, uint16_t *__restrict__ zb,
                                                       float *__restrict__ ssp) {
    constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;
    __shared__ __bf16 As[2][BM][LDK];
    __shared__ __bf16 Bs[2][BN][LDK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int Kp = K / S, kz = blockIdx.z * Kp;
    // loaders: load i of thread t reads row 32 i + t/8, 8 bf16 at 8 (t%8) of the
    // tile (8 consecutive threads read one 128-byte row run)
    const int lr = tid >> 3, lc = (tid & 7) * 8;
    const uint16_t *arow[4], *brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int am = m0 + 32 * i + lr < M ? m0 + 32 * i + lr : M - 1;
        arow[i] = A + (size_t)am * lda + kz + lc;
        if (SWIGLU) {  // tile column c: gate row 64x + c, or up row 64x + c - 64
            // (a select of the two pointers: indexing W.w by the lane's column
            // made the compiler reload them from the argument block and wait)
            const int c = 32 * i + lr;
            const void *wsel = c < 64 ? W.w[0] : W.w[1];
            brow[i] = reinterpret_cast<const uint16_t *>(wsel) + (size_t)(blockIdx.x * 64 + (c & 63)) * K + kz + lc;
        } else {
            const int bn = n0 + 32 * i + lr < N ? n0 + 32 * i + lr : N - 1;
            brow[i] = seg_row<uint16_t>(W, bn, K) + kz + lc;
        }
    }
    // the SwiGLU epilogue's gate and up scales, loaded with the first tiles
    // (after the loop they cost a round trip of their own)
    float sgv[2] = {0.f, 0.f}, suv[2] = {0.f, 0.f};
    if constexpr (SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            sgv[j] = sg[blockIdx.x * 64 + j * 32 + (lane & 31)];
            suv[j] = su[blockIdx.x * 64 + j * 32 + (lane & 31)];
        }
    }
    u32x4_t ra0[4], rb0[4];
    // (macros rather than lambdas over array references: the latter left the
    // staging registers in scratch memory)
#define GLOAD(ra, rb, ks)                                                                   \
    do {                                                                                    \
        const int k_ = (ks) * BK;                                                           \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) ra[i] =                               \
            *reinterpret_cast<const u32x4_t *>(arow[i] + k_);                               \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) rb[i] =                               \
            *reinterpret_cast<const u32x4_t *>(brow[i] + k_);                               \
    } while (0)
#define SSTORE(buf, ra, rb)                                                                 \
    do {                                                                                    \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                       \
            *reinterpret_cast<u32x4_t *>(&As[buf][32 * i + lr][lc]) = ra[i];                \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                       \
            *reinterpret_cast<u32x4_t *>(&Bs[buf][32 * i + lr][lc]) = rb[i];                \
    } while (0)
#define COMPUTE(buf)                                                                        \
    do {                                                                                    \
        _Pragma("unroll") for (int kk = 0; kk < BK; kk += 16) {                             \
            bf16x8 a_[2], b_[2];                                                            \
            _Pragma("unroll") for (int i = 0; i < 2; ++i) a_[i] = *reinterpret_cast<const bf16x8 *>( \
                &As[buf][wm * 64 + i * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);            \
            _Pragma("unroll") for (int j = 0; j < 2; ++j) b_[j] = *reinterpret_cast<const bf16x8 *>( \
                &Bs[buf][wn * 64 + j * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);            \
            _Pragma("unroll") for (int i = 0; i < 2; ++i)                                   \
                _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] =                   \
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_[i], b_[j], acc[i][j], 0, 0, 0); \
        }                                                                                   \
    } while (0)
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    // One K step of loads in flight in registers while the other LDS buffer is
    // computed on.  The loads are unconditional (past the last step they repeat
    // it), so the compiler's count of outstanding loads stays exact.
    const int nks = Kp / BK, last = nks - 1;
    GLOAD(ra0, rb0, 0);
    SSTORE(0, ra0, rb0);
    GLOAD(ra0, rb0, 1 < last ? 1 : last);
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
        const int buf = ks & 1;
        COMPUTE(buf);
        if (ks + 1 < nks) {
            SSTORE(buf ^ 1, ra0, rb0);
            GLOAD(ra0, rb0, ks + 2 < last ? ks + 2 : last);
        }
        __syncthreads();
    }
#undef GLOAD
#undef SSTORE
#undef COMPUTE
    if constexpr (SWIGLU) {
        // The two waves of a 64-row block hold the gate (wn 0) and up (wn 1)
        // halves of the same (row, ffn index) elements in the same lanes.  Each
        // hands the other its accumulators of one 32-row tile through LDS (the
        // operand tiles are free after the loop's last barrier) and finishes
        // the other tile: wn 0 rows 0..31 of the block, wn 1 rows 32..63.
        float *ex = reinterpret_cast<float *>(&As[0][0][0]);
        float *mine = ex + (wn * 2 + wm) * (2 * 16 * 64);          // [j][e][lane]
        const float *other = ex + ((1 - wn) * 2 + wm) * (2 * 16 * 64);
        if (wn == 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) mine[(j * 16 + e) * 64 + lane] = acc[1][j][e];
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) mine[(j * 16 + e) * 64 + lane] = acc[0][j][e];
        }
        __syncthreads();
        const int F = N / 2, x = blockIdx.x;
        const int i = wn;  // the 32-row tile this wave finishes
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float a = wn == 0 ? acc[0][j][e] : other[(j * 16 + e) * 64 + lane];
                const float b = wn == 0 ? other[(j * 16 + e) * 64 + lane] : acc[1][j][e];
                const float g = a * sgv[j];
                const float z = g / (1.0f + expf(-g)) * (b * suv[j]);
                ss += z * z;
                if (row < M) zb[(size_t)row * F + x * 64 + j * 32 + (lane & 31)] = f2bf(z);
            }
            // the row's 64 indices lie in the 32 lanes of this lane's half: DPP
            // row sums, then row 0's sum into row 1 and row 2's into row 3
            ss = group_sum<16>(ss);
            ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x142, 0xA, 0xF, false));
            if ((lane & 31) == 31 && row < M) ssp[(size_t)row * (F / 64) + x] = ss;
        }
        return;
    }
    float *Cz = C + (size_t)blockIdx.z * pstride;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (row < M) Cz[(size_t)row * ldc + col] = acc[i][j][e];
            }
        }
}


// The same tiles fed by LDS DMA (global_load_lds_dwordx4: lane i of a wave's
// load writes 16 bytes at the wave's LDS address + 16 i, no staging
// registers), STAGES deep: the loads of STAGES-1 K steps stay in flight while
// one step is computed, which covers the memory latency that a one-step
// register prefetch left exposed.  A tile row (64 bf16 = 8 chunks of 16 bytes)
// is stored with chunk c at position c ^ ((row / 2) % 8), so the rows a wave
// reads for one MFMA operand fall in different banks.  One workgroup per CU
// (STAGES x 32 KB of LDS).
// LDS byte address of a shared-memory pointer
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

template <int STAGES>
__global__ __launch_bounds__(512) void k_gemm_dma(const uint16_t *__restrict__ A, int lda, const GemmW W, int N, int K,
                                                  float *__restrict__ C, int ldc, int M, int S, size_t pstride) {
    constexpr int BM = 128, BN = 128, BK = 64, TE = BM * BK;  // elements of one operand tile
    __shared__ __attribute__((aligned(16))) uint16_t lds[STAGES][2][TE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;  // 8 waves: 2 per SIMD
    const int wm = wave >> 2, wn = wave & 3;                        // wave block: rows 64 wm, cols 32 wn
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int Kp = K / S, kz = blockIdx.z * Kp;
    // DMA: load j (0..1) of wave w covers tile rows 16 w + 8 j .. +7; lane l
    // reads row r = 16 w + 8 j + l/8, global chunk (l % 8) ^ sw(r), and lands at
    // chunk l % 8 of that row.  sw(r) = (r / 2) % 8: the 16 rows a group of 16
    // lanes reads at one logical chunk then sit in 16 different bank groups
    // (two 128-byte rows share a 256-byte bank line).
    const int crow = lane >> 3;
    const uint16_t *asrc[2], *bsrc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 16 * wave + 8 * j + crow;
        const int csrc = (lane & 7) ^ ((row >> 1) & 7);
        const int gm = m0 + row < M ? m0 + row : M - 1;
        const int gn = n0 + row < N ? n0 + row : N - 1;
        asrc[j] = A + (size_t)gm * lda + kz + 8 * csrc;
        bsrc[j] = seg_row<uint16_t>(W, gn, K) + kz + 8 * csrc;
    }
    auto issue = [&](int st, int ks) {
        const int k = ks * BK;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(asrc[j] + k),
                                             (__attribute__((address_space(3))) void *)(&lds[st][0][(16 * wave + 8 * j) * BK]),
                                             16, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(bsrc[j] + k),
                                             (__attribute__((address_space(3))) void *)(&lds[st][1][(16 * wave + 8 * j) * BK]),
                                             16, 0, 0);
    };
    f32x16 acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
    const int nks = Kp / BK, last = nks - 1;
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st) issue(st, st < last ? st : last);
    for (int ks = 0; ks < nks; ++ks) {
        // refill the buffer step ks-1 used (every wave passed the barrier after
        // computing it); unconditional, so every wave always has the same loads
        // outstanding: steps ks .. ks+STAGES-1, 4 per step, oldest first
        const int nx = ks + STAGES - 1;
        issue(nx % STAGES, nx < last ? nx : last);
        // this wave's loads of step ks have landed; the barrier makes every
        // wave's (plain s_barrier: a fence here would wait for all loads)
        if constexpr (STAGES == 4) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        else if constexpr (STAGES == 3) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        const uint32_t As = lds_addr(lds[ks % STAGES][0]), Bs = lds_addr(lds[ks % STAGES][1]);
        const int ra0 = wm * 64 + (lane & 31), ra1 = ra0 + 32, rb = wn * 32 + (lane & 31);
        // the step's 12 operand fragments in one batch and one wait, then its
        // 8 MFMAs back to back.  LDS reads in asm: the compiler cannot tell them
        // from the DMA's destinations and would otherwise wait for every load
        // in flight.  Early-clobber outputs: no output shares a register with
        // an address still to be read.
        bf16x8 a0[4], a1[4], b[4];
        uint32_t ad0[4], ad1[4], bd[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ch = 2 * q + (lane >> 5);   // the global 16-byte chunk this lane supplies
            ad0[q] = As + 2 * (ra0 * BK + 8 * (ch ^ ((ra0 >> 1) & 7)));
            ad1[q] = As + 2 * (ra1 * BK + 8 * (ch ^ ((ra1 >> 1) & 7)));
            bd[q] = Bs + 2 * (rb * BK + 8 * (ch ^ ((rb >> 1) & 7)));
        }
        asm volatile(
            "ds_read_b128 %0, %12\n\t"
            "ds_read_b128 %1, %13\n\t"
            "ds_read_b128 %2, %14\n\t"
            "ds_read_b128 %3, %15\n\t"
            "ds_read_b128 %4, %16\n\t"
            "ds_read_b128 %5, %17\n\t"
            "ds_read_b128 %6, %18\n\t"
            "ds_read_b128 %7, %19\n\t"
            "ds_read_b128 %8, %20\n\t"
            "ds_read_b128 %9, %21\n\t"
            "ds_read_b128 %10, %22\n\t"
            "ds_read_b128 %11, %23\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a0[0]), "=&v"(a1[0]), "=&v"(b[0]), "=&v"(a0[1]), "=&v"(a1[1]), "=&v"(b[1]),
              "=&v"(a0[2]), "=&v"(a1[2]), "=&v"(b[2]), "=&v"(a0[3]), "=&v"(a1[3]), "=&v"(b[3])
            : "v"(ad0[0]), "v"(ad1[0]), "v"(bd[0]), "v"(ad0[1]), "v"(ad1[1]), "v"(bd[1]),
              "v"(ad0[2]), "v"(ad1[2]), "v"(bd[2]), "v"(ad0[3]), "v"(ad1[3]), "v"(bd[3]));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[q], b[q], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[q], b[q], acc[1], 0, 0, 0);
        }
        // every wave's reads of this buffer are done (lgkmcnt 0 above) before
        // the next iteration's loads refill it
        __builtin_amdgcn_s_barrier();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated tail loads, before the workgroup ends
    float *Cz = C + (size_t)blockIdx.z * pstride;
    const int col = n0 + wn * 32 + (lane & 31);
    if (col < N) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (row < M) Cz[(size_t)row * ldc + col] = acc[i][e];
            }
    }
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Few-row projections (batched decode, short chunks): M <= 16*MT rows of bf16
// activations against bf16 weights, on v_mfma_f32_16x16x32_bf16.  Workgroup =
// 64 weight rows (output columns), wave w the 16 rows 16w..; K blocks of 128
// in order, the workgroup's share of them when K is split (part z of S writes
// C + z * pstride, the reader adds the slabs).  Each activation block (M rows
// x 128) is loaded once per workgroup, coalesced, into LDS and read by all four
// waves; each wave streams its weight rows straight into registers, four K
// blocks ahead.  Operand layout of the 16x16x32 MFMA: lane l supplies row
// l % 16 and k-slots 8 (l/16) .. +7 of A (and of B), and receives
// C[4 (l/16) + i][l % 16] in accumulator i; MFMA t of a block takes k = 32t ..
// 32t+31.
template <int MT>
__global__ __launch_bounds__(256) void k_gemm_skinny(const uint16_t *__restrict__ A, int lda, const GemmW W, int N,
                                                     int K, float *__restrict__ C, int ldc, int M, int S,
                                                     size_t pstride) {
    constexpr int AP = 128 + 8;                    // LDS row pitch (bf16)
    __shared__ __attribute__((aligned(16))) __bf16 As[2][16 * MT][AP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 64 + 16 * wave;
    const int nkb = K / 128, kb0 = (int)((long)blockIdx.y * nkb / S), kb1 = (int)((long)(blockIdx.y + 1) * nkb / S);
    const int nk = kb1 - kb0, last = nk - 1;
    const uint16_t *wrow = seg_row<uint16_t>(W, n0 + r < N ? n0 + r : N - 1, K) + (size_t)kb0 * 128 + 8 * g;
    // activation loader: thread t takes row t / 4 (rows >= 16 MT idle), the 32
    // bf16 at 32 (t % 4) of the block
    const int arw = tid >> 2, acl = (tid & 3) * 32;
    const bool aload = arw < 16 * MT;
    const uint16_t *arow = A + (size_t)(arw < M ? arw : M - 1) * lda + (size_t)kb0 * 128 + acl;
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    u4 w0[4], w1[4], w2[4], w3[4], a0[4], a1[4], a2[4], a3[4];
#define WLOAD(wv, j)                                                                        \
    do {                                                                                    \
        const int k_ = ((j) < last ? (j) : last) * 128;                                     \
        _Pragma("unroll") for (int t = 0; t < 4; ++t) wv[t] = *reinterpret_cast<const u4 *>(wrow + k_ + 32 * t); \
    } while (0)
#define ALOAD(av, j)                                                                        \
    do {                                                                                    \
        const int k_ = ((j) < last ? (j) : last) * 128;                                     \
        _Pragma("unroll") for (int t = 0; t < 4; ++t) av[t] = *reinterpret_cast<const u4 *>(arow + k_ + 8 * t); \
    } while (0)
#define ASTORE(buf, av)                                                                     \
    do {                                                                                    \
        if (aload) _Pragma("unroll") for (int t = 0; t < 4; ++t)                            \
            *reinterpret_cast<u4 *>(&As[buf][arw][acl + 8 * t]) = av[t];                    \
    } while (0)
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#define MMA(wv, buf)                                                                        \
    do {                                                                                    \
        _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                     \
            const bf16x8 b_ = __builtin_bit_cast(bf16x8, wv[t]);                            \
            _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                             \
                const bf16x8 a_ = *reinterpret_cast<const bf16x8 *>(&As[buf][16 * mt + r][32 * t + 8 * g]); \
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_, b_, acc[mt], 0, 0, 0); \
            }                                                                               \
        }                                                                                   \
    } while (0)
    // Unconditional loads (past the last block they repeat it) and a loop
    // unrolled by four keep the compiler's count of outstanding loads exact.
    // activations and weights both four K blocks ahead: block j sits in
    // registers a(j%4) and w(j%4) until it is consumed
    ALOAD(a0, 0);
    ALOAD(a1, 1);
    ALOAD(a2, 2);
    ALOAD(a3, 3);
    WLOAD(w0, 0);
    WLOAD(w1, 1);
    WLOAD(w2, 2);
    WLOAD(w3, 3);
    ASTORE(0, a0);
    ALOAD(a0, 4);
    __syncthreads();
#define STEP(j, wv, an, buf)                                                                \
    MMA(wv, buf);                                                                           \
    if (kb + (j) + 1 >= nk) break;                                                          \
    ASTORE((buf) ^ 1, an);                                                                  \
    ALOAD(an, kb + (j) + 5);                                                                \
    WLOAD(wv, kb + (j) + 4);                                                                \
    __syncthreads();
    for (int kb = 0; kb < nk; kb += 4) {
        STEP(0, w0, a1, 0)
        STEP(1, w1, a2, 1)
        STEP(2, w2, a3, 0)
        STEP(3, w3, a0, 1)
    }
#undef STEP
#undef MMA
#undef ASTORE
#undef ALOAD
#undef WLOAD
    float *Cz = C + (size_t)blockIdx.y * pstride;
    const int nn = n0 + r;
    if (nn < N)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * mt + 4 * g + i;
                if (m < M) Cz[(size_t)m * ldc + nn] = acc[mt][i];
            }
}

}  // namespace

hipError_t launch_gemm(int wtype, const float *A, const uint16_t *Ab, int lda, const GemmW &Wb, int N, int K,
                       float *C, int ldc, int M, hipStream_t s, int kparts, size_t pstride) {
    if (kparts < 1 || (kparts > 1 && !gemm_splits_ok(wtype, Ab != nullptr, M, K, kparts))) return hipErrorInvalidValue;
    if (K % 4 || lda % 4 || Wb.nseg < 1 || Wb.nseg > 4 || Wb.seg_end[Wb.nseg - 1] != N) return hipErrorInvalidValue;
    const GemmW W = Wb;
    if (wtype == kBF16 && Ab && lda % 8 == 0) {
        if (M <= 64 && K % 128 == 0) {
            const dim3 grid((N + 63) / 64, kparts);
            if (M <= 16) hipLaunchKernelGGL((k_gemm_skinny<1>), grid, dim3(256), 0, s, Ab, lda, W, N, K, C, ldc, M, kparts, pstride);
            else if (M <= 32) hipLaunchKernelGGL((k_gemm_skinny<2>), grid, dim3(256), 0, s, Ab, lda, W, N, K, C, ldc, M, kparts, pstride);
            else hipLaunchKernelGGL((k_gemm_skinny<4>), grid, dim3(256), 0, s, Ab, lda, W, N, K, C, ldc, M, kparts, pstride);
            return hipGetLastError();
        }
        if (M > 64 && K % 64 == 0) {
            // one workgroup per CU when the tiles fit the chip in one round (LDS
            // DMA, 4 stages); two per CU otherwise (register prefetch, 2 stages)
            const dim3 grid((N + 127) / 128, (M + 127) / 128, kparts);
            if ((long)grid.x * grid.y * grid.z <= 256)
                hipLaunchKernelGGL(k_gemm_dma<4>, grid, dim3(512), 0, s, Ab, lda, W, N, K, C, ldc, M, kparts, pstride);
            else
                hipLaunchKernelGGL(k_gemm_mfma2<false>, grid, dim3(256), 0, s, Ab, lda, W, N, K, C, ldc, M, kparts,
                                   pstride, nullptr, nullptr, nullptr, nullptr);
            return hipGetLastError();
        }
        if (M >= 32 && K % 8 == 0) {
            // bf16 MFMA; narrower tiles when the 128-wide ones would leave CUs idle
            const int mt = (M + 127) / 128;
            if ((long)mt * ((N + 127) / 128) >= 256)
                hipLaunchKernelGGL((k_gemm_mfma<128>), dim3((N + 127) / 128, mt), dim3(256), 0, s, Ab, lda, W, N, K,
                                   C, ldc, M);
            else
                hipLaunchKernelGGL((k_gemm_mfma<64>), dim3((N + 63) / 64, mt), dim3(256), 0, s, Ab, lda, W, N, K, C,
                                   ldc, M);
            return hipGetLastError();
        }
    }
    dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(256);
    if (wtype == kBF16) hipLaunchKernelGGL((k_gemm_tiled<kBF16>), grid, block, 0, s, A, lda, W, N, K, C, ldc, M);
    else hipLaunchKernelGGL((k_gemm_tiled<kF32>), grid, block, 0, s, A, lda, W, N, K, C, ldc, M);
    return hipGetLastError();
}

hipError_t launch_gemm_swiglu(const uint16_t *Ab, int lda, const void *wgate, const void *wup, int F, int K,
                              const float *sg, const float *su, uint16_t *zb, float *ssp, int M, hipStream_t s) {
    if (!gemm_swiglu_ok(kBF16, M, F, K, lda) || !Ab || !zb || !ssp) return hipErrorInvalidValue;
    const GemmW W{{wgate, wup, wup, wup}, {F, 2 * F, 2 * F, 2 * F}, 2};
    const dim3 grid(F / 64, (M + 127) / 128, 1);
    hipLaunchKernelGGL(k_gemm_mfma2<true>, grid, dim3(256), 0, s, Ab, lda, W, 2 * F, K, nullptr, 0, M, 1, (size_t)0,
                       sg, su, zb, ssp);
    return hipGetLastError();
}

}  // namespace dk
