// gemm.hip -- projections of multi-row calls: C[m][n] = sum_k A[m][k] W[n][k]
// (dory.rs `attn_layer` / `mlp_layer`, the matmat branches), A fp32 [T][K]
// activations, W [N][K] weights in bf16 or fp32, fp32 accumulation.
//
// This is the portable tiled form: 64x64 output tiles, K in steps of 16 staged
// through LDS, 4x4 outputs per thread.  It keeps fp32 activations, so it also
// serves the fp32-weight geometries exactly.
#include "device.h"

namespace dk {

namespace {

constexpr int BM = 64, BN = 64, BK = 16;

template <int WT>
__global__ __launch_bounds__(256) void k_gemm_tiled(const float *__restrict__ A, int lda,
                                                    const void *__restrict__ Wv, int N, int K,
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
                    const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(Wv) +
                                                                     (size_t)n * K + k);
                    v = make_float4(bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y));
                } else {
                    v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(Wv) + (size_t)n * K + k);
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

}  // namespace

hipError_t launch_gemm(int wtype, const float *A, int lda, const void *W, int N, int K, float *C, int ldc,
                       int M, hipStream_t s) {
    if (K % 4 || lda % 4) return hipErrorInvalidValue;
    dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(256);
    if (wtype == kBF16) hipLaunchKernelGGL((k_gemm_tiled<kBF16>), grid, block, 0, s, A, lda, W, N, K, C, ldc, M);
    else hipLaunchKernelGGL((k_gemm_tiled<kF32>), grid, block, 0, s, A, lda, W, N, K, C, ldc, M);
    return hipGetLastError();
}

}  // namespace dk
