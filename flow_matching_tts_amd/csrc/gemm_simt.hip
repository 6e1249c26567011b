// fp32 FMA GEMM (no matrix cores): C[m, n] = sum_k act(A[m, k]) W[n, k], fp32 accumulation.
//
// Used where fp32 arithmetic is the contract: every GEMM of the fp32 sampler,
// and the hoisted conditioning GEMMs of the bf16 sampler (timestep MLP,
// speaker projection, adaLN modulation for all steps), whose activations stay
// fp32 against bf16 weights. 64x64 output tile per 256 threads, 4x4 outputs
// per thread, K staged through LDS in steps of 16.
#include "epilogue.h"

namespace cfm {
namespace {

constexpr int TM = 64, TN = 64, TK = 16, NT = 256;

template <typename WT> __device__ __forceinline__ float ld_w(const WT* p);
template <> __device__ __forceinline__ float ld_w<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_w<bf16>(const bf16* p) { return (float)*p; }

template <typename WT, bool SILU_A, int EPI>
__global__ void __launch_bounds__(NT)
gemm_simt_kernel(const float* __restrict__ A, int lda, const WT* __restrict__ W, int ldw,
                 int M, int N, int K, EpiParams ep) {
    __shared__ float As[TK][TM + 4];
    __shared__ float Ws[TK][TN + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
    if (ep.m_dev) {                 // device row count (at most M): whole block, before any barrier
        M = min(M, *ep.m_dev);
        if (m0 >= M) return;
    }
    float acc[4][4] = {};

    for (int k0 = 0; k0 < K; k0 += TK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * NT, row = e >> 4, kk = e & 15;
            const int m = m0 + row, n = n0 + row, k = k0 + kk;
            float a = (m < M && k < K) ? A[(long long)m * lda + k] : 0.0f;
            if (SILU_A) a = (m < M && k < K) ? silu(a) : 0.0f;
            As[kk][row] = a;
            Ws[kk][row] = (n < N && k < K) ? ld_w<WT>(W + (long long)n * ldw + k) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = Ws[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
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
            if (n < N) epi_store<EPI, float>(ep, m, n, acc[i][j]);
        }
    }
}

template <typename WT, bool SILU_A>
void launch_w(int epi, const float* A, int lda, const WT* W, int ldw, int M, int N, int K,
              const EpiParams& ep, hipStream_t s) {
    dim3 grid((N + TN - 1) / TN, (M + TM - 1) / TM);
    switch (epi) {
        case EPI_F32: gemm_simt_kernel<WT, SILU_A, EPI_F32><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        case EPI_ACT: gemm_simt_kernel<WT, SILU_A, EPI_ACT><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        case EPI_GELU_ACT: gemm_simt_kernel<WT, SILU_A, EPI_GELU_ACT><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        case EPI_GATED: gemm_simt_kernel<WT, SILU_A, EPI_GATED><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        case EPI_INPROJ: gemm_simt_kernel<WT, SILU_A, EPI_INPROJ><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        case EPI_VOUT: gemm_simt_kernel<WT, SILU_A, EPI_VOUT><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        default: break;
    }
}

}  // namespace

void launch_gemm_simt(bool w_bf16, bool silu_a, int epi, const float* A, int lda, const void* W,
                      int ldw, int M, int N, int K, const EpiParams& ep, hipStream_t s) {
    if (M <= 0 || N <= 0) return;
    if (w_bf16) {
        if (silu_a) launch_w<bf16, true>(epi, A, lda, (const bf16*)W, ldw, M, N, K, ep, s);
        else launch_w<bf16, false>(epi, A, lda, (const bf16*)W, ldw, M, N, K, ep, s);
    } else {
        if (silu_a) launch_w<float, true>(epi, A, lda, (const float*)W, ldw, M, N, K, ep, s);
        else launch_w<float, false>(epi, A, lda, (const float*)W, ldw, M, N, K, ep, s);
    }
}

}  // namespace cfm
