// bf16 MFMA GEMM for gfx950: C[m, n] = sum_k A[m, k] W[n, k] with fused epilogues.
//
// Both operands are K-contiguous (A row-major [M, K], W in Linear layout
// [N, K]), which is the natural operand order of v_mfma_f32_32x32x16_bf16:
// every lane feeds 8 consecutive k of one A row and 8 consecutive k of one W
// row, so LDS tiles are read with 16-byte loads and never transposed.
//
// Tiling: 256 threads (4 waves) per 128x128 output tile, each wave a 64x64
// quadrant = 2x2 MFMA 32x32 blocks (64 fp32 accumulators per lane). K advances
// in steps of 32 through a double-buffered LDS tile; the next tile's global
// loads are in flight while the current one feeds the MFMAs.
// fp32 A operands (the latent x and the condition features) are rounded to
// bf16 while being staged, so no separate conversion pass touches HBM.
#include "epilogue.h"

namespace cfm {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDK = BK + 8;          // LDS row pitch in bf16 (80 B): spreads rows over banks
constexpr int NT = 256;

template <typename AT> struct AStage;

// bf16 A: 128 rows x 4 chunks of 8 = 512 chunks, 2 per thread
template <> struct AStage<bf16> {
    bf16x8 v[2];
    __device__ __forceinline__ void load(const bf16* A, int lda, int M, int K, int m0, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c = tid + i * NT, row = c >> 2, kc = (c & 3) * 8;
            int m = m0 + row, k = k0 + kc;
            if (m < M && k < K) v[i] = *(const bf16x8*)(A + (long long)m * lda + k);
            else v[i] = bf16x8{};
        }
    }
    __device__ __forceinline__ void store(bf16* As, int tid) const {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c = tid + i * NT, row = c >> 2, kc = (c & 3) * 8;
            *(bf16x8*)(As + row * LDK + kc) = v[i];
        }
    }
};

// fp32 A: 128 rows x 8 chunks of 4 = 1024 chunks, 4 per thread, rounded to bf16
template <> struct AStage<float> {
    f32x4 v[4];
    __device__ __forceinline__ void load(const float* A, int lda, int M, int K, int m0, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int c = tid + i * NT, row = c >> 3, kc = (c & 7) * 4;
            int m = m0 + row, k = k0 + kc;
            if (m < M && k < K) v[i] = *(const f32x4*)(A + (long long)m * lda + k);
            else v[i] = f32x4{};
        }
    }
    __device__ __forceinline__ void store(bf16* As, int tid) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int c = tid + i * NT, row = c >> 3, kc = (c & 7) * 4;
            bf16x4 b;
            b[0] = (bf16)v[i][0]; b[1] = (bf16)v[i][1]; b[2] = (bf16)v[i][2]; b[3] = (bf16)v[i][3];
            *(bf16x4*)(As + row * LDK + kc) = b;
        }
    }
};

struct WStage {
    bf16x8 v[2];
    __device__ __forceinline__ void load(const bf16* W, int ldw, int N, int K, int n0, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c = tid + i * NT, row = c >> 2, kc = (c & 3) * 8;
            int n = n0 + row, k = k0 + kc;
            if (n < N && k < K) v[i] = *(const bf16x8*)(W + (long long)n * ldw + k);
            else v[i] = bf16x8{};
        }
    }
    __device__ __forceinline__ void store(bf16* Ws, int tid) const {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c = tid + i * NT, row = c >> 2, kc = (c & 3) * 8;
            *(bf16x8*)(Ws + row * LDK + kc) = v[i];
        }
    }
};

template <typename AT, int EPI>
__global__ void __launch_bounds__(NT)
gemm_bf16_kernel(const AT* __restrict__ A, int lda, const bf16* __restrict__ W, int ldw,
                 int M, int N, int K, EpiParams ep) {
    __shared__ __attribute__((aligned(16))) bf16 As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) bf16 Ws[2][BN * LDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    AStage<AT> sa;
    WStage sw;
    const int nk = (K + BK - 1) / BK;
    sa.load(A, lda, M, K, m0, 0, tid);
    sw.load(W, ldw, N, K, n0, 0, tid);
    sa.store(As[0], tid);
    sw.store(Ws[0], tid);
    __syncthreads();

    int cur = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) {
            sa.load(A, lda, M, K, m0, (kt + 1) * BK, tid);
            sw.load(W, ldw, N, K, n0, (kt + 1) * BK, tid);
        }
        const bf16* as = As[cur];
        const bf16* ws = Ws[cur];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *(const bf16x8*)(as + (wm * 64 + i * 32 + li) * LDK + ks * 16 + lh * 8);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *(const bf16x8*)(ws + (wn * 64 + j * 32 + li) * LDK + ks * 16 + lh * 8);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            sa.store(As[cur ^ 1], tid);
            sw.store(Ws[cur ^ 1], tid);
        }
        __syncthreads();
        cur ^= 1;
    }

    // accumulator layout of a 32x32 block: register g*4 + r holds
    // row 8g + 4*(lane/32) + r, column lane%32.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + j * 32 + li;
            if (n >= N) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + wm * 64 + i * 32 + 8 * g + 4 * lh + r;
                    if (m < M) epi_store<EPI, bf16>(ep, m, n, acc[i][j][g * 4 + r]);
                }
        }
}

template <typename AT>
void launch_a(int epi, const AT* A, int lda, const bf16* W, int ldw, int M, int N, int K,
              const EpiParams& ep, hipStream_t s) {
    dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
    switch (epi) {
        case EPI_F32: gemm_bf16_kernel<AT, EPI_F32><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        case EPI_ACT: gemm_bf16_kernel<AT, EPI_ACT><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        case EPI_GELU_ACT: gemm_bf16_kernel<AT, EPI_GELU_ACT><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        case EPI_GATED: gemm_bf16_kernel<AT, EPI_GATED><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        case EPI_INPROJ: gemm_bf16_kernel<AT, EPI_INPROJ><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        case EPI_VOUT: gemm_bf16_kernel<AT, EPI_VOUT><<<grid, NT, 0, s>>>(A, lda, W, ldw, M, N, K, ep); break;
        default: break;
    }
}

}  // namespace

void launch_gemm_bf16(bool a_f32, int epi, const void* A, int lda, const bf16* W, int ldw,
                      int M, int N, int K, const EpiParams& ep, hipStream_t s) {
    if (M <= 0 || N <= 0) return;
    if (a_f32) launch_a<float>(epi, (const float*)A, lda, W, ldw, M, N, K, ep, s);
    else launch_a<bf16>(epi, (const bf16*)A, lda, W, ldw, M, N, K, ep, s);
}

}  // namespace cfm
