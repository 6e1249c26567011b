// Per-element GEMM epilogues (bias, GELU, gated residual, input-projection
// scatter into the branch rows, masked velocity store).
#pragma once
#include "kernels.h"

namespace cfm {

template <typename OutT> __device__ __forceinline__ OutT to_out(float v);
template <> __device__ __forceinline__ float to_out<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 to_out<bf16>(float v) { return (bf16)v; }

template <int EPI, typename ActT>
__device__ __forceinline__ void epi_store(const EpiParams& p, int m, int n, float acc) {
    const float b = p.bias ? p.bias[n] : 0.0f;
    if constexpr (EPI == EPI_F32) {
        ((float*)p.out)[(long long)m * p.ldo + n] = acc + b;
    } else if constexpr (EPI == EPI_ACT) {
        ((ActT*)p.out)[(long long)m * p.ldo + n] = to_out<ActT>(acc + b);
    } else if constexpr (EPI == EPI_GELU_ACT) {
        ((ActT*)p.out)[(long long)m * p.ldo + n] = to_out<ActT>(gelu_erf(acc + b));
    } else if constexpr (EPI == EPI_GATED) {
        float* h = (float*)p.out + (long long)m * p.ldo + n;
        *h += p.gate.at((long long)m)[n] * (acc + b);
    } else if constexpr (EPI == EPI_INPROJ) {
        const int r = m / p.Tx, t = m - r * p.Tx;
        const float plain = acc + b;
        const float withc = p.cproj ? acc + p.cproj[(long long)m * p.ldo + n] : plain;
        for (int br = 0; br < p.nb; ++br) {
            long long tok = (long long)(br * p.R + r) * p.T + p.P + t;
            ((float*)p.out)[tok * p.ldo + n] = br >= p.cond_branch0 ? withc : plain;
        }
    } else if constexpr (EPI == EPI_QKV) {
        if (n < p.d2) {
            ((bf16*)p.out)[(long long)m * p.ldo + n] = (bf16)(acc + b);
        } else {
            const int row = m / p.T, t = m - row * p.T;
            const int c = n - p.d2, hh = c >> 6, e = c & 63;
            p.vt[((long long)(row * p.H + hh) * 64 + e) * p.Tp + t] = (bf16)(acc + b);
        }
    } else if constexpr (EPI == EPI_VOUT) {
        const int row = m / p.Tx, t = m - row * p.Tx;
        const int r = row % p.R;
        const bool valid = p.mask == nullptr || p.mask[(long long)r * p.Tx + t] != 0;
        ((float*)p.out)[(long long)m * p.ldo + n] = valid ? acc + b : 0.0f;
    }
}

// Four consecutive rows m0..m0+3 of one column (one lane's registers g*4 + 0..3).
// EPI_QKV stores the four transposed values of a value column as one 8-byte
// write when they belong to the same sequence row; everything else goes per element.
template <int EPI, typename ActT>
__device__ __forceinline__ void epi_store4(const EpiParams& p, int m0, int M, int n, const float* acc4) {
    if constexpr (EPI == EPI_QKV) {
        if (n >= p.d2 && m0 + 3 < M) {
            const int row = m0 / p.T, t = m0 - row * p.T;
            if (t + 3 < p.T && (t & 3) == 0) {
                const float b = p.bias ? p.bias[n] : 0.0f;
                const int c = n - p.d2, hh = c >> 6, e = c & 63;
                bf16x4 v;
                v[0] = (bf16)(acc4[0] + b); v[1] = (bf16)(acc4[1] + b);
                v[2] = (bf16)(acc4[2] + b); v[3] = (bf16)(acc4[3] + b);
                *(bf16x4*)(p.vt + ((long long)(row * p.H + hh) * 64 + e) * p.Tp + t) = v;
                return;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (m0 + r < M) epi_store<EPI, ActT>(p, m0 + r, n, acc4[r]);
}

}  // namespace cfm
