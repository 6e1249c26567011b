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
    } else if constexpr (EPI == EPI_VOUT) {
        const int row = m / p.Tx, t = m - row * p.Tx;
        const int r = row % p.R;
        const bool valid = p.mask == nullptr || p.mask[(long long)r * p.Tx + t] != 0;
        ((float*)p.out)[(long long)m * p.ldo + n] = valid ? acc + b : 0.0f;
    }
}

}  // namespace cfm
