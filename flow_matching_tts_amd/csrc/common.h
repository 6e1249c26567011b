// Shared device helpers for the gfx950 kernels: bf16 packing, wave64
// reductions, MFMA vector types and the row -> modulation-vector mapping.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cfm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float gelu_erf(float x) {
    // exact GELU: x * Phi(x) = x/2 (1 + erf(x / sqrt 2)), erf from the device math library
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

// GELU for bf16 outputs: x * Phi(x) with the complementary error function from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erfc(z) ~= t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2), t = 1 / (1 + p z),
// z >= 0, absolute error at most 1.5e-7, far below a bf16 ulp. Branch-free,
// one hardware reciprocal and one hardware exp2; Phi(x) = 1 - erfc(z)/2 for
// x >= 0 and erfc(z)/2 below, with z = |x| / sqrt 2 (no cancellation for x < 0).
__device__ __forceinline__ float gelu_as(float x) {
    const float z = fabsf(x) * 0.70710678118654752440f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
    float q = fmaf(t, 1.061405429f, -1.453152027f);
    q = fmaf(t, q, 1.421413741f);
    q = fmaf(t, q, -0.284496736f);
    q = fmaf(t, q, 0.254829592f);
    const float half_erfc = 0.5f * t * q * __builtin_amdgcn_exp2f(-1.44269504088896341f * z * z);
    return x * (x >= 0.0f ? 1.0f - half_erfc : half_erfc);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// Where a row's modulation vectors live. Rows are branch-major (row = b*R + r);
// token m belongs to row m / tokens_per_row, or to row tok_row[m] in the packed
// layout of a variable-length batch. Every row reads conditioning
// vector 0 except the rows of branch `spk_branch`, whose condition carries the
// request's speaker vector and reads vector 1 + r.
struct RowMod {
    const float* base = nullptr;       // vector 0 of the current step, already offset to the chunk
    long long cvec_stride = 0;         // floats between consecutive conditioning vectors
    int tokens_per_row = 1;
    int n_requests = 1;
    int spk_branch = -1;               // -1: every row uses vector 0
    const int32_t* tok_row = nullptr;  // packed rows: row of each token (else m / tokens_per_row)

    __device__ __forceinline__ const float* at(long long m) const {
        if (spk_branch < 0) return base;
        int row = tok_row ? tok_row[m] : (int)(m / tokens_per_row);
        int b = row / n_requests;
        int r = row - b * n_requests;
        return base + (b == spk_branch ? (long long)(1 + r) * cvec_stride : 0);
    }
};

}  // namespace cfm
