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

// GELU for bf16 outputs. With y = min(|x|, 6),
//   GELU(x) = x Phi(x) = (x + |x| - y erfc(y / sqrt 2)) / 2   for |x| <= 6
// (erf is odd), and erfc(y / sqrt 2) = exp2(P(y)) with P a degree-8 polynomial
// fitted to log2 erfc(y / sqrt 2) on [0, 6] (flow_matching_tts_amd/gelu_fit.py
// derives the coefficients). The fit is in the log domain, so the relative error
// is bounded everywhere, tails included: below 1e-5 relative (5.2e-7 absolute)
// on [-6, 6], against a bf16 rounding of 2^-9. Past 6 the erfc term is below
// 6e-9 and is held at its value at 6. Horner by fused multiply-adds and one
// hardware exp2: no division, no branch, NaN propagates.
__device__ __forceinline__ float gelu_bf16(float x) {
    const float ax = fabsf(x);
    const float y = fminf(ax, 6.0f);
    float p = 6.125587149e-09f;
    p = fmaf(p, y, -2.091931947e-06f);
    p = fmaf(p, y, 6.530121027e-05f);
    p = fmaf(p, y, -9.562799823e-04f);
    p = fmaf(p, y, 8.603745140e-03f);
    p = fmaf(p, y, -5.415251106e-02f);
    p = fmaf(p, y, -4.582694471e-01f);
    p = fmaf(p, y, -1.151334286e+00f);
    p = fmaf(p, y, 1.387941666e-05f);
    return 0.5f * fmaf(-y, __builtin_amdgcn_exp2f(p), x + ax);
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
