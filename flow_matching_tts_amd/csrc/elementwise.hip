// Bandwidth-bound kernels: fused CFG combine + Euler update, adaLN-modulated
// LayerNorm, and the small set-up kernels of a sampling call (timestep
// embedding, per-request key lengths, conditioning vectors, prefix tokens).
#include <math.h>
#include "kernels.h"

namespace cfm {
namespace {

// ---------------------------------------------------------------------------
// Fused CFG combine + Euler update (VoiceHub "Custom Triton and CUDA kernels":
// packed CFG combination plus an Euler update in one pass). One float4 of x per
// thread: x += sum_b (dt * w_b) * v_b, read once, written once; masked frames
// are neither read nor written.
__global__ void __launch_bounds__(256)
cfg_euler_kernel(const f32x4* __restrict__ v, int nb, float w0, float w1, float w2,
                 const uint8_t* __restrict__ mask, long long n4, int c4, long long branch4,
                 f32x4* __restrict__ x) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    if (mask != nullptr && mask[i / c4] == 0) return;
    f32x4 acc = x[i];
    acc += w0 * v[i];
    if (nb > 1) acc += w1 * v[branch4 + i];
    if (nb > 2) acc += w2 * v[2 * branch4 + i];
    x[i] = acc;
}

// ---------------------------------------------------------------------------
// adaLN LayerNorm, one wave per token: the row is held in registers, mean and
// biased variance by two wave reductions (exact two-pass), then
// y = (h - mean) * rsqrt(var + 1e-6) * (1 + scale) + shift.
constexpr int LN_MAX4 = 16;   // d <= 4096

template <bool OUT_BF16>
__global__ void __launch_bounds__(256)
adaln_kernel(LnParams p) {
    const long long o = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (o >= p.n_out) return;
    const long long row = o / p.Tout;
    const int t = (int)(o - row * p.Tout);
    const long long in_tok = row * p.Tin + p.off + t;
    const int d4 = p.d >> 2;
    const f32x4* src = (const f32x4*)(p.h + in_tok * p.d);

    f32x4 v[LN_MAX4];
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < LN_MAX4; ++i) {
        const int c = lane + i * 64;
        if (c < d4) {
            v[i] = src[c];
            sum += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
        }
    }
    const float mean = wave_sum(sum) / (float)p.d;
    float sq = 0.0f;
#pragma unroll
    for (int i = 0; i < LN_MAX4; ++i) {
        const int c = lane + i * 64;
        if (c < d4) {
            const f32x4 z = v[i] - mean;
            sq += (z[0] * z[0] + z[1] * z[1]) + (z[2] * z[2] + z[3] * z[3]);
        }
    }
    const float rstd = rsqrtf(wave_sum(sq) / (float)p.d + 1e-6f);
    const f32x4* sh = (const f32x4*)p.shift.at(o);
    const f32x4* sc = (const f32x4*)p.scale.at(o);
#pragma unroll
    for (int i = 0; i < LN_MAX4; ++i) {
        const int c = lane + i * 64;
        if (c < d4) {
            const f32x4 y = (v[i] - mean) * rstd * (1.0f + sc[c]) + sh[c];
            if constexpr (OUT_BF16) {
                bf16x4 b;
                b[0] = (bf16)y[0]; b[1] = (bf16)y[1]; b[2] = (bf16)y[2]; b[3] = (bf16)y[3];
                ((bf16x4*)((bf16*)p.y + o * p.d))[c] = b;
            } else {
                ((f32x4*)((float*)p.y + o * p.d))[c] = y;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// temb[k, i] = cos(1000 t_k w_i) for i < F/2, sin(1000 t_k w_(i-F/2)) otherwise,
// w_i = 10000^(-i/(F/2)), t_k = k/S; phase computed in fp64.
__global__ void timestep_embedding_kernel(float* temb, int S, int F) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int k = blockIdx.y;
    if (i >= F || k >= S) return;
    const int half = F / 2;
    const int fi = i < half ? i : i - half;
    const double t = (double)k / (double)S;
    const double w = exp(-log(10000.0) * (double)fi / (double)half);
    const double arg = 1000.0 * t * w;
    temb[(long long)k * F + i] = (float)(i < half ? cos(arg) : sin(arg));
}

// Per-request key validity (see launch_key_prep). One block per request.
__global__ void key_prep_kernel(const uint8_t* mask, int mask_stride, const int32_t* kv_len_in, int P,
                                int T, int Tp, int32_t* kv_len_out, uint8_t* kvalid, uint8_t* tile_full) {
    __shared__ int last;
    const int r = blockIdx.x;
    const int Tx = T - P;
    if (threadIdx.x == 0) last = 0;
    __syncthreads();
    int kvl;
    if (kv_len_in != nullptr) {
        kvl = min(max(kv_len_in[r], 0), T);
    } else {
        int mine = 0;
        for (int t = threadIdx.x; t < Tx; t += blockDim.x)
            if (mask == nullptr || mask[(long long)r * mask_stride + t]) mine = t + 1;
        atomicMax(&last, mine);
        __syncthreads();
        kvl = P + last;
    }
    uint8_t* kv = kvalid + (long long)r * Tp;
    for (int t = threadIdx.x; t < Tp; t += blockDim.x) {
        bool ok = t < kvl;
        if (ok && mask != nullptr && t >= P) ok = mask[(long long)r * mask_stride + (t - P)] != 0;
        kv[t] = ok ? 1 : 0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < Tp / 64; i += blockDim.x) {
        int all = 1;
        for (int e = 0; e < 64; ++e) all &= kv[i * 64 + e];
        tile_full[(long long)r * (Tp / 64) + i] = (uint8_t)all;
    }
    if (threadIdx.x == 0) kv_len_out[r] = kvl;
}

__global__ void assemble_cvec_kernel(const float* ct, const float* bs, const float* spkproj,
                                     int nc, int d, float* cvec) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    const int ci = blockIdx.y, k = blockIdx.z;
    if (n >= d) return;
    float v = ct[(long long)k * d + n];
    if (bs != nullptr) v += ci == 0 ? bs[n] : spkproj[(long long)(ci - 1) * d + n];
    cvec[((long long)k * nc + ci) * d + n] = v;
}

__global__ void prefix_init_kernel(const float* cproj, const float* bias, int R, int cond_branch0,
                                   int P, int T, int d, float* h) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    const int pr = blockIdx.y;            // r * P + p
    const int b = blockIdx.z;
    if (n >= d) return;
    const int r = pr / P, pp = pr - r * P;
    const float v = b >= cond_branch0 ? cproj[(long long)pr * d + n] : bias[n];
    h[((long long)(b * R + r) * T + pp) * d + n] = v;
}

}  // namespace

void launch_cfg_euler(const float* v, int nb, float w0, float w1, float w2, const uint8_t* mask,
                      int R, int Tx, int C, float* x, hipStream_t s) {
    const long long n4 = (long long)R * Tx * C / 4;
    if (n4 <= 0) return;
    const int blocks = (int)((n4 + 255) / 256);
    cfg_euler_kernel<<<blocks, 256, 0, s>>>((const f32x4*)v, nb, w0, w1, w2, mask, n4, C / 4, n4,
                                             (f32x4*)x);
}

void launch_adaln(const LnParams& p, hipStream_t s) {
    if (p.n_out <= 0) return;
    const int blocks = (int)((p.n_out + 3) / 4);
    if (p.out_bf16) adaln_kernel<true><<<blocks, 256, 0, s>>>(p);
    else adaln_kernel<false><<<blocks, 256, 0, s>>>(p);
}

void launch_timestep_embedding(float* temb, int S, int F, hipStream_t s) {
    if (S <= 0) return;
    timestep_embedding_kernel<<<dim3((F + 127) / 128, S), 128, 0, s>>>(temb, S, F);
}

void launch_key_prep(const uint8_t* mask, int mask_stride, const int32_t* kv_len_in, int R, int P,
                     int T, int Tp, int32_t* kv_len_out, uint8_t* kvalid, uint8_t* tile_full,
                     hipStream_t s) {
    if (R <= 0) return;
    key_prep_kernel<<<R, 256, 0, s>>>(mask, mask_stride, kv_len_in, P, T, Tp, kv_len_out, kvalid, tile_full);
}

void launch_assemble_cvec(const float* ct, const float* bs, const float* spkproj, int S, int nc,
                          int d, float* cvec, hipStream_t s) {
    if (S <= 0) return;
    assemble_cvec_kernel<<<dim3((d + 255) / 256, nc, S), 256, 0, s>>>(ct, bs, spkproj, nc, d, cvec);
}

void launch_prefix_init(const float* cproj, const float* bias, int R, int nb, int cond_branch0,
                        int P, int T, int d, float* h, hipStream_t s) {
    if (R <= 0 || P <= 0) return;
    prefix_init_kernel<<<dim3((d + 255) / 256, R * P, nb), 256, 0, s>>>(cproj, bias, R, cond_branch0,
                                                                       P, T, d, h);
}

}  // namespace cfm
