// Bandwidth-bound kernels: fused CFG combine + Euler update, adaLN-modulated
// LayerNorm, and the small set-up kernels of a sampling call (timestep
// embedding, per-request key lengths, conditioning vectors, prefix tokens).
#include <algorithm>
#include <math.h>
#include "kernels.h"

namespace cfm {
namespace {

// ---------------------------------------------------------------------------
// Fused CFG combine + Euler update (VoiceHub "Diffusion and flow TTS
// optimization", section "Custom Triton and CUDA kernels", names the guidance
// combine fused with the Euler step as a kernel worth writing):
// x_out = x_in + sum_b (dt * w_b) * v_b, one float4 of x per thread, read once,
// written once. The loads of x and of every branch's velocity are issued before
// the frame's mask byte is looked at (all are in range whatever the mask), so the
// mask does not put a second dependent round trip in front of them. Masked frames
// are not written when the update is in place; with a separate output (the
// midpoint solver's half step) they are copied, so the output is defined
// everywhere. Requests whose unconditional lane is off (adaptive guidance) take
// the fully conditioned branch alone: x_out = x_in + w_full * v_{nb-1}.
__global__ void __launch_bounds__(256)
cfg_euler_kernel(const f32x4* __restrict__ v, int nb, float w0, float w1, float w2,
                 const uint8_t* __restrict__ mask, long long n4, int c4, long long branch4, int Tx,
                 const f32x4* x_in, f32x4* x_out, const int32_t* __restrict__ lane_off, float w_full) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const f32x4 xv = x_in[i];
    const f32x4 a = v[i];
    f32x4 b = f32x4{}, c = f32x4{};
    if (nb > 1) b = v[branch4 + i];
    if (nb > 2) c = v[2 * branch4 + i];
    const long long f = i / c4;                       // frame r * Tx + t
    const bool ok = mask == nullptr || mask[f] != 0;
    const bool off = lane_off != nullptr && lane_off[f / Tx] != 0;
    if (!ok) {
        if (x_out != x_in) x_out[i] = xv;
        return;
    }
    f32x4 acc;
    if (off) {
        acc = xv + w_full * (nb > 2 ? c : nb > 1 ? b : a);
    } else {
        acc = xv + w0 * a;
        if (nb > 1) acc += w1 * b;
        if (nb > 2) acc += w2 * c;
    }
    x_out[i] = acc;
}

// Adaptive guidance, once per step after its first (left-endpoint) evaluation:
// one block per request reduces, over the request's valid frames,
// sum |v_full - v_u| and sum |v_full| (fixed order: per-thread strided sums,
// then a tree in LDS), and advances the request's lane state from st_in to
// st_out (state: count [R], off [R], guided evaluations [R]). Steps before
// `warmup` never count; from then on a metric below the threshold increments
// the count and any other resets it; the lane stops once the count reaches
// `patience`. A stopped lane stays stopped.
constexpr int AG_NT = 256;
__global__ void __launch_bounds__(AG_NT)
adaptive_update_kernel(const float* __restrict__ v, int nb, long long branch_stride, const uint8_t* __restrict__ mask,
                       int Tx, int C, const int32_t* __restrict__ st_in, int32_t* __restrict__ st_out, int R,
                       int step, int warmup, int patience, float threshold, int evals_per_step) {
    __shared__ float sn[AG_NT], sd[AG_NT];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int count = st_in[r], off = st_in[R + r], guided = st_in[2 * R + r];
    if (off) {
        if (tid == 0) { st_out[r] = count; st_out[R + r] = 1; st_out[2 * R + r] = guided; }
        return;
    }
    const float* vu = v + (long long)r * Tx * C;
    const float* vf = vu + (long long)(nb - 1) * branch_stride;
    float num = 0.0f, den = 0.0f;
    const long long n = (long long)Tx * C;
    for (long long e = tid; e < n; e += AG_NT) {
        if (mask != nullptr && mask[(long long)r * Tx + e / C] == 0) continue;
        const float f = vf[e];
        num += fabsf(f - vu[e]);
        den += fabsf(f);
    }
    sn[tid] = num;
    sd[tid] = den;
    __syncthreads();
    for (int o = AG_NT / 2; o > 0; o >>= 1) {
        if (tid < o) { sn[tid] += sn[tid + o]; sd[tid] += sd[tid + o]; }
        __syncthreads();
    }
    if (tid == 0) {
        const float metric = sd[0] > 0.0f ? sn[0] / sd[0] : 0.0f;
        int c2 = count;
        if (step >= warmup) c2 = metric < threshold ? count + 1 : 0;
        st_out[r] = c2;
        st_out[R + r] = c2 >= patience ? 1 : 0;
        st_out[2 * R + r] = guided + evals_per_step;
    }
}

// ---------------------------------------------------------------------------
// Block-residual cache (one lane: the whole batch of a call). The probe is the
// hidden state after the front blocks; its score against the previous
// evaluation's probe is sum |h - prev| / sum |prev| over valid tokens, reduced in a
// fixed order (per-thread strided sums, an LDS tree per block, the blocks' partials
// summed by one block), so that every run takes the same decisions.
__device__ __forceinline__ bool cache_token_valid(const CacheTok& tk, long long m) {
    int row, t;
    if (tk.tok_row != nullptr) {
        row = tk.tok_row[m];
        if (row < 0) return false;
        t = (int)(m - tk.row_off[row]);
    } else {
        row = (int)(m / tk.T);
        t = (int)(m - (long long)row * tk.T);
    }
    return t < tk.Tp && tk.kvalid[(long long)(row % tk.R) * tk.Tp + t] != 0;
}

constexpr int CS_NT = 256;
__global__ void __launch_bounds__(CS_NT)
cache_score_kernel(const f32x4* __restrict__ h, f32x4* __restrict__ prev, int d4, CacheTok tk, float* parts) {
    __shared__ float sn[CS_NT], sd[CS_NT];
    const long long ntok = tk.n_dev ? min(tk.cap, (long long)*tk.n_dev) : tk.cap;
    const long long n = ntok * d4;
    float num = 0.0f, den = 0.0f;
    for (long long e = (long long)blockIdx.x * CS_NT + threadIdx.x; e < n; e += (long long)gridDim.x * CS_NT) {
        const f32x4 a = h[e], b = prev[e];
        if (cache_token_valid(tk, e / d4)) {
            const f32x4 df = a - b;
            num += (fabsf(df[0]) + fabsf(df[1])) + (fabsf(df[2]) + fabsf(df[3]));
            den += (fabsf(b[0]) + fabsf(b[1])) + (fabsf(b[2]) + fabsf(b[3]));
        }
        prev[e] = a;
    }
    sn[threadIdx.x] = num;
    sd[threadIdx.x] = den;
    __syncthreads();
    for (int o = CS_NT / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) { sn[threadIdx.x] += sn[threadIdx.x + o]; sd[threadIdx.x] += sd[threadIdx.x + o]; }
        __syncthreads();
    }
    if (threadIdx.x == 0) { parts[2 * blockIdx.x] = sn[0]; parts[2 * blockIdx.x + 1] = sd[0]; }
}

__global__ void __launch_bounds__(CS_NT)
cache_decide_kernel(const float* parts, int32_t* st, int forced, float threshold, float budget, int max_consecutive,
                    int max_cached, CacheTok tk) {
    __shared__ float sn[CS_NT], sd[CS_NT];
    float num = 0.0f, den = 0.0f;
    for (int i = threadIdx.x; i < kCacheParts; i += CS_NT) { num += parts[2 * i]; den += parts[2 * i + 1]; }
    sn[threadIdx.x] = num;
    sd[threadIdx.x] = den;
    __syncthreads();
    for (int o = CS_NT / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) { sn[threadIdx.x] += sn[threadIdx.x + o]; sd[threadIdx.x] += sd[threadIdx.x + o]; }
        __syncthreads();
    }
    if (threadIdx.x != 0) return;
    const int consecutive = st[1], hits = st[2], has_res = st[3], has_prev = st[6];
    const float acc = __int_as_float(st[7]);
    const float score = has_prev ? (sd[0] > 0.0f ? sn[0] / sd[0] : 0.0f) : __builtin_nanf("");
    const bool compute = forced || !has_res || (max_cached >= 0 && hits >= max_cached) ||
                         consecutive >= max_consecutive || !(score < threshold) || acc + score > budget;
    st[0] += 1;
    if (compute) {
        st[1] = 0;
        st[3] = 1;                          // the residual is saved after the middle blocks
        st[7] = __float_as_int(0.0f);
    } else {
        st[1] = consecutive + 1;
        st[2] = hits + 1;
        st[7] = __float_as_int(acc + score);
    }
    st[4] = compute ? 1 : 0;
    st[5] = compute ? (int)(tk.n_dev ? min(tk.cap, (long long)*tk.n_dev) : tk.cap) : 0;
    st[6] = 1;
}

__global__ void __launch_bounds__(256)
cache_apply_kernel(f32x4* __restrict__ h, f32x4* __restrict__ res, const f32x4* __restrict__ prev, int d4, CacheTok tk,
                   const int32_t* st) {
    const long long ntok = tk.n_dev ? min(tk.cap, (long long)*tk.n_dev) : tk.cap;
    const long long n = ntok * d4;
    const bool compute = st[4] != 0;
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
        if (compute) res[e] = h[e] - prev[e];
        else h[e] = h[e] + res[e];
    }
}

__global__ void fill_i32_kernel(int32_t* p, int n, int value) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

__global__ void copy_i32_kernel(const int32_t* src, int32_t* dst, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// adaLN LayerNorm. A wave normalises tpw (1..TPW) consecutive tokens; the row is held in
// registers (V float4 per lane), mean and biased variance come from two wave
// reductions (exact two-pass), then y = (h - mean) * rsqrt(var + 1e-6) *
// (1 + scale) + shift. The shift/scale vectors are loaded once per wave and
// reloaded only when a token belongs to another modulation group, and the next
// token's row is loaded before the current one is reduced.
constexpr int TPW = 4;

template <bool OUT_BF16, int V>
__global__ void __launch_bounds__(256)
adaln_kernel(LnParams p, int tpw) {
    const long long o0 = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * tpw;
    const int lane = threadIdx.x & 63;
    const int d4 = p.d >> 2;
    if (p.n_dev) p.n_out = min(p.n_out, (long long)*p.n_dev);
    if (o0 >= p.n_out) return;
    // output token o -> its token in the row-major output order (rows of Tout), from
    // which the input token and the modulation vectors follow
    auto rm_of = [&](long long o) {
        if (p.inter_nb == 0) return o;
        const long long fr = o / p.inter_nb;
        const int b = (int)(o - fr * p.inter_nb);
        const long long r = fr / p.Tout;
        return ((long long)b * p.inter_R + r) * p.Tout + (fr - r * p.Tout);
    };
    auto src_of = [&](long long o) {
        const long long om = rm_of(o);
        const long long row = om / p.Tout;
        const int t = (int)(om - row * p.Tout);
        return (const f32x4*)(p.h + (row * p.Tin + p.off + t) * p.d);
    };
    f32x4 cur[V], nxt[V], sh[V], sc[V];
    const float* sh_ptr = nullptr;
    {
        const f32x4* src = src_of(o0);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int c = lane + i * 64;
            cur[i] = c < d4 ? src[c] : f32x4{};
        }
    }
#pragma unroll 1
    for (int it = 0; it < tpw; ++it) {
        const long long o = o0 + it;
        if (o >= p.n_out) break;
        // modulation vectors first, the next token's row after them: the output
        // below waits only for the vectors (loads complete in issue order), so its
        // stores go out while the next row is still in flight
        const float* shp = p.shift.at(rm_of(o));
        if (shp != sh_ptr) {              // wave-uniform
            sh_ptr = shp;
            const f32x4* s4 = (const f32x4*)shp;
            const f32x4* c4 = (const f32x4*)p.scale.at(rm_of(o));
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int c = lane + i * 64;
                sh[i] = c < d4 ? s4[c] : f32x4{};
                sc[i] = c < d4 ? c4[c] + 1.0f : f32x4{};
            }
        }
        const bool more = it + 1 < tpw && o + 1 < p.n_out;
        if (more) {
            const f32x4* src = src_of(o + 1);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int c = lane + i * 64;
                nxt[i] = c < d4 ? src[c] : f32x4{};
            }
        }
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < V; ++i) sum += (cur[i][0] + cur[i][1]) + (cur[i][2] + cur[i][3]);
        const float mean = p.rms ? 0.0f : wave_sum(sum) / (float)p.d;
        float sq = 0.0f;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int c = lane + i * 64;
            if (c < d4) {
                const f32x4 z = cur[i] - mean;
                sq += (z[0] * z[0] + z[1] * z[1]) + (z[2] * z[2] + z[3] * z[3]);
            }
        }
        const float rstd = rsqrtf(wave_sum(sq) / (float)p.d + 1e-6f);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int c = lane + i * 64;
            if (c < d4) {
                const f32x4 y = (cur[i] - mean) * rstd * sc[i] + sh[i];
                if constexpr (OUT_BF16) {
                    bf16x4 b;
                    b[0] = (bf16)y[0]; b[1] = (bf16)y[1]; b[2] = (bf16)y[2]; b[3] = (bf16)y[3];
                    ((bf16x4*)((bf16*)p.y + o * p.d))[c] = b;
                } else {
                    ((f32x4*)((float*)p.y + o * p.d))[c] = y;
                }
            }
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < V; ++i) cur[i] = nxt[i];
        }
    }
}

// ---------------------------------------------------------------------------
// Time of evaluation j of a sampling call (fp64). Step k runs from t_k to t_k+1 on
// the grid of S steps: u = k / S and t_k = u (uniform), u^2 (quadratic),
// 1 - (1 - u)^2 (trailing), or n_k / N with n_k = round(k N / S), halves up, on a
// native grid of N uniform steps. With one evaluation per step (Euler) evaluation
// j is at t_j; with two (midpoint) evaluation 2k is at t_k and 2k + 1 at
// t_k + (t_k+1 - t_k) / 2. The host computes the same times for the step sizes.
__host__ __device__ inline double grid_time(int kind, int S, int N, int k) {
    if (k <= 0) return 0.0;
    if (k >= S) return 1.0;
    const double u = (double)k / (double)S;
    switch (kind) {
        case 1: return u * u;
        case 2: return 1.0 - (1.0 - u) * (1.0 - u);
        case 3: return (double)((2LL * k * N + S) / (2LL * S)) / (double)N;
        default: return u;
    }
}

__host__ __device__ inline double eval_time(int kind, int S, int N, int per_step, int j) {
    const int k = j / per_step;
    const double t0 = grid_time(kind, S, N, k);
    if (j % per_step == 0) return t0;
    return t0 + 0.5 * (grid_time(kind, S, N, k + 1) - t0);
}

// temb[j, i] = cos(1000 t_j w_i) for i < F/2, sin(1000 t_j w_(i-F/2)) otherwise,
// w_i = 10000^(-i/(F/2)), t_j the time of evaluation j; phase computed in fp64.
__global__ void timestep_embedding_kernel(float* temb, int n_eval, int F, int kind, int S, int N, int per_step) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int j = blockIdx.y;
    if (i >= F || j >= n_eval) return;
    const int half = F / 2;
    const int fi = i < half ? i : i - half;
    const double t = eval_time(kind, S, N, per_step, j);
    const double w = exp(-log(10000.0) * (double)fi / (double)half);
    const double arg = 1000.0 * t * w;
    temb[(long long)j * F + i] = (float)(i < half ? cos(arg) : sin(arg));
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

// Row offsets of the packed layout: one block, each thread sums a contiguous
// run of rows, the run totals are scanned in LDS (Hillis-Steele), and the runs
// are written out. Row i = b*R + r holds kv_len[r] tokens rounded up to a
// multiple of 8, so that every row starts 8-token aligned.
constexpr int PACK_NT = 256;
// With lane_off (adaptive guidance), the rows of every branch but the last of a
// request whose unconditional lane is off hold no token.
__device__ __forceinline__ int packed_len(const int32_t* kv_len, const int32_t* lane_off, int R, int nb, int i) {
    const int r = i % R;
    if (lane_off != nullptr && i / R < nb - 1 && lane_off[r] != 0) return 0;
    return (kv_len[r] + 7) & ~7;
}

__global__ void __launch_bounds__(PACK_NT) pack_offsets_kernel(const int32_t* kv_len, const int32_t* lane_off, int R,
                                                              int nb, int N, int32_t* row_off) {
    __shared__ int part[PACK_NT];
    const int tid = threadIdx.x;
    const int per = (N + PACK_NT - 1) / PACK_NT;
    const int lo = min(N, tid * per), hi = min(N, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += packed_len(kv_len, lane_off, R, nb, i);
    part[tid] = sum;
    __syncthreads();
    for (int o = 1; o < PACK_NT; o <<= 1) {
        const int v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - sum;   // exclusive prefix of this thread's run
    for (int i = lo; i < hi; ++i) {
        row_off[i] = run;
        run += packed_len(kv_len, lane_off, R, nb, i);
    }
    if (tid == PACK_NT - 1) row_off[N] = part[tid];
}

// tok_row[t] = the row holding packed token t (the last row whose offset is
// <= t, which skips empty rows), -1 from row_off[N] on.
__global__ void pack_rows_kernel(const int32_t* row_off, int N, int NTmax, int32_t* tok_row) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= NTmax) return;
    if (t >= row_off[N]) { tok_row[t] = -1; return; }
    int lo = 0, hi = N - 1;   // row_off[lo] <= t < row_off[hi + 1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (row_off[mid] <= t) lo = mid; else hi = mid - 1;
    }
    tok_row[t] = lo;
}

__global__ void assemble_cvec_kernel(const float* ct, const float* bs, const float* spkproj,
                                     int nc, int d, float* cvec, bf16* silu_bf16) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    const int ci = blockIdx.y, k = blockIdx.z;
    if (n >= d) return;
    float v = ct[(long long)k * d + n];
    if (bs != nullptr) v += ci == 0 ? bs[n] : spkproj[(long long)(ci - 1) * d + n];
    const long long o = ((long long)k * nc + ci) * d + n;
    if (silu_bf16) silu_bf16[o] = (bf16)silu(v);
    else cvec[o] = v;
}

__global__ void rope_table_kernel(float* tab, int T, int half, double base) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * half) return;
    const int t = i / half, k = i - t * half;
    const double a = (double)t * pow(base, -2.0 * k / (2.0 * half));
    tab[2 * i] = (float)cos(a);
    tab[2 * i + 1] = (float)sin(a);
}

// one thread per (token, pair of q|k columns)
__global__ void rope_f32_kernel(float* qkv, long long n_tok, int ld, int T, int d, int hd, const float* tab,
                                const int32_t* n_dev) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long n = n_dev ? min(n_tok, (long long)*n_dev) : n_tok;
    if (i >= n * d) return;
    const long long m = i / d;
    const int pr = (int)(i - m * d);              // pair index over the 2d q|k columns
    const int col = 2 * pr, k = (col % hd) >> 1;
    const int t = (int)(m % T);
    const float c = tab[2 * (t * (hd >> 1) + k)], sn = tab[2 * (t * (hd >> 1) + k) + 1];
    float* x = qkv + m * ld + col;
    const float a = x[0], b = x[1];
    x[0] = a * c - b * sn;
    x[1] = a * sn + b * c;
}

__global__ void swiglu_f32_kernel(const float* gu, float* act, long long M, int f, const int32_t* n_dev) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long Mv = n_dev ? min(M, (long long)*n_dev) : M;
    if (i >= Mv * f) return;
    const long long m = i / f;
    const int j = (int)(i - m * f), b = j >> 4, e = j & 15;
    const float* r = gu + m * 2 * f + 32 * b + e;
    act[i] = silu(r[0]) * r[16];
}

__global__ void silu_bf16_kernel(const float* in, bf16* out, long long n) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = (bf16)silu(in[i]);
}

__global__ void expand_context_kernel(const float* cond, float* xctx, int R, int cond0, long long per_row) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int row = blockIdx.y, b = row / R, r = row - b * R;
    if (i >= per_row) return;
    xctx[(long long)row * per_row + i] = b >= cond0 ? cond[(long long)r * per_row + i] : 0.0f;
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

void launch_cfg_euler(const CfgEulerArgs& a, hipStream_t s) {
    const long long n4 = (long long)a.R * a.Tx * a.C / 4;
    if (n4 <= 0) return;
    const int blocks = (int)((n4 + 255) / 256);
    cfg_euler_kernel<<<blocks, 256, 0, s>>>((const f32x4*)a.v, a.nb, a.w0, a.w1, a.w2, a.mask, n4, a.C / 4, n4, a.Tx,
                                             (const f32x4*)a.x_in, (f32x4*)a.x_out, a.lane_off, a.w_full);
}

void launch_adaptive_update(const float* v, int nb, const uint8_t* mask, int R, int Tx, int C, const int32_t* st_in,
                            int32_t* st_out, int step, int warmup, int patience, float threshold, int evals_per_step,
                            hipStream_t s) {
    if (R <= 0) return;
    adaptive_update_kernel<<<R, AG_NT, 0, s>>>(v, nb, (long long)R * Tx * C, mask, Tx, C, st_in, st_out, R, step,
                                               warmup, patience, threshold, evals_per_step);
}

void launch_cache_score(const float* h, float* prev, int d, const CacheTok& tk, float* parts, hipStream_t s) {
    cache_score_kernel<<<kCacheParts, CS_NT, 0, s>>>((const f32x4*)h, (f32x4*)prev, d / 4, tk, parts);
}

void launch_cache_decide(const float* parts, int32_t* state, int forced, float threshold, float budget,
                         int max_consecutive, int max_cached, const CacheTok& tk, hipStream_t s) {
    cache_decide_kernel<<<1, CS_NT, 0, s>>>(parts, state, forced, threshold, budget, max_consecutive, max_cached, tk);
}

void launch_cache_apply(float* h, float* res, const float* prev, int d, const CacheTok& tk, const int32_t* state,
                        hipStream_t s) {
    const long long n = tk.cap * (d / 4);
    const int blocks = (int)std::min<long long>(4096, (n + 255) / 256);
    if (blocks > 0) cache_apply_kernel<<<blocks, 256, 0, s>>>((f32x4*)h, (f32x4*)res, (const f32x4*)prev, d / 4, tk, state);
}

void launch_fill_i32(int32_t* p, int n, int value, hipStream_t s) {
    if (n > 0) fill_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n, value);
}

void launch_copy_i32(const int32_t* src, int32_t* dst, int n, hipStream_t s) {
    if (n > 0) copy_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(src, dst, n);
}

double host_eval_time(int kind, int S, int N, int per_step, int j) { return eval_time(kind, S, N, per_step, j); }
double host_grid_time(int kind, int S, int N, int k) { return grid_time(kind, S, N, k); }

template <int V>
void launch_adaln_v(const LnParams& p, hipStream_t s) {
    // several tokens per wave only when there are enough waves to fill the chip
    const int tpw = (int)std::max<long long>(1, std::min<long long>(TPW, p.n_out / 2048));
    const int blocks = (int)((p.n_out + 4 * tpw - 1) / (4 * tpw));
    if (p.out_bf16) adaln_kernel<true, V><<<blocks, 256, 0, s>>>(p, tpw);
    else adaln_kernel<false, V><<<blocks, 256, 0, s>>>(p, tpw);
}

void launch_adaln(const LnParams& p, hipStream_t s) {
    if (p.n_out <= 0) return;
    const int v = (p.d / 4 + 63) / 64;     // float4 per lane
    if (v <= 1) launch_adaln_v<1>(p, s);
    else if (v <= 2) launch_adaln_v<2>(p, s);
    else if (v <= 4) launch_adaln_v<4>(p, s);
    else if (v <= 8) launch_adaln_v<8>(p, s);
    else launch_adaln_v<16>(p, s);
}

void launch_timestep_embedding(float* temb, int n_eval, int F, int kind, int S, int N, int per_step, hipStream_t s) {
    if (n_eval <= 0) return;
    timestep_embedding_kernel<<<dim3((F + 127) / 128, n_eval), 128, 0, s>>>(temb, n_eval, F, kind, S, N, per_step);
}

void launch_key_prep(const uint8_t* mask, int mask_stride, const int32_t* kv_len_in, int R, int P,
                     int T, int Tp, int32_t* kv_len_out, uint8_t* kvalid, uint8_t* tile_full,
                     hipStream_t s) {
    if (R <= 0) return;
    key_prep_kernel<<<R, 256, 0, s>>>(mask, mask_stride, kv_len_in, P, T, Tp, kv_len_out, kvalid, tile_full);
}

void launch_pack_rows(const int32_t* kv_len, const int32_t* lane_off, int R, int nb, int NTmax, int32_t* row_off,
                      int32_t* tok_row, hipStream_t s) {
    const int N = nb * R;
    if (N <= 0) return;
    pack_offsets_kernel<<<1, PACK_NT, 0, s>>>(kv_len, lane_off, R, nb, N, row_off);
    if (NTmax > 0) pack_rows_kernel<<<(NTmax + 255) / 256, 256, 0, s>>>(row_off, N, NTmax, tok_row);
}

void launch_assemble_cvec(const float* ct, const float* bs, const float* spkproj, int S, int nc,
                          int d, float* cvec, hipStream_t s, bf16* silu_bf16) {
    if (S <= 0) return;
    assemble_cvec_kernel<<<dim3((d + 255) / 256, nc, S), 256, 0, s>>>(ct, bs, spkproj, nc, d, cvec, silu_bf16);
}

void launch_rope_table(float* tab, int T, int hd, double base, hipStream_t s) {
    const int n = T * (hd / 2);
    if (n <= 0) return;
    rope_table_kernel<<<(n + 255) / 256, 256, 0, s>>>(tab, T, hd / 2, base);
}

void launch_rope_f32(float* qkv, long long n_tok, int ld, int T, int d, int hd, const float* tab,
                     const int32_t* n_dev, hipStream_t s) {
    const long long n = n_tok * d;
    if (n <= 0) return;
    rope_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(qkv, n_tok, ld, T, d, hd, tab, n_dev);
}

void launch_swiglu_f32(const float* gu, float* act, long long M, int f, const int32_t* n_dev, hipStream_t s) {
    const long long n = M * f;
    if (n <= 0) return;
    swiglu_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(gu, act, M, f, n_dev);
}

void launch_silu_bf16(const float* in, bf16* out, long long n, hipStream_t s) {
    if (n <= 0) return;
    silu_bf16_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(in, out, n);
}

void launch_expand_context(const float* cond, float* xctx, int R, int nb, int cond0, long long per_row,
                           hipStream_t s) {
    if (R <= 0 || per_row <= 0) return;
    expand_context_kernel<<<dim3((unsigned)((per_row + 255) / 256), nb * R), 256, 0, s>>>(cond, xctx, R, cond0,
                                                                                        per_row);
}

void launch_prefix_init(const float* cproj, const float* bias, int R, int nb, int cond_branch0,
                        int P, int T, int d, float* h, hipStream_t s) {
    if (R <= 0 || P <= 0) return;
    prefix_init_kernel<<<dim3((d + 255) / 256, R * P, nb), 256, 0, s>>>(cproj, bias, R, cond_branch0,
                                                                       P, T, d, h);
}

}  // namespace cfm
