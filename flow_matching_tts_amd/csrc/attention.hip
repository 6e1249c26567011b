// Key-padding-masked multi-head attention over latent frames (non-causal).
//
// bf16 path (head_dim 64): flash-style, one block = 4 waves = 128 queries of
// one (row, head); keys stream through LDS in tiles of 64 with the online
// softmax recurrence (running max m, running sum l, rescale of the partial
// output by exp(m_old - m_new)), so the T x T score matrix never exists.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, C[i][j] = sum_k A[i][k] B[k][j]):
//   S^T = K Q^T : A = the K tile (rows = keys), B = Q^T held in registers for
//                 the whole loop. The accumulator keeps one query per lane
//                 (column = lane % 32) and 32 keys in its 16 registers x 2
//                 lane halves, so a query's row max / row sum needs only a
//                 swap with lane ^ 32, and the rescale factor is per lane.
//   O^T += V^T P^T : B = P^T comes straight from the softmax registers (same
//                 query per lane); the k slots of that operand are a fixed
//                 permutation of the tile's keys, and the V^T operand is read
//                 from LDS in that same key order.
// Masked keys are zero-filled in K and V and get a -inf score bias, so a
// non-finite value behind a padded frame can never reach a valid output.
//
// fp32 path: one thread per query, exact fp32 online softmax, for the fp32
// sampler (small head dims).
#include <math.h>
#include "kernels.h"

namespace cfm {
namespace {

constexpr int HD = 64;
constexpr int QT = 128;        // queries per block
constexpr int KT = 64;         // keys per LDS tile
constexpr int KP = HD + 8;     // K tile row pitch (bf16): 144 B
constexpr int VP = KT + 8;     // V^T tile row pitch (bf16): 144 B

__device__ __forceinline__ bool key_valid(const AttnParams& p, const uint8_t* km, int key, int kvl) {
    if (key >= kvl) return false;
    if (km == nullptr || key < p.P) return true;
    return km[key - p.P] != 0;
}

__global__ void __launch_bounds__(256)
attn_bf16_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) bf16 Ks[KT * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vt[HD * VP];
    __shared__ float kbias[KT];

    const int row = blockIdx.z, head = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, h = lane >> 5;
    const int T = p.T, d = p.H * HD;
    const long long ld = 3LL * d;
    const bf16* base = (const bf16*)p.qkv + (long long)row * T * ld;
    const int q = blockIdx.x * QT + wave * 32 + j;

    bf16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        qf[kk] = q < T ? *(const bf16x8*)(base + (long long)q * ld + head * HD + kk * 16 + h * 8) : bf16x8{};

    const int rr = row % p.kv_mod;
    const int kvl = min(p.kv_len[rr], T);
    const uint8_t* km = p.key_mask ? p.key_mask + (long long)rr * p.mask_stride : nullptr;
    const float sl2 = 1.4426950408889634f / sqrtf((float)HD);   // 1/sqrt(hd) in base-2 units

    f32x16 oacc[2] = {f32x16{}, f32x16{}};
    float m_run = -1e30f, l_part = 0.0f;

    for (int k0 = 0; k0 < kvl; k0 += KT) {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int c = tid + pass * 256, key = c >> 3, ch = (c & 7) * 8;
            const int kg = k0 + key;
            const bool ok = key_valid(p, km, kg, kvl);
            bf16x8 kv = bf16x8{}, vv = bf16x8{};
            if (ok) {
                const bf16* src = base + (long long)kg * ld + head * HD + ch;
                kv = *(const bf16x8*)(src + d);
                vv = *(const bf16x8*)(src + 2 * d);
            }
            *(bf16x8*)(Ks + key * KP + ch) = kv;
#pragma unroll
            for (int e = 0; e < 8; ++e) Vt[(ch + e) * VP + key] = vv[e];
            if (ch == 0) kbias[key] = ok ? 0.0f : -INFINITY;
        }
        __syncthreads();

        f32x16 s[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            s[kh] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 a = *(const bf16x8*)(Ks + (kh * 32 + j) * KP + kk * 16 + h * 8);
                s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kh], 0, 0, 0);
            }
        }
        // s[kh][g*4 + r] = score(key = kh*32 + 8g + 4h + r, query q)
        float mx = -INFINITY;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = s[kh][g * 4 + r] * sl2 + kbias[kh * 32 + 8 * g + 4 * h + r];
                    s[kh][g * 4 + r] = v;
                    mx = fmaxf(mx, v);
                }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        float ls = 0.0f;
        bf16x8 pb[2][2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pv = exp2f(s[kh][g * 4 + r] - m_new);
                    ls += pv;
                    pb[kh][g >> 1][(g & 1) * 4 + r] = (bf16)pv;
                }
        l_part = l_part * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) oacc[dt] *= alpha;

        // B operand slot e of lane half h (k-step st of key half kh) is key
        // kh*32 + 16 st + 4h + e for e < 4 and kh*32 + 16 st + 8 + 4h + (e - 4) for e >= 4.
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const bf16* vr = Vt + (dt * 32 + j) * VP + kh * 32 + 16 * st + 4 * h;
                    const bf16x4 lo = *(const bf16x4*)(vr);
                    const bf16x4 hi = *(const bf16x4*)(vr + 8);
                    bf16x8 a;
                    a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
                    a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kh][st], oacc[dt], 0, 0, 0);
                }
        __syncthreads();
    }

    const float l = l_part + __shfl_xor(l_part, 32, 64);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (q < T) {
        bf16* dst = (bf16*)p.o + ((long long)row * T + q) * d + head * HD;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 o4;
#pragma unroll
                for (int r = 0; r < 4; ++r) o4[r] = (bf16)(oacc[dt][g * 4 + r] * inv);
                *(bf16x4*)(dst + dt * 32 + 8 * g + 4 * h) = o4;
            }
    }
}

constexpr int FQ = 64;          // queries per block on the fp32 path
constexpr int FHD = 64;         // max head dim on the fp32 path

__global__ void __launch_bounds__(FQ)
attn_f32_kernel(AttnParams p) {
    const int row = blockIdx.z, head = blockIdx.y;
    const int q = blockIdx.x * FQ + threadIdx.x;
    const int T = p.T, hd = p.hd, d = p.H * hd;
    const long long ld = 3LL * d;
    const float* base = (const float*)p.qkv + (long long)row * T * ld;
    const int rr = row % p.kv_mod;
    const int kvl = min(p.kv_len[rr], T);
    const uint8_t* km = p.key_mask ? p.key_mask + (long long)rr * p.mask_stride : nullptr;
    const float scale = 1.0f / sqrtf((float)hd);
    const int qc = q < T ? q : T - 1;

    float qv[FHD], acc[FHD];
#pragma unroll
    for (int e = 0; e < FHD; ++e) {
        qv[e] = e < hd ? base[(long long)qc * ld + head * hd + e] : 0.0f;
        acc[e] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    for (int key = 0; key < kvl; ++key) {
        if (!key_valid(p, km, key, kvl)) continue;
        const float* kr = base + (long long)key * ld + d + head * hd;
        float sdot = 0.0f;
#pragma unroll
        for (int e = 0; e < FHD; ++e)
            if (e < hd) sdot = fmaf(qv[e], kr[e], sdot);
        sdot *= scale;
        const float m_new = fmaxf(m, sdot);
        const float corr = expf(m - m_new);
        const float pv = expf(sdot - m_new);
        l = l * corr + pv;
        const float* vr = kr + d;
#pragma unroll
        for (int e = 0; e < FHD; ++e)
            if (e < hd) acc[e] = fmaf(pv, vr[e], acc[e] * corr);
        m = m_new;
    }
    if (q < T) {
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        float* dst = (float*)p.o + ((long long)row * T + q) * d + head * hd;
#pragma unroll
        for (int e = 0; e < FHD; ++e)
            if (e < hd) dst[e] = acc[e] * inv;
    }
}

}  // namespace

void launch_attention_bf16(const AttnParams& p, hipStream_t s) {
    if (p.rows <= 0 || p.T <= 0) return;
    dim3 grid((p.T + QT - 1) / QT, p.H, p.rows);
    attn_bf16_kernel<<<grid, 256, 0, s>>>(p);
}

void launch_attention_f32(const AttnParams& p, hipStream_t s) {
    if (p.rows <= 0 || p.T <= 0) return;
    dim3 grid((p.T + FQ - 1) / FQ, p.H, p.rows);
    attn_f32_kernel<<<grid, FQ, 0, s>>>(p);
}

}  // namespace cfm
