// Key-padding-masked multi-head attention over latent frames (non-causal).
//
// bf16 path (head_dim 64): flash-style, one block = 8 waves = 256 queries of
// one (row, head), 32 per wave, all sharing each K and V^T tile staged in LDS;
// keys stream through double-buffered LDS tiles
// of 64 with the online softmax recurrence (running max m, running sum l,
// rescale of the partial output by exp(m_old - m_new)), so the T x T score
// matrix never exists. V arrives already transposed per head (the QKV GEMM
// epilogue writes it that way), so every LDS tile is filled with plain
// 16-byte loads and stores.
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
// Occupancy is what hides latency here: the kernel is limited to 128 VGPRs so
// that two 8-wave blocks share a CU (4 waves per SIMD), and tiles alternate
// between two LDS buffers so one barrier per tile suffices.
// Masked keys are zero-filled in K and V and get a -inf score bias, so a
// non-finite value behind a padded frame can never reach a valid output; tiles
// whose 64 keys are all valid skip the bias. The 1/sqrt(hd) scale is folded into
// the exp2 argument, and the running max moves lazily (see RESCALE_SLACK).
//
// fp32 path: one thread per query, exact fp32 online softmax, for the fp32
// sampler (small head dims).
#include <math.h>
#include "kernels.h"

namespace cfm {
namespace {

constexpr int HD = 64;
constexpr int KT = 64;         // keys per LDS tile
constexpr int KP = HD + 8;     // K tile row pitch (bf16): 144 B
constexpr int VP = KT + 8;     // V^T tile row pitch (bf16): 144 B
// The running max is only moved when a tile's max exceeds it by more than
// 2^8 in probability (8 in base-2 exponent): until then p = 2^(s - m) <= 256,
// far from overflow in fp32 and in bf16, and softmax does not depend on the
// constant subtracted, so skipping the rescale changes nothing but rounding.
constexpr float RESCALE_SLACK = 8.0f;

__device__ __forceinline__ bool key_valid(const AttnParams& p, const uint8_t* km, int key, int kvl) {
    if (key >= kvl) return false;
    if (km == nullptr || key < p.P) return true;
    return km[key - p.P] != 0;
}

// One KV tile in registers on its way to LDS: KV_CH chunks of K (one key, 8
// head dims each) and of V^T (one head dim, 8 keys each) per thread, with the
// validity bytes of their keys. Masked keys are written as zeros.
template <int NT>
struct KvStage {
    static constexpr int KV_CH = KT * HD / 8 / NT;
    static_assert(KV_CH >= 1 && KT * HD / 8 % NT == 0, "tile split");
    bf16x8 k[KV_CH], v[KV_CH];
    uint8_t kok[KV_CH];
    uint64_t vok[KV_CH];
    __device__ __forceinline__ void load(const bf16* kbase, long long ldk, int kmax, const bf16* vtbase,
                                         int Tp, const uint8_t* kv, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < KV_CH; ++i) {
            const int c = tid + i * NT;
            const int key = k0 + (c >> 3), ch = (c & 7) * 8;
            kok[i] = kv[key];
            k[i] = *(const bf16x8*)(kbase + (long long)min(key, kmax) * ldk + ch);
            const int hd = c >> 3, kc = k0 + (c & 7) * 8;
            vok[i] = *(const uint64_t*)(kv + kc);
            v[i] = *(const bf16x8*)(vtbase + (long long)hd * Tp + kc);
        }
    }
    __device__ __forceinline__ void store(bf16* Ks, bf16* Vt, float* kbias, int tid) const {
#pragma unroll
        for (int i = 0; i < KV_CH; ++i) {
            const int c = tid + i * NT;
            const int kr = c >> 3, ch = (c & 7) * 8;
            *(bf16x8*)(Ks + kr * KP + ch) = kok[i] ? k[i] : bf16x8{};
            if (ch == 0) kbias[kr] = kok[i] ? 0.0f : -INFINITY;
            const int hd = c >> 3, kc = (c & 7) * 8;
            bf16x8 vv = v[i];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (((vok[i] >> (8 * e)) & 0xff) == 0) vv[e] = (bf16)0.0f;
            *(bf16x8*)(Vt + hd * VP + kc) = vv;
        }
    }
};

// NW waves per block, 32 queries each, all sharing every K / V^T tile: 8 for
// long sequences; 1 for short ones (a block per 32 queries, no idle waves).
template <int NW>
__global__ void __launch_bounds__(64 * NW, 4)   // 4 waves per SIMD
attn_bf16_kernel(AttnParams p) {
    constexpr int QT = 32 * NW;    // queries per block
    constexpr int NT = 64 * NW;
    __shared__ __attribute__((aligned(16))) bf16 Ks[2][KT * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vt[2][HD * VP];
    __shared__ float kbias[2][KT];

    const int row = blockIdx.z, head = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, h = lane >> 5;
    // first token of the row and its length: padded rows hold T tokens each,
    // packed rows row_off[row + 1] - row_off[row]
    long long rbase;
    int T;
    if (p.row_off) {
        rbase = p.row_off[row];
        T = p.row_off[row + 1] - (int)rbase;
        if (blockIdx.x * QT >= T) return;     // block-uniform: no query of this block exists
    } else {
        rbase = (long long)row * p.T;
        T = p.T;
    }
    const int d = p.H * HD;
    const long long ldk = 2LL * d;
    const bf16* qbase = (const bf16*)p.qkv + rbase * ldk + head * HD;
    const bf16* kbase = qbase + d;
    const bf16* vtbase = (const bf16*)p.vt + (long long)(row * p.H + head) * HD * p.Tp;
    const int q = blockIdx.x * QT + wave * 32 + j;

    bf16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        qf[kk] = q < T ? *(const bf16x8*)(qbase + (long long)q * ldk + kk * 16 + h * 8) : bf16x8{};

    const int rr = row % p.kv_mod;
    const int kvl = min(p.kv_len[rr], T);
    const uint8_t* kv = p.kvalid + (long long)rr * p.Tp;
    const uint8_t* tfull = p.tile_full + (long long)rr * (p.Tp / KT);
    const float sl2 = 1.4426950408889634f / sqrtf((float)HD);   // 1/sqrt(hd) in base-2 units

    f32x16 oacc[2] = {f32x16{}, f32x16{}};
    // running max of the scaled scores (base 2); finite start so that a tile with
    // no valid key (all scores -inf) gives exp2(-inf) = 0, never inf - inf
    float m_run = -1e30f;
    float l_part = 0.0f;

    const int ntiles = (kvl + KT - 1) / KT;
    for (int it = 0; it < ntiles; ++it) {
        const int cur = it & 1;
        const bool full = tfull[it] != 0;
        {
            KvStage<NT> st;
            st.load(kbase, ldk, T - 1, vtbase, p.Tp, kv, it * KT, tid);
            st.store(Ks[cur], Vt[cur], kbias[cur], tid);
        }
        __syncthreads();
        const bf16* ks = Ks[cur];
        const bf16* vt = Vt[cur];

        // S^T = K Q^T: s[kh][g*4 + r] = score(key kh*32 + 8g + 4h + r, query q)
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 a = *(const bf16x8*)(ks + (kh * 32 + j) * KP + kk * 16 + h * 8);
                s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kh], 0, 0, 0);
            }
        if (!full) {   // partial tile: masked keys get -inf
            const float* kb = kbias[cur];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int r = 0; r < 4; ++r) s[kh][g * 4 + r] += kb[kh * 32 + 8 * g + 4 * h + r];
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kh][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
        // move the running max only when the tile max clears it by the slack
        const bool move = mx > m_run + RESCALE_SLACK;
        if (__any(move)) {   // some lane of the wave moves its max
            const float m_new = move ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 1 for lanes that keep their max
            l_part *= alpha;
            oacc[0] *= alpha;
            oacc[1] *= alpha;
            m_run = m_new;
        }
        float ls = 0.0f;
        bf16x8 pb[2][2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pv = __builtin_amdgcn_exp2f(fmaf(s[kh][g * 4 + r], sl2, -m_run));
                    ls += pv;
                    pb[kh][g >> 1][(g & 1) * 4 + r] = (bf16)pv;
                }
        l_part += ls;

        // O^T += V^T P^T. B-operand slot e of lane half h (k-step ss of key half kh)
        // is key kh*32 + 16 ss + 4h + e (e < 4) or kh*32 + 16 ss + 8 + 4h + (e - 4).
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int ss = 0; ss < 2; ++ss) {
                    const bf16* vr = vt + (dt * 32 + j) * VP + kh * 32 + 16 * ss + 4 * h;
                    const bf16x4 lo = *(const bf16x4*)(vr);
                    const bf16x4 hi = *(const bf16x4*)(vr + 8);
                    bf16x8 a;
                    a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
                    a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kh][ss], oacc[dt], 0, 0, 0);
                }

        // no barrier here: the next tile goes to the other buffer, and the barrier
        // after that store orders it after every wave's reads of this one
    }

    const float l = l_part + __shfl_xor(l_part, 32, 64);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (q < T) {
        bf16* dst = (bf16*)p.o + (rbase + q) * d + head * HD;
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
constexpr int FKT = 64;         // keys per LDS tile on the fp32 path

// fp32 path: one thread per query, exact fp32 online softmax; the block's keys
// and values pass through LDS in tiles of 64 (HD = head dim, a multiple of 4).
template <int HD_>
__global__ void __launch_bounds__(FQ)
attn_f32_kernel(AttnParams p) {
    __shared__ float Kt[FKT][HD_ + 1];
    __shared__ float Vs[FKT][HD_ + 1];
    __shared__ float kb[FKT];
    const int row = blockIdx.z, head = blockIdx.y;
    const int q = blockIdx.x * FQ + threadIdx.x;
    const int T = p.T, d = p.H * HD_;
    const long long ld = 3LL * d;
    const float* base = (const float*)p.qkv + (long long)row * T * ld;
    const int rr = row % p.kv_mod;
    const int kvl = min(p.kv_len[rr], T);
    const uint8_t* km = p.key_mask ? p.key_mask + (long long)rr * p.mask_stride : nullptr;
    const float scale = 1.0f / sqrtf((float)HD_);
    const int qc = q < T ? q : T - 1;

    float qv[HD_], acc[HD_];
#pragma unroll
    for (int e = 0; e < HD_; ++e) {
        qv[e] = base[(long long)qc * ld + head * HD_ + e] * scale;
        acc[e] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    for (int k0 = 0; k0 < kvl; k0 += FKT) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < FKT * HD_; idx += FQ) {
            const int kr = idx / HD_, e = idx % HD_;
            const int key = k0 + kr;
            const bool ok = key < kvl;
            Kt[kr][e] = ok ? base[(long long)key * ld + d + head * HD_ + e] : 0.0f;
            Vs[kr][e] = ok ? base[(long long)key * ld + 2 * d + head * HD_ + e] : 0.0f;
        }
        for (int kr = threadIdx.x; kr < FKT; kr += FQ) {
            const int key = k0 + kr;
            kb[kr] = key_valid(p, km, key, kvl) ? 1.0f : 0.0f;
        }
        __syncthreads();
        const int nk = min(FKT, kvl - k0);
        for (int kr = 0; kr < nk; ++kr) {
            if (kb[kr] == 0.0f) continue;
            float sdot = 0.0f;
#pragma unroll
            for (int e = 0; e < HD_; ++e) sdot = fmaf(qv[e], Kt[kr][e], sdot);
            const float m_new = fmaxf(m, sdot);
            const float corr = expf(m - m_new);
            const float pv = expf(sdot - m_new);
            l = l * corr + pv;
#pragma unroll
            for (int e = 0; e < HD_; ++e) acc[e] = fmaf(pv, Vs[kr][e], acc[e] * corr);
            m = m_new;
        }
    }
    if (q < T) {
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        float* dst = (float*)p.o + ((long long)row * T + q) * d + head * HD_;
#pragma unroll
        for (int e = 0; e < HD_; ++e) dst[e] = acc[e] * inv;
    }
}

}  // namespace

void launch_attention_bf16(const AttnParams& p, hipStream_t s) {
    if (p.rows <= 0 || p.T <= 0) return;
    if (p.T <= 64) {
        dim3 grid((p.T + 31) / 32, p.H, p.rows);
        attn_bf16_kernel<1><<<grid, 64, 0, s>>>(p);
    } else {
        dim3 grid((p.T + 255) / 256, p.H, p.rows);
        attn_bf16_kernel<8><<<grid, 512, 0, s>>>(p);
    }
}

template <int HD_>
void launch_f32_hd(const AttnParams& p, hipStream_t s) {
    dim3 grid((p.T + FQ - 1) / FQ, p.H, p.rows);
    attn_f32_kernel<HD_><<<grid, FQ, 0, s>>>(p);
}

void launch_attention_f32(const AttnParams& p, hipStream_t s) {
    if (p.rows <= 0 || p.T <= 0) return;
    switch (p.hd) {   // head dims the fp32 path supports: multiples of 4 up to 64
        case 4: launch_f32_hd<4>(p, s); break;      case 8: launch_f32_hd<8>(p, s); break;
        case 12: launch_f32_hd<12>(p, s); break;    case 16: launch_f32_hd<16>(p, s); break;
        case 20: launch_f32_hd<20>(p, s); break;    case 24: launch_f32_hd<24>(p, s); break;
        case 28: launch_f32_hd<28>(p, s); break;    case 32: launch_f32_hd<32>(p, s); break;
        case 36: launch_f32_hd<36>(p, s); break;    case 40: launch_f32_hd<40>(p, s); break;
        case 44: launch_f32_hd<44>(p, s); break;    case 48: launch_f32_hd<48>(p, s); break;
        case 52: launch_f32_hd<52>(p, s); break;    case 56: launch_f32_hd<56>(p, s); break;
        case 60: launch_f32_hd<60>(p, s); break;    default: launch_f32_hd<64>(p, s); break;
    }
}

}  // namespace cfm
