// Key-padding-masked multi-head attention over latent frames (non-causal).
//
// bf16 path (head_dim 64): flash-style, one block = 8 waves = 256 queries of
// one (row, head), 32 per wave, all sharing each K and V^T tile staged in LDS;
// keys stream through a ring of LDS tiles
// of 64 with the online softmax recurrence (running max m, running sum l,
// rescale of the partial output by exp(m_old - m_new)), so the T x T score
// matrix never exists. V arrives already transposed per head (the QKV GEMM
// epilogue writes it that way), so every LDS tile is 64 rows of 128 contiguous
// bytes in HBM, loaded straight into LDS.
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
// The kernel is limited to 128 VGPRs so that two 8-wave blocks share a CU (4
// waves per SIMD); one barrier per tile suffices because the ring has a slot
// more than the tiles in flight.
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
// The running max is only moved when a tile's max exceeds it by more than
// 2^8 in probability (8 in base-2 exponent): until then p = 2^(s - m) <= 256,
// far from overflow in fp32 and in bf16, and softmax does not depend on the
// constant subtracted, so skipping the rescale changes nothing but rounding.
constexpr float RESCALE_SLACK = 8.0f;
constexpr int OOB = 0x7ffffff0;   // buffer offset past every range: the load returns zeros

// LDS tile = 64 rows (keys of K, head dims of V^T) of 128 data bytes at a
// 144-byte stride: the 16 rows that 16 lanes read at one chunk (one 128-bit
// LDS read cycle) fall on 16 distinct bank groups, and every fragment read
// is a per-lane base plus an immediate offset. Tiles arrive by direct
// buffer-to-LDS loads: one load instruction fills 1 KiB at M0 + 16 * lane, so
// instruction g covers rows 7g .. 7g + 6 (9 lanes per row: 8 data chunks and the
// pad chunk) at M0 = 7g * 144, and its last lane rewrites the first chunk of
// row 7g + 7 with the same data the next instruction brings. Ten instructions
// cover a tile; the last spills past row 63 into a slack area nobody reads.
constexpr int RS = 144;                    // row stride, bytes
constexpr int GRP = 7;                     // rows per load instruction
constexpr int NLD = (KT + GRP - 1) / GRP;  // load instructions per tile (10)
constexpr int TILE_B = NLD * GRP * RS + 1024 - GRP * RS;   // bytes per tile incl. slack (10096)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t arsrc(const void* p, long long bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                             (int)min(bytes, (long long)0x7fffffff), 0x00020000);
}
// buffer_load_dwordx4 ... lds: 16 bytes per lane land at M0 + 16 * lane
__device__ __forceinline__ void adma16(__amdgpu_buffer_rsrc_t rs, int voff, unsigned lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rs) : "memory");
}
template <int N>
__device__ __forceinline__ void await_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }
__device__ __forceinline__ void abarrier() { asm volatile("s_barrier" ::: "memory"); }

template <int NW> struct AttnCfg {
    static constexpr int NS = NW == 1 ? 2 : 3;                       // ring slots
    static constexpr int PER = (2 * NLD + NW - 1) / NW;               // load instructions per wave per tile
    static constexpr int SLOT_B = 2 * TILE_B + 1024;                  // K tile, V^T tile, 1 KiB sink
    static constexpr int RING_B = NS * SLOT_B;
};

template <int NW>
size_t attn_lds_bytes(int Tp) {
    using A = AttnCfg<NW>;
    return (size_t)A::RING_B + (size_t)A::NS * KT * 4 + (size_t)Tp + (size_t)Tp / KT;
}

// NW waves per block (8: 256 queries), 32 queries each, all sharing every
// K / V^T tile; sequences of one tile use attn_short_kernel instead.
//
// K and V^T tiles go from HBM straight into an LDS ring of NS slots, issued
// NS - 1 tiles ahead and awaited with explicit vmcnt waits, so the loop holds
// no staging registers. K rows of keys at or past the row's key length are out
// of the load's range and arrive as zeros. A tile that is not entirely valid
// (tail or mask holes) is then patched in LDS: the K rows and V^T columns of its
// invalid keys are zeroed and their score bias set to -inf, so a non-finite
// value behind a masked key never reaches a valid output.
template <int NW>
__global__ void __launch_bounds__(64 * NW, 4)   // 4 waves per SIMD
attn_bf16_kernel(AttnParams p) {
    using A = AttnCfg<NW>;
    constexpr int QT = 32 * NW;    // queries per block
    constexpr int NT = 64 * NW;
    constexpr int NS = A::NS, PER = A::PER;
    extern __shared__ __attribute__((aligned(16))) char asmem[];
    float* const kbias = (float*)(asmem + A::RING_B);               // NS x 64
    uint8_t* const kvs = (uint8_t*)(kbias + NS * KT);               // Tp validity bytes, then tile flags
    const unsigned ring_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)asmem;

    if (p.active != nullptr && *p.active == 0) return;   // skipped (block-uniform)
    const int row = blockIdx.z, head = blockIdx.y;
    // the wave index picks the load instructions: keep it in a scalar register
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    // keys: the row's own tokens, or (cross-attention) its Tk context tokens
    const bool cross = p.kx != nullptr;
    const int Tk = cross ? p.Tk : T;
    const long long ldkk = cross ? p.ldkx : ldk;
    const bf16* kbase = cross ? (const bf16*)p.kx + (long long)row * p.Tk * p.ldkx + head * HD : qbase + d;
    const bf16* vtbase = (const bf16*)p.vt + (long long)(row * p.H + head) * HD * p.Tp;
    const int q = blockIdx.x * QT + wave * 32 + j;

    const int rr = row % p.kv_mod;
    const int kvl = min(p.kv_len[rr], Tk);
    const int ntiles = (kvl + KT - 1) / KT;
    const int Tp = p.Tp;

    bf16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        qf[kk] = q < T ? *(const bf16x8*)(qbase + (long long)q * ldk + kk * 16 + h * 8) : bf16x8{};
    // key validity and per-tile "all valid" flags into LDS (read while patching)
    {
        const uint8_t* kv = p.kvalid + (long long)rr * Tp;
        const uint8_t* tf = p.tile_full + (long long)rr * (Tp / KT);
        for (int i = tid; i < ntiles * KT / 16; i += NT) ((uint4*)kvs)[i] = ((const uint4*)kv)[i];
        for (int i = tid; i < ntiles; i += NT) kvs[Tp + i] = tf[i];
    }
    // drain every load above with a wait the compiler sees: its bookkeeping then
    // knows q is resident and puts no vmcnt wait inside the loop (such a wait
    // would also wait for the ring's loads, which it does not see)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // K rows past the key length are out of range: they load as zeros
    const __amdgpu_buffer_rsrc_t rk = arsrc(kbase, kvl > 0 ? ((long long)(kvl - 1) * ldkk + HD) * 2 : 0);
    const __amdgpu_buffer_rsrc_t rv = arsrc(vtbase, (long long)HD * Tp * 2);
    const int lrow = lane / 9, lchunk = lane - 9 * (lane / 9);   // this lane's row / chunk in a load
    auto issue = [&](int it) {
        const unsigned slot = ring_addr + (unsigned)((it % NS) * A::SLOT_B);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int g = wave * PER + i;             // load instruction (uniform): 0..9 K, 10..19 V^T, 20+ none
            if (g >= 2 * NLD) {
                if constexpr (NW > 1) adma16(rv, OOB, slot + 2 * TILE_B);   // keeps every wave's count equal
                continue;
            }
            const bool isk = g < NLD;
            const int gg = isk ? g : g - NLD;
            const int r = gg * GRP + lrow;            // tile row
            const bool ok = r < KT && lchunk < 8;
            const unsigned dst = slot + (isk ? 0u : (unsigned)TILE_B) + (unsigned)(gg * GRP * RS);
            if (isk) {
                const int key = it * KT + r;
                adma16(rk, ok && key < kvl ? (int)(((long long)key * ldkk + lchunk * 8) * 2) : OOB, dst);
            } else {
                adma16(rv, ok ? (int)(((long long)r * Tp + it * KT + lchunk * 8) * 2) : OOB, dst);
            }
        }
    };
    auto wait_tiles = [&](int later) {   // this wave's loads done but those of `later` younger tiles
        if constexpr (NS >= 3) { if (later >= 2) { await_vm<2 * PER>(); return; } }
        if (later == 1) await_vm<PER>();
        else await_vm<0>();
    };

    const float sl2 = 1.4426950408889634f / sqrtf((float)HD);   // 1/sqrt(hd) in base-2 units
    f32x16 oacc[2] = {f32x16{}, f32x16{}};
    // running max of the scaled scores (base 2); finite start so that a tile with
    // no valid key (all scores -inf) gives exp2(-inf) = 0, never inf - inf
    float m_run = -1e30f;
    float l_part = 0.0f;
    // per-lane fragment bases: K row j at chunk h, V^T row j at half h
    const int kl = j * RS + h * 16, vl = TILE_B + j * RS + h * 8;

    for (int it = 0; it < NS - 1 && it < ntiles; ++it) issue(it);
    for (int it = 0; it < ntiles; ++it) {
        const int cur = it % NS;
        wait_tiles(min(ntiles - 1, it + NS - 2) - it);
        abarrier();   // tile it is in LDS for every wave; slot (it - 1) % NS is free
        const bool full = kvs[Tp + it] != 0;
        const char* sb = asmem + cur * A::SLOT_B;
        if (!full) {
            // patch: zero the K rows and V^T columns of invalid keys, set their bias
            char* ks = (char*)sb;
            char* vt = ks + TILE_B;
            const uint8_t* kv = kvs + it * KT;
            for (int e = tid; e < KT * 8; e += NT) {
                const int r = e >> 3, c = e & 7;      // K: key r, chunk c; V^T: head dim r, keys 8c .. 8c + 7
                if (!kv[r]) *(bf16x8*)(ks + r * RS + c * 16) = bf16x8{};
                bf16x8* vp = (bf16x8*)(vt + r * RS + c * 16);
                const uint64_t okb = *(const uint64_t*)(kv + 8 * c);
                if (okb != 0x0101010101010101ull) {
                    bf16x8 vv = *vp;
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (((okb >> (8 * u)) & 0xff) == 0) vv[u] = (bf16)0.0f;
                    *vp = vv;
                }
            }
            for (int e = tid; e < KT; e += NT) kbias[cur * KT + e] = kv[e] ? 0.0f : -INFINITY;
            __syncthreads();
        }
        if (it + NS - 1 < ntiles) issue(it + NS - 1);

        // S^T = K Q^T: s[kh][g*4 + r] = score(key kh*32 + 8g + 4h + r, query q)
        const char* kb0 = sb + kl;
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 a = *(const bf16x8*)(kb0 + kh * 32 * RS + kk * 32);
                s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kh], 0, 0, 0);
            }
        if (!full) {   // partial tile: masked keys get -inf
            const float* kbp = kbias + cur * KT;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int r = 0; r < 4; ++r) s[kh][g * 4 + r] += kbp[kh * 32 + 8 * g + 4 * h + r];
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
        const char* vb0 = sb + vl;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int ss = 0; ss < 2; ++ss) {
                    const char* vr = vb0 + dt * 32 * RS + (kh * 32 + 16 * ss) * 2;
                    const bf16x4 lo = *(const bf16x4*)(vr);
                    const bf16x4 hi = *(const bf16x4*)(vr + 16);
                    bf16x8 a;
                    a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
                    a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kh][ss], oacc[dt], 0, 0, 0);
                }
        // no barrier here: this slot is refilled only after a later iteration's
        // barrier, which every wave reaches after these reads
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

constexpr int KP = HD + 8;     // short kernel: K tile row pitch (bf16), 144 B
constexpr int VP = KT + 8;     // short kernel: V^T tile row pitch (bf16), 144 B

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

// Tiny sequences (at most 32 queries and 32 keys per row, the LocDiT decode tail):
// one wave per (row, head), four heads per block, no LDS and no barrier. Every
// operand comes straight from global memory into MFMA fragments (K rows and Q rows
// 16 bytes per lane, V^T rows 8 bytes per lane in the key order of the P^T
// fragments), so the wave issues all its loads at once; S^T = K Q^T is one 32x32
// block (4 MFMAs), the softmax runs on its accumulators (one query per lane pair),
// and O^T = V^T P^T takes 4 more MFMAs. At these sizes a launch is bound by load
// latency, not by arithmetic.
constexpr int TINY_T = 32;
constexpr int TINY_W = 4;   // heads (waves) per block

__global__ void __launch_bounds__(64 * TINY_W)
attn_tiny_kernel(AttnParams p) {
    if (p.active != nullptr && *p.active == 0) return;   // skipped (block-uniform)
    const int row = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int head = blockIdx.x * TINY_W + wave;
    if (head >= p.H) return;           // wave-uniform; nothing below synchronises waves
    const int j = lane & 31, h = lane >> 5;
    long long rbase;
    int T;
    if (p.row_off) {
        rbase = p.row_off[row];
        T = p.row_off[row + 1] - (int)rbase;
    } else {
        rbase = (long long)row * p.T;
        T = p.T;
    }
    const int d = p.H * HD;
    const long long ldk = 2LL * d;
    const bf16* qbase = (const bf16*)p.qkv + rbase * ldk + head * HD;
    const bool cross = p.kx != nullptr;
    const int Tk = cross ? p.Tk : T;
    const long long ldkk = cross ? p.ldkx : ldk;
    const bf16* kbase = cross ? (const bf16*)p.kx + (long long)row * p.Tk * p.ldkx + head * HD : qbase + d;
    const bf16* vtbase = (const bf16*)p.vt + (long long)(row * p.H + head) * HD * p.Tp;
    const int rr = row % p.kv_mod;
    const int kvl = min(p.kv_len[rr], Tk);

    // fragments: K row j (A of S^T), Q row j (B of S^T), V^T rows dt*32 + j in the key
    // order of the P^T fragments (slot e of k-step ss: key 16 ss + 4h + e, e < 4, or
    // 16 ss + 8 + 4h + e - 4)
    bf16x8 ka[4], qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        ka[kk] = j < Tk ? *(const bf16x8*)(kbase + (long long)j * ldkk + kk * 16 + h * 8) : bf16x8{};
        qf[kk] = j < T ? *(const bf16x8*)(qbase + (long long)j * ldk + kk * 16 + h * 8) : bf16x8{};
    }
    bf16x4 vlo[2][2], vhi[2][2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            const bf16* vr = vtbase + (long long)(dt * 32 + j) * p.Tp + 16 * ss + 4 * h;
            vlo[dt][ss] = *(const bf16x4*)vr;
            vhi[dt][ss] = *(const bf16x4*)(vr + 8);
        }
    // key validity: lane j's key j, gathered into one 32-bit mask
    const bool kj = j < kvl && p.kvalid[(long long)rr * p.Tp + j] != 0;
    const uint32_t vmask = (uint32_t)__ballot(kj);
    auto valid = [&](int key) { return ((vmask >> key) & 1u) != 0; };

    // S^T = K Q^T: s[g*4 + r] = score(key 8g + 4h + r, query j)
    f32x16 sc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[kk], sc, 0, 0, 0);
    const float sl2 = 1.4426950408889634f / sqrtf((float)HD);   // 1/sqrt(hd) in base-2 units
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = 8 * g + 4 * h + r;
            if (!valid(key)) sc[g * 4 + r] = -INFINITY;
            mx = fmaxf(mx, sc[g * 4 + r]);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m = mx == -INFINITY ? 0.0f : mx * sl2;     // no valid key: every p is 0
    float ls = 0.0f;
    bf16x8 pb[2];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(sc[g * 4 + r], sl2, -m));
            ls += pv;
            pb[g >> 1][(g & 1) * 4 + r] = (bf16)pv;
        }
    const float l = ls + __shfl_xor(ls, 32, 64);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;

    // O^T = V^T P^T; values of invalid keys are zeroed (their p is 0, and 0 times a
    // non-finite value behind the padding must not reach the output)
    f32x16 oacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            bf16x8 a;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[e] = valid(16 * ss + 4 * h + e) ? vlo[dt][ss][e] : (bf16)0.0f;
                a[4 + e] = valid(16 * ss + 8 + 4 * h + e) ? vhi[dt][ss][e] : (bf16)0.0f;
            }
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ss], oacc[dt], 0, 0, 0);
        }
    if (j < T) {
        bf16* dst = (bf16*)p.o + (rbase + j) * d + head * HD;
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

// Short sequences (one key tile, T <= 64): one wave per 32 queries, the tile
// staged through registers into a padded LDS layout (72-element rows) in one
// step; with a single tile there is nothing to prefetch. The staged tile, the
// fragments and both accumulator pairs take more than 128 registers, so the
// kernel runs at the occupancy its registers allow (no waves-per-SIMD target).
template <int NW>
__global__ void __launch_bounds__(64 * NW, 1)
attn_short_kernel(AttnParams p) {
    constexpr int QT = 32 * NW;    // queries per block
    constexpr int NT = 64 * NW;
    __shared__ __attribute__((aligned(16))) bf16 Ks[2][KT * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vt[2][HD * VP];
    __shared__ float kbias[2][KT];

    if (p.active != nullptr && *p.active == 0) return;   // skipped (block-uniform)
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
    const bool cross = p.kx != nullptr;        // keys from the context (one tile: Tk <= 64)
    const int Tk = cross ? p.Tk : T;
    const long long ldkk = cross ? p.ldkx : ldk;
    const bf16* kbase = cross ? (const bf16*)p.kx + (long long)row * p.Tk * p.ldkx + head * HD : qbase + d;
    const bf16* vtbase = (const bf16*)p.vt + (long long)(row * p.H + head) * HD * p.Tp;
    const int q = blockIdx.x * QT + wave * 32 + j;

    bf16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        qf[kk] = q < T ? *(const bf16x8*)(qbase + (long long)q * ldk + kk * 16 + h * 8) : bf16x8{};

    const int rr = row % p.kv_mod;
    const int kvl = min(p.kv_len[rr], Tk);
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
            st.load(kbase, ldkk, Tk - 1, vtbase, p.Tp, kv, it * KT, tid);
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


__device__ __forceinline__ bool key_valid(const AttnParams& p, const uint8_t* km, int key, int kvl) {
    if (key >= kvl) return false;
    if (km == nullptr || key < p.P) return true;
    return km[key - p.P] != 0;
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
    if (p.active != nullptr && *p.active == 0) return;   // skipped (block-uniform)
    const int row = blockIdx.z, head = blockIdx.y;
    const int q = blockIdx.x * FQ + threadIdx.x;
    const int T = p.T, d = p.H * HD_;
    const long long ld = 3LL * d;
    const float* base = (const float*)p.qkv + (long long)row * T * ld;
    // key | value rows: the row's own tokens (at column d of its q|k|v rows), or
    // (cross-attention) its Tk context tokens
    const bool cross = p.kx != nullptr;
    const int Tk = cross ? p.Tk : T;
    const long long ldkv = cross ? p.ldkx : ld;
    const float* kvb = cross ? (const float*)p.kx + (long long)row * p.Tk * p.ldkx : base + d;
    const int rr = row % p.kv_mod;
    const int kvl = min(p.kv_len[rr], Tk);
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
            Kt[kr][e] = ok ? kvb[(long long)key * ldkv + head * HD_ + e] : 0.0f;
            Vs[kr][e] = ok ? kvb[(long long)key * ldkv + d + head * HD_ + e] : 0.0f;
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

template <int NW>
void launch_attn_nw(const AttnParams& p, hipStream_t s) {
    static const bool attr = [] {
        return hipFuncSetAttribute((const void*)attn_bf16_kernel<NW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   160 * 1024) == hipSuccess;
    }();
    (void)attr;
    dim3 grid((p.T + 32 * NW - 1) / (32 * NW), p.H, p.rows);
    attn_bf16_kernel<NW><<<grid, 64 * NW, attn_lds_bytes<NW>(p.Tp), s>>>(p);
}

bool attention_bf16_fits(long long T) {
    if (T <= 64) return true;   // one key tile: the short kernel, static LDS
    const long long Tp = (T + 63) / 64 * 64;
    return Tp <= (1LL << 30) && attn_lds_bytes<8>((int)Tp) <= 160 * 1024;
}

void launch_attention_bf16(const AttnParams& p, hipStream_t s) {
    if (p.rows <= 0 || p.T <= 0) return;
    const int tq = p.row_off ? (p.T + 7) / 8 * 8 : p.T;     // largest row: packed rows round to 8
    const int tk = p.kx ? p.Tk : tq;
    if (tq <= TINY_T && tk <= TINY_T) {
        attn_tiny_kernel<<<dim3((p.H + TINY_W - 1) / TINY_W, p.rows), 64 * TINY_W, 0, s>>>(p);
        return;
    }
    if (p.T <= 64 && (p.kx == nullptr || p.Tk <= 64)) {
        dim3 grid((p.T + 31) / 32, p.H, p.rows);
        attn_short_kernel<1><<<grid, 64, 0, s>>>(p);
    } else {
        launch_attn_nw<8>(p, s);
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
