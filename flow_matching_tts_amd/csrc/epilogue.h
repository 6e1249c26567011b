// Per-element GEMM epilogues (bias, GELU, gated residual, input-projection
// scatter into the branch rows, masked velocity store).
#pragma once
#include <type_traits>
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
        // bf16 outputs: the approximation is exact to far below the output rounding
        const float g = std::is_same<ActT, bf16>::value ? gelu_bf16(acc + b) : gelu_erf(acc + b);
        ((ActT*)p.out)[(long long)m * p.ldo + n] = to_out<ActT>(g);
    } else if constexpr (EPI == EPI_GATED) {
        float* h = (float*)p.out + (long long)m * p.ldo + n;
        *h += p.gate.at((long long)m)[n] * (acc + b);
    } else if constexpr (EPI == EPI_INPROJ) {
        const int r = m / p.Tx, t = m - r * p.Tx;
        const float plain = acc + b;
        const float withc = p.cproj ? acc + p.cproj[(long long)m * p.ldo + n] : plain;
        for (int br = 0; br < p.nb; ++br) {
            long long tok;
            if (p.row_off) {
                const int row = br * p.R + r;
                if (t >= p.row_off[row + 1] - p.row_off[row]) continue;   // past the row's last valid frame
                tok = p.row_off[row] + t;
            } else {
                tok = (long long)(br * p.R + r) * p.T + p.P + t;
            }
            ((float*)p.out)[tok * p.ldo + n] = br >= p.cond_branch0 ? withc : plain;
        }
    } else if constexpr (EPI == EPI_QKV) {
        if (n < p.d2) {
            ((bf16*)p.out)[(long long)m * p.ldo + n] = (bf16)(acc + b);
        } else {
            const int row = p.tok_row ? p.tok_row[m] : m / p.T;
            const int t = m - (p.tok_row ? p.row_off[row] : row * p.T);
            const int c = n - p.d2, hh = c >> 6, e = c & 63;
            p.vt[((long long)(row * p.H + hh) * 64 + e) * p.Tp + t] = (bf16)(acc + b);
        }
    } else if constexpr (EPI == EPI_VOUT) {
        const int row = p.tok_row ? p.tok_row[m] : m / p.Tx;
        const int t = m - (p.tok_row ? p.row_off[row] : row * p.Tx);
        if (t >= p.Tx) return;   // packed rows: alignment tokens past the last frame
        const int r = row % p.R;
        const bool valid = p.mask == nullptr || p.mask[(long long)r * p.Tx + t] != 0;
        ((float*)p.out)[((long long)row * p.Tx + t) * p.ldo + n] = valid ? acc + b : 0.0f;
    }
}

// Vector epilogue of 4 consecutive columns n..n+3 of one row m (in range, 16-byte
// aligned). Same arithmetic as epi_store, one wide access per operand.
template <int EPI>
__device__ __forceinline__ void epi_store_vec4(const EpiParams& p, int m, int n, f32x4 v,
                                               const f32x4* bias4 = nullptr) {
    // the in-projection's conditioned branches add the condition term (which holds
    // the bias) to the bare accumulator, as every other in-projection path does
    const f32x4 acc = v;
    if (bias4) v += *bias4;                        // preloaded by the caller (same columns)
    else if (p.bias) v += *(const f32x4*)(p.bias + n);
    if constexpr (EPI == EPI_F32) {
        *(f32x4*)((float*)p.out + (long long)m * p.ldo + n) = v;
    } else if constexpr (EPI == EPI_ACT || EPI == EPI_GELU_ACT || EPI == EPI_QKV) {
        if constexpr (EPI == EPI_GELU_ACT) {
            v[0] = gelu_bf16(v[0]); v[1] = gelu_bf16(v[1]); v[2] = gelu_bf16(v[2]); v[3] = gelu_bf16(v[3]);
        }
        if constexpr (EPI == EPI_QKV) {
            if (p.rope != nullptr) {
                // q or k columns n .. n+3 (n % 4 == 0): pairs (n, n+1) and (n+2, n+3) of their
                // head turn by the table's angles of pair indices i0, i0 + 1 at position t
                const int t = p.tok_row ? m - p.row_off[p.tok_row[m]] : m % p.T;
                const int i0 = (n % p.rope_hd) >> 1;
                const f32x4 cs = *(const f32x4*)(p.rope + ((long long)t * (p.rope_hd >> 1) + i0) * 2);
                const float a0 = v[0], a1 = v[1], b0 = v[2], b1 = v[3];
                v[0] = a0 * cs[0] - a1 * cs[1];
                v[1] = a0 * cs[1] + a1 * cs[0];
                v[2] = b0 * cs[2] - b1 * cs[3];
                v[3] = b0 * cs[3] + b1 * cs[2];
            }
        }
        bf16x4 b;
        b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
        *(bf16x4*)((bf16*)p.out + (long long)m * p.ldo + n) = b;
    } else if constexpr (EPI == EPI_GATED) {
        f32x4* h = (f32x4*)((float*)p.out + (long long)m * p.ldo + n);
        *h += *(const f32x4*)(p.gate.at((long long)m) + n) * v;
    } else if constexpr (EPI == EPI_INPROJ) {
        const int r = m / p.Tx, t = m - r * p.Tx;
        // v holds acc + bias; the conditioned branches use acc + cproj instead
        const f32x4 withc = p.cproj ? acc + *(const f32x4*)(p.cproj + (long long)m * p.ldo + n) : v;
        for (int br = 0; br < p.nb; ++br) {
            long long tok;
            if (p.row_off) {
                const int row = br * p.R + r;
                if (t >= p.row_off[row + 1] - p.row_off[row]) continue;   // past the row's last valid frame
                tok = p.row_off[row] + t;
            } else {
                tok = (long long)(br * p.R + r) * p.T + p.P + t;
            }
            *(f32x4*)((float*)p.out + tok * p.ldo + n) = br >= p.cond_branch0 ? withc : v;
        }
    } else if constexpr (EPI == EPI_VOUT) {
        const int row = p.tok_row ? p.tok_row[m] : m / p.Tx;
        const int t = m - (p.tok_row ? p.row_off[row] : row * p.Tx);
        if (t >= p.Tx) return;   // packed rows: alignment tokens past the last frame
        const int r = row % p.R;
        const bool valid = p.mask == nullptr || p.mask[(long long)r * p.Tx + t] != 0;
        *(f32x4*)((float*)p.out + ((long long)row * p.Tx + t) * p.ldo + n) = valid ? v : f32x4{};
    }
}

// Epilogue of one 32x32 MFMA accumulator block through a wave-private LDS
// scratch area (32 rows x 32 floats, row-major, 4 KiB): each lane writes its column
// (16 scalar writes; a write instruction covers 32 consecutive columns of a
// row), then reads back four consecutive columns of one row per access, so
// every global access of the epilogue is 16 bytes wide (8 for bf16 outputs)
// instead of one element. Value columns of the QKV projection are read back
// down a column instead and written transposed (8 consecutive sequence
// positions per store).
constexpr int EPI_RP = 32;
constexpr int EPI_WAVE_FLOATS = 32 * EPI_RP;

// bias4 / bias1, when given, hold the bias of this lane's columns (nb0 + 4 (lane % 8)
// .. + 3; nb0 + lane % 32 for the transposed V columns), loaded by the caller before
// any store: a global load placed after stores waits for those stores as well (one
// vmcnt counter for both), which serialises an epilogue on store completion. PK =
// false drops the packed-row lookups (tok_row must then be null), so that path
// issues no load at all.
template <int EPI, bool PK = true>
__device__ __forceinline__ void epi_block(const EpiParams& p, const f32x16& acc, float* wl, int mb, int nb0,
                                          int M, int N, int lane, const f32x4* bias4 = nullptr,
                                          const float* bias1 = nullptr) {
    const int li = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) wl[(8 * g + 4 * lh + r) * EPI_RP + li] = acc[g * 4 + r];
    __builtin_amdgcn_wave_barrier();
    if constexpr (EPI == EPI_SWIGLU) {
        // fused gate-up block: columns nb0 .. nb0 + 15 are the gate of features
        // nb0 / 2 .. + 15, columns nb0 + 16 .. + 31 their up values. Lane: row
        // (lane / 4) + 16 q, features 4 (lane % 4) .. + 3.
        if (nb0 < N) {
            const int c = (lane & 3) * 4;
            const f32x4 bg = p.bias ? *(const f32x4*)(p.bias + nb0 + c) : f32x4{};
            const f32x4 bu = p.bias ? *(const f32x4*)(p.bias + nb0 + 16 + c) : f32x4{};
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int row = (lane >> 2) + 16 * q, m = mb + row;
                if (m >= M) continue;
                const f32x4 g = *(const f32x4*)(wl + row * EPI_RP + c) + bg;
                const f32x4 u = *(const f32x4*)(wl + row * EPI_RP + 16 + c) + bu;
                bf16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (bf16)(silu(g[e]) * u[e]);
                *(bf16x4*)((bf16*)p.out + (long long)m * p.ldo + (nb0 >> 1) + c) = o;
            }
        }
        __builtin_amdgcn_wave_barrier();
        return;
    }
    if constexpr (EPI == EPI_VOUT_EULER) {
        // the block's 32 rows are 32 / nb frames with their nb branch rows next to each
        // other; lane: frame (lane / 8) + 8 q of the block, columns 4 (lane % 8) .. + 3
        const int nbv = p.nb, c0 = (lane & 7) * 4, n = nb0 + c0;
        const long long nfr = (long long)p.R * p.Tx;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int fi = (lane >> 3) + 8 * q;
            const long long fr = mb / nbv + fi;
            if (fi * nbv >= 32 || fr >= nfr || n >= N) continue;
            const bool valid = p.mask == nullptr || p.mask[fr] != 0;
            const float* xi = p.x_in + fr * p.ldo;
            float* xo = p.x_out + fr * p.ldo;
            if (n + 3 < N) {
                const f32x4 b4 = p.bias ? *(const f32x4*)(p.bias + n) : f32x4{};
                const f32x4 xv = *(const f32x4*)(xi + n);
                if (valid) {
                    f32x4 acc = xv + p.cw[0] * (*(const f32x4*)(wl + (fi * nbv) * EPI_RP + c0) + b4);
                    if (nbv > 1) acc += p.cw[1] * (*(const f32x4*)(wl + (fi * nbv + 1) * EPI_RP + c0) + b4);
                    *(f32x4*)(xo + n) = acc;
                } else if (xo != xi) {
                    *(f32x4*)(xo + n) = xv;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (n + e >= N) continue;
                    const float b1 = p.bias ? p.bias[n + e] : 0.0f;
                    const float xv = xi[n + e];
                    if (valid) {
                        float acc = xv + p.cw[0] * (wl[(fi * nbv) * EPI_RP + c0 + e] + b1);
                        if (nbv > 1) acc += p.cw[1] * (wl[(fi * nbv + 1) * EPI_RP + c0 + e] + b1);
                        xo[n + e] = acc;
                    } else if (xo != xi) {
                        xo[n + e] = xv;
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        return;
    }
    if constexpr (EPI == EPI_QKV) {
        if (nb0 >= p.d2) {
            // lane: column li, rows 16 lh .. 16 lh + 15 (consecutive sequence positions)
            const int n = nb0 + li;
            if (n < N) {
                const float b = bias1 ? *bias1 : p.bias ? p.bias[n] : 0.0f;
                const int c = n - p.d2, hh = c >> 6, e = c & 63;
#pragma unroll
                for (int q8 = 0; q8 < 2; ++q8) {
                    const int r0 = 16 * lh + 8 * q8, m = mb + r0;
                    float vals[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) vals[r] = wl[(r0 + r) * EPI_RP + li] + b;
                    if (m >= M) continue;
                    const bool pk = PK && p.tok_row != nullptr;
                    const int row = pk ? p.tok_row[m] : m / p.T;
                    const int t = m - (pk ? p.row_off[row] : row * p.T);
                    const int len = pk ? p.row_off[row + 1] - p.row_off[row] : p.T;
                    if (m + 7 < M && t + 7 < len && (t & 7) == 0) {
                        bf16x8 o;
#pragma unroll
                        for (int r = 0; r < 8; ++r) o[r] = (bf16)vals[r];
                        *(bf16x8*)(p.vt + ((long long)(row * p.H + hh) * 64 + e) * p.Tp + t) = o;
                    } else if (pk) {   // rare (row boundaries): rolled, reads LDS again
#pragma unroll 1
                        for (int r = 0; r < 8 && m + r < M; ++r) {
                            const int rw = p.tok_row[m + r], tt = (m + r) - p.row_off[rw];
                            p.vt[((long long)(rw * p.H + hh) * 64 + e) * p.Tp + tt] =
                                (bf16)(wl[(r0 + r) * EPI_RP + li] + b);
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 8; ++r)
                            if (m + r < M) {
                                const int rw = (m + r) / p.T, tt = (m + r) - rw * p.T;
                                p.vt[((long long)(rw * p.H + hh) * 64 + e) * p.Tp + tt] = (bf16)vals[r];
                            }
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            return;
        }
    }
    // lane: row (lane / 8) + 8 q, columns 4 (lane % 8) .. +3
    const int c0 = (lane & 7) * 4;
    if constexpr (EPI == EPI_INPROJ) {
        // the in-projection reads the condition term of each row: load all four rows'
        // operands first, then store (a load after a store waits for the store too)
        const int n = nb0 + c0;
        if (n + 3 < N && p.row_off == nullptr) {
            const f32x4 b = p.bias ? *(const f32x4*)(p.bias + n) : f32x4{};
            f32x4 v[4], vc[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = min(mb + (lane >> 3) + 8 * q, M - 1);
                v[q] = *(const f32x4*)(wl + ((lane >> 3) + 8 * q) * EPI_RP + c0);
                vc[q] = p.cproj ? v[q] + *(const f32x4*)(p.cproj + (long long)m * p.ldo + n) : v[q] + b;
                v[q] += b;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = mb + (lane >> 3) + 8 * q;
                if (m >= M) continue;
                const int r = m / p.Tx, t = m - r * p.Tx;
                for (int br = 0; br < p.nb; ++br) {
                    const long long tok = (long long)(br * p.R + r) * p.T + p.P + t;
                    *(f32x4*)((float*)p.out + tok * p.ldo + n) = br >= p.cond_branch0 ? vc[q] : v[q];
                }
            }
            __builtin_amdgcn_wave_barrier();
            return;
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = (lane >> 3) + 8 * q;
        const f32x4 v = *(const f32x4*)(wl + row * EPI_RP + c0);
        const int m = mb + row, n = nb0 + c0;
        if (m >= M) continue;
        if (n + 3 < N) {
            epi_store_vec4<EPI>(p, m, n, v, bias4);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < N) epi_store<EPI, bf16>(p, m, n + e, v[e]);
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// Gated-residual epilogue of a wave's TM x TN accumulator blocks with the
// residual stream and the gate read ahead: the h and gate values of block b +
// AHEAD are loaded before block b is stored (distinct addresses), and the bias of
// every column before the first store, so no load result is waited for behind
// stores (one vmcnt counter covers both). Tiles with ragged columns take the
// per-element path of epi_block. Same arithmetic as epi_block<EPI_GATED>.
template <int TM, int TN>
__device__ __forceinline__ void epi_tile_gated(const EpiParams& p, const f32x16 (&acc)[TM][TN], float* wl, int mb0,
                                               int nb0, int M, int N, int lane) {
    if (nb0 + TN * 32 > N) {   // ragged columns somewhere in this wave's tile
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) epi_block<EPI_GATED>(p, acc[i][j], wl, mb0 + i * 32, nb0 + j * 32, M, N, lane);
        return;
    }
    const int c0 = (lane & 7) * 4;
    f32x4 bias[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) bias[j] = p.bias ? *(const f32x4*)(p.bias + nb0 + j * 32 + c0) : f32x4{};
    if (p.gate.spk_branch < 0) {
        // every row reads the same gate vector: preload it per column like the bias
        // and read only the residual ahead, four blocks deep (64 VGPRs)
        f32x4 gate[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) gate[j] = *(const f32x4*)(p.gate.base + nb0 + j * 32 + c0);
        constexpr int AH = 4;
        f32x4 hq[AH + 1][4];
        auto fetch_h = [&](int b, f32x4 (&hv)[4]) {
            const int i = b / TN, j = b % TN;
            const int n = nb0 + j * 32 + c0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = mb0 + i * 32 + (lane >> 3) + 8 * q;
                hv[q] = m < M ? *(const f32x4*)((const float*)p.out + (long long)m * p.ldo + n) : f32x4{};
            }
        };
#pragma unroll
        for (int b = 0; b < AH && b < TM * TN; ++b) fetch_h(b, hq[b]);
#pragma unroll
        for (int b = 0; b < TM * TN; ++b) {
            const int i = b / TN, j = b % TN;
            if (b + AH < TM * TN) fetch_h(b + AH, hq[(b + AH) % (AH + 1)]);
            const f32x4 (&hcur)[4] = hq[b % (AH + 1)];
            const int mb = mb0 + i * 32, n = nb0 + j * 32 + c0;
            const int li = lane & 31, lh = lane >> 5;
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r) wl[(8 * g + 4 * lh + r) * EPI_RP + li] = acc[i][j][g * 4 + r];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = (lane >> 3) + 8 * q;
                const int m = mb + row;
                if (m >= M) continue;
                const f32x4 v = *(const f32x4*)(wl + row * EPI_RP + c0) + bias[j];
                *(f32x4*)((float*)p.out + (long long)m * p.ldo + n) = hcur[q] + gate[j] * v;
            }
            __builtin_amdgcn_wave_barrier();
        }
        return;
    }
    // Per-row gate vectors (a speaker branch: its rows read their request's own
    // modulation). Tokens are laid out row after row, so the 32 tokens of a block
    // nearly always belong to one row: the gate pointers of a block's first and
    // last token are compared (wave-uniform), and when they are equal every token
    // of the block reads that one vector (rows are monotone in the token index and
    // the speaker branch is the last branch, so equal pointers mean one row, or
    // only rows that share vector 0). Such a block's gate is read ahead with its
    // residual, one 16-byte load per lane; a block that straddles rows with
    // different vectors looks its gates up per row when it is stored.
    const float* gbase[TM];
    bool guni[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const long long mf = mb0 + i * 32, ml = min(mf + 31, (long long)M - 1);
        gbase[i] = mf < M ? p.gate.at(mf) : p.gate.base;
        guni[i] = mf >= M || gbase[i] == p.gate.at(ml);
    }
    constexpr int AH = 3;
    f32x4 hq[AH + 1][4], gq[AH + 1];
    auto fetch = [&](int b, f32x4 (&hv)[4], f32x4& gv) {
        const int i = b / TN, j = b % TN;
        const int n = nb0 + j * 32 + c0;
        gv = guni[i] ? *(const f32x4*)(gbase[i] + n) : f32x4{};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = mb0 + i * 32 + (lane >> 3) + 8 * q;
            hv[q] = m < M ? *(const f32x4*)((const float*)p.out + (long long)m * p.ldo + n) : f32x4{};
        }
    };
#pragma unroll
    for (int b = 0; b < AH && b < TM * TN; ++b) fetch(b, hq[b], gq[b]);
#pragma unroll
    for (int b = 0; b < TM * TN; ++b) {
        const int i = b / TN, j = b % TN;
        if (b + AH < TM * TN) fetch(b + AH, hq[(b + AH) % (AH + 1)], gq[(b + AH) % (AH + 1)]);
        const f32x4 (&hcur)[4] = hq[b % (AH + 1)];
        const f32x4 gcur = gq[b % (AH + 1)];
        const int mb = mb0 + i * 32, n = nb0 + j * 32 + c0;
        const int li = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) wl[(8 * g + 4 * lh + r) * EPI_RP + li] = acc[i][j][g * 4 + r];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = (lane >> 3) + 8 * q;
            const int m = mb + row;
            if (m >= M) continue;
            const f32x4 v = *(const f32x4*)(wl + row * EPI_RP + c0) + bias[j];
            const f32x4 g = guni[i] ? gcur : *(const f32x4*)(p.gate.at((long long)m) + n);
            *(f32x4*)((float*)p.out + (long long)m * p.ldo + n) = hcur[q] + g * v;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace cfm
