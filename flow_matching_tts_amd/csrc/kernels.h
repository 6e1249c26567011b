// Launchers of the gfx950 kernels (host side), shared by the C-ABI runtime.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "common.h"

namespace cfm {

// GEMM epilogues: what happens to acc[m, n] = sum_k A[m,k] W[n,k].
enum Epi {
    EPI_F32 = 0,       // out f32 [m, n] = acc + bias
    EPI_ACT = 1,       // out act (bf16 on the MFMA path, f32 on the SIMT path) = acc + bias
    EPI_GELU_ACT = 2,  // out act = GELU(acc + bias)
    EPI_GATED = 3,     // out f32 [m, n] += gate(m)[n] * (acc + bias)
    EPI_INPROJ = 4,    // input projection of latent token m = r*Tx + t into every branch row
    EPI_VOUT = 5,      // velocity: out f32 [m, n] = frame valid ? acc + bias : 0
    EPI_QKV = 6,       // q|k columns -> out bf16 [m, 2d]; v columns -> vt bf16 [row, head, hd, Tp] (transposed)
    EPI_SWIGLU = 7,    // fused gate-up: block of 32 columns 32b .. 32b+31 = 16 gate then 16 up columns of
                       // features 16b .. 16b+15; out bf16 [m, 16b + i] = SiLU(gate_i + bias) * (up_i + bias)
    EPI_VOUT_EULER = 8,  // velocity rows interleaved by frame (m = frame * nb + b, nb = 1 or 2), guidance
                         // combine and Euler step in the epilogue: x_out[frame, n] = x_in[frame, n] +
                         // sum_b cw[b] (acc + bias) on valid frames; masked frames keep x_in
};

struct EpiParams {
    const float* bias = nullptr;     // [N] or null
    void* out = nullptr;
    long long ldo = 0;               // row stride of out, elements
    RowMod gate{};                   // EPI_GATED: gate vector of token m
    // EPI_INPROJ: latent token m = r*Tx + t lands at token (b*R + r)*T + P + t
    // of every branch b; branches b >= cond_branch0 add the condition
    // projection cproj[m, n] (which already holds the bias), the others add bias.
    int R = 0, Tx = 0, T = 0, P = 0, nb = 0, cond_branch0 = 1;
    const float* cproj = nullptr;
    // EPI_VOUT: m = row*Tx + t, request r = row % R, mask [R, Tx] or null
    const uint8_t* mask = nullptr;
    // EPI_QKV: token m = row*T + t; value column n - 2d of head hh = (n-2d)/64 lands at
    // vt[((row*H + hh)*64 + (n-2d)%64)*Tp + t]; q and k columns go to out with row stride ldo (= 2d)
    bf16* vt = nullptr;
    int H = 0, Tp = 0, d2 = 0;
    // packed rows (variable-length batches): token m of the packed layout
    // belongs to row tok_row[m] at position m - row_off[row]; row i holds
    // row_off[i + 1] - row_off[i] tokens (its frame count rounded up to a
    // multiple of 8; positions past Tx are never stored). Null: rows padded to
    // T (or Tx) tokens.
    const int32_t* tok_row = nullptr;
    const int32_t* row_off = nullptr;
    // optional device row count (at most M): the grid is sized for M and the
    // tiles past *m_dev exit at once
    const int32_t* m_dev = nullptr;
    // optional room for split-K partial products (fp32): a bf16 GEMM with few tiles and
    // a long K may then split K (the library picks the split; M * N * splits floats)
    float* split_ws = nullptr;
    long long split_ws_floats = 0;
    // EPI_VOUT_EULER: latent x [R * Tx frames, ldo] in and out (may be the same), branch
    // weights (dt already applied), frame mask [R * Tx] or null (R, Tx, nb above)
    const float* x_in = nullptr;
    float* x_out = nullptr;
    float cw[3] = {0.0f, 0.0f, 0.0f};
    // EPI_GATED, optional: when the GEMM runs split in K, its row-wise reduction also
    // applies the next adaLN norm to the updated rows, ln_y bf16 [m, N] =
    // norm(h[m]) (1 + ln_scale(m)) + ln_shift(m) (LayerNorm, or RMSNorm with ln_rms);
    // launch_gemm_bf16 returns whether it did
    void* ln_y = nullptr;
    RowMod ln_shift{}, ln_scale{};
    int ln_rms = 0;
    // EPI_QKV, optional: rotary embedding of the q|k columns, table [T, rope_hd / 2] of
    // (cos, sin) pairs by token position t (m - row_off[tok_row[m]], or m % T)
    const float* rope = nullptr;
    int rope_hd = 0;
};

// bf16 MFMA GEMM, A bf16 or f32 (rounded to bf16 while staging), W bf16 [N, K].
// tile: 0 = pick by problem size; 1 = 128x128, 6 = 128x128 with K stage 64, 10 = 64x64,
// 14 = 256x256 ping-pong (bf16 A only above 1)
// Returns true when the epilogue also produced ep.ln_y (see EpiParams).
bool launch_gemm_bf16(bool a_f32, int epi, const void* A, int lda, const bf16* W, int ldw,
                      int M, int N, int K, const EpiParams& ep, hipStream_t s, int tile = 0);
// fp32 SIMT GEMM, A f32 (optionally SiLU on load), W f32 or bf16 [N, K]; EPI_ACT stores f32.
void launch_gemm_simt(bool w_bf16, bool silu_a, int epi, const float* A, int lda, const void* W,
                      int ldw, int M, int N, int K, const EpiParams& ep, hipStream_t s);

struct AttnParams {
    const void* qkv;          // fp32 path: [rows, T, 3d]; bf16 path: q|k [rows, T, 2d]
    const void* vt;           // bf16 path: V transposed per head [rows, H, 64, Tp]
    int Tp;                   // padded key count of vt (multiple of 64)
    void* o;                  // [rows, T, d]
    int rows, T, H, hd;
    const int32_t* kv_len;    // per (row % kv_mod): keys >= kv_len are masked
    int kv_mod;
    const uint8_t* key_mask;  // [(row % kv_mod), Tm] for keys >= P, or null
    int mask_stride;          // Tm
    int P;                    // keys < P are always valid (condition prefix)
    // bf16 path: per-key validity bytes [(row % kv_mod), Tp] and per-64-key-tile
    // "all valid" bytes [(row % kv_mod), Tp / 64], made by launch_key_prep
    const uint8_t* kvalid;
    const uint8_t* tile_full;
    // packed rows: row i's q|k rows start at token row_off[i] (else i * T); the
    // row's query count is then its key length
    const int32_t* row_off = nullptr;
    // optional device flag: when it reads 0 every block exits at once (a skipped block)
    const int32_t* active = nullptr;
    // cross-attention: keys come from kx instead of the row's own tokens, Tk per row
    // (row i's keys at kx + i * Tk * ldkx; bf16 path: keys only, values in vt as
    // usual; fp32 path: [key | value] rows of 2d); kv_len / kvalid / tile_full and
    // Tp then describe those Tk keys. Null: self-attention.
    const void* kx = nullptr;
    long long ldkx = 0;
    int Tk = 0;
};
void launch_attention_bf16(const AttnParams& p, hipStream_t s);
// whether the bf16 attention's LDS (key ring plus per-key tables) holds sequences of T keys
bool attention_bf16_fits(long long T);
void launch_attention_f32(const AttnParams& p, hipStream_t s);

// adaLN LayerNorm: output token o = row*Tout + t reads input token row*Tin + off + t.
struct LnParams {
    const float* h;
    void* y;
    int d;
    long long n_out;          // output tokens
    int Tin, Tout, off;
    RowMod shift, scale;      // RowMod evaluated on the OUTPUT token index
    int out_bf16;
    const int32_t* n_dev = nullptr;   // optional device count of output tokens (at most n_out)
    int rms = 0;                      // RMSNorm h / sqrt(mean(h^2) + 1e-6) instead of LayerNorm
    // optional output order interleaved by frame: output token o = (r * Tout + t) * inter_nb + b
    // holds what the row-major order puts at (b * inter_R + r) * Tout + t (0 = row-major)
    int inter_nb = 0, inter_R = 0;
};
void launch_adaln(const LnParams& p, hipStream_t s);

// x_out = x_in + sum_b w_b v_b on valid frames (v [nb, R, Tx, C]); masked frames are
// left alone in place, copied when x_out != x_in; requests with lane_off[r] != 0 take
// x_in + w_full v_{nb-1}.
struct CfgEulerArgs {
    const float* v = nullptr;
    int nb = 1;
    float w0 = 0.0f, w1 = 0.0f, w2 = 0.0f;
    const uint8_t* mask = nullptr;
    int R = 0, Tx = 0, C = 0;
    const float* x_in = nullptr;
    float* x_out = nullptr;
    const int32_t* lane_off = nullptr;
    float w_full = 0.0f;
};
void launch_cfg_euler(const CfgEulerArgs& a, hipStream_t s);
// adaptive guidance state update after a step's first evaluation (state [count R | off R | guided R])
void launch_adaptive_update(const float* v, int nb, const uint8_t* mask, int R, int Tx, int C, const int32_t* st_in,
                            int32_t* st_out, int step, int warmup, int patience, float threshold, int evals_per_step,
                            hipStream_t s);
void launch_fill_i32(int32_t* p, int n, int value, hipStream_t s);
// Block-residual cache (one lane per call). State: int32 [8] = evaluations, consecutive
// hits, hits, residual saved, compute flag, middle-block token count, probe saved,
// accumulated score (float bits). kCacheParts partial sums per score.
constexpr int kCacheParts = 512;
struct CacheTok {              // which tokens of the hidden state exist and are valid frames
    long long cap = 0;         // token capacity (grid size)
    const int32_t* n_dev = nullptr;   // device token count (packed layout) or null: cap tokens
    int T = 1;                 // tokens per row (padded layout)
    const int32_t* tok_row = nullptr, *row_off = nullptr;   // packed layout
    const uint8_t* kvalid = nullptr;  // [R, Tp] key validity
    int R = 1, Tp = 64;
};
// partial sums of |h - prev| and |prev| over valid tokens (parts [kCacheParts][2]); then prev = h
void launch_cache_score(const float* h, float* prev, int d, const CacheTok& tk, float* parts, hipStream_t s);
// the decision of one evaluation from the partial sums (reads the token count for the
// middle blocks from tk.n_dev, or uses tk.cap)
void launch_cache_decide(const float* parts, int32_t* state, int forced, float threshold, float budget,
                         int max_consecutive, int max_cached, const CacheTok& tk, hipStream_t s);
// after the middle blocks: compute flag set -> res = h - prev; else h += res
void launch_cache_apply(float* h, float* res, const float* prev, int d, const CacheTok& tk, const int32_t* state,
                        hipStream_t s);
void launch_copy_i32(const int32_t* src, int32_t* dst, int n, hipStream_t s);
// Evaluation times of a sampling call: grid kind 0 uniform, 1 quadratic, 2 trailing,
// 3 native subsequence of N uniform steps; per_step evaluations per step (1 Euler,
// 2 midpoint). The host and the timestep-embedding kernel use the same function.
double host_grid_time(int kind, int S, int N, int k);
double host_eval_time(int kind, int S, int N, int per_step, int j);
// temb [n_eval, F] = sinusoidal embedding of every evaluation time (phase in fp64)
void launch_timestep_embedding(float* temb, int n_eval, int F, int kind, int S, int N, int per_step, hipStream_t s);
// Key validity of every request's sequence (P prefix keys, then Tx = T - P frames):
// kv_len_out[r] = min(kv_len_in[r], T) if kv_len_in is given, else P + 1 + the
// index of the last valid frame (P if none); kvalid[r, t] = t < kv_len_out[r] and
// (t < P or mask[r, t - P] != 0 or no mask), zero for t in [T, Tp); tile_full[r, i]
// = 1 when keys 64i .. 64i+63 are all valid.
// Rotary table tab[t, i] = (cos, sin)(t * base^(-2i / hd)), t < T, i < hd / 2 (angles in fp64).
void launch_rope_table(float* tab, int T, int hd, double base, hipStream_t s);
// In-place rotary embedding of the q and k columns (0 .. 2d) of fp32 rows qkv [n_tok, ld],
// token m at position m % T; n_dev optional device token count.
void launch_rope_f32(float* qkv, long long n_tok, int ld, int T, int d, int hd, const float* tab,
                     const int32_t* n_dev, hipStream_t s);
// act[m, 16b + i] = SiLU(gu[m, 32b + i]) * gu[m, 32b + 16 + i] (fp32, the interleaved gate-up rows).
void launch_swiglu_f32(const float* gu, float* act, long long M, int f, const int32_t* n_dev, hipStream_t s);
// out[i] = bf16(SiLU(in[i])).
void launch_silu_bf16(const float* in, bf16* out, long long n, hipStream_t s);
// Context of every branch row: xctx[b*R + r] = b >= cond0 ? cond[r] : 0 (per_row floats each).
void launch_expand_context(const float* cond, float* xctx, int R, int nb, int cond0, long long per_row,
                           hipStream_t s);
void launch_key_prep(const uint8_t* mask, int mask_stride, const int32_t* kv_len_in, int R, int P,
                     int T, int Tp, int32_t* kv_len_out, uint8_t* kvalid, uint8_t* tile_full,
                     hipStream_t s);
// Packed row layout of a variable-length batch: rows are branch-major (row =
// b*R + r) and row i holds kv_len[r] tokens rounded up to a multiple of 8 (none
// when b < nb - 1 and lane_off[r] != 0, lane_off optional); row_off[N + 1] prefix
// offsets (row_off[N] = total tokens) and tok_row[t] = row of packed token t (-1
// past the end, up to NTmax).
void launch_pack_rows(const int32_t* kv_len, const int32_t* lane_off, int R, int nb, int NTmax, int32_t* row_off,
                      int32_t* tok_row, hipStream_t s);
// cvec[(k*nc + ci), :] = ct[k, :] + (spk ? (ci == 0 ? bs : spkproj[ci-1]) : 0); with
// silu_bf16 set, silu of that vector rounded to bf16 goes there instead (the A operand
// of the modulation GEMM on matrix cores)
void launch_assemble_cvec(const float* ct, const float* bs, const float* spkproj, int S, int nc,
                          int d, float* cvec, hipStream_t s, bf16* silu_bf16 = nullptr);
// prefix tokens of every branch row: h[(b*R + r)*T + p] = b >= cond_branch0 ? cproj[r*P + p] : bias
void launch_prefix_init(const float* cproj, const float* bias, int R, int nb, int cond_branch0,
                        int P, int T, int d, float* h, hipStream_t s);

}  // namespace cfm
