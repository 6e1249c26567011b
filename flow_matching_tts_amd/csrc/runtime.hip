// Host runtime behind include/cfm.h: argument validation, weight manifest,
// workspace carve-up and the launch sequence of one sampling call.
//
// A call enqueues, on the caller's stream and with no host synchronisation:
//   set-up (once per call): out <- x0; per-request key lengths; timestep
//     embeddings of every step; timestep MLP; speaker projection; the adaLN
//     modulation vectors of every step and layer; the projection of the
//     condition features (constant over steps). VoiceHub's "Recommended
//     optimization boundaries" asks to cache masks and conditioning outside the
//     repeated estimator; this is that hoisting.
//   per Euler step: input projection into every branch row, L DiT blocks
//     (adaLN-LN, QKV GEMM, masked attention, out-proj GEMM + gated residual,
//     adaLN-LN, FC1 GEMM + GELU, FC2 GEMM + gated residual), final adaLN-LN,
//     output projection to the branch velocities, fused CFG combine + Euler.
// The step loop never reads device memory back: the step size and guidance
// weights are kernel arguments computed on the host (the vLLM-Omni blog's
// "CFM/LocDiT decode-tail batching" section removes exactly such per-step
// host syncs from its Euler loop).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/cfm.h"
#include "kernels.h"

using namespace cfm;

namespace {

thread_local std::string g_detail;

cfm_status fail(cfm_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
cfm_status fail(cfm_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_detail = buf;
    return s;
}

constexpr long long kMaxOperandBytes = (1LL << 31) - 256;
constexpr int kSwigluGroup = 16;          // gate/up row interleave of the fused SwiGLU FC1 (half a 32-column block)
constexpr size_t kSplitKTokens = 4096;   // batches up to this many tokens may split K

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline long long round8(long long v) { return (v + 7) / 8 * 8; }

cfm_status check_config(const cfm_config* c) {
    if (c == nullptr) return fail(CFM_E_NULL, "config is NULL");
    if (c->n_layers < 0 || c->d_model <= 0 || c->n_heads <= 0 || c->ffn_dim <= 0 ||
        c->latent_dim <= 0 || c->cond_dim < 0 || c->n_prefix < 0 || c->spk_dim < 0 ||
        c->t_freq_dim <= 0 || c->max_requests < 0 || c->max_frames < 0 || c->max_steps < 0)
        return fail(CFM_E_VALUE, "negative or zero size in config");
    if (c->dtype != CFM_F32 && c->dtype != CFM_BF16) return fail(CFM_E_UNSUPPORTED, "dtype %d", c->dtype);
    if (c->cond_mode != CFM_COND_CHANNEL && c->cond_mode != CFM_COND_PREFIX && c->cond_mode != CFM_COND_CROSS)
        return fail(CFM_E_UNSUPPORTED, "cond_mode %d", c->cond_mode);
    if (c->norm != CFM_NORM_LAYER && c->norm != CFM_NORM_RMS) return fail(CFM_E_UNSUPPORTED, "norm %d", c->norm);
    if (c->mlp != CFM_MLP_GELU && c->mlp != CFM_MLP_SWIGLU) return fail(CFM_E_UNSUPPORTED, "mlp %d", c->mlp);
    if (c->mlp == CFM_MLP_SWIGLU && c->ffn_dim % 16)
        return fail(CFM_E_UNSUPPORTED, "the SwiGLU MLP needs ffn_dim %% 16 == 0");
    if (c->rope && !(std::isfinite(c->rope_base) && c->rope_base > 0.0f))
        return fail(CFM_E_VALUE, "rope_base must be positive and finite");
    if (c->n_branches < 1 || c->n_branches > 3) return fail(CFM_E_UNSUPPORTED, "n_branches %d", c->n_branches);
    if (c->d_model % c->n_heads) return fail(CFM_E_UNSUPPORTED, "d_model %% n_heads != 0");
    const int hd = c->d_model / c->n_heads;
    if (c->d_model % 8 || c->ffn_dim % 8) return fail(CFM_E_UNSUPPORTED, "d_model and ffn_dim must be multiples of 8");
    if (c->d_model > 4096) return fail(CFM_E_UNSUPPORTED, "d_model above 4096");
    if (c->latent_dim % 4 || c->cond_dim % 4) return fail(CFM_E_UNSUPPORTED, "latent_dim and cond_dim must be multiples of 4");
    if (c->t_freq_dim % 8) return fail(CFM_E_UNSUPPORTED, "t_freq_dim must be a multiple of 8");
    if (c->spk_dim % 4) return fail(CFM_E_UNSUPPORTED, "spk_dim must be a multiple of 4");
    if (c->dtype == CFM_BF16 && hd != 64) return fail(CFM_E_UNSUPPORTED, "bf16 path needs head_dim 64 (got %d)", hd);
    if (c->dtype == CFM_F32 && (hd % 4 || hd > 64)) return fail(CFM_E_UNSUPPORTED, "fp32 path needs head_dim %% 4 == 0 and <= 64");
    {
        // the matrix-core GEMMs address each operand with 32-bit byte offsets
        const long long es = c->dtype == CFM_BF16 ? 2 : 4;
        const long long P = c->cond_mode == CFM_COND_PREFIX ? c->n_prefix : 0;
        const long long tokens = (long long)c->n_branches * c->max_requests * round8(c->max_frames + P);
        const long long wide = std::max<long long>(3LL * c->d_model, 2LL * c->ffn_dim);
        const long long cond_rows = (long long)c->max_requests * (c->cond_mode == CFM_COND_CHANNEL ? c->max_frames : c->n_prefix);
        const long long ctx_rows = c->cond_mode == CFM_COND_CROSS ? (long long)c->n_branches * c->max_requests * c->n_prefix : 0;
        if (tokens * wide * es >= kMaxOperandBytes || ctx_rows * 2LL * c->d_model * es >= kMaxOperandBytes ||
            ctx_rows * c->cond_dim * 4 >= kMaxOperandBytes ||
            (long long)c->max_requests * c->max_frames * c->latent_dim * 4 >= kMaxOperandBytes ||
            cond_rows * std::max(c->cond_dim, c->latent_dim) * 4 >= kMaxOperandBytes)
            return fail(CFM_E_UNSUPPORTED, "capacity too large: an activation operand would exceed 2 GiB");
    }
    {
        // launch limits of the kernels a call enqueues: rejected here so that a call
        // never fails half-way through its launch sequence
        const long long P = c->cond_mode == CFM_COND_PREFIX ? c->n_prefix : 0;
        const long long rows = (long long)c->n_branches * c->max_requests;
        if (rows > 65535 || c->n_heads > 65535)
            return fail(CFM_E_UNSUPPORTED, "n_branches * max_requests and n_heads must be <= 65535 (attention grid)");
        if (c->max_steps > 65535) return fail(CFM_E_UNSUPPORTED, "max_steps must be <= 65535");
        if (c->spk_dim > 0 && c->max_requests + 1LL > 65535)
            return fail(CFM_E_UNSUPPORTED, "max_requests must be < 65535 with a speaker path");
        if ((long long)c->max_requests * P > 65535)
            return fail(CFM_E_UNSUPPORTED, "max_requests * n_prefix must be <= 65535");
        if (c->dtype == CFM_BF16 && !attention_bf16_fits(c->max_frames + P))
            return fail(CFM_E_UNSUPPORTED, "max_frames + n_prefix = %lld: the attention key tables exceed LDS",
                        (long long)c->max_frames + P);
        if (c->dtype == CFM_BF16 && c->cond_mode == CFM_COND_CROSS && !attention_bf16_fits(c->n_prefix))
            return fail(CFM_E_UNSUPPORTED, "n_prefix = %d context keys exceed the attention's LDS tables", c->n_prefix);
    }
    if (c->cond_mode == CFM_COND_PREFIX) {
        if (c->n_prefix <= 0) return fail(CFM_E_UNSUPPORTED, "prefix mode needs n_prefix > 0");
        if (c->cond_dim != c->latent_dim) return fail(CFM_E_UNSUPPORTED, "prefix mode needs cond_dim == latent_dim");
    } else if (c->cond_mode == CFM_COND_CROSS) {
        if (c->n_prefix <= 0) return fail(CFM_E_UNSUPPORTED, "cross mode needs n_prefix (context tokens) > 0");
        if (c->cond_dim <= 0) return fail(CFM_E_UNSUPPORTED, "cross mode needs cond_dim > 0");
    } else {
        if (c->n_prefix != 0) return fail(CFM_E_UNSUPPORTED, "channel mode needs n_prefix == 0");
        if (c->cond_dim <= 0) return fail(CFM_E_UNSUPPORTED, "channel mode needs cond_dim > 0");
    }
    return CFM_OK;
}

struct Slot {
    long long off = -1;   // bytes
    int ld = 0;           // elements
};

struct Manifest {
    std::vector<cfm_tensor_desc> d;
    size_t bytes = 0;
};

// Builds the slot list; the same function fixes the offsets for the binding
// (through cfm_weight_manifest) and for the runtime (through find()).
Manifest build_manifest(const cfm_config& c) {
    Manifest m;
    const int mat_dt = c.dtype;
    const size_t mat_es = c.dtype == CFM_BF16 ? 2 : 4;
    size_t off = 0;
    auto add = [&](const char* name, long long row0, long long col0, long long rows, long long cols,
                   bool vec, bool packed, int interleave = 0) {
        cfm_tensor_desc t;
        std::memset(&t, 0, sizeof t);
        std::snprintf(t.name, sizeof t.name, "%s", name);
        t.row0 = row0; t.col0 = col0; t.rows = rows; t.cols = cols;
        t.interleave = interleave;
        t.dtype = vec ? CFM_F32 : mat_dt;
        t.ld = vec ? cols : round8(cols);
        const size_t es = vec ? 4 : mat_es;
        if (!packed) off = align_up(off, 256);
        t.offset = (long long)off;
        off += (size_t)rows * t.ld * es;
        m.d.push_back(t);
    };
    const long long d = c.d_model, f = c.ffn_dim, C = c.latent_dim;
    char nm[64];
    add("t_embed.fc1.weight", 0, 0, d, c.t_freq_dim, false, false);
    add("t_embed.fc1.bias", 0, 0, 1, d, true, false);
    add("t_embed.fc2.weight", 0, 0, d, d, false, false);
    add("t_embed.fc2.bias", 0, 0, 1, d, true, false);
    if (c.spk_dim > 0) {
        add("spk_proj.weight", 0, 0, d, c.spk_dim, false, false);
        add("spk_proj.bias", 0, 0, 1, d, true, false);
    }
    add("in_proj.weight", 0, 0, d, C, false, false);
    if (c.cond_mode == CFM_COND_CHANNEL) add("in_proj.weight", 0, C, d, c.cond_dim, false, false);
    add("in_proj.bias", 0, 0, 1, d, true, false);
    // all adaLN projections back to back: one GEMM produces every layer's modulation
    for (int l = 0; l < c.n_layers; ++l) {
        std::snprintf(nm, sizeof nm, "blocks.%d.ada.weight", l);
        add(nm, 0, 0, 6 * d, d, false, l > 0);
    }
    add("final.ada.weight", 0, 0, 2 * d, d, false, c.n_layers > 0);
    for (int l = 0; l < c.n_layers; ++l) {
        std::snprintf(nm, sizeof nm, "blocks.%d.ada.bias", l);
        add(nm, 0, 0, 1, 6 * d, true, l > 0);
    }
    add("final.ada.bias", 0, 0, 1, 2 * d, true, c.n_layers > 0);
    // SwiGLU: the fused gate-up FC1 (2f rows, gate rows first) is stored interleaved
    // in groups of 16, so every 32-column output block pairs 16 gate and 16 up columns
    const bool swiglu = c.mlp == CFM_MLP_SWIGLU;
    for (int l = 0; l < c.n_layers; ++l) {
        const char* parts[4] = {"qkv", "proj", "fc1", "fc2"};
        const long long rows[4] = {3 * d, d, swiglu ? 2 * f : f, d};
        const long long cols[4] = {d, d, d, f};
        for (int i = 0; i < 4; ++i) {
            const int il = swiglu && i == 2 ? kSwigluGroup : 0;
            std::snprintf(nm, sizeof nm, "blocks.%d.%s.weight", l, parts[i]);
            add(nm, 0, 0, rows[i], cols[i], false, false, il);
            std::snprintf(nm, sizeof nm, "blocks.%d.%s.bias", l, parts[i]);
            add(nm, 0, 0, 1, rows[i], true, false, il);
        }
        if (c.cond_mode == CFM_COND_CROSS) {
            const char* xp[3] = {"q", "kv", "out"};
            const long long xr[3] = {d, 2 * d, d};
            const long long xc[3] = {d, c.cond_dim, d};
            for (int i = 0; i < 3; ++i) {
                std::snprintf(nm, sizeof nm, "blocks.%d.xattn.%s.weight", l, xp[i]);
                add(nm, 0, 0, xr[i], xc[i], false, false);
                std::snprintf(nm, sizeof nm, "blocks.%d.xattn.%s.bias", l, xp[i]);
                add(nm, 0, 0, 1, xr[i], true, false);
            }
        }
    }
    add("final.out.weight", 0, 0, C, d, false, false);
    add("final.out.bias", 0, 0, 1, C, true, false);
    m.bytes = align_up(off, 256);
    return m;
}

Slot find(const Manifest& m, const char* name, long long col0 = 0) {
    for (const auto& t : m.d)
        if (std::strcmp(t.name, name) == 0 && t.col0 == col0) return Slot{t.offset, (int)t.ld};
    return Slot{};
}

struct Layout {   // workspace regions, byte offsets
    size_t h, act, big, vt, v, cproj, temb, tpre, ct, spkproj, cvec, mod, kvlen, kvalid, tfull, rowoff, tokrow,
        xmid, lanes, probe, resid, cstate, cparts, splitk, rope, gu, unit, xctx, xk, xvt, xkvlen, xkvalid, xtfull,
        total;
};

inline long long round64(long long v) { return (v + 63) / 64 * 64; }

Layout plan_workspace(const cfm_config& c) {
    const size_t es = c.dtype == CFM_BF16 ? 2 : 4;
    const size_t Rm = c.max_requests, Tx = c.max_frames, S = c.max_steps;
    const size_t P = c.cond_mode == CFM_COND_PREFIX ? c.n_prefix : 0;
    const size_t N = (size_t)c.n_branches * Rm, d = c.d_model;
    // packed layout of masked batches (bf16 path, frame-aligned condition): rows
    // are rounded up to 8 tokens, so token buffers hold N * round8(T) tokens
    const bool packable = c.dtype == CFM_BF16 && c.cond_mode != CFM_COND_PREFIX;
    const size_t T = Tx + P, TT = packable ? (T + 7) / 8 * 8 : T;
    const size_t Tc = c.cond_mode == CFM_COND_PREFIX ? P : c.cond_mode == CFM_COND_CHANNEL ? Tx : 0;
    const size_t nc = 1 + (c.spk_dim > 0 ? Rm : 0);
    const size_t ML = (6 * (size_t)c.n_layers + 2) * d;
    const size_t wide = std::max<size_t>(3 * d, c.ffn_dim);
    const bool cross = c.cond_mode == CFM_COND_CROSS;
    const size_t Tk = cross ? c.n_prefix : 0, Tkp = (size_t)round64(Tk), L_ = c.n_layers;
    Layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
    L.h = take(N * TT * d * 4);
    L.act = take(N * TT * d * es);
    L.big = take(N * TT * wide * es);
    // bf16 path: V transposed per head, [rows, H, 64, T rounded up to 64]
    L.vt = take(c.dtype == CFM_BF16 ? N * d * (size_t)round64(T) * 2 : 0);
    L.v = take(N * Tx * c.latent_dim * 4);
    L.cproj = take(Rm * Tc * d * 4);
    L.temb = take(S * c.t_freq_dim * 4);
    L.tpre = take(S * d * 4);
    L.ct = take(S * d * 4);
    L.spkproj = take(c.spk_dim > 0 ? Rm * d * 4 : 0);
    L.cvec = take(S * nc * d * 4);
    L.mod = take(S * nc * ML * 4);
    L.kvlen = take(Rm * 4);
    L.kvalid = take(Rm * (size_t)round64(T));           // per-key validity bytes
    L.tfull = take(Rm * (size_t)round64(T) / 64);       // per-64-key-tile "all valid" bytes
    L.rowoff = take(packable ? (N + 1) * 4 : 0);
    L.tokrow = take(packable ? N * TT * 4 : 0);
    L.xmid = take(Rm * Tx * c.latent_dim * 4);          // midpoint solver: x at the half step
    L.lanes = take(2 * 3 * Rm * 4);                      // adaptive guidance: two states [count | off | guided]
    L.probe = take(N * TT * d * 4);                      // block-residual cache: previous probe
    L.resid = take(N * TT * d * 4);                      // ... and the saved middle-block residual
    L.cstate = take(8 * 4);
    L.cparts = take(kCacheParts * 2 * 4);
    // split-K partial products of the gated-residual GEMMs (N = d) of small batches:
    // up to 4 fp32 planes of [tokens, d]; large batches never split
    L.splitk = take(c.dtype == CFM_BF16 && N * TT <= kSplitKTokens ? 4 * N * TT * d * 4 : 0);
    // rotary table: (cos, sin) of every token position and pair index (positions up to
    // the row capacity rounded to 8: the packed layout's alignment tokens have some)
    L.rope = take(c.rope ? round8(T) * (d / c.n_heads / 2) * 2 * 4 : 0);
    // fp32 SwiGLU: the GEMM's interleaved gate-up output before the SwiGLU kernel
    L.gu = take(c.dtype == CFM_F32 && c.mlp == CFM_MLP_SWIGLU ? N * TT * 2 * c.ffn_dim * 4 : 0);
    L.unit = take(2 * d * 4);                            // d zeros then d ones (unmodulated norm, ungated residual)
    // cross-attention: the context of every branch row, then per layer its keys and
    // values (bf16: K [rows, Tk, d] and V^T [rows, H, 64, Tk rounded to 64]; fp32:
    // [rows, Tk, 2d] key | value rows), and the key tables of the Tk context keys
    L.xctx = take(cross ? N * Tk * c.cond_dim * 4 : 0);
    L.xk = take(cross ? L_ * N * Tk * d * (c.dtype == CFM_BF16 ? 2 : 8) : 0);
    L.xvt = take(cross && c.dtype == CFM_BF16 ? L_ * N * d * Tkp * 2 : 0);
    L.xkvlen = take(cross ? Rm * 4 : 0);
    L.xkvalid = take(cross ? Rm * Tkp : 0);
    L.xtfull = take(cross ? Rm * Tkp / 64 : 0);
    L.total = off;
    return L;
}

}  // namespace

struct cfm_ctx {
    cfm_config cfg;
    const char* w = nullptr;
    char* ws = nullptr;
    size_t ws_bytes = 0;
    Manifest man;
    Layout lay;
    Slot t1w, t1b, t2w, t2b, spkw, spkb, inxw, incw, inb, adaw, adab, outw, outb;
    struct LayerW { Slot qkvw, qkvb, projw, projb, fc1w, fc1b, fc2w, fc2b, xqw, xqb, xkvw, xkvb, xow, xob; };
    std::vector<LayerW> layers;
    // kernel timing
    int prof_class = -1, prof_cap = 0, prof_used = 0, prof_dropped = 0;
    std::vector<hipEvent_t> ev0, ev1;
};

namespace {

template <typename T> const T* wp(const cfm_ctx* c, Slot s) { return (const T*)(c->w + s.off); }
template <typename T> T* wsp(const cfm_ctx* c, size_t off) { return (T*)(c->ws + off); }

// Runs `fn` (one kernel launch) bracketed by timing events when its class is profiled.
template <typename F>
void timed(cfm_ctx* c, int cls, hipStream_t s, F&& fn) {
    if (cls == c->prof_class && c->prof_class >= 0) {
        if (c->prof_used < c->prof_cap) {
            (void)hipEventRecord(c->ev0[c->prof_used], s);
            fn();
            (void)hipEventRecord(c->ev1[c->prof_used], s);
            ++c->prof_used;
            return;
        }
        ++c->prof_dropped;
    }
    fn();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" {

const char* cfm_status_string(cfm_status s) {
    switch (s) {
        case CFM_OK: return "ok";
        case CFM_E_NULL: return "null pointer";
        case CFM_E_SHAPE: return "bad shape or layout";
        case CFM_E_CAPACITY: return "above create-time capacity";
        case CFM_E_VALUE: return "bad value";
        case CFM_E_UNSUPPORTED: return "unsupported configuration";
        case CFM_E_WORKSPACE: return "workspace too small";
        case CFM_E_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* cfm_last_error_detail(void) { return g_detail.c_str(); }

size_t cfm_weights_bytes(const cfm_config* cfg) {
    if (check_config(cfg) != CFM_OK) return 0;
    return build_manifest(*cfg).bytes;
}

size_t cfm_workspace_bytes(const cfm_config* cfg) {
    if (check_config(cfg) != CFM_OK) return 0;
    return plan_workspace(*cfg).total;
}

int cfm_weight_manifest(const cfm_config* cfg, cfm_tensor_desc* out, int cap) {
    cfm_status st = check_config(cfg);
    if (st != CFM_OK) return -(int)st;
    if (cap > 0 && out == nullptr) return -(int)fail(CFM_E_NULL, "manifest output is NULL");
    Manifest m = build_manifest(*cfg);
    for (int i = 0; i < cap && i < (int)m.d.size(); ++i) out[i] = m.d[i];
    return (int)m.d.size();
}

cfm_status cfm_create(const cfm_config* cfg, const void* weights, void* workspace,
                      size_t workspace_bytes, cfm_ctx** out_ctx) {
    if (out_ctx == nullptr) return fail(CFM_E_NULL, "out_ctx is NULL");
    *out_ctx = nullptr;
    cfm_status st = check_config(cfg);
    if (st != CFM_OK) return st;
    if (weights == nullptr) return fail(CFM_E_NULL, "weights is NULL");
    Layout lay = plan_workspace(*cfg);
    if (lay.total > 0 && workspace == nullptr) return fail(CFM_E_NULL, "workspace is NULL");
    if (workspace_bytes < lay.total)
        return fail(CFM_E_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, lay.total);
    if (((uintptr_t)weights & 255) || ((uintptr_t)workspace & 255))
        return fail(CFM_E_SHAPE, "weights and workspace must be 256-byte aligned");
    cfm_ctx* c = new (std::nothrow) cfm_ctx;
    if (c == nullptr) return fail(CFM_E_VALUE, "host allocation failed");
    c->cfg = *cfg;
    c->w = (const char*)weights;
    c->ws = (char*)workspace;
    c->ws_bytes = workspace_bytes;
    c->man = build_manifest(*cfg);
    c->lay = lay;
    c->t1w = find(c->man, "t_embed.fc1.weight");
    c->t1b = find(c->man, "t_embed.fc1.bias");
    c->t2w = find(c->man, "t_embed.fc2.weight");
    c->t2b = find(c->man, "t_embed.fc2.bias");
    if (cfg->spk_dim > 0) {
        c->spkw = find(c->man, "spk_proj.weight");
        c->spkb = find(c->man, "spk_proj.bias");
    }
    c->inxw = find(c->man, "in_proj.weight", 0);
    if (cfg->cond_mode == CFM_COND_CHANNEL) c->incw = find(c->man, "in_proj.weight", cfg->latent_dim);
    c->inb = find(c->man, "in_proj.bias");
    c->adaw = cfg->n_layers > 0 ? find(c->man, "blocks.0.ada.weight") : find(c->man, "final.ada.weight");
    c->adab = cfg->n_layers > 0 ? find(c->man, "blocks.0.ada.bias") : find(c->man, "final.ada.bias");
    c->outw = find(c->man, "final.out.weight");
    c->outb = find(c->man, "final.out.bias");
    char nm[64];
    for (int l = 0; l < cfg->n_layers; ++l) {
        cfm_ctx::LayerW L;
        auto s = [&](const char* part, const char* kind) {
            std::snprintf(nm, sizeof nm, "blocks.%d.%s.%s", l, part, kind);
            return find(c->man, nm);
        };
        L.qkvw = s("qkv", "weight"); L.qkvb = s("qkv", "bias");
        L.projw = s("proj", "weight"); L.projb = s("proj", "bias");
        L.fc1w = s("fc1", "weight"); L.fc1b = s("fc1", "bias");
        L.fc2w = s("fc2", "weight"); L.fc2b = s("fc2", "bias");
        if (cfg->cond_mode == CFM_COND_CROSS) {
            L.xqw = s("xattn.q", "weight"); L.xqb = s("xattn.q", "bias");
            L.xkvw = s("xattn.kv", "weight"); L.xkvb = s("xattn.kv", "bias");
            L.xow = s("xattn.out", "weight"); L.xob = s("xattn.out", "bias");
        }
        c->layers.push_back(L);
    }
    *out_ctx = c;
    return CFM_OK;
}

void cfm_destroy(cfm_ctx* c) {
    if (c == nullptr) return;
    for (auto e : c->ev0) (void)hipEventDestroy(e);
    for (auto e : c->ev1) (void)hipEventDestroy(e);
    delete c;
}

cfm_status cfm_profile_enable(cfm_ctx* c, int kernel_class, int capacity) {
    if (c == nullptr) return fail(CFM_E_NULL, "ctx is NULL");
    if (kernel_class < 0 || kernel_class >= CFM_K_COUNT || capacity < 0)
        return fail(CFM_E_VALUE, "bad kernel class or capacity");
    while ((int)c->ev0.size() < capacity) {
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) return fail(CFM_E_HIP, "hipEventCreate failed");
        if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return fail(CFM_E_HIP, "hipEventCreate failed"); }
        c->ev0.push_back(a);
        c->ev1.push_back(b);
    }
    c->prof_class = kernel_class;
    c->prof_cap = capacity;
    c->prof_used = 0;
    c->prof_dropped = 0;
    return CFM_OK;
}

cfm_status cfm_profile_read(cfm_ctx* c, double* total_ms, int* launches, int* dropped) {
    if (c == nullptr || total_ms == nullptr || launches == nullptr || dropped == nullptr)
        return fail(CFM_E_NULL, "NULL argument");
    double sum = 0.0;
    for (int i = 0; i < c->prof_used; ++i) {
        if (hipEventSynchronize(c->ev1[i]) != hipSuccess) return fail(CFM_E_HIP, "hipEventSynchronize failed");
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, c->ev0[i], c->ev1[i]) != hipSuccess)
            return fail(CFM_E_HIP, "hipEventElapsedTime failed");
        sum += ms;
    }
    *total_ms = sum;
    *launches = c->prof_used;
    *dropped = c->prof_dropped;
    return CFM_OK;
}

cfm_status cfm_profile_disable(cfm_ctx* c) {
    if (c == nullptr) return fail(CFM_E_NULL, "ctx is NULL");
    c->prof_class = -1;
    return CFM_OK;
}

namespace {

struct Opts {                  // validated cfm_sample_options
    int schedule = CFM_SCHEDULE_UNIFORM, native = 0, solver = CFM_SOLVER_EULER, mode = CFM_GUIDANCE_FULL;
    double start = 0.0, end = 1.0;
    float threshold = 0.0f;
    int warmup = 0, patience = 1;
    int32_t* guided_out = nullptr;
    bool cache = false;
    int c_front = 1, c_back = 1, c_warmup = 0, c_consec = 0, c_max = -1;
    float c_threshold = 0.0f, c_budget = 0.0f;
    const uint8_t* c_force = nullptr;
    int32_t* c_hits = nullptr;
};

cfm_status read_options(const cfm_sample_options* o, int S, Opts& out) {
    out = Opts{};
    if (o == nullptr) return CFM_OK;
    if (o->schedule < CFM_SCHEDULE_UNIFORM || o->schedule > CFM_SCHEDULE_NATIVE)
        return fail(CFM_E_VALUE, "schedule %d", o->schedule);
    if (o->solver != CFM_SOLVER_EULER && o->solver != CFM_SOLVER_MIDPOINT) return fail(CFM_E_VALUE, "solver %d", o->solver);
    if (o->guidance_mode < CFM_GUIDANCE_FULL || o->guidance_mode > CFM_GUIDANCE_ADAPTIVE)
        return fail(CFM_E_VALUE, "guidance_mode %d", o->guidance_mode);
    if (o->schedule == CFM_SCHEDULE_NATIVE && (o->native_steps < S || o->native_steps <= 0))
        return fail(CFM_E_VALUE, "native schedule: native_steps %d must be >= n_steps %d and > 0", o->native_steps, S);
    if (o->guidance_mode == CFM_GUIDANCE_INTERVAL && (!std::isfinite(o->interval_start) || !std::isfinite(o->interval_end)))
        return fail(CFM_E_VALUE, "guidance interval must be finite");
    if (o->guidance_mode == CFM_GUIDANCE_ADAPTIVE) {
        if (std::isnan(o->adaptive_threshold) || o->adaptive_threshold < 0.0f)
            return fail(CFM_E_VALUE, "adaptive threshold must be >= 0 (infinity allowed)");
        if (o->adaptive_warmup < 0 || o->adaptive_patience < 1)
            return fail(CFM_E_VALUE, "adaptive warmup must be >= 0 and patience >= 1");
    }
    out.schedule = o->schedule;
    out.native = o->native_steps;
    out.solver = o->solver;
    out.mode = o->guidance_mode;
    out.start = o->interval_start;
    out.end = o->interval_end;
    out.threshold = o->adaptive_threshold;
    out.warmup = o->adaptive_warmup;
    out.patience = o->adaptive_patience;
    out.guided_out = o->guided_evals;
    out.c_hits = o->cache_hits;
    if (o->cache != 0) {
        if (o->cache != 1) return fail(CFM_E_VALUE, "cache %d", o->cache);
        if (o->guidance_mode != CFM_GUIDANCE_FULL)
            return fail(CFM_E_UNSUPPORTED, "the block-residual cache needs guidance_mode FULL");
        if (o->cache_front < 1 || o->cache_back < 0 || o->cache_warmup < 0 || o->cache_max_consecutive < 0 ||
            o->cache_max_cached < -1)
            return fail(CFM_E_VALUE, "cache block counts / warm-up / limits out of range");
        if (std::isnan(o->cache_threshold) || o->cache_threshold < 0.0f || std::isnan(o->cache_budget) ||
            o->cache_budget < 0.0f)
            return fail(CFM_E_VALUE, "cache threshold and budget must be >= 0 (infinity allowed)");
        out.cache = true;
        out.c_front = o->cache_front;
        out.c_back = o->cache_back;
        out.c_warmup = o->cache_warmup;
        out.c_consec = o->cache_max_consecutive;
        out.c_max = o->cache_max_cached;
        out.c_threshold = o->cache_threshold;
        out.c_budget = o->cache_budget;
        out.c_force = o->cache_force;
    }
    return CFM_OK;
}

}  // namespace

cfm_status cfm_sample(cfm_ctx* c, const float* x0, const float* cond, const float* spk,
                      const uint8_t* frame_mask, int R, int Tx, int S,
                      const float* guidance, float* out, void* stream) {
    return cfm_sample_ex(c, x0, cond, spk, frame_mask, R, Tx, S, guidance, nullptr, out, stream);
}

cfm_status cfm_sample_ex(cfm_ctx* c, const float* x0, const float* cond, const float* spk,
                         const uint8_t* frame_mask, int R, int Tx, int S, const float* guidance,
                         const cfm_sample_options* options, float* out, void* stream) {
    if (c == nullptr) return fail(CFM_E_NULL, "ctx is NULL");
    const cfm_config& g = c->cfg;
    if (R < 0 || Tx < 0 || S < 0) return fail(CFM_E_VALUE, "negative n_requests, n_frames or n_steps");
    Opts op;
    {
        cfm_status st = read_options(options, S, op);
        if (st != CFM_OK) return st;
    }
    const int per_step = op.solver == CFM_SOLVER_MIDPOINT ? 2 : 1;
    const long long n_eval_ll = (long long)S * per_step;
    if (R > g.max_requests || Tx > g.max_frames || n_eval_ll > g.max_steps)
        return fail(CFM_E_CAPACITY, "R=%d Tx=%d evaluations=%lld above capacity %d/%d/%d", R, Tx, n_eval_ll,
                    g.max_requests, g.max_frames, g.max_steps);
    const int n_eval = (int)n_eval_ll;
    const int nb = g.n_branches;
    if (nb > 1 && guidance == nullptr) return fail(CFM_E_NULL, "guidance is NULL");
    float scales[2] = {0.0f, 0.0f};
    for (int i = 0; i < nb - 1; ++i) {
        scales[i] = guidance[i];
        if (!std::isfinite(scales[i])) return fail(CFM_E_VALUE, "guidance scale %d is not finite", i);
    }
    if (R == 0 || Tx == 0) return CFM_OK;
    if (x0 == nullptr || out == nullptr || cond == nullptr) return fail(CFM_E_NULL, "x0, cond or out is NULL");
    if (g.spk_dim > 0 && spk == nullptr) return fail(CFM_E_NULL, "spk is NULL");
    if (!aligned16(x0) || !aligned16(out) || !aligned16(cond) || (spk && !aligned16(spk)))
        return fail(CFM_E_SHAPE, "x0, cond, spk and out must be 16-byte aligned");
    if ((op.guided_out != nullptr && ((uintptr_t)op.guided_out & 3)) || (op.c_hits && ((uintptr_t)op.c_hits & 3)))
        return fail(CFM_E_SHAPE, "guided_evals and cache_hits must be 4-byte aligned");
    const int C = g.latent_dim, d = g.d_model, L = g.n_layers;
    const size_t xbytes = (size_t)R * Tx * C * sizeof(float);
    {
        const char* a = (const char*)x0;
        const char* b = (const char*)out;
        if (a != b && a < b + xbytes && b < a + xbytes)
            return fail(CFM_E_SHAPE, "out partially overlaps x0 (only exact aliasing is allowed)");
    }
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();   // clear a stale error of an earlier, unrelated call
    if (out != x0 && hipMemcpyAsync(out, x0, xbytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return fail(CFM_E_HIP, "hipMemcpyAsync failed");
    int32_t* lanes = wsp<int32_t>(c, c->lay.lanes);   // two adaptive states of 3R ints
    if (S == 0) {
        if (op.guided_out) launch_fill_i32(op.guided_out, R, 0, s);
        if (op.c_hits) launch_fill_i32(op.c_hits, 1, 0, s);
        hipError_t e = hipGetLastError();
        return e == hipSuccess ? CFM_OK : fail(CFM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }

    const bool bf = g.dtype == CFM_BF16;
    const bool prefix = g.cond_mode == CFM_COND_PREFIX;
    const bool cross = g.cond_mode == CFM_COND_CROSS;
    const bool rms = g.norm == CFM_NORM_RMS, swiglu = g.mlp == CFM_MLP_SWIGLU;
    const int P = prefix ? g.n_prefix : 0;
    const int Tk = cross ? g.n_prefix : 0, Tkp = (int)round64(Tk);
    const int T = Tx + P, N = nb * R;
    const int nc = 1 + (g.spk_dim > 0 ? R : 0);
    const long long ML = (6LL * L + 2) * d;
    const int H = g.n_heads, hd = d / H, f = g.ffn_dim;
    const Layout& ly = c->lay;
    const bool adaptive = op.mode == CFM_GUIDANCE_ADAPTIVE && nb > 1;

    float* h = wsp<float>(c, ly.h);
    void* act = c->ws + ly.act;
    void* big = c->ws + ly.big;
    bf16* vt = (bf16*)(c->ws + ly.vt);
    const int Tp = (int)round64(T);
    float* vel = wsp<float>(c, ly.v);
    float* cproj = wsp<float>(c, ly.cproj);
    float* temb = wsp<float>(c, ly.temb);
    float* tpre = wsp<float>(c, ly.tpre);
    float* ct = wsp<float>(c, ly.ct);
    float* spkproj = wsp<float>(c, ly.spkproj);
    float* cvec = wsp<float>(c, ly.cvec);
    float* mod = wsp<float>(c, ly.mod);
    float* xmid = wsp<float>(c, ly.xmid);
    float* probe = wsp<float>(c, ly.probe);
    float* splitk = ly.splitk < ly.total && bf ? wsp<float>(c, ly.splitk) : nullptr;
    const long long splitk_floats = splitk ? (long long)((ly.total - ly.splitk) / 4) : 0;
    float* resid = wsp<float>(c, ly.resid);
    int32_t* cstate = wsp<int32_t>(c, ly.cstate);
    float* cparts = wsp<float>(c, ly.cparts);
    // block-residual cache: front blocks [0, cf), middle [cf, cb), back [cb, L)
    const int cf = std::min(op.c_front, L), cb = std::max(cf, L - op.c_back);
    const bool caching = op.cache && cf < cb;
    float* rope_tab = g.rope ? wsp<float>(c, ly.rope) : nullptr;
    float* gu = wsp<float>(c, ly.gu);
    float* unit = wsp<float>(c, ly.unit);               // d zeros, then d ones
    float* xctx = wsp<float>(c, ly.xctx);
    int32_t* xkvlen = wsp<int32_t>(c, ly.xkvlen);
    uint8_t* xkvalid = wsp<uint8_t>(c, ly.xkvalid);
    uint8_t* xtfull = wsp<uint8_t>(c, ly.xtfull);
    // per layer: keys (bf16 [N*Tk, d]; fp32 key|value rows [N*Tk, 2d]) and bf16 V^T
    auto xk_of = [&](int l) { return c->ws + ly.xk + (size_t)l * N * Tk * d * (bf ? 2 : 8); };
    auto xvt_of = [&](int l) { return (bf16*)(c->ws + ly.xvt) + (size_t)l * N * d * Tkp; };
    int32_t* kvlen = wsp<int32_t>(c, ly.kvlen);
    uint8_t* kvalid = wsp<uint8_t>(c, ly.kvalid);
    uint8_t* tfull = wsp<uint8_t>(c, ly.tfull);
    // The bf16 channel-condition path runs packed when a batch is masked (row b*R + r
    // keeps only its first kv_len[r] frames, up to the last valid one, rounded up to
    // 8 tokens; rows follow each other and every token-parallel kernel works on the
    // packed token count, read on the device) and under adaptive guidance (the rows
    // of a request whose unconditional lane has stopped hold no token, so they cost
    // nothing). The outputs are those of the padded layout: every operation but
    // attention is token-local, attention masks every key from kv_len on, and the
    // frames cut off are masked keys whose velocities are never used.
    const bool packable = bf && !prefix;   // channel or cross condition: frame-aligned rows
    const bool packed = packable && (frame_mask != nullptr || adaptive);
    const long long Trow = packed ? (T + 7) / 8 * 8 : T;     // token capacity per row
    int32_t* rowoff = packed ? wsp<int32_t>(c, ly.rowoff) : nullptr;
    int32_t* tokrow = packed ? wsp<int32_t>(c, ly.tokrow) : nullptr;

    // GEMM through matrix cores (bf16 sampler) or fp32 FMA (fp32 sampler)
    // (returns whether the GEMM also produced ep.ln_y, the next norm's output)
    auto gemm = [&](int cls, bool a_f32, const void* A, int lda, Slot w, int M, int Nn, int K, int epi,
                    const EpiParams& ep) -> bool {
        bool ln_done = false;
        timed(c, cls, s, [&] {
            if (bf) ln_done = launch_gemm_bf16(a_f32, epi, A, lda, wp<bf16>(c, w), w.ld, M, Nn, K, ep, s);
            else launch_gemm_simt(false, false, epi, (const float*)A, lda, c->w + w.off, w.ld, M, Nn, K, ep, s);
        });
        return ln_done;
    };
    // hoisted fp32-activation GEMMs against config-dtype weights
    auto hoisted = [&](bool silu_a, const float* A, int lda, Slot w, Slot b, int M, int Nn, int K,
                       float* o, long long ldo) {
        EpiParams ep;
        ep.bias = wp<float>(c, b);
        ep.out = o;
        ep.ldo = ldo;
        timed(c, CFM_K_HOISTED, s, [&] {
            launch_gemm_simt(bf, silu_a, EPI_F32, A, lda, c->w + w.off, w.ld, M, Nn, K, ep, s);
        });
    };

    // ---- set-up, once per call: key tables, the packed layout of a masked batch,
    // timestep embeddings and modulation vectors of every evaluation, the condition
    // projection (constant over steps)
    timed(c, CFM_K_HOISTED, s, [&] {
        launch_key_prep(frame_mask, Tx, nullptr, R, P, T, Tp, kvlen, kvalid, tfull, s);
        if (packed && !adaptive) launch_pack_rows(kvlen, nullptr, R, nb, (int)(N * Trow), rowoff, tokrow, s);
        if (adaptive) launch_fill_i32(lanes, 3 * R, 0, s);
        if (op.cache) launch_fill_i32(cstate, 8, 0, s);
    });
    timed(c, CFM_K_HOISTED, s, [&] {
        launch_timestep_embedding(temb, n_eval, g.t_freq_dim, op.schedule, S, op.native, per_step, s);
    });
    if (bf) {
        // bf16 sampler: the timestep MLP and the speaker projection on matrix cores
        // (operands rounded to bf16 like every GEMM operand of that path); the SiLU
        // between the two MLP layers writes the second layer's bf16 A operand into the
        // condition-vector region, which is only filled after that layer
        auto f32gemm = [&](bool a_f32, const void* A, int lda, Slot w, Slot b, int M, int K, float* o) {
            EpiParams ep;
            ep.bias = wp<float>(c, b);
            ep.out = o;
            ep.ldo = d;
            gemm(CFM_K_HOISTED, a_f32, A, lda, w, M, d, K, EPI_F32, ep);
        };
        f32gemm(true, temb, g.t_freq_dim, c->t1w, c->t1b, n_eval, g.t_freq_dim, tpre);
        timed(c, CFM_K_HOISTED, s, [&] { launch_silu_bf16(tpre, (bf16*)cvec, (long long)n_eval * d, s); });
        f32gemm(false, cvec, d, c->t2w, c->t2b, n_eval, d, ct);
        if (g.spk_dim > 0) f32gemm(true, spk, g.spk_dim, c->spkw, c->spkb, R, g.spk_dim, spkproj);
    } else {
        hoisted(false, temb, g.t_freq_dim, c->t1w, c->t1b, n_eval, d, g.t_freq_dim, tpre, d);
        hoisted(true, tpre, d, c->t2w, c->t2b, n_eval, d, d, ct, d);
        if (g.spk_dim > 0) hoisted(false, spk, g.spk_dim, c->spkw, c->spkb, R, d, g.spk_dim, spkproj, d);
    }
    // the modulation vectors of every evaluation, layer and conditioning vector: one
    // GEMM over the stacked adaLN weights (bf16 sampler: silu(c) rounded to bf16 as
    // the A operand on matrix cores, like every other GEMM operand of that path)
    bf16* cvec_silu = bf ? (bf16*)cvec : nullptr;
    timed(c, CFM_K_HOISTED, s, [&] {
        launch_assemble_cvec(ct, g.spk_dim > 0 ? wp<float>(c, c->spkb) : nullptr, spkproj, n_eval, nc, d, cvec, s,
                             cvec_silu);
    });
    if (bf) {
        EpiParams ep;
        ep.bias = wp<float>(c, c->adab);
        ep.out = mod;
        ep.ldo = ML;
        gemm(CFM_K_HOISTED, false, cvec_silu, d, c->adaw, n_eval * nc, (int)ML, d, EPI_F32, ep);
    } else {
        hoisted(true, cvec, d, c->adaw, c->adab, n_eval * nc, (int)ML, d, mod, ML);
    }
    {
        EpiParams ep;
        ep.bias = wp<float>(c, c->inb);
        ep.out = cproj;
        ep.ldo = d;
        if (prefix) gemm(CFM_K_HOISTED, true, cond, C, c->inxw, R * P, d, C, EPI_F32, ep);
        else if (!cross) gemm(CFM_K_HOISTED, true, cond, g.cond_dim, c->incw, R * Tx, d, g.cond_dim, EPI_F32, ep);
    }
    // block variants: the rotary table, the unit vectors, and the cross-attention keys
    // and values of every layer (the context is fixed over the steps)
    timed(c, CFM_K_HOISTED, s, [&] {
        if (rope_tab) launch_rope_table(rope_tab, (int)round8(T), hd, (double)g.rope_base, s);
        launch_fill_i32((int32_t*)unit, d, 0, s);
        launch_fill_i32((int32_t*)unit + d, d, 0x3f800000, s);   // 1.0f
    });
    if (cross) {
        timed(c, CFM_K_HOISTED, s, [&] {
            launch_key_prep(nullptr, Tk, nullptr, R, 0, Tk, Tkp, xkvlen, xkvalid, xtfull, s);
            launch_expand_context(cond, xctx, R, nb, nb == 1 ? 0 : 1, (long long)Tk * g.cond_dim, s);
        });
        for (int l = 0; l < L; ++l) {
            const auto& W = c->layers[l];
            EpiParams ek;
            ek.bias = wp<float>(c, W.xkvb);
            ek.out = xk_of(l);
            if (bf) {   // keys to [row token, d], values transposed per head
                ek.ldo = d; ek.vt = xvt_of(l); ek.H = H; ek.T = Tk; ek.Tp = Tkp; ek.d2 = d;
                gemm(CFM_K_HOISTED, true, xctx, g.cond_dim, W.xkvw, N * Tk, 2 * d, g.cond_dim, EPI_QKV, ek);
            } else {
                ek.ldo = 2 * d;
                gemm(CFM_K_HOISTED, true, xctx, g.cond_dim, W.xkvw, N * Tk, 2 * d, g.cond_dim, EPI_ACT, ek);
            }
        }
    }

    // One estimator evaluation at evaluation index j over nbe branch rows per
    // request (nbe = nb, or 1: the fully conditioned branch alone, an unguided
    // evaluation), latent input xl [R, Tx, C]; velocities to vel [nbe, R, Tx, C].
    // Rows are branch-major (row = b * R + r): with nbe = 1 the single row of a
    // request is row r, and in the packed layout rows 0 .. R - 1 are a prefix of the
    // layout, whose token count is row_off[R].
    // `fuse`, when given, is the guidance combine + Euler step that follows this
    // evaluation: where the layout allows (bf16, rows not packed, one or two branch
    // rows, no adaptive lanes) it runs in the velocity projection's epilogue and the
    // lambda returns true; otherwise the velocities go to `vel` and the caller combines.
    auto estimate = [&](int j, int nbe, const float* xl, const CfgEulerArgs* fuse) -> bool {
        const int Ne = nbe * R;
        const int cond0 = nbe == 1 ? 0 : 1;
        const int spk_branch = g.spk_dim > 0 ? nbe - 1 : -1;
        const long long NTk = (long long)Ne * Trow;                 // token capacity of the grid
        const int32_t* ntok = packed ? rowoff + Ne : nullptr;       // packed: device token count
        const float* modk = mod + (long long)j * nc * ML;
        auto rowmod = [&](const float* base, int tokens_per_row) {
            RowMod m;
            m.base = base;
            m.cvec_stride = ML;
            m.tokens_per_row = tokens_per_row;
            m.n_requests = R;
            m.spk_branch = spk_branch;
            m.tok_row = tokrow;
            return m;
        };
        AttnParams ap;
        ap.qkv = big; ap.vt = vt; ap.Tp = Tp; ap.o = act; ap.rows = Ne; ap.T = T; ap.H = H; ap.hd = hd;
        ap.kv_len = kvlen; ap.kv_mod = R; ap.key_mask = frame_mask; ap.mask_stride = Tx; ap.P = P;
        ap.kvalid = kvalid; ap.tile_full = tfull; ap.row_off = rowoff;
        if (prefix)
            timed(c, CFM_K_GEMM_IN, s, [&] {
                launch_prefix_init(cproj, wp<float>(c, c->inb), R, nbe, cond0, P, T, d, h, s);
            });
        {
            EpiParams ep;
            ep.bias = wp<float>(c, c->inb);
            ep.out = h; ep.ldo = d;
            ep.R = R; ep.Tx = Tx; ep.T = T; ep.P = P; ep.nb = nbe; ep.cond_branch0 = cond0;
            ep.cproj = prefix || cross ? nullptr : cproj;
            ep.row_off = rowoff;
            gemm(CFM_K_GEMM_IN, true, xl, C, c->inxw, R * Tx, d, C, EPI_INPROJ, ep);
        }
        CacheTok tk;
        tk.cap = NTk; tk.n_dev = ntok; tk.T = T; tk.tok_row = tokrow; tk.row_off = rowoff; tk.kvalid = kvalid;
        tk.R = R; tk.Tp = Tp;
        // the gated-residual GEMMs of small batches (split in K) may also apply the next
        // adaLN norm in their row-wise reduction (same bits as the adaLN kernel);
        // act_ready records that LN1 is done. Not across the cache's residual update.
        const bool ln_fuse = bf && !cross;
        bool act_ready = false;
        for (int l = 0; l < L; ++l) {
            if (caching && l == cf) {
                // probe: the state after the front blocks, scored against the previous one
                timed(c, CFM_K_HOISTED, s, [&] {
                    launch_cache_score(h, probe, d, tk, cparts, s);
                    const int forced = j < op.c_warmup || (op.c_force != nullptr && op.c_force[j] != 0);
                    launch_cache_decide(cparts, cstate, forced, op.c_threshold, op.c_budget, op.c_consec, op.c_max,
                                        tk, s);
                });
            }
            // middle blocks under the cache: their kernels read the token count the
            // decision left (0 on a hit: every block exits at once)
            const bool mid = caching && l >= cf && l < cb;
            const int32_t* ntok_l = mid ? cstate + 5 : ntok;
            const auto& W = c->layers[l];
            const float* ml = modk + (long long)l * 6 * d;
            LnParams ln;
            ln.h = h; ln.y = act; ln.d = d; ln.n_out = NTk; ln.Tin = T; ln.Tout = T; ln.off = 0;
            ln.shift = rowmod(ml + 0 * d, T); ln.scale = rowmod(ml + 1 * d, T); ln.out_bf16 = bf;
            ln.n_dev = ntok_l; ln.rms = rms;
            if (!act_ready) timed(c, CFM_K_ADALN, s, [&] { launch_adaln(ln, s); });
            act_ready = false;
            EpiParams e1; e1.bias = wp<float>(c, W.qkvb); e1.out = big;
            if (bf) {   // q|k rows of 2d (rotated in the epilogue), v transposed per head
                e1.ldo = 2 * d; e1.vt = vt; e1.H = H; e1.T = T; e1.Tp = Tp; e1.d2 = 2 * d;
                e1.tok_row = tokrow; e1.row_off = rowoff; e1.m_dev = ntok_l;
                e1.rope = rope_tab; e1.rope_hd = hd;
            } else {
                e1.ldo = 3 * d;
                e1.m_dev = ntok_l;
            }
            gemm(CFM_K_GEMM_QKV, false, act, d, W.qkvw, (int)NTk, 3 * d, d, bf ? EPI_QKV : EPI_ACT, e1);
            if (rope_tab && !bf)
                timed(c, CFM_K_GEMM_QKV, s, [&] { launch_rope_f32((float*)big, NTk, 3 * d, T, d, hd, rope_tab, ntok_l, s); });
            ap.active = mid ? cstate + 4 : nullptr;
            timed(c, CFM_K_ATTENTION, s, [&] {
                if (bf) launch_attention_bf16(ap, s); else launch_attention_f32(ap, s);
            });
            EpiParams e2; e2.bias = wp<float>(c, W.projb); e2.out = h; e2.ldo = d; e2.gate = rowmod(ml + 2 * d, T);
            e2.m_dev = ntok_l;
            e2.split_ws = splitk; e2.split_ws_floats = splitk_floats;
            if (ln_fuse) {   // LN2 of this block
                e2.ln_y = act; e2.ln_shift = rowmod(ml + 3 * d, T); e2.ln_scale = rowmod(ml + 4 * d, T);
                e2.ln_rms = rms;
            }
            const bool ln2_done = gemm(CFM_K_GEMM_PROJ, false, act, d, W.projw, (int)NTk, d, d, EPI_GATED, e2);
            if (cross) {
                // cross-attention sublayer: unmodulated norm, queries, attention over the
                // row's context keys, ungated residual (gate vector of ones)
                LnParams lx = ln;
                RowMod zero = rowmod(unit, T), one = rowmod(unit + d, T);
                zero.spk_branch = one.spk_branch = -1;
                lx.shift = zero; lx.scale = zero;
                timed(c, CFM_K_ADALN, s, [&] { launch_adaln(lx, s); });
                EpiParams eq; eq.bias = wp<float>(c, W.xqb); eq.out = big; eq.ldo = bf ? 2 * d : 3 * d;
                eq.m_dev = ntok_l;
                gemm(CFM_K_GEMM_XATTN, false, act, d, W.xqw, (int)NTk, d, d, EPI_ACT, eq);
                AttnParams ax = ap;
                const int kv0 = nbe == 1 ? (nb - 1) * R : 0;      // rows of the fully conditioned branch
                ax.kx = xk_of(l) + (size_t)kv0 * Tk * d * (bf ? 2 : 8);
                ax.ldkx = bf ? d : 2 * d; ax.Tk = Tk;
                ax.vt = xvt_of(l) + (size_t)kv0 * d * Tkp; ax.Tp = Tkp;
                ax.kv_len = xkvlen; ax.kv_mod = R; ax.key_mask = nullptr; ax.mask_stride = 0; ax.P = 0;
                ax.kvalid = xkvalid; ax.tile_full = xtfull;
                timed(c, CFM_K_XATTN, s, [&] {
                    if (bf) launch_attention_bf16(ax, s); else launch_attention_f32(ax, s);
                });
                EpiParams eo; eo.bias = wp<float>(c, W.xob); eo.out = h; eo.ldo = d; eo.gate = one;
                eo.m_dev = ntok_l;
                eo.split_ws = splitk; eo.split_ws_floats = splitk_floats;
                gemm(CFM_K_GEMM_XATTN, false, act, d, W.xow, (int)NTk, d, d, EPI_GATED, eo);
            }
            ln.shift = rowmod(ml + 3 * d, T); ln.scale = rowmod(ml + 4 * d, T);
            if (!ln2_done) timed(c, CFM_K_ADALN, s, [&] { launch_adaln(ln, s); });
            EpiParams e3; e3.bias = wp<float>(c, W.fc1b); e3.out = big; e3.ldo = f; e3.m_dev = ntok_l;
            if (!swiglu) {
                gemm(CFM_K_GEMM_FC1, false, act, d, W.fc1w, (int)NTk, f, d, EPI_GELU_ACT, e3);
            } else if (bf) {   // fused gate-up GEMM, SwiGLU in its epilogue
                gemm(CFM_K_GEMM_FC1, false, act, d, W.fc1w, (int)NTk, 2 * f, d, EPI_SWIGLU, e3);
            } else {
                e3.out = gu; e3.ldo = 2 * f;
                gemm(CFM_K_GEMM_FC1, false, act, d, W.fc1w, (int)NTk, 2 * f, d, EPI_ACT, e3);
                timed(c, CFM_K_GEMM_FC1, s, [&] { launch_swiglu_f32(gu, (float*)big, NTk, f, ntok_l, s); });
            }
            EpiParams e4; e4.bias = wp<float>(c, W.fc2b); e4.out = h; e4.ldo = d; e4.gate = rowmod(ml + 5 * d, T);
            e4.m_dev = ntok_l;
            e4.split_ws = splitk; e4.split_ws_floats = splitk_floats;
            if (ln_fuse && l + 1 < L && !(caching && l == cb - 1)) {   // LN1 of the next block
                const float* mn = modk + (long long)(l + 1) * 6 * d;
                e4.ln_y = act; e4.ln_shift = rowmod(mn, T); e4.ln_scale = rowmod(mn + d, T); e4.ln_rms = rms;
            }
            act_ready = gemm(CFM_K_GEMM_FC2, false, big, f, W.fc2w, (int)NTk, d, f, EPI_GATED, e4);
            if (caching && l == cb - 1)   // computed: save the residual; hit: add the saved one
                timed(c, CFM_K_HOISTED, s, [&] { launch_cache_apply(h, resid, probe, d, tk, cstate, s); });
        }
        const bool fused = fuse != nullptr && bf && !packed && !adaptive && nbe <= 2 && fuse->lane_off == nullptr;
        {
            const float* mf = modk + (long long)L * 6 * d;
            LnParams ln;
            ln.h = h; ln.y = act; ln.d = d; ln.n_out = (long long)Ne * Tx; ln.Tin = T; ln.Tout = Tx; ln.off = P;
            ln.shift = rowmod(mf, Tx); ln.scale = rowmod(mf + d, Tx); ln.out_bf16 = bf; ln.rms = rms;
            if (packed) { ln.n_out = NTk; ln.Tin = ln.Tout = 1; ln.n_dev = ntok; }   // tokens map one to one
            if (fused) { ln.inter_nb = nbe; ln.inter_R = R; }   // the nbe rows of a frame next to each other
            timed(c, CFM_K_ADALN, s, [&] { launch_adaln(ln, s); });
            EpiParams ep; ep.bias = wp<float>(c, c->outb); ep.ldo = C;
            ep.R = R; ep.Tx = Tx; ep.mask = frame_mask;
            if (fused) {
                ep.nb = nbe; ep.x_in = fuse->x_in; ep.x_out = fuse->x_out;
                ep.cw[0] = fuse->w0; ep.cw[1] = fuse->w1;
                gemm(CFM_K_GEMM_OUT, false, act, d, c->outw, Ne * Tx, C, d, EPI_VOUT_EULER, ep);
            } else {
                ep.out = vel;
                ep.tok_row = tokrow; ep.row_off = rowoff; ep.m_dev = ntok;
                gemm(CFM_K_GEMM_OUT, false, act, d, c->outw, packed ? (int)NTk : Ne * Tx, C, d, EPI_VOUT, ep);
            }
        }
        return fused;
    };

    // guidance weights of a guided evaluation (weights of the branch velocities
    // that give the guidance equation)
    float w[3] = {1.0f, 0.0f, 0.0f};
    if (nb == 2) { w[0] = 1.0f - scales[0]; w[1] = scales[0]; }
    if (nb == 3) { w[0] = 1.0f - scales[0]; w[1] = scales[0] - scales[1]; w[2] = scales[1]; }
    // whether an evaluation at time t runs guided (host-decided policies)
    auto guided_at = [&](double t) {
        if (nb == 1) return false;
        if (op.mode == CFM_GUIDANCE_INTERVAL) return op.start <= t && t <= op.end;
        return true;   // full CFG; adaptive lanes are decided on the device
    };
    // x_out = x_in + dt * (guided combine of the nbe rows just evaluated)
    auto combine_args = [&](int nbe, float dt, const float* xin, float* xout, const int32_t* lane_off) {
        CfgEulerArgs a;
        a.v = vel; a.nb = nbe; a.mask = frame_mask; a.R = R; a.Tx = Tx; a.C = C;
        a.x_in = xin; a.x_out = xout; a.lane_off = lane_off; a.w_full = dt;
        if (nbe == 1) a.w0 = dt;
        else { a.w0 = dt * w[0]; a.w1 = dt * w[1]; a.w2 = dt * w[2]; }
        return a;
    };

    // ---- steps: the grid is rebuilt before the loop (uniform, quadratic, trailing or
    // a subsequence of a native grid), then one (Euler) or two (midpoint) evaluations
    // per step; step sizes and guidance weights are kernel arguments
    long long guided_evals = 0;
    for (int k = 0; k < S; ++k) {
        const double t0 = host_grid_time(op.schedule, S, op.native, k);
        const double t1 = host_grid_time(op.schedule, S, op.native, k + 1);
        const float dt = (float)(t1 - t0);
        const int32_t* st_cur = lanes + (k & 1) * 3 * R;        // lane state this step runs with
        int32_t* st_next = lanes + ((k + 1) & 1) * 3 * R;
        const int32_t* lane_off = adaptive ? st_cur + R : nullptr;
        // this step's packed layout: stopped lanes hold no unconditional rows (only
        // where the layout is packed; elsewhere every row is computed and the stopped
        // lanes' rows are not used)
        if (adaptive && packed)
            timed(c, CFM_K_HOISTED, s, [&] {
                launch_pack_rows(kvlen, lane_off, R, nb, (int)(N * Trow), rowoff, tokrow, s);
            });
        for (int e = 0; e < per_step; ++e) {
            const int j = k * per_step + e;
            const double te = host_eval_time(op.schedule, S, op.native, per_step, j);
            const int nbe = guided_at(te) ? nb : 1;
            guided_evals += nbe > 1 ? 1 : 0;
            const CfgEulerArgs a = per_step == 2 && e == 0 ? combine_args(nbe, 0.5f * dt, out, xmid, lane_off)  // half step
                                                           : combine_args(nbe, dt, out, out, lane_off);
            const bool fused = estimate(j, nbe, e == 0 ? out : xmid, &a);
            if (adaptive && e == 0)
                launch_adaptive_update(vel, nb, frame_mask, R, Tx, C, st_cur, st_next, k, op.warmup, op.patience,
                                       op.threshold, per_step, s);
            if (!fused) timed(c, CFM_K_CFG_EULER, s, [&] { launch_cfg_euler(a, s); });
        }
    }
    if (op.guided_out != nullptr) {
        if (adaptive) launch_copy_i32(lanes + (S & 1) * 3 * R + 2 * R, op.guided_out, R, s);
        else launch_fill_i32(op.guided_out, R, (int)guided_evals, s);
    }
    if (op.c_hits != nullptr) {
        if (caching) launch_copy_i32(cstate + 2, op.c_hits, 1, s);
        else launch_fill_i32(op.c_hits, 1, 0, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CFM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return CFM_OK;
}

// ------------------------------------------------------------ single kernels

cfm_status cfm_cfg_euler(const float* v, const float* w, int nb, float dt, const uint8_t* mask,
                         int R, int Tx, int C, float* x, void* stream) {
    if (nb < 1 || nb > 3 || R < 0 || Tx < 0 || C < 0) return fail(CFM_E_VALUE, "bad nb/R/Tx/C");
    if (C % 4) return fail(CFM_E_SHAPE, "C must be a multiple of 4");
    if ((long long)R * Tx * C == 0) return CFM_OK;
    if (v == nullptr || w == nullptr || x == nullptr) return fail(CFM_E_NULL, "v, w or x is NULL");
    if (!aligned16(v) || !aligned16(x)) return fail(CFM_E_SHAPE, "v and x must be 16-byte aligned");
    float ww[3] = {0.0f, 0.0f, 0.0f};
    for (int b = 0; b < nb; ++b) {
        if (!std::isfinite(w[b])) return fail(CFM_E_VALUE, "non-finite branch weight");
        ww[b] = dt * w[b];
    }
    if (!std::isfinite(dt)) return fail(CFM_E_VALUE, "non-finite dt");
    (void)hipGetLastError();
    CfgEulerArgs a;
    a.v = v; a.nb = nb; a.w0 = ww[0]; a.w1 = ww[1]; a.w2 = ww[2]; a.mask = mask; a.R = R; a.Tx = Tx; a.C = C;
    a.x_in = x; a.x_out = x;
    launch_cfg_euler(a, (hipStream_t)stream);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CFM_OK : fail(CFM_E_HIP, "launch failed: %s", hipGetErrorString(e));
}

cfm_status cfm_gemm_bf16(const void* A, int a_is_f32, int lda, const void* W, int ldw,
                         const float* bias, int M, int N, int K, int epilogue,
                         const float* gate, void* C, int ldc, int tile, void* stream) {
    if (M < 0 || N < 0 || K < 0) return fail(CFM_E_VALUE, "negative size");
    if (!(tile == 0 || tile == 1 || tile == 6 || tile == 10 || tile == 14 || tile == 15) || (tile > 1 && a_is_f32))
        return fail(CFM_E_VALUE, "tile %d", tile);
    if (epilogue < 0 || epilogue > 4) return fail(CFM_E_VALUE, "epilogue %d", epilogue);
    if (epilogue == 4 && N % 32) return fail(CFM_E_SHAPE, "the SwiGLU epilogue needs N %% 32 == 0");
    if (M == 0 || N == 0) return CFM_OK;
    if (A == nullptr || W == nullptr || C == nullptr) return fail(CFM_E_NULL, "A, W or C is NULL");
    if (epilogue == 3 && gate == nullptr) return fail(CFM_E_NULL, "gate is NULL");
    const int kq = a_is_f32 ? 4 : 8;
    const int ncols = epilogue == 4 ? N / 2 : N;
    if (K % kq || lda % kq || ldw % 8 || lda < K || ldw < round8(K) || ldc < ncols || (ncols > 3 && ldc % 4))
        return fail(CFM_E_SHAPE, "K/lda/ldw/ldc do not meet the layout rules");
    if (!aligned16(A) || !aligned16(W) || !aligned16(C) || (bias && !aligned16(bias)) || (gate && !aligned16(gate)))
        return fail(CFM_E_SHAPE, "A, W, C, bias and gate must be 16-byte aligned");
    if ((long long)M * lda * (a_is_f32 ? 4 : 2) >= kMaxOperandBytes || (long long)N * ldw * 2 >= kMaxOperandBytes)
        return fail(CFM_E_SHAPE, "operand above 2 GiB");
    static const int map[5] = {EPI_F32, EPI_ACT, EPI_GELU_ACT, EPI_GATED, EPI_SWIGLU};
    EpiParams ep;
    ep.bias = bias;
    ep.out = C;
    ep.ldo = ldc;
    ep.gate.base = gate;
    ep.gate.cvec_stride = 0;
    ep.gate.tokens_per_row = 1;
    ep.gate.n_requests = 1;
    ep.gate.spk_branch = -1;
    (void)hipGetLastError();
    launch_gemm_bf16(a_is_f32 != 0, map[epilogue], A, lda, (const bf16*)W, ldw, M, N, K, ep, (hipStream_t)stream,
                     tile);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CFM_OK : fail(CFM_E_HIP, "launch failed: %s", hipGetErrorString(e));
}

namespace {
// bytes of key-validity tables the attention of `rows` rows of T keys needs: key
// lengths, then (from the next 16-byte boundary, which the 64 bytes of slack
// cover) per-key validity bytes and per-64-key-tile flags
size_t attention_scratch_bytes(int rows, int T) {
    const long long Tp = round64(T);
    return (size_t)rows * 4 + (size_t)rows * Tp + (size_t)rows * (Tp / 64) + 64;
}

// key tables + attention over caller-checked arguments, the tables in device memory `tables`
cfm_status attention_bf16_run(const void* qk, const void* vt, const int32_t* kv_len, const uint8_t* key_mask,
                              int rows, int T, int H, void* tables, void* o, hipStream_t s) {
    const long long Tp = round64(T);
    int32_t* kvl = (int32_t*)tables;
    uint8_t* kvalid = (uint8_t*)tables + align_up((size_t)rows * 4, 16);
    uint8_t* tfull = kvalid + (size_t)rows * Tp;
    AttnParams p;
    p.qkv = qk; p.vt = vt; p.Tp = (int)Tp; p.o = o; p.rows = rows; p.T = T; p.H = H; p.hd = 64;
    p.kv_len = kvl; p.kv_mod = rows; p.key_mask = key_mask; p.mask_stride = T; p.P = 0;
    p.kvalid = kvalid; p.tile_full = tfull;
    (void)hipGetLastError();
    launch_key_prep(key_mask, T, kv_len, rows, 0, T, (int)Tp, kvl, kvalid, tfull, s);
    launch_attention_bf16(p, s);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CFM_OK : fail(CFM_E_HIP, "launch failed: %s", hipGetErrorString(e));
}

cfm_status attention_bf16_check(const void* qk, const void* vt, const int32_t* kv_len, int rows, int T, int H,
                                const void* o) {
    if (rows < 0 || T < 0 || H <= 0) return fail(CFM_E_VALUE, "bad rows/T/H");
    if (rows > 65535 || H > 65535) return fail(CFM_E_SHAPE, "rows and H must be <= 65535");
    if (rows == 0 || T == 0) return CFM_OK;
    if (qk == nullptr || vt == nullptr || kv_len == nullptr || o == nullptr)
        return fail(CFM_E_NULL, "qk, vt, kv_len or o is NULL");
    if (!aligned16(qk) || !aligned16(vt) || ((uintptr_t)o & 7))
        return fail(CFM_E_SHAPE, "qk, vt 16-byte / o 8-byte alignment");
    if (!attention_bf16_fits(T)) return fail(CFM_E_UNSUPPORTED, "T = %d: the key tables exceed LDS", T);
    return CFM_OK;
}

constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
}  // namespace

// Scratch of cfm_attention_bf16_noalloc (key-validity tables): one copy per GPU,
// held until the process ends. Host code never passes `scratch` itself (on the
// host the name is only a stand-in for the symbol); it passes the device address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
cfm_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(CFM_E_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return fail(CFM_E_UNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(CFM_E_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CFM_OK;
}
}  // namespace

cfm_status cfm_attention_bf16(const void* qk, const void* vt, const int32_t* kv_len,
                              const uint8_t* key_mask, int rows, int T, int H, void* scratch_buf,
                              size_t scratch_bytes, void* o, void* stream) {
    cfm_status st = attention_bf16_check(qk, vt, kv_len, rows, T, H, o);
    if (st != CFM_OK || rows == 0 || T == 0) return st;
    if (scratch_buf == nullptr) return fail(CFM_E_NULL, "scratch is NULL");
    if ((uintptr_t)scratch_buf & 15) return fail(CFM_E_SHAPE, "scratch must be 16-byte aligned");
    const size_t need = attention_scratch_bytes(rows, T);
    if (scratch_bytes < need) return fail(CFM_E_WORKSPACE, "scratch %zu bytes, need %zu", scratch_bytes, need);
    return attention_bf16_run(qk, vt, kv_len, key_mask, rows, T, H, scratch_buf, o, (hipStream_t)stream);
}

cfm_status cfm_attention_bf16_noalloc(const void* qk, const void* vt, const int32_t* kv_len,
                                      const uint8_t* key_mask, int rows, int T, int H, void* o, void* stream) {
    cfm_status st = attention_bf16_check(qk, vt, kv_len, rows, T, H, o);
    if (st != CFM_OK || rows == 0 || T == 0) return st;
    const size_t need = attention_scratch_bytes(rows, T);
    if (need > kNoAllocScratchBytes)
        return fail(CFM_E_CAPACITY, "rows = %d, T = %d need %zu bytes of key tables; the built-in scratch holds %zu",
                    rows, T, need, kNoAllocScratchBytes);
    void* p = nullptr;
    st = scratch_on_current_device(&p);
    if (st != CFM_OK) return st;
    return attention_bf16_run(qk, vt, kv_len, key_mask, rows, T, H, p, o, (hipStream_t)stream);
}

cfm_status cfm_adaln(const float* hsrc, const float* shift, const float* scale, int M, int d,
                     int out_bf16, void* y, void* stream) {
    if (M < 0 || d <= 0) return fail(CFM_E_VALUE, "bad M/d");
    if (d % 4 || d > 4096) return fail(CFM_E_SHAPE, "d must be a multiple of 4 and <= 4096");
    if (M == 0) return CFM_OK;
    if (hsrc == nullptr || shift == nullptr || scale == nullptr || y == nullptr) return fail(CFM_E_NULL, "NULL argument");
    if (!aligned16(hsrc) || !aligned16(shift) || !aligned16(scale) || ((uintptr_t)y & 7))
        return fail(CFM_E_SHAPE, "alignment");
    LnParams p;
    p.h = hsrc; p.y = y; p.d = d; p.n_out = M; p.Tin = 1; p.Tout = 1; p.off = 0;
    p.shift.base = shift; p.shift.cvec_stride = 0; p.shift.tokens_per_row = 1; p.shift.n_requests = 1; p.shift.spk_branch = -1;
    p.scale = p.shift;
    p.scale.base = scale;
    p.out_bf16 = out_bf16 != 0;
    (void)hipGetLastError();
    launch_adaln(p, (hipStream_t)stream);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? CFM_OK : fail(CFM_E_HIP, "launch failed: %s", hipGetErrorString(e));
}

}  // extern "C"
