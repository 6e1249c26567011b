/*
 * cfm.h -- C ABI of the MI355X (gfx950) batched conditional-flow-matching sampler.
 *
 * What the library computes (sources: the VoiceHub page "Diffusion and flow TTS
 * optimization", sections "Active families", "Custom Triton and CUDA kernels",
 * "Static shapes and CUDA graphs" and its table "Semantic-preserving and
 * approximate changes"; the vLLM-Omni TTS blog, section "CFM/LocDiT decode-tail
 * batching"):
 *
 *   Euler sampling of a flow-matching / rectified-flow ODE from noise x0 (t = 0)
 *   to data (t = 1) on the uniform grid t_k = k / S. At every step one DiT
 *   velocity estimator runs over ALL requests of the batch at once, each request
 *   expanded into its classifier-free-guidance branch rows ("packed CFG": rows
 *   are branch-major, row = b * R + r). The branch velocities are combined with
 *   the guidance equation and the Euler update x <- x + dt * v is applied:
 *
 *     2 branches (uncond, cond):            v = v_u + s (v_c - v_u)
 *     3 branches (uncond, text, text+spk):  v = v_u + s_t (v_t - v_u) + s_s (v_ts - v_t)
 *     1 branch:                             v = v_c
 *
 *   Estimator per row: c = W2 SiLU(W1 e(t) + b1) + b2 (+ Ws spk + bs), e(t) the
 *   256-wide sinusoidal embedding of 1000 t; h = input projection of the frames
 *   (latent channels concatenated with per-frame condition channels, or
 *   condition frames placed before the latent frames); L DiT blocks, each
 *     h += gate1 * Proj(MHA(LN(h) (1 + scale1) + shift1))
 *     h += gate2 * FC2(GELU(FC1(LN(h) (1 + scale2) + shift2)))
 *   with (shift1, scale1, gate1, shift2, scale2, gate2) = Wada_l SiLU(c) + bada_l,
 *   key-padding-masked non-causal attention; v = Out(LN(h)(1 + scale_f) + shift_f).
 *   Branches without a condition see it zeroed. Padded frames are masked as keys,
 *   get v = 0, and are returned unchanged (out = x0 there, bit for bit).
 *
 * Conventions for every function:
 *   - All device pointers are HIP device (or managed) memory on the current
 *     device; host pointers are marked "host". Tensors are dense row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *     is enqueued asynchronously on it; no function here synchronises the host,
 *     allocates device memory or reads device memory back, except where stated.
 *   - Every argument is validated BEFORE anything is enqueued: on an error
 *     return nothing was launched and no output was touched. Errors detected
 *     after enqueue (a failed launch) return CFM_E_HIP and leave outputs
 *     undefined. No function aborts or throws. The detail of the last error of
 *     the calling thread is available from cfm_last_error_detail().
 *   - A context is not safe for concurrent cfm_sample calls (they share its
 *     workspace); separate contexts are independent.
 */
#ifndef CFM_MI355X_H
#define CFM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cfm_status {
    CFM_OK = 0,
    CFM_E_NULL = 1,          /* a required pointer is NULL                          */
    CFM_E_SHAPE = 2,         /* inconsistent sizes or layout                        */
    CFM_E_CAPACITY = 3,      /* request/frame/step count above the create-time max  */
    CFM_E_VALUE = 4,         /* negative count, non-finite guidance scale, ...      */
    CFM_E_UNSUPPORTED = 5,   /* configuration this build does not implement         */
    CFM_E_WORKSPACE = 6,     /* workspace smaller than cfm_workspace_bytes()        */
    CFM_E_HIP = 7            /* a HIP runtime call or kernel launch failed          */
} cfm_status;

typedef enum cfm_dtype { CFM_F32 = 0, CFM_BF16 = 1 } cfm_dtype;
typedef enum cfm_cond_mode { CFM_COND_CHANNEL = 0, CFM_COND_PREFIX = 1, CFM_COND_CROSS = 2 } cfm_cond_mode;
/* Block variants (VoiceHub "Diffusion and flow TTS optimization", section "Custom
 * Triton and CUDA kernels": RMSNorm and SwiGLU patterns; vLLM-Omni TTS blog, section
 * "CFM/LocDiT decode-tail batching": the LocDiT's fused gate-up MLP). */
typedef enum cfm_norm { CFM_NORM_LAYER = 0, CFM_NORM_RMS = 1 } cfm_norm;
typedef enum cfm_mlp { CFM_MLP_GELU = 0, CFM_MLP_SWIGLU = 1 } cfm_mlp;

/* Model and capacity description. Plain data; copied by cfm_create.
 *   cond_mode CHANNEL: cond is [R, Tx, cond_dim], concatenated after the latent
 *                      channels of each frame before the input projection.
 *   cond_mode PREFIX:  cond is [R, n_prefix, latent_dim]: condition frames placed
 *                      before the Tx latent frames (cond_dim must equal latent_dim).
 *   cond_mode CROSS:   cond is a context [R, n_prefix, cond_dim] that every block
 *                      reads through a cross-attention sublayer placed between its
 *                      self-attention and its MLP, h += Wo attn(Wq N(h) + bq, K, V) + bo,
 *                      N the block's norm without modulation, [K | V] = Wkv ctx + bkv
 *                      over all n_prefix context tokens (computed once per call: the
 *                      context is fixed over the steps; VoiceHub, "Recommended
 *                      optimization boundaries" table, rows Echo and Irodori-TTS:
 *                      cached condition keys/values). The input projection sees the
 *                      latent alone; the unconditional branch sees a zero context.
 *   norm:  LAYER (h - mean) / sqrt(var + 1e-6), or RMS h / sqrt(mean(h^2) + 1e-6);
 *          every norm of the estimator follows it.
 *   mlp:   GELU: FC2(GELU(FC1 u)); SWIGLU: FC1 is a fused gate-up weight of 2 ffn_dim
 *          rows (gate rows first, as given), FC2(SiLU(gate) * up); needs ffn_dim % 16 == 0.
 *   rope:  nonzero: rotary position embedding (RoFormer) of the self-attention
 *          queries and keys: feature pairs (2i, 2i+1) of each head turn by the
 *          angle p * rope_base^(-2i / head_dim), p the token's index in its row's
 *          sequence (prefix tokens first); rope_base > 0 and finite.
 *   dtype BF16: weights and GEMM/attention operands bfloat16 with fp32
 *               accumulation; residual stream, LayerNorm statistics, softmax,
 *               modulation, velocities and x are fp32.
 *   dtype F32:  fp32 end to end.
 * Supported: d_model % 8 == 0, ffn_dim % 8 == 0, latent_dim % 4 == 0,
 * cond_dim % 4 == 0, t_freq_dim even and % 8 == 0, 1 <= n_branches <= 3;
 * BF16 needs head_dim == 64, F32 needs head_dim % 4 == 0 and head_dim <= 64. */
typedef struct cfm_config {
    int32_t n_layers, d_model, n_heads, ffn_dim;
    int32_t latent_dim, cond_dim, cond_mode, n_prefix;
    int32_t spk_dim;          /* 0 = no speaker path                                 */
    int32_t t_freq_dim;       /* width of the sinusoidal timestep embedding (256)   */
    int32_t n_branches;       /* CFG branch rows per request: 1, 2 or 3             */
    int32_t dtype;            /* cfm_dtype                                          */
    int32_t max_requests, max_frames, max_steps;   /* capacity of the workspace    */
    int32_t norm;             /* cfm_norm                                           */
    int32_t mlp;              /* cfm_mlp                                            */
    int32_t rope;             /* 0 = off                                            */
    float rope_base;          /* rotary frequency base (10000 in RoFormer)          */
} cfm_config;

/* One slot of the flat weight buffer. The slot holds
 * source[row0 : row0 + rows, col0 : col0 + cols] of the named parameter
 * (PyTorch Linear convention: weight [out, in], bias [out]) with a row stride
 * of `ld` elements, starting `offset` bytes into the buffer. `dtype` is the
 * element type of the slot (matrices: the config dtype; biases: always F32).
 * `interleave` = k > 0 reorders the slot's rows: the source rows form two halves
 * (rows/2 each), and slot row group g (rows [2k g, 2k g + 2k)) holds rows
 * [k g, k g + k) of the first half followed by rows [k g, k g + k) of the second
 * half (for a bias, the same on its elements); 0 = source order. (The fused
 * gate-up weight is stored this way, so that each 2k-wide output block of its
 * GEMM holds k gate columns and the k up columns that pair with them.)
 * Bytes of the buffer not covered by a slot (row padding) must be zero. */
typedef struct cfm_tensor_desc {
    char name[48];
    int64_t row0, col0, rows, cols, ld;
    int64_t offset;
    int32_t dtype;
    int32_t interleave;
} cfm_tensor_desc;

typedef struct cfm_ctx cfm_ctx;

/* Host-only size queries. Return 0 / a negative cfm_status for an unsupported
 * or invalid config. */
size_t cfm_weights_bytes(const cfm_config* cfg);
size_t cfm_workspace_bytes(const cfm_config* cfg);
/* Writes up to `cap` slot descriptors to `out` (host) and returns the total
 * number of slots, or -(cfm_status) on error. out may be NULL when cap == 0. */
int cfm_weight_manifest(const cfm_config* cfg, cfm_tensor_desc* out, int cap);

/* Creates a sampler context (host memory only; no HIP call). BORROWS
 * `weights` (cfm_weights_bytes, filled per the manifest) and `workspace`
 * (cfm_workspace_bytes): both are caller-owned device memory that must outlive
 * the context and every call still in flight. All state of a call lives in that
 * caller-visible workspace and the library allocates nothing, the condition the
 * vox-serve page "Adding a Model" sets for graph-captured model code (buffers
 * allocated up front, shapes taken from arguments, no allocation in the captured
 * region). The config is validated here, so that an unsupported request fails
 * before anything is mutated (VoiceHub "Diffusion and flow TTS optimization",
 * section "Attention": an explicit request the backend cannot honour fails
 * before model mutation). Errors: CFM_E_NULL, CFM_E_UNSUPPORTED, CFM_E_VALUE,
 * CFM_E_WORKSPACE, CFM_E_SHAPE (weights or workspace not 256-byte aligned). */
cfm_status cfm_create(const cfm_config* cfg, const void* weights, void* workspace,
                      size_t workspace_bytes, cfm_ctx** out_ctx);

/* Runs the whole sampler: S = n_steps Euler steps over R = n_requests requests.
 *   x0         device fp32 [R, Tx, latent_dim]         noise (t = 0)
 *   cond       device fp32 [R, Tx, cond_dim] (CHANNEL), [R, n_prefix, latent_dim] (PREFIX)
 *              or [R, n_prefix, cond_dim] (CROSS)
 *   spk        device fp32 [R, spk_dim], or NULL when spk_dim == 0
 *   frame_mask device uint8 [R, Tx], 1 = valid frame, or NULL = all valid
 *   guidance   host fp32 [n_branches - 1] guidance scales (NULL allowed when n_branches == 1)
 *   out        device fp32 [R, Tx, latent_dim]; may alias x0 exactly
 * Tx = n_frames. R == 0 is a no-op; S == 0 gives out = x0. A request with no
 * valid frame gives out = x0. Inputs must stay alive and unmodified until the
 * stream has passed this call. Errors: CFM_E_NULL, CFM_E_SHAPE, CFM_E_CAPACITY,
 * CFM_E_VALUE (negative count, non-finite scale), CFM_E_HIP.
 * Sources of the contract:
 *   - every request's CFG rows go through ONE estimator call per step (the
 *     vLLM-Omni TTS blog, section "CFM/LocDiT decode-tail batching", batches the
 *     two CFG rows of many requests into one estimator call);
 *   - the step loop has no host synchronisation: step sizes and guidance
 *     weights are computed on the host before enqueue and passed by value (the
 *     same section removes the per-step host syncs of the Euler loop);
 *   - nothing is allocated and every shape comes from the arguments (vox-serve,
 *     "Adding a Model": graph-capture rules), so the call can be captured;
 *   - packed CFG rows give what separate branch calls give, and padded frames
 *     are fully masked and returned untouched (VoiceHub "Diffusion and flow TTS
 *     optimization", table "Semantic-preserving and approximate changes");
 *   - randomness belongs to the request: the noise x0 is an input and the
 *     library draws no random numbers (vox-serve, "Adding a Model"; the
 *     Breeze-TTS-2 recipe's per-request generators);
 *   - arguments are validated before anything is enqueued, so a rejected call
 *     leaves out untouched (VoiceHub, section "Attention"). */
cfm_status cfm_sample(cfm_ctx* ctx, const float* x0, const float* cond, const float* spk,
                      const uint8_t* frame_mask, int n_requests, int n_frames, int n_steps,
                      const float* guidance, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * Sampler-level options (cfm_sample_ex). Sources: VoiceHub "Diffusion and flow TTS
 * optimization", sections "Reduce a 50-step sampler before optimizing its
 * kernels" (the grid is rebuilt before the loop, keeps both endpoints and strict
 * monotonicity; native / uniform / quadratic / trailing shapes) and "Guidance
 * reduction" (limited-interval and adaptive CFG, independent per-request lanes),
 * and its "Active families" table (Euler or midpoint for the F5-TTS family).
 * The pages give no formulas; the readings implemented here:
 *   schedules on S steps, u = k / S: UNIFORM t_k = u, QUADRATIC t_k = u^2 (small
 *     steps near the noise end), TRAILING t_k = 1 - (1 - u)^2 (small steps near the
 *     data end), NATIVE t_k = round(k N / S) / N (halves up) on a native grid of
 *     N = native_steps uniform steps (N >= S);
 *   MIDPOINT: x_k+1 = x_k + dt v(t_k + dt/2, x_k + (dt/2) v(t_k, x_k)): two estimator
 *     evaluations per step, so n_steps * 2 must not exceed the config's max_steps
 *     (which bounds estimator evaluations per call);
 *   INTERVAL guidance: an evaluation at time t runs the CFG branch rows only when
 *     interval_start <= t <= interval_end; otherwise only the fully conditioned
 *     branch row of every request is evaluated (half the rows with two branches)
 *     and its velocity is used as is (guidance scale 1);
 *   ADAPTIVE guidance, per request: after a step's first evaluation the metric
 *     sum |v_full - v_u| / sum |v_full| over the request's valid frames is compared
 *     with adaptive_threshold; steps below adaptive_warmup never count, later steps
 *     below the threshold increment a counter and others reset it; once the counter
 *     reaches adaptive_patience the request's unconditional lane stops for all later
 *     steps, which run the fully conditioned row alone. Decided on the device, with
 *     no host synchronisation; on the bf16 channel-condition path the stopped rows
 *     are dropped from the packed row layout, elsewhere they are still computed and
 *     not used.
 * Block-residual caching (VoiceHub, section "Approximate block-residual caching"),
 * readings: the cache lane is the whole batch of one call (the packed CFG batch);
 * every estimator evaluation is a cache step; the probe is the hidden state after
 * the first cache_front blocks, scored against the previous evaluation's probe as
 * sum |probe - prev| / sum |prev| over valid frames; an evaluation computes the
 * middle blocks when forced (cache_force, or one of the first cache_warmup
 * evaluations), when no residual is saved yet, when cache_max_cached hits have been
 * taken, after cache_max_consecutive hits in a row, when the score is not below
 * cache_threshold, or when the scores accepted since the last computation plus this
 * one exceed cache_budget; a computing evaluation saves the middle blocks' residual
 * (state after minus state before), a hit adds it instead of running them. The
 * last cache_back blocks always run. Decided on the device (no host
 * synchronisation); skipped blocks' kernels exit at once. Needs guidance_mode FULL
 * (a changing row set would invalidate the probe), else CFM_E_UNSUPPORTED. */
typedef enum cfm_schedule {
    CFM_SCHEDULE_UNIFORM = 0, CFM_SCHEDULE_QUADRATIC = 1, CFM_SCHEDULE_TRAILING = 2, CFM_SCHEDULE_NATIVE = 3
} cfm_schedule;
typedef enum cfm_solver { CFM_SOLVER_EULER = 0, CFM_SOLVER_MIDPOINT = 1 } cfm_solver;
typedef enum cfm_guidance_mode {
    CFM_GUIDANCE_FULL = 0, CFM_GUIDANCE_INTERVAL = 1, CFM_GUIDANCE_ADAPTIVE = 2
} cfm_guidance_mode;

typedef struct cfm_sample_options {
    int32_t schedule;            /* cfm_schedule                                         */
    int32_t native_steps;        /* NATIVE: steps of the native uniform grid (>= n_steps) */
    int32_t solver;              /* cfm_solver                                           */
    int32_t guidance_mode;       /* cfm_guidance_mode                                    */
    float interval_start, interval_end;                 /* INTERVAL (finite)            */
    float adaptive_threshold;    /* ADAPTIVE: >= 0, +infinity allowed                    */
    int32_t adaptive_warmup;     /* ADAPTIVE: >= 0                                       */
    int32_t adaptive_patience;   /* ADAPTIVE: >= 1                                       */
    int32_t reserved;
    int32_t* guided_evals;       /* optional device int32 [R]: per request, the number of
                                    estimator evaluations that ran its unconditional rows */
    /* Block-residual cache (DBCache; 0 = off): see the reading below.               */
    int32_t cache;               /* 1 = on                                               */
    int32_t cache_front;         /* Fn >= 1 blocks always run first                      */
    int32_t cache_back;          /* Bn >= 0 blocks always run last                       */
    int32_t cache_warmup;        /* the first evaluations that always compute (>= 0)     */
    int32_t cache_max_consecutive;  /* hits in a row before a forced computation (>= 0)  */
    int32_t cache_max_cached;    /* total hits allowed per call, -1 = unlimited          */
    float cache_threshold;       /* hit when the probe score is below it (>= 0, inf ok)  */
    float cache_budget;          /* refresh when accepted scores add up past it (>= 0)   */
    const uint8_t* cache_force;  /* optional host [evaluations]: nonzero forces computing */
    int32_t* cache_hits;         /* optional device int32 [1]: evaluations that reused the
                                    saved residual                                       */
} cfm_sample_options;

/* cfm_sample with sampler-level options (NULL = uniform grid, Euler, full CFG,
 * i.e. exactly cfm_sample). Same arguments, rules and errors as cfm_sample, plus
 * CFM_E_VALUE for an option out of range and CFM_E_CAPACITY when the estimator
 * evaluations (n_steps, twice that for MIDPOINT) exceed max_steps. */
cfm_status cfm_sample_ex(cfm_ctx* ctx, const float* x0, const float* cond, const float* spk,
                         const uint8_t* frame_mask, int n_requests, int n_frames, int n_steps,
                         const float* guidance, const cfm_sample_options* options, float* out,
                         void* stream);

/* Frees host state only: the borrowed weight and workspace buffers stay the
 * caller's (vox-serve, "Adding a Model": buffers are owned by the caller and
 * outlive the captured work). Work already enqueued keeps using them, so the
 * caller frees them only after the stream has passed its last call. NULL-safe. */
void cfm_destroy(cfm_ctx* ctx);

const char* cfm_status_string(cfm_status s);
/* Thread-local text describing the last error returned on this thread. */
const char* cfm_last_error_detail(void);

/* ---------------------------------------------------------------------------
 * Kernel timing. While enabled, every launch of the selected kernel class is
 * bracketed by two hipEvents recorded on the launch stream. cfm_profile_read
 * SYNCHRONISES on those events (host wait) and returns the summed elapsed
 * milliseconds and the launch count since the last enable; the event pool holds
 * `capacity` launches (extra launches are not timed and counted in *dropped).
 * Class ids are the CFM_K_* values below (XATTN: the cross-attention kernel of the
 * CROSS mode; GEMM_XATTN: its query and output projections; a fp32 rotary or SwiGLU
 * pass counts with its QKV or FC1 GEMM; the unmodulated cross-attention norm with
 * ADALN). */
enum {
    CFM_K_GEMM_QKV = 0, CFM_K_GEMM_PROJ = 1, CFM_K_GEMM_FC1 = 2, CFM_K_GEMM_FC2 = 3,
    CFM_K_ATTENTION = 4, CFM_K_ADALN = 5, CFM_K_CFG_EULER = 6, CFM_K_GEMM_IN = 7,
    CFM_K_GEMM_OUT = 8, CFM_K_HOISTED = 9, CFM_K_XATTN = 10, CFM_K_GEMM_XATTN = 11, CFM_K_COUNT = 12
};
cfm_status cfm_profile_enable(cfm_ctx* ctx, int kernel_class, int capacity);
cfm_status cfm_profile_read(cfm_ctx* ctx, double* total_ms, int* launches, int* dropped);
cfm_status cfm_profile_disable(cfm_ctx* ctx);

/* ---------------------------------------------------------------------------
 * Single-kernel entry points (the same kernels cfm_sample launches), for
 * kernel-level parity tests and roofline measurement.
 *
 * Fused CFG combine + Euler update (VoiceHub "Diffusion and flow TTS optimization",
 * section "Custom Triton and CUDA kernels", lists the guidance combine fused with
 * the Euler step among the kernels worth writing):
 *   for every valid frame (r, t): x[r,t,:] += dt * sum_b w[b] * v[b,r,t,:]
 * v device fp32 [nb, R, Tx, C]; w host fp32 [nb] branch weights (for guidance
 * scale s: w = (1 - s, s); three branches: (1 - s_t, s_t - s_s, s_s));
 * mask device uint8 [R, Tx] or NULL; x device fp32 [R, Tx, C] updated in place.
 * Masked frames of x are not written. C % 4 == 0. */
cfm_status cfm_cfg_euler(const float* v, const float* w, int nb, float dt, const uint8_t* mask,
                         int R, int Tx, int C, float* x, void* stream);

/* bf16 MFMA GEMM with a plain epilogue: C[m,n] = sum_k A[m,k] W[n,k] + bias[n].
 *   A device bf16 (a_is_f32 = 0) or fp32 (a_is_f32 = 1, rounded to bf16 on load)
 *   [M, K] row stride lda; W device bf16 [N, K] row stride ldw; bias device fp32
 *   [N] or NULL. epilogue 0: C fp32; 1: C bf16; 2: C bf16 of GELU(exact erf);
 *   3: gated residual C(fp32) += gate[n] * (acc + bias[n]) with gate device fp32 [N];
 *   4: SwiGLU of a fused gate-up weight stored interleaved in groups of 16 rows
 *      (cfm_tensor_desc, interleave 16): C bf16 [M, N/2],
 *      C[m, 16b + i] = SiLU(acc[m, 32b + i] + bias) * (acc[m, 32b + 16 + i] + bias),
 *      N % 32 == 0 (VoiceHub "Custom Triton and CUDA kernels": SwiGLU; vLLM-Omni
 *      TTS blog "CFM/LocDiT decode-tail batching": fused gate-up MLP).
 * K % 8 == 0 (bf16 A) or K % 4 == 0 (fp32 A); lda, ldw multiples of 8 (bf16)
 * or 4 (fp32 A); ldw >= K rounded up to 8 with zero padding.
 * tile: 0 = chosen from the problem size (what cfm_sample uses); 1 = 128x128
 * tiles, 6 = 128x128 with a K stage of 64, 10 = 64x64, 14 = 256x256 with two
 * wave groups alternating loads and MFMAs (K stage 64), 15 = as 14 on 128x128
 * tiles. Any other value returns
 * CFM_E_VALUE, as does a tile other than 0 or 1 with an fp32 A operand. The GELU
 * of epilogue 2 is evaluated with an erfc approximation of relative error below
 * 1e-5 (bf16 rounding: 2^-9).
 * Layout rules (CFM_E_SHAPE otherwise): ldc >= N (N/2 for epilogue 4), and ldc % 4 == 0 when N > 3
 * (rows of four or more columns are written with vector stores); A, W, C, bias
 * and gate 16-byte aligned. */
cfm_status cfm_gemm_bf16(const void* A, int a_is_f32, int lda, const void* W, int ldw,
                         const float* bias, int M, int N, int K, int epilogue,
                         const float* gate, void* C, int ldc, int tile, void* stream);

/* Key-padding-masked multi-head attention, bf16 in / bf16 out, fp32 softmax
 * (VoiceHub, "Attention" and the padding row of "Semantic-preserving and
 * approximate changes": padded frames are fully masked):
 *   o[row, q, head] = sum_k softmax_k(q.k / sqrt(64), masked keys excluded) v_k
 *   qk device bf16 [rows, T, 2 * H * 64]: q at columns head*64, k at H*64 + head*64
 *   vt device bf16 [rows, H, 64, Tp]: v transposed per head, Tp = T rounded up
 *      to a multiple of 64 (entries past T are never used)
 *   kv_len device int32 [rows]: keys >= kv_len[row] are masked;
 *   key_mask device uint8 [rows, T] (1 = valid key) or NULL;
 *   scratch device memory (16-byte aligned) of at least
 *      rows * 4 + rows * Tp + rows * Tp / 64 + 64 bytes (key validity tables);
 *   o device bf16 [rows, T, H * 64]. A row with no valid key gives o = 0. */
cfm_status cfm_attention_bf16(const void* qk, const void* vt, const int32_t* kv_len,
                              const uint8_t* key_mask, int rows, int T, int H, void* scratch,
                              size_t scratch_bytes, void* o, void* stream);

/* The same attention for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the key-validity tables live in a buffer built into the
 * library, one 8 MiB copy per GPU held until the process ends, so this call
 * allocates nothing. Arguments as cfm_attention_bf16 without scratch; rows * 4
 * + rows * Tp + rows * Tp / 64 + 64 (the scratch size cfm_attention_bf16 asks for)
 * must not exceed 8 MiB
 * (CFM_E_CAPACITY otherwise; e.g. 128 rows of up to 64 000 keys). Every call on a
 * GPU uses that GPU's one buffer: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must be serialised by
 * the caller. Nothing in the buffer needs clearing: each call writes every table
 * entry it reads. Errors as cfm_attention_bf16, plus CFM_E_HIP if the buffer's
 * device address cannot be looked up. */
cfm_status cfm_attention_bf16_noalloc(const void* qk, const void* vt, const int32_t* kv_len,
                                      const uint8_t* key_mask, int rows, int T, int H, void* o,
                                      void* stream);

/* adaLN-modulated LayerNorm: y = LN(h) * (1 + scale) + shift, eps 1e-6, biased
 * variance, stats in fp32. h device fp32 [M, d]; shift, scale device fp32 [d];
 * y device bf16 (out_bf16 = 1) or fp32 [M, d]. d % 4 == 0. */
cfm_status cfm_adaln(const float* h, const float* shift, const float* scale, int M, int d,
                     int out_bf16, void* y, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CFM_MI355X_H */
