// bf16 MFMA GEMM for gfx950: C[m, n] = sum_k A[m, k] W[n, k] with fused epilogues.
//
// Both operands are K-contiguous (A row-major [M, K], W in Linear layout
// [N, K]), the natural operand order of v_mfma_f32_32x32x16_bf16: every lane
// feeds 8 consecutive k of one A row and 8 consecutive k of one W row, so LDS
// tiles are read with 16-byte loads and never transposed.
//
// Kernel family (the `tile` argument selects one; 0 picks by problem size):
//  - gemm_bf16_kernel: register-staged. A block computes a BM x BN tile with
//    WGM x WGN waves; K is staged BK at a time through two padded LDS buffers
//    (global loads of the next stage issued at the top of an iteration, written
//    to the other buffer at its end; fragments of k-step ks+1 read while the
//    MFMAs of ks run). Small and medium problems (128x128 and 64x64 tiles) and
//    fp32 A operands (rounded to bf16 while staging, so no conversion pass
//    touches HBM).
//  - gemm_pp64_kernel: 256x256 tiles for large problems; operands loaded
//    straight into an LDS ring by buffer_load ... lds, with the 8 waves in two
//    groups that alternate load and multiply phases (ping-pong), K stage 64.
// Every variant writes its output through the same per-wave LDS-staged
// epilogues (epilogue.h).
//
// Blocks are numbered so that the tiles one XCD runs at the same time share
// operand rows in that XCD's L2: the hardware deals block ids round-robin to
// the 8 XCDs, so each XCD's ids are mapped to a contiguous range of tile
// numbers, and tiles are walked in groups of GROUP_M block-rows; under a device
// row count the ids follow the walk directly, spreading the working leading
// rows over all XCDs (tile_map.h).
#include <algorithm>
#include <type_traits>

#include "epilogue.h"
#include "tile_map.h"

namespace cfm {
namespace {

constexpr int PAD = 8;        // bf16 elements of padding per LDS row

template <int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
    static constexpr int NT = 64 * WGM * WGN;
    static constexpr int WM = BM / WGM, WN = BN / WGN;         // wave sub-tile
    static constexpr int TM = WM / 32, TN = WN / 32;           // MFMA blocks per wave
    static constexpr int LDK = BK + PAD;
    static constexpr int CPR = BK / 8;                         // 16-byte chunks per row
    static constexpr int LDS_BYTES = 2 * (BM + BN) * LDK * 2;
    static_assert(TM >= 1 && TN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile");
    static_assert(LDS_BYTES >= WGM * WGN * EPI_WAVE_FLOATS * 4, "epilogue staging fits in the operand LDS");
    static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "chunk split");
};

// Raw buffer resource over [rows x ld] elements: loads outside it return 0, so
// the staging loads below need no branches for ragged M, N or K edges (an
// out-of-range chunk is given an offset past the end of the buffer).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, long long bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
constexpr int OOB = 0x7ffffff0;

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int ROWS, int CPR, int NT, int LDK>
struct Bf16Stage {
    static constexpr int CHUNKS = ROWS * CPR / NT;
    i32x4 v[CHUNKS];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int ld, int rows_total, int K, int r0, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = tid + i * NT, row = c / CPR, kc = (c % CPR) * 8;
            const int r = r0 + row, k = k0 + kc;
            const int off = (r < rows_total && k < K) ? (r * ld + k) * 2 : OOB;
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        }
    }
    __device__ __forceinline__ void store(bf16* S, int tid) const {
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = tid + i * NT, row = c / CPR, kc = (c % CPR) * 8;
            *(i32x4*)(S + row * LDK + kc) = v[i];
        }
    }
};

// fp32 A operand: chunks of 4 floats, rounded to bf16 when written to LDS
template <int ROWS, int BK, int NT, int LDK>
struct F32Stage {
    static constexpr int CPR = BK / 4;
    static constexpr int CHUNKS = ROWS * CPR / NT;
    i32x4 v[CHUNKS];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int ld, int rows_total, int K, int r0, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = tid + i * NT, row = c / CPR, kc = (c % CPR) * 4;
            const int r = r0 + row, k = k0 + kc;
            const int off = (r < rows_total && k < K) ? (r * ld + k) * 4 : OOB;
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        }
    }
    __device__ __forceinline__ void store(bf16* S, int tid) const {
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = tid + i * NT, row = c / CPR, kc = (c % CPR) * 4;
            const f32x4 f = __builtin_bit_cast(f32x4, v[i]);
            bf16x4 b;
            b[0] = (bf16)f[0]; b[1] = (bf16)f[1]; b[2] = (bf16)f[2]; b[3] = (bf16)f[3];
            *(bf16x4*)(S + row * LDK + kc) = b;
        }
    }
};

template <typename AT, typename C> struct AStageOf { using type = Bf16Stage<C::BM, C::CPR, C::NT, C::LDK>; };
template <typename C> struct AStageOf<float, C> { using type = F32Stage<C::BM, C::BK, C::NT, C::LDK>; };

template <typename C, typename AT, int EPI>
__global__ void __launch_bounds__(C::NT)
gemm_bf16_kernel(const AT* __restrict__ A, int lda, const bf16* __restrict__ W, int ldw,
                 int M, int N, int K, int tm, int tn, EpiParams ep) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16* const as_base = (bf16*)smem;                          // 2 stages of [BM][LDK]
    bf16* const ws_base = (bf16*)smem + 2 * C::BM * C::LDK;     // 2 stages of [BN][LDK]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int wm = wave / C::WGN, wn = wave % C::WGN;
    int mt, nt;
    tile_of(blockIdx.x, tm * tn, tm, tn, ep.m_dev != nullptr, mt, nt);
    const int m0 = mt * C::BM, n0 = nt * C::BN;
    if (ep.m_dev) {
        M = min(M, *ep.m_dev);
        if (m0 >= M) return;
    }

    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x16{};

    typename AStageOf<AT, C>::type sa;
    Bf16Stage<C::BN, C::CPR, C::NT, C::LDK> sw;
    const __amdgpu_buffer_rsrc_t ra = rsrc_of(A, (long long)M * lda * sizeof(AT));
    const __amdgpu_buffer_rsrc_t rw = rsrc_of(W, (long long)N * ldw * 2);
    const int nk = (K + C::BK - 1) / C::BK;
    sa.load(ra, lda, M, K, m0, 0, tid);
    sw.load(rw, ldw, N, K, n0, 0, tid);
    sa.store(as_base, tid);
    sw.store(ws_base, tid);
    __syncthreads();

    constexpr int KS = C::BK / 16;
    int cur = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) {
            sa.load(ra, lda, M, K, m0, (kt + 1) * C::BK, tid);
            sw.load(rw, ldw, N, K, n0, (kt + 1) * C::BK, tid);
        }
        const bf16* as = as_base + cur * C::BM * C::LDK + (wm * C::WM + li) * C::LDK + lh * 8;
        const bf16* ws = ws_base + cur * C::BN * C::LDK + (wn * C::WN + li) * C::LDK + lh * 8;
        bf16x8 a[2][C::TM], b[2][C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i) a[0][i] = *(const bf16x8*)(as + i * 32 * C::LDK);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) b[0][j] = *(const bf16x8*)(ws + j * 32 * C::LDK);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = ks & 1;
            if (ks + 1 < KS) {
#pragma unroll
                for (int i = 0; i < C::TM; ++i) a[c ^ 1][i] = *(const bf16x8*)(as + i * 32 * C::LDK + (ks + 1) * 16);
#pragma unroll
                for (int j = 0; j < C::TN; ++j) b[c ^ 1][j] = *(const bf16x8*)(ws + j * 32 * C::LDK + (ks + 1) * 16);
            }
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            sa.store(as_base + (cur ^ 1) * C::BM * C::LDK, tid);
            sw.store(ws_base + (cur ^ 1) * C::BN * C::LDK, tid);
        }
        __syncthreads();
        cur ^= 1;
    }

    // epilogue through LDS, reusing the operand buffers (every wave is past its
    // last read of them once it passes this barrier)
    __syncthreads();
    float* wl = (float*)smem + wave * EPI_WAVE_FLOATS;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            epi_block<EPI>(ep, acc[i][j], wl, m0 + wm * C::WM + i * 32, n0 + wn * C::WN + j * 32, M, N, lane);
}

template <typename C, typename AT, int EPI>
void launch_cfg(const AT* A, int lda, const bf16* W, int ldw, int M, int N, int K,
                const EpiParams& ep, hipStream_t s) {
    const int tn = (N + C::BN - 1) / C::BN, tm = (M + C::BM - 1) / C::BM;
    static const bool attr = [] {
        return hipFuncSetAttribute((const void*)gemm_bf16_kernel<C, AT, EPI>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES) == hipSuccess;
    }();
    (void)attr;
    gemm_bf16_kernel<C, AT, EPI><<<tm * tn, C::NT, C::LDS_BYTES, s>>>(A, lda, W, ldw, M, N, K, tm, tn, ep);
}

// ---------------------------------------------------------------------------
// Large problems: operand tiles go from HBM straight into LDS
// (buffer_load_dwordx4 ... lds: each lane's 16 bytes land at M0 + 16 * lane),
// so no registers stage them. The loads are issued from inline assembly and
// their completion is awaited explicitly (s_waitcnt vmcnt before the barrier
// that publishes a stage), so the compiler neither knows about nor waits on
// them; the main loop contains no other vector-memory instruction, and
// everything is drained before the epilogue issues its own loads. M0 is written
// only by these sequences (the compiler reserves M0 and sets it itself right
// before each of its own uses; these kernels have none).
template <int BM_, int BN_, int WGM_, int WGN_>
struct PCfg {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int TM = WM / 32, TN = WN / 32;
    static_assert(TM >= 1 && TN >= 1, "wave tile");
};

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, int voff, unsigned lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rs) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Ping-pong with K stage 64 (tile 14): 128-byte LDS rows (one cache line per
// row per stage, eight rows per load instruction), a 2-slot ring of 64 KiB
// slots, and phases of 32 MFMAs, so a barrier pair is paid per 64 of K instead
// of 32. A slot is refilled only when every other reader of the rows a wave
// loads has passed a barrier after reading them. Group 0's waves load A (64 rows
// each, read by the waves of both groups) at the start of their M(j - 1), after
// the barrier that ends group 1's reads of stage j - 2 (same slot; group 0 read
// it a phase earlier). Group 1's waves load W, each exactly the 64 rows of the
// column quarter it multiplies, at the end of their M(j - 2), right after their
// own reads of the slot: the only other reader of those rows, the group-0 wave
// of the same quarter, read them a phase earlier. (A split in which every wave
// loads rows that other waves of its own group read would race here.) Group 0
// awaits its part at the end of its C(j - 1), group 1 at the end of its M(j - 1):
// both waits come before the barrier after which group 0 reads stage j, and both
// leave two phases for the loads to land.
constexpr int BK64 = 64;

__device__ __forceinline__ int swz64(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// One operand's share of a K-64 stage: INSTR loads of 8 rows each. Per lane
// only the row base and the swizzled chunk are kept (the swizzle of a row group
// alternates between two patterns, c and c ^ 4); everything else is uniform.
template <int INSTR>
__device__ __forceinline__ void dma_stage64(__amdgpu_buffer_rsrc_t rs, int ld, int rows_total, int K, int r0,
                                            int k0, unsigned slot_addr, int w4, int lane) {
    const int lr = lane >> 3;                              // row within a group
    const int c0 = (lane & 7) ^ (lane >> 4);               // chunk fetched in even groups (odd: c0 ^ 4)
    const int g0 = w4 * INSTR;                             // first group of this wave (uniform)
    const int rbase = (r0 + g0 * 8 + lr) * ld * 2;        // byte offset of this lane's row in group g0
    const int rows_left = rows_total - r0 - g0 * 8 - lr;   // rows of this lane's column still in range
    const int k_left = K - k0;
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
        const int c = ((g0 + i) & 1) ? (c0 ^ 4) : c0;
        const bool ok = i * 8 < rows_left && c * 8 < k_left;
        const int off = ok ? rbase + i * 8 * ld * 2 + (k0 + c * 8) * 2 : OOB;
        dma16(rs, off, __builtin_amdgcn_readfirstlane(slot_addr + (g0 + i) * 8 * BK64 * 2));
    }
}

template <typename C> struct Frags64 {
    bf16x8 a[BK64 / 16][C::TM], b[BK64 / 16][C::TN];
};

template <typename C>
__device__ __forceinline__ void read_frags64(Frags64<C>& f, const bf16* as, const bf16* ws, int wm, int wn, int li,
                                             int lh) {
#pragma unroll
    for (int ks = 0; ks < BK64 / 16; ++ks) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const int row = wm * C::WM + i * 32 + li;
            f.a[ks][i] = *(const bf16x8*)(as + row * BK64 + swz64(row, ks * 2 + lh) * 8);
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int row = wn * C::WN + j * 32 + li;
            f.b[ks][j] = *(const bf16x8*)(ws + row * BK64 + swz64(row, ks * 2 + lh) * 8);
        }
    }
}

// kchunk > 0: split-K. Block b computes the partial product over K-slice b / (tm tn)
// ([kchunk * slice, kchunk * (slice + 1))) of tile b % (tm tn), written as fp32 to
// ep.out + slice * ep.ldo * M (the epilogue must be EPI_F32 with no bias).
template <typename C, int EPI>
__global__ void __launch_bounds__(C::NT)
gemm_pp64_kernel(const bf16* __restrict__ A, int lda, const bf16* __restrict__ W, int ldw,
                 int M, int N, int K, int tm, int tn, EpiParams ep, int kchunk) {
    static_assert(C::WGM == 2 && C::WGN == 4, "two groups of four waves");
    constexpr int SLOT = (C::BM + C::BN) * BK64;                // bf16 elements
    // group 0's waves load A (64 rows each), group 1's waves W (each the 64 rows of
    // the column quarter it multiplies): L loads of 8 rows per wave per stage
    static_assert(C::BM == C::BN && C::BM % (8 * C::WGN) == 0, "equal shares");
    constexpr int L = C::BM / 8 / C::WGN;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16* const ring = (bf16*)smem;
    const unsigned ring_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    // the group decides control flow around barriers: make it provably wave-uniform
    const int grp = __builtin_amdgcn_readfirstlane(wave) / C::WGN, wn = wave % C::WGN;
    int bid = blockIdx.x;
    long long koff = 0;
    if (kchunk > 0) {               // split-K: this block's K-slice and partial-sum plane
        const int slice = bid / (tm * tn);
        bid -= slice * tm * tn;
        koff = (long long)slice * kchunk;
        K = min(kchunk, K - (int)koff);
        ep.out = (float*)ep.out + (long long)slice * M * ep.ldo;
    }
    int mt, nt;
    tile_of(bid, tm * tn, tm, tn, ep.m_dev != nullptr, mt, nt);
    const int m0 = mt * C::BM, n0 = nt * C::BN;
    if (ep.m_dev) {
        M = min(M, *ep.m_dev);
        if (m0 >= M) return;   // whole block, before any barrier
    }
    const __amdgpu_buffer_rsrc_t ra = rsrc_of(A + koff, ((long long)M * lda - koff) * 2);
    const __amdgpu_buffer_rsrc_t rw = rsrc_of(W + koff, ((long long)N * ldw - koff) * 2);
    const int nk = (K + BK64 - 1) / BK64;

    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x16{};

    auto issue = [&](int stage) {   // this wave's share of the stage's rows
        const unsigned slot = ring_addr + (unsigned)((stage & 1) * SLOT * 2);
        if (grp == 0) dma_stage64<L>(ra, lda, M, K, m0, stage * BK64, slot, wn, lane);
        else dma_stage64<L>(rw, ldw, N, K, n0, stage * BK64, slot + C::BM * BK64 * 2, wn, lane);
    };
    auto sync = [&] {
        __builtin_amdgcn_sched_barrier(0);
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
    };
    Frags64<C> f;
    auto reads = [&](int k) {
        const bf16* sl = ring + (k & 1) * SLOT;
        read_frags64<C>(f, sl, sl + C::BM * BK64, grp, wn, li, lh);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    auto compute = [&] {
#pragma unroll
        for (int ks = 0; ks < BK64 / 16; ++ks)
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks][i], f.b[ks][j], acc[i][j], 0, 0, 0);
    };

    issue(0);
    if (nk > 1) { issue(1); wait_vm<L>(); } else { wait_vm<0>(); }
    sync();
    if (grp == 0) {
        for (int k = 0; k < nk; ++k) {
            if (k >= 1 && k + 1 < nk) issue(k + 1);   // first: needed by the end of the next phase
            reads(k);
            sync();
            compute();
            if (k + 1 < nk) wait_vm<0>();   // this wave's part of stage k + 1 has landed
            sync();
        }
    } else {
        for (int k = 0; k < nk; ++k) {
            if (k == 0) sync();
            // stage k + 2 reuses the slot of stage k. This wave refills only the W
            // rows it multiplies itself (reads complete just above); their only
            // other reader, the group-0 wave of the same column quarter, read
            // them a phase earlier, before the last barrier.
            reads(k);
            if (k + 2 < nk) issue(k + 2);
            if (k + 1 < nk) {               // this wave's part of stage k + 1 has landed
                if (k + 2 < nk) wait_vm<L>();
                else wait_vm<0>();
            }
            sync();
            compute();
            if (k + 1 < nk) sync();
        }
    }
    // No block barrier before the epilogue: after its last barrier no wave reads
    // the ring again (group 1's last multiply works from registers) and no load is
    // in flight, so group 0 stages its output in its own 4 KiB area at once,
    // while group 1 is still multiplying.
    wait_vm<0>();
    float* wl = (float*)smem + wave * EPI_WAVE_FLOATS;
    if constexpr (EPI == EPI_GATED) {
        epi_tile_gated<C::TM, C::TN>(ep, acc, wl, m0 + grp * C::WM, n0 + wn * C::WN, M, N, lane);
    } else if constexpr (EPI == EPI_F32 || EPI == EPI_ACT || EPI == EPI_GELU_ACT || EPI == EPI_QKV) {
        // the bias of every column this lane stores, loaded before the first store
        f32x4 b4[C::TN];
        float b1[C::TN];
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int nj = n0 + wn * C::WN + j * 32;
            const int n4 = nj + (lane & 7) * 4, n1 = nj + li;
            b4[j] = ep.bias && n4 + 3 < N ? *(const f32x4*)(ep.bias + n4) : f32x4{};
            b1[j] = ep.bias && n1 < N ? ep.bias[n1] : 0.0f;
        }
        // one wait the compiler sees: from here on no load is outstanding, so no
        // store below is followed by a wait for it (the counter covers stores too)
        __builtin_amdgcn_s_waitcnt(0);
        auto blocks = [&](auto pk) {
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    epi_block<EPI, decltype(pk)::value>(ep, acc[i][j], wl, m0 + grp * C::WM + i * 32,
                                                        n0 + wn * C::WN + j * 32, M, N, lane, &b4[j], &b1[j]);
        };
        // packed rows (their lookups load) and plain rows (no load) as separate code
        if (EPI == EPI_QKV && ep.tok_row != nullptr) blocks(std::true_type{});
        else blocks(std::false_type{});
    } else {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                epi_block<EPI>(ep, acc[i][j], wl, m0 + grp * C::WM + i * 32, n0 + wn * C::WN + j * 32, M, N, lane);
    }
}

using PP = PCfg<256, 256, 2, 4>;   // 8 waves in two groups of four, 128x64 per wave
using PP128 = PCfg<128, 128, 2, 4>;   // the same schedule on 128x128 tiles, 64x32 per wave

template <typename C, int EPI>
void launch_pp64(const bf16* A, int lda, const bf16* W, int ldw, int M, int N, int K,
                 const EpiParams& ep, hipStream_t s, int splits = 1, int kchunk = 0) {
    const int tn = (N + C::BN - 1) / C::BN, tm = (M + C::BM - 1) / C::BM;
    constexpr int LDS = 2 * (C::BM + C::BN) * BK64 * 2;
    static_assert(LDS >= C::NW * EPI_WAVE_FLOATS * 4, "epilogue staging fits in the ring");
    static const bool attr = [] {
        return hipFuncSetAttribute((const void*)gemm_pp64_kernel<C, EPI>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, LDS) == hipSuccess;
    }();
    (void)attr;
    gemm_pp64_kernel<C, EPI><<<tm * tn * splits, C::NT, LDS, s>>>(A, lda, W, ldw, M, N, K, tm, tn, ep, kchunk);
}

// Split-K reduction: out tile = epilogue(sum over the slices' fp32 partial products),
// four columns per thread, slices summed in order (the result does not depend on
// how the blocks ran). Rows past the device row count are skipped.
template <int EPI>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N, EpiParams ep) {
    const long long plane = (long long)M * N;     // one slice's partial products, [M, N]
    if (ep.m_dev) M = min(M, *ep.m_dev);
    const int n4 = N / 4;
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)M * n4) return;
    const int m = (int)(i / n4), n = (int)(i - (long long)m * n4) * 4;
    f32x4 v = *(const f32x4*)(part + (long long)m * N + n);
    for (int sl = 1; sl < splits; ++sl) v += *(const f32x4*)(part + sl * plane + (long long)m * N + n);
    epi_store_vec4<EPI>(ep, m, n, v);
}

// Row-wise reduction of the gated-residual epilogue fused with the next adaLN norm:
// one block of 256 threads per row (up to 4096 columns: 4 float4 per thread), every
// load of the row (its K-slices, bias, gate and residual) issued at once, the slices
// summed in slice order plus bias and gated into the residual row (the arithmetic of
// epi_store_vec4<EPI_GATED>), then the two-pass mean / variance of the updated row
// (mean 0 for RMSNorm) and the modulated, bf16-rounded norm output. The row sums
// follow the adaLN kernel's order exactly (per lane l of a 64-lane wave, the float4
// chunks l, l + 64, l + 128, ... in turn, then the wave's butterfly), so the norm
// output has the same bits as the separate adaLN kernel's.
constexpr int LNF_V = 4;          // float4 per thread
constexpr int LNF_SPLITS = 4;     // most K-slices the split-K path makes
// sum over the row in the adaLN kernel's order: part[k][l] holds chunk 64 k + l's
// contribution (k < nk); lane l of wave 0 adds its chunks in k order, the wave sums
// the lanes, and every thread gets the result
__device__ __forceinline__ float row_sum_adaln_order(float (*part)[64], int nk, float* out) {
    __syncthreads();
    if (threadIdx.x < 64) {
        float v = 0.0f;
        for (int k = 0; k < nk; ++k) v += part[k][threadIdx.x];
        v = wave_sum(v);
        if (threadIdx.x == 0) *out = v;
    }
    __syncthreads();
    return *out;
}
__global__ void __launch_bounds__(256)
splitk_reduce_ln_kernel(const float* __restrict__ part, int splits, int M, int N, EpiParams ep) {
    __shared__ float rp[LNF_V * 4][64];
    __shared__ float rsum[2];
    const long long plane = (long long)M * N;
    if (ep.m_dev) M = min(M, *ep.m_dev);
    const int m = blockIdx.x, t = threadIdx.x;
    if (m >= M) return;                              // block-uniform
    const int n4 = N / 4;
    // the adaLN kernel's float4 count per lane: the next power of two of ceil(n4 / 64)
    const int q = (n4 + 63) / 64, nk = q <= 1 ? 1 : q <= 2 ? 2 : q <= 4 ? 4 : q <= 8 ? 8 : 16;
    const float* g = ep.gate.at(m);
    float* hrow = (float*)ep.out + (long long)m * ep.ldo;
    f32x4 sl[LNF_V][LNF_SPLITS], hv[LNF_V], gv[LNF_V], bv[LNF_V];
#pragma unroll
    for (int i = 0; i < LNF_V; ++i) {
        const int c = t + 256 * i, n = 4 * c;
        const bool in = c < n4;
#pragma unroll
        for (int k = 0; k < LNF_SPLITS; ++k)
            sl[i][k] = in && k < splits ? *(const f32x4*)(part + k * plane + (long long)m * N + n) : f32x4{};
        hv[i] = in ? *(const f32x4*)(hrow + n) : f32x4{};
        gv[i] = in ? *(const f32x4*)(g + n) : f32x4{};
        bv[i] = in && ep.bias ? *(const f32x4*)(ep.bias + n) : f32x4{};
    }
#pragma unroll
    for (int i = 0; i < LNF_V; ++i) {
        const int c = t + 256 * i;
        if (c < n4) {
            f32x4 v = sl[i][0];
#pragma unroll
            for (int k = 1; k < LNF_SPLITS; ++k)
                if (k < splits) v += sl[i][k];
            v += bv[i];
            hv[i] += gv[i] * v;
            *(f32x4*)(hrow + 4 * c) = hv[i];
        }
        if (c / 64 < nk) rp[c / 64][c & 63] = c < n4 ? (hv[i][0] + hv[i][1]) + (hv[i][2] + hv[i][3]) : 0.0f;
    }
    const float mean = ep.ln_rms ? 0.0f : row_sum_adaln_order(rp, nk, &rsum[0]) / (float)N;
#pragma unroll
    for (int i = 0; i < LNF_V; ++i) {
        const int c = t + 256 * i;
        if (c / 64 < nk) {
            float sq = 0.0f;
            if (c < n4) {
                const f32x4 z = hv[i] - mean;
                sq = (z[0] * z[0] + z[1] * z[1]) + (z[2] * z[2] + z[3] * z[3]);
            }
            rp[c / 64][c & 63] = sq;
        }
    }
    const float rstd = rsqrtf(row_sum_adaln_order(rp, nk, &rsum[1]) / (float)N + 1e-6f);
    const float* sh = ep.ln_shift.at(m);
    const float* sc = ep.ln_scale.at(m);
    bf16* yrow = (bf16*)ep.ln_y + (long long)m * N;
#pragma unroll
    for (int i = 0; i < LNF_V; ++i) {
        const int c = t + 256 * i;
        if (c < n4) {
            const int n = 4 * c;
            const f32x4 y = (hv[i] - mean) * rstd * (*(const f32x4*)(sc + n) + 1.0f) + *(const f32x4*)(sh + n);
            bf16x4 b;
            b[0] = (bf16)y[0]; b[1] = (bf16)y[1]; b[2] = (bf16)y[2]; b[3] = (bf16)y[3];
            *(bf16x4*)(yrow + n) = b;
        }
    }
}

// The partial products of a split-K GEMM (EPI_F32, no bias, fp32 planes in the
// caller's split workspace), then the reduction with the real epilogue (and, for the
// gated residual with ep.ln_y set, the next norm: returns true then).
template <int EPI>
bool launch_splitk(const bf16* A, int lda, const bf16* W, int ldw, int M, int N, int K, const EpiParams& ep,
                   int splits, hipStream_t s) {
    const int kchunk = (K / splits + BK64 - 1) / BK64 * BK64;
    EpiParams pe;
    pe.out = ep.split_ws;
    pe.ldo = N;
    pe.m_dev = ep.m_dev;
    launch_pp64<PP128, EPI_F32>(A, lda, W, ldw, M, N, K, pe, s, splits, kchunk);
    if constexpr (EPI == EPI_GATED) {
        if (ep.ln_y != nullptr && N <= LNF_V * 4 * 256 && splits <= LNF_SPLITS) {
            splitk_reduce_ln_kernel<<<M, 256, 0, s>>>(ep.split_ws, splits, M, N, ep);
            return true;
        }
    }
    const long long n = (long long)M * (N / 4);
    splitk_reduce_kernel<EPI><<<(int)((n + 255) / 256), 256, 0, s>>>(ep.split_ws, splits, M, N, ep);
    return false;
}


// tile configurations (index = the `tile` argument; 0 = automatic)
using C1 = Cfg<128, 128, 32, 2, 2>;     // 4 waves, 64x64 per wave
using C6 = Cfg<128, 128, 64, 2, 2>;     // 4 waves, 64x64 per wave, deeper K stage
using C10 = Cfg<64, 64, 64, 2, 2>;      // 4 waves, 32x32 per wave: small problems
using CF = Cfg<128, 128, 32, 2, 2>;     // fp32 A operands

template <typename AT, int EPI>
bool launch_epi(int tile, const AT* A, int lda, const bf16* W, int ldw, int M, int N, int K,
                const EpiParams& ep, hipStream_t s) {
    if constexpr (std::is_same<AT, float>::value) {
        launch_cfg<CF, AT, EPI>(A, lda, W, ldw, M, N, K, ep, s);
    } else {
        if (tile == 0) {
            // the largest tile that still gives about one tile per CU or more; 256x256
            // and 128x128 tiles run the K-64 ping-pong kernel, unless N and K are both
            // small (then the register-staged 128x128 kernel, whose fixed cost is
            // lower, wins)
            const long long big = (long long)((M + 255) / 256) * ((N + 255) / 256);
            const long long mid = (long long)((M + 127) / 128) * ((N + 127) / 128);
            tile = big >= 192 ? (N >= 1024 || K >= 1024 ? 14 : 1) : mid >= 160 ? 15 : 10;
            // few 128x128 tiles and a long K: split K over 128x128 tiles when the
            // caller provides room for the partial products (gated-residual and plain
            // fp32 epilogues, which take four columns at a time). The slice count
            // depends on K alone, so a row's result does not depend on how many other
            // rows share the call while the batch stays in this regime.
            if (tile == 10 && (EPI == EPI_GATED || EPI == EPI_F32) && ep.split_ws != nullptr && N % 4 == 0) {
                const int splits = (int)std::min(4, K / 512);
                if (splits >= 2 && (long long)M * N * splits <= ep.split_ws_floats)
                    return launch_splitk<EPI>(A, lda, W, ldw, M, N, K, ep, splits, s);
            }
        }
        switch (tile) {
            case 6: launch_cfg<C6, AT, EPI>(A, lda, W, ldw, M, N, K, ep, s); break;
            case 10: launch_cfg<C10, AT, EPI>(A, lda, W, ldw, M, N, K, ep, s); break;
            case 14: launch_pp64<PP, EPI>(A, lda, W, ldw, M, N, K, ep, s); break;
            case 15: launch_pp64<PP128, EPI>(A, lda, W, ldw, M, N, K, ep, s); break;
            default: launch_cfg<C1, AT, EPI>(A, lda, W, ldw, M, N, K, ep, s); break;
        }
    }
    return false;
}

template <typename AT>
bool launch_a(int tile, int epi, const AT* A, int lda, const bf16* W, int ldw, int M, int N, int K,
              const EpiParams& ep, hipStream_t s) {
    switch (epi) {
        case EPI_F32: launch_epi<AT, EPI_F32>(tile, A, lda, W, ldw, M, N, K, ep, s); break;
        case EPI_ACT: launch_epi<AT, EPI_ACT>(tile, A, lda, W, ldw, M, N, K, ep, s); break;
        case EPI_GELU_ACT: launch_epi<AT, EPI_GELU_ACT>(tile, A, lda, W, ldw, M, N, K, ep, s); break;
        case EPI_GATED: return launch_epi<AT, EPI_GATED>(tile, A, lda, W, ldw, M, N, K, ep, s);
        case EPI_INPROJ: launch_epi<AT, EPI_INPROJ>(tile, A, lda, W, ldw, M, N, K, ep, s); break;
        case EPI_VOUT: launch_epi<AT, EPI_VOUT>(tile, A, lda, W, ldw, M, N, K, ep, s); break;
        case EPI_QKV: launch_epi<AT, EPI_QKV>(tile, A, lda, W, ldw, M, N, K, ep, s); break;
        case EPI_SWIGLU: launch_epi<AT, EPI_SWIGLU>(tile, A, lda, W, ldw, M, N, K, ep, s); break;
        case EPI_VOUT_EULER: launch_epi<AT, EPI_VOUT_EULER>(tile, A, lda, W, ldw, M, N, K, ep, s); break;
        default: break;
    }
    return false;
}

}  // namespace

bool launch_gemm_bf16(bool a_f32, int epi, const void* A, int lda, const bf16* W, int ldw,
                      int M, int N, int K, const EpiParams& ep, hipStream_t s, int tile) {
    if (M <= 0 || N <= 0) return false;
    if (a_f32) return launch_a<float>(tile, epi, (const float*)A, lda, W, ldw, M, N, K, ep, s);
    return launch_a<bf16>(tile, epi, (const bf16*)A, lda, W, ldw, M, N, K, ep, s);
}

}  // namespace cfm
