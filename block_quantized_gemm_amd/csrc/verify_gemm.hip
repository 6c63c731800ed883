// verify_gemm.hip -- the verification matmul for a draft block of <= 16 rows.
//
// "Qwen3.8-27B on the AMD R9700: up to 227 tok/s", section "A block-diffusion
// drafter, verified exactly": the target checks a whole draft block in one
// batched forward that reads the weights once, so 16 rows cost about what one
// row costs.  This file is that product for two weight formats:
//   Q4_0 -- "Qwen3.8-27B at 45.7 tok/s ...", section "Prompt processing":
//           4-bit codes with offset 8 in blocks of 32, one fp16 scale per block;
//   FP8  -- "r9k: a from-scratch inference engine ...", opening paragraph:
//           E4M3 weights with one scale per 128 x 128 tile.
//
// Arithmetic (gfx950, wave64):
//  * One MFMA 16x16x32 (bf16 or fp16) per (16 output features x 32 k); A is
//    the activation block (rows zero-padded to 16), B the weights.  The same
//    instruction sequence runs for every N <= 16, so an output row never
//    depends on N (the pages compare outputs byte for byte across block
//    widths, "What 'lossless' means here, precisely").
//  * Q4_0: every lane streams one 16-byte block of one feature; a 4x4
//    lane-group transpose (permlane swaps) hands each lane its 4-byte slice of
//    each block; codes become the exact 16-bit values MAGIC + q; an MFMA with
//    the constant -(MAGIC + 8) forms the per-row offset term (once per block,
//    shared by all of the wave's tiles), which enters the block MFMA as its
//    accumulator, so the MFMA returns the block sum (q - 8) x in fp32.  The
//    fp16 block scale is one fp32 FMA per output.
//  * FP8: 32 contiguous bytes per lane per 128-wide step, hardware E4M3 ->
//    16-bit conversion (exact), 4 MFMAs per step, one FMA with the fp32 tile
//    scale.
//
// Data movement (the kernels are bound by HBM and by memory latency):
//  * A workgroup is W waves; each wave owns T tiles of 16 features, so a
//    workgroup covers a tile group of TG = T * W tiles.  Weights stream with
//    16-byte raw buffer loads (rows past M read as zeros) PF steps of 128 k
//    ahead of the math, in registers.
//  * Activations (16 rows) are staged in LDS with buffer loads that write LDS
//    directly; every staged element serves the TG tiles.  Q4_0 block scales
//    are staged the same way.
//  * With a workspace (the normal case) the walk kernel runs persistent
//    workgroups, each walking one contiguous share of the launch's chunks
//    (tile group x 8 steps, 4 on panel weights): the weight pipeline never drains between
//    chunks, the next chunk's activations and scales load into the other of
//    two LDS buffers, a tile group inside the share is summed in registers
//    over all of K, and a tile group cut between two shares is finished from
//    its fp32 parts added in share order (the same result on every run):
//    by the last of its workgroups to arrive, from pieces in the workspace,
//    or, when the next share's part is in before a share's last chunk, by
//    the share's own workgroup, from registers.
//  * Q4_0 weights come row-major or in the panel layout, where each chunk (4
//    steps) of a 256-feature tile group is one 72 KiB record read front to
//    back with non-temporal loads.
//  * Without a workspace the one-shot kernel gives each workgroup a whole
//    tile group over all of K, staged chunk by chunk.
#include "vq_device.h"
#include "vq_internal.h"

#include <atomic>

namespace vq {

constexpr int kStepK = 128;  // k per step: 4 Q4_0 blocks or one FP8 chunk

// One problem of a launch (kernel arguments, by value).
struct KProblem {
    const uint8_t *w;     // Q4_0 codes [M][K/2] or E4M3 bytes [M][K]
    const void *scales;   // Q4_0 f16 [M][K/32] or FP8 f32 [ceil(M/128)][K/128]
    const uint16_t *act;  // this row group's [<=16][K] activations
    void *out;            // this row group's [<=16][M] outputs
    int M, K;
    int chunk;            // one-shot kernel: steps per LDS chunk
    int cpt;              // walk kernel: chunks (8 steps, 4 on panel weights) per tile group
    int ntg;              // tile groups
    int item0;            // first item of this problem in the launch (a tile group, or a chunk)
};

// A launch: up to kGroupPerLaunch problems sharing the launch shape, the row
// count (<= 16), the output dtype and alpha.  Item i belongs to the last
// problem whose item0 <= i.  The walk kernel's pieces and arrival counters
// live in the caller's workspace.
struct KGroup {
    KProblem p[kGroupPerLaunch];
    int item0[kGroupPerLaunch];  // p[i].item0, packed for one batch of scalar loads
    int count, items, N, out_dtype;
    int share, extra;            // walk kernel: items = share * grid + extra (range arithmetic in 32 bits); the
                                 // walk kernel takes these, count and N as scalar arguments
    float alpha;
    float *part;    // pieces: [workgroups][2 sides][TG tiles][64 lanes][4]
    uint32_t *cnt;  // arrival counters: [workgroups][waves], zero between calls
};

// LDS layout:
//  activations: 16 rows x kActPitch bytes, row-major (row r, element k of the
//    staged chunk at r * kActPitch + 2k), one chunk of at most 8 steps; the
//    16 bytes of padding stagger the rows over the LDS banks;
//  Q4_0 scales: a row of 4 * CH fp16 per feature (CH = the chunk bound).
constexpr int kActPitch = 2 * 1024 + 16;
constexpr int kActLdsBytes = 16 * kActPitch;
constexpr int kOut = 0x7FFFFFF0;  // an offset past every buffer: the load returns zeros

// Most steps per LDS chunk for a workgroup of W waves (the activation chunk is
// moved by 32 load instructions of 1 KB shared out over the waves).
__host__ __device__ constexpr int max_chunk_steps(int W) { return W >= 4 ? 8 : 4; }

__host__ __device__ inline int verify_tile_groups_dev(int M, int tg) { return ((M + 15) / 16 + tg - 1) / tg; }

// Pipeline depth: stages of weight loads in flight per wave.
__host__ __device__ constexpr int pipeline_depth(bool fp8, int T) { return ((fp8 ? 2 * T : T) >= 4) ? 2 : 4; }

// Q4_0 scale pieces (16 bytes) per feature row, and load instructions for the
// rows of T tiles (one instruction moves 64 pieces).
__host__ __device__ constexpr int scale_pieces(int W) { return max_chunk_steps(W) / 2; }
__host__ __device__ constexpr int scale_insts(int T, int W) { return (T * 16 * scale_pieces(W) + 63) / 64; }

__device__ __forceinline__ int steps_of(bool fp8, int K) { return fp8 ? (K >> 7) : (((K >> 5) + 3) >> 2); }

// ---------------------------------------------------------------------------
// The math of one step of 128 k for one wave's T tiles.
//   row  -- LDS: activation row j (= lane & 15); element e' of the step sits
//           at byte o0 + 2e' from it (o0: the step's byte offset in the
//           staged chunk)
//   sc   -- LDS (Q4_0): scale row of feature j of tile 0 at the step's first
//           block; tile t's row is 16 * t * scrow halves further
//   w    -- the step's weight registers; ts -- FP8 tile scales
//   PRE  -- Q4_0 codes already in lane-group order (dword q of lane group g =
//           dword g of block q), as the panel layout stores them
// ---------------------------------------------------------------------------
template <int ACT, bool FP8, int T, int WB, bool PRE = false>
__device__ __forceinline__ void step_math(const uint8_t *row, int o0, int g, const uint16_t *sc,
                                          int scrow, const u32x4 (&w)[T][WB], const float (&ts)[T],
                                          f32x4 (&acc)[T]) {
    using A16 = Act16<ACT>;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    auto at = [&](int byte) { return row + o0 + byte; };
    // A operand of lane (g, r): row r; Q4_0 block q: x[4g..4g+3] and
    // x[16+4g..16+4g+3] of the block (the order q4_operand gives the codes);
    // FP8 MFMA u: x[32g + 8u .. +8] of the step
    auto a_operand = [&](int q) {
        if constexpr (FP8) {
            return *reinterpret_cast<const u32x4 *>(at(2 * (32 * g + 8 * q)));
        } else {
            const u32x2 lo = *reinterpret_cast<const u32x2 *>(at(2 * (32 * q + 4 * g)));
            const u32x2 hi = *reinterpret_cast<const u32x2 *>(at(2 * (32 * q + 16 + 4 * g)));
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    };
    if constexpr (FP8) {
        u32x4 av[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            av[q] = a_operand(q);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            f32x4 part = zero4;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4 src = w[t][u >> 1];
                const uint32_t e0 = src[2 * (u & 1)], e1 = src[2 * (u & 1) + 1];
                const u32x4 bop = {A16::template fp8x2<false>(e0), A16::template fp8x2<true>(e0),
                                   A16::template fp8x2<false>(e1), A16::template fp8x2<true>(e1)};
                part = A16::mfma(av[u], bop, part);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[t][r] = __builtin_fmaf(ts[t], part[r], acc[t][r]);
        }
    } else {
        // block-major: per 32-k block one offset MFMA shared by the T tiles,
        // then each tile's block MFMA and scale FMA
        const u32x4 negc = {A16::kNegOffset, A16::kNegOffset, A16::kNegOffset, A16::kNegOffset};
        uint32_t d[T][4];
        u32x2 scp[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            d[t][0] = w[t][0][0];
            d[t][1] = w[t][0][1];
            d[t][2] = w[t][0][2];
            d[t][3] = w[t][0][3];
            if constexpr (!PRE)  // lane group g: dword g of blocks 0..3 (panel codes arrive that way)
                transpose_lane_groups(d[t][0], d[t][1], d[t][2], d[t][3]);
            scp[t] = *reinterpret_cast<const u32x2 *>(sc + t * 16 * scrow);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 aq = a_operand(q);
            const f32x4 corr = A16::mfma(aq, negc, zero4);  // -(MAGIC + 8) * sum x, per row
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const f32x4 dot = A16::mfma(aq, q4_operand<A16::kMagicByte>(d[t][q]), corr);
                const float s = h2f((q & 1) ? (scp[t][q >> 1] >> 16) : (scp[t][q >> 1] & 0xFFFFu));
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[t][r] = __builtin_fmaf(s, dot[r], acc[t][r]);
            }
        }
    }
}

// Activation chunk into LDS: rows of this launch's row group, steps
// [s_first, s_first + nc) of K.  Instruction (row r, half h) moves 64
// consecutive 16-byte pieces -- 1 KB of whole cache lines -- of row r; the 32
// instructions are shared out over the W waves.  Pieces past the chunk or past
// K deliver zeros, and so do rows past N (the buffer ends there).
template <int W>
__device__ __forceinline__ void stage_act(uint8_t *act_lds, rsrc_t ra, int K, int s_first, int nc, int wave,
                                          int lane) {
    const int kb = s_first * kStepK;
#pragma unroll
    for (int i = 0; i < 32 / W; ++i) {
        const int inst = wave + W * i;
        const int r = inst >> 1, h = inst & 1;
        const int p = 64 * h + lane;
        const bool ok = p < 16 * nc && kb + 8 * p < K;
        bload16_lds(ra, act_lds + r * kActPitch + h * 1024, ok ? r * K * 2 + 2 * kb + 16 * p : kOut);
    }
}

// Q4_0 scales of `nfeat` feature rows (the buffer starts at the first one)
// for steps [s_first, s_first + nc): row f gets the 4 * CH scales from block
// 4 * s_first on, 16 bytes per lane; instructions inst0, inst0 + inst_step,
// ... (SI of them).  Needs every row start 16-byte aligned (NB % 8 == 0).
template <int W, int SI>
__device__ __forceinline__ void stage_scales(uint8_t *sc_lds, rsrc_t rs, int NB, int nfeat, int s_first, int nc,
                                             int inst0, int inst_step, int lane) {
    constexpr int PPF = scale_pieces(W);
#pragma unroll
    for (int i = 0; i < SI; ++i) {
        const int inst = inst0 + inst_step * i;
        const int f = inst * (64 / PPF) + lane / PPF, pc = lane % PPF;
        const bool ok = f < nfeat && 2 * pc < nc;
        bload16_lds(rs, sc_lds + inst * 1024, ok ? (f * NB + 4 * s_first + 8 * pc) * 2 : kOut);
    }
}

// ---------------------------------------------------------------------------
// One-shot kernel (no workspace): workgroup = one tile group over all of K.
// Items are handed out so that each XCD (workgroups go to the 8 XCDs in
// turn, b % 8) gets one contiguous range of them.
// ---------------------------------------------------------------------------
template <int ACT, bool FP8, int T, int W, int PF>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(T >= 4 ? 2 : 4))) void oneshot_kernel(
    const KGroup grp) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int TG = T * W;
    constexpr int NT = 64 * W;
    constexpr int WB = FP8 ? 2 : 1;
    constexpr int kStepBytes = FP8 ? 128 : 64;
    constexpr int CH = max_chunk_steps(W);
    constexpr int SIW = FP8 ? 0 : (scale_insts(TG, W) + W - 1) / W;
    constexpr int SPT = FP8 ? 1 : (TG * 16 * CH + NT - 1) / NT;
    constexpr int scrow = 4 * CH;
    static_assert(CH % PF == 0, "chunks hold whole pipeline rounds");

    const int b = (int)blockIdx.x;
    const int nq = grp.items >> 3, nr = grp.items & 7;
    const int xcd = b & 7, loc = b >> 3;
    const int item = xcd < nr ? xcd * (nq + 1) + loc : nr * (nq + 1) + (xcd - nr) * nq + loc;
    int pi = 0;
    for (int q = 1; q < grp.count; ++q)
        if (item >= grp.p[q].item0)
            pi = q;
    const KProblem &a = grp.p[pi];
    const int lane = threadIdx.x & 63, wave = wave_id(), j = lane & 15, g = lane >> 4;
    const int M = a.M, K = a.K, NB = K >> 5;
    const int steps = steps_of(FP8, K);
    const int tg = item - a.item0;
    const int nrows = grp.N;
    const int fwg = tg * TG * 16, fwv = fwg + wave * T * 16;
    const int wrow = FP8 ? K : (K >> 1);
    const int chunk = a.chunk;

    uint8_t *act_lds = lds;
    uint8_t *sc_lds = lds + kActLdsBytes;

    const int wfeat = max(0, min(M - fwv, T * 16));
    const rsrc_t rw = make_rsrc(a.w + (size_t)min(fwv, M) * wrow, (uint32_t)wfeat * (uint32_t)wrow);
    const int vw = j * wrow + (FP8 ? 32 : 16) * g;
    const float *tsrow[T];
    if constexpr (FP8) {
#pragma unroll
        for (int t = 0; t < T; ++t)
            tsrow[t] = static_cast<const float *>(a.scales) + (size_t)(min(fwv + 16 * t, M - 1) >> 7) * steps;
    }
    u32x4 wb[PF][T][WB];
    float tsb[PF][T];
    // the step offset is part of the range-checked per-lane offset: the
    // partial last Q4_0 step of the last row reads zeros, not past the array
    auto issue = [&](auto U, int st) {
        const int koff = vw + kStepBytes * st;
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
            for (int h = 0; h < WB; ++h)
                wb[U.value][t][h] = bload16<kAuxCached>(rw, koff + t * 16 * wrow + 16 * h, 0);
            if constexpr (FP8)
                tsb[U.value][t] = tsrow[t][st];
            else
                tsb[U.value][t] = 0.f;
        }
    };

    const rsrc_t ra = make_rsrc(a.act, (uint32_t)nrows * (uint32_t)K * 2u);
    const int wgfeat = max(0, min(M - fwg, TG * 16));
    const uint8_t *sbase = FP8 ? nullptr : static_cast<const uint8_t *>(a.scales) + (size_t)min(fwg, M) * NB * 2;
    const rsrc_t rs = make_rsrc(sbase, FP8 ? 0u : (uint32_t)wgfeat * (uint32_t)NB * 2u);
    const bool sc_dma = (NB & 7) == 0;
    u32x2 ss[SPT];
    auto stage_sc_load = [&](int c0, int nc) {  // scales through registers (NB % 8 != 0)
        if constexpr (!FP8) {
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                const int e = threadIdx.x + NT * i;
                const int fi = e / CH, st = e % CH;
                const int blk = 4 * (c0 + st);
                const bool ok = st < nc && fi < TG * 16;
                const int off = (fi * NB + blk) * 2;
                uint32_t hw[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    hw[q] = bload2<kAuxCached>(rs, ok && blk + q < NB ? off + 2 * q : kOut, 0);
                ss[i] = u32x2{hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16)};
            }
        }
    };
    auto stage_sc_store = [&]() {
        if constexpr (!FP8) {
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                const int e = threadIdx.x + NT * i;
                const int fi = e / CH, st = e % CH;
                if (fi < TG * 16)
                    *reinterpret_cast<u32x2 *>(sc_lds + (fi * scrow + 4 * st) * 2) = ss[i];
            }
        }
    };
    auto stage = [&](int c0, int nc) {
        stage_act<W>(act_lds, ra, K, c0, nc, wave, lane);
        if constexpr (!FP8) {
            if (sc_dma)
                stage_scales<W, SIW>(sc_lds, rs, NB, wgfeat, c0, nc, wave, W, lane);
            else
                stage_sc_load(c0, nc);
        }
    };

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](auto U, int st, int c0) {
        const uint16_t *sc =
            reinterpret_cast<const uint16_t *>(sc_lds) + ((wave * T) * 16 + j) * scrow + 4 * (st - c0);
        step_math<ACT, FP8, T, WB>(act_lds + j * kActPitch, (st - c0) * (2 * kStepK), g, sc, scrow, wb[U.value],
                                   tsb[U.value], acc);
    };

    // prologue: the first chunk's staging, the first PF steps of weights
    const int nc0 = min(chunk, steps);
    stage(0, nc0);
    if (steps >= PF) {
        static_for<PF>([&](auto U) { issue(U, U.value); });
        wait_vmcnt<PF * T * WB>();  // this wave's staging has landed
    } else {
        static_for<PF>([&](auto U) {
            if (U.value < steps)
                issue(U, U.value);
        });
        wait_vmcnt<0>();
    }
    if (!FP8 && !sc_dma)
        stage_sc_store();
    __syncthreads();

    for (int c0 = 0; c0 < steps; c0 += chunk) {
        const int c1 = min(steps, c0 + chunk);
        if (c0 > 0) {
            __syncthreads();
            stage(c0, c1 - c0);
            wait_vmcnt<0>();
            if (!FP8 && !sc_dma)
                stage_sc_store();
            __syncthreads();
        }
        int i = c0;
        while (i + 2 * PF <= c1) {
            static_for<PF>([&](auto U) {
                compute(U, i + U.value, c0);
                __builtin_amdgcn_sched_barrier(0);
                issue(U, i + U.value + PF);
                __builtin_amdgcn_sched_barrier(0);
            });
            i += PF;
        }
        static_for<2 * PF>([&](auto V) {
            constexpr int U = V.value % PF;
            const int st = i + V.value;
            if (st < c1) {
                compute(std::integral_constant<int, U>{}, st, c0);
                if (st + PF < steps)
                    issue(std::integral_constant<int, U>{}, st + PF);
            }
        });
    }

#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int feat = fwv + t * 16 + j;
        if (feat < M) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * g + r;
                if (row < nrows)
                    store_out(a.out, grp.out_dtype, (size_t)row * M + feat, grp.alpha * acc[t][r]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Walk kernel (workspace): persistent workgroups, each walking one contiguous
// range of chunks.  A chunk is one tile group x 8 steps (4 on panel weights); chunks are numbered
// problem by problem, tile group by tile group, along K within a tile group,
// so a workgroup's range is a run of whole tile groups with at most one
// partial tile group at each end.  A tile group that lies inside the range is
// accumulated in registers over all of K and written out directly.  The piece
// of a tile group cut by a range boundary goes to the workspace (fp32, one
// slot per workgroup and side), and the last of its workgroups to arrive adds
// the pieces in range order and writes the outputs.
// ---------------------------------------------------------------------------
constexpr int kWalkSteps = 8;                   // steps per chunk
constexpr int kActBuf = kActLdsBytes;  // one activation buffer: 16 rows x 1024 k at a pitch of kActPitch

// Activation chunk into one buffer, row r at r * kActPitch: the 16 bytes of
// padding per row spread the 16 rows' reads of one element over the LDS
// banks, and keep every read at a constant offset from the lane's row.
// Instruction (row r, half h) moves 64 consecutive 16-byte pieces (1 KiB of
// whole cache lines); a load instruction into LDS writes lane l's 16 bytes to
// byte 16 l of its destination.  The 32 instructions are shared out over the
// W waves; pieces past the chunk or past K, and rows past N, read zeros.
template <int W, int HALVES = 2>
__device__ __forceinline__ void stage_act_rows(uint8_t *buf, rsrc_t ra, int K, int s_first, int nc, int wave,
                                               int lane) {
    const int kb = s_first * kStepK;
    constexpr int kInsts = 16 * HALVES;
#pragma unroll
    for (int i = 0; i < (kInsts + W - 1) / W; ++i) {
        const int inst = wave + W * i;
        if (kInsts % W != 0 && inst >= kInsts)
            break;
        const int r = inst / HALVES, h = inst % HALVES;
        const int p = 64 * h + lane;
        const bool ok = p < 16 * nc && kb + 8 * p < K;
        bload16_lds(ra, buf + r * kActPitch + h * 1024, ok ? r * K * 2 + 2 * kb + 16 * p : kOut);
    }
}

// Position of a chunk: problem, tile group, chunk within the tile group.
struct ChunkRef {
    int pi, tg, c;
};

// The problem that holds chunk `it` (a linear search over the launch's
// problems: once per workgroup; later chunks are reached by next_chunk).
__device__ __forceinline__ int find_problem(const int (&item0)[kGroupPerLaunch], int count, int it) {
    int pi = 0;
#pragma unroll
    for (int q = 1; q < kGroupPerLaunch; ++q)
        pi += (q < count && it >= item0[q]) ? 1 : 0;
    return pi;
}
__device__ __forceinline__ ChunkRef chunk_in(const KProblem &a, int pi, int it) {
    const int loc = it - a.item0;
    const int tg = loc / a.cpt;
    return ChunkRef{pi, tg, loc - tg * a.cpt};
}

// The chunk after r, a chunk of problem a (past the launch's last chunk it
// stays on the last problem; such chunks are never real).
__device__ __forceinline__ ChunkRef next_chunk(int count, const KProblem &a, ChunkRef r) {
    if (++r.c == a.cpt) {
        r.c = 0;
        if (++r.tg == a.ntg) {
            r.tg = 0;
            r.pi = min(r.pi + 1, count - 1);
        }
    }
    return r;
}

// Problems whose first chunk the walk kernel takes as a scalar argument.
constexpr int kPreloadFirst = 8;

// First chunk of workgroup b's range, floor(b * items / G), and the workgroup
// whose range holds chunk c.  Ranges hold share or share + 1 chunks, and the
// longer ones are spread evenly over the logical ids (so over the XCDs, which
// take contiguous runs of ids); items = share * G + extra keeps the start in
// 32 bits.
__device__ __forceinline__ int range_start(int b, int share, int extra, int G) {
    return b * share + (b * extra) / G;
}
__device__ __forceinline__ int range_owner(const KGroup &grp, int c, int G) {
    return (int)(((int64_t)(c + 1) * G - 1) / grp.items);
}

// The launch constants that place a workgroup's first chunk come first, as
// plain scalar arguments: the command processor writes them into SGPRs
// before the first instruction (kernel-argument preloading, enabled for this
// file by the build), so the first chunk's problem records are the kernel's
// first memory round trip.  G is the grid size, i1..i8 the first chunks of
// problems 1..8 (launches of more than 9 problems load item0 instead).
template <int ACT, bool FP8, int T, int W, int PF, bool PANEL>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void walk_kernel(
    int G, int share, int extra, int count, int nrows, int i1, int i2, int i3, int i4, int i5, int i6, int i7, int i8,
    const KGroup grp) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int TG = T * W;
    constexpr int WB = FP8 ? 2 : 1;
    constexpr int kStepBytes = FP8 ? 128 : 64;
    constexpr int CH = (PANEL && !FP8) ? kPanelSteps : kWalkSteps;
    constexpr int SIW = FP8 ? 0 : T;       // scale loads per wave per chunk: 16 feature rows x 64 bytes each
    constexpr int kScBuf = SIW * 1024;     // one wave's scale buffer
    constexpr int scrow = 4 * CH;          // scales per feature row in the buffer
    constexpr int kIssueLoads = PF * T * WB;
    constexpr int kCoherent = 0x10;        // sc1: agent-coherent, no cache maintenance needed
    static_assert(CH % PF == 0, "chunks hold whole pipeline rounds");
    static_assert(PANEL || scale_pieces(4) * 2 == CH, "scale rows of one chunk");
    static_assert(!PANEL || FP8 ||
                      (T == kPanelWaveTiles && W == kPanelWaves && CH == kPanelSteps &&
                       T * kPanelTileScaleBytes == 1024),
                  "one Q4_0 panel record per chunk, one 1 KiB scale load per wave");
    static_assert(!PANEL || !FP8 || (T == 1 && W * 16 == kFp8PanelFeatures && CH == kFp8PanelSteps),
                  "one FP8 panel record per chunk, one tile per wave");

    const int lane = threadIdx.x & 63, wave = wave_id(), j = lane & 15, g = lane >> 4;
    float *const part = grp.part;
    // Workgroups go to the 8 XCDs in turn (blockIdx % 8); give each XCD a
    // contiguous run of ranges, so that the workgroups sharing an L2 walk
    // neighbouring tile groups and reuse each other's activation chunks.
    const int b = xcd_run_index((int)blockIdx.x, G);
    // (ib < ie: the grid never exceeds the launch's chunks)
    const int ib = range_start(b, share, extra, G), ie = range_start(b + 1, share, extra, G);
    uint8_t *sc_wave = lds + 2 * kActBuf + wave * 2 * kScBuf;  // this wave's two scale buffers

    // ---- weights of a chunk for this wave's T tiles (chunks past the range read zeros)
    struct Src {
        rsrc_t rw;
        int vw, s0, steps, wrow;
        const float *ts[T];
    };
    auto make_src = [&](const ChunkRef &r, const KProblem &a, bool real) {
        Src src;
        const int M = a.M, K = a.K;
        src.wrow = FP8 ? K : (K >> 1);
        src.steps = steps_of(FP8, K);
        src.s0 = r.c * CH;
        if constexpr (PANEL && !FP8) {  // the chunk's record; tile t of step s at 16 KiB * s + 1 KiB * t
            src.rw = make_rsrc(a.w + ((size_t)r.tg * a.cpt + r.c) * kPanelRecordBytes,
                               real ? (uint32_t)kPanelRecordBytes : 0u);
            src.vw = wave * T * 1024 + 16 * lane;
            return src;
        }
        const int fwv = (r.tg * TG + wave * T) * 16;
        if constexpr (PANEL && FP8) {  // the chunk's record; this wave's step s, half h at 16 KiB * s + 1 KiB * h
            src.rw = make_rsrc(a.w + ((size_t)r.tg * a.cpt + r.c) * kFp8RecordBytes,
                               real ? (uint32_t)kFp8RecordBytes : 0u);
            src.vw = wave * 2048 + 16 * lane;
            src.ts[0] = static_cast<const float *>(a.scales) + (size_t)(min(fwv, M - 1) >> 7) * src.steps;
            return src;
        }
        const int wfeat = real ? max(0, min(M - fwv, T * 16)) : 0;
        src.rw = make_rsrc(a.w + (size_t)min(fwv, M) * src.wrow, (uint32_t)wfeat * (uint32_t)src.wrow);
        src.vw = j * src.wrow + (FP8 ? 32 : 16) * g;
        if constexpr (FP8) {
#pragma unroll
            for (int t = 0; t < T; ++t)
                src.ts[t] = static_cast<const float *>(a.scales) +
                            (size_t)(min(fwv + 16 * t, M - 1) >> 7) * src.steps;
        }
        return src;
    };
    u32x4 wb[PF][T][WB];
    float tsb[PF][T];
    auto issue = [&](auto U, const Src &src, int st) {
        const int gs = src.s0 + st;
        const bool ok = gs < src.steps;
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
            for (int h = 0; h < WB; ++h)
                // Panel records are read whole, once, front to back: non-temporal
                // loads (measured +6% per layer).  Row-major Q4_0 rows are read 64
                // bytes per step, the other half of each 128-byte line a step
                // later, which the default policy keeps in L2 (non-temporal: -7%).
                // A panel record holds zeros for its steps past K, so its loads
                // need no step check (a chunk past the range has a resource of
                // size 0); dropping the per-load select gained 0.6-1.2% per layer.
                wb[U.value][t][h] = bload16<(PANEL ? kAuxStream : kAuxCached)>(
                    src.rw,
                    PANEL && FP8 ? src.vw + (W * 2048) * st + 1024 * h
                    : PANEL      ? src.vw + kPanelTiles * 1024 * st + 1024 * t
                    : !ok        ? kOut
                                 : src.vw + kStepBytes * gs + t * 16 * src.wrow + 16 * h,
                    0);
            if constexpr (FP8)
                tsb[U.value][t] = src.ts[t][min(gs, src.steps - 1)];
            else
                tsb[U.value][t] = 0.f;
        }
    };

    // ---- a chunk's activations (whole workgroup) and this wave's scales
    auto act_for = [&](const ChunkRef &r, const KProblem &a, bool real, int buf) {
        const int steps = steps_of(FP8, a.K);
        const int s0 = r.c * CH;
        const rsrc_t ra = make_rsrc(a.act, real ? (uint32_t)nrows * (uint32_t)a.K * 2u : 0u);
        stage_act_rows<W, CH / 4>(lds + buf * kActBuf, ra, a.K, s0, min(CH, steps - s0), wave, lane);
    };
    auto scales_for = [&](const ChunkRef &r, const KProblem &a, bool real, int buf) {
        if constexpr (PANEL && !FP8) {  // this wave's 1 KiB of the record's scale rows (its T tiles)
            // non-temporal like the record's codes: read once (+0.6 to +0.8%
            // per layer in three alternating pairs against the default policy)
            const rsrc_t rs = make_rsrc(a.w + ((size_t)r.tg * a.cpt + r.c) * kPanelRecordBytes,
                                        real ? (uint32_t)kPanelRecordBytes : 0u);
            bload16_lds<kAuxStream>(rs, sc_wave + buf * kScBuf, kPanelCodeBytes + wave * 1024 + 16 * lane);
        } else if constexpr (!FP8) {
            const int NB = a.K >> 5, M = a.M;
            const int steps = steps_of(false, a.K);
            const int s0 = r.c * CH;
            const int fwv = (r.tg * TG + wave * T) * 16;
            const int nfeat = real ? max(0, min(M - fwv, T * 16)) : 0;
            const rsrc_t rs = make_rsrc(static_cast<const uint8_t *>(a.scales) + (size_t)min(fwv, M) * NB * 2,
                                        (uint32_t)nfeat * (uint32_t)NB * 2u);
            stage_scales<4, SIW>(sc_wave + buf * kScBuf, rs, NB, nfeat, s0, min(CH, steps - s0), 0, 1, lane);
        }
    };

    // ---- outputs and pieces
    const rsrc_t rp = make_rsrc(part, (uint32_t)G * 2u * TG * 1024u);
    auto slot_off = [&](int wg, int side, int t) { return ((wg * 2 + side) * TG + wave * T + t) * 1024 + lane * 16; };
    auto store_tiles = [&](const KProblem &a, int tg, const f32x4 (&v)[T]) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int feat = (tg * TG + wave * T + t) * 16 + j;
            if (feat < a.M) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * g + r;
                    if (row < nrows)
                        store_out(a.out, grp.out_dtype, (size_t)row * a.M + feat, grp.alpha * v[t][r]);
                }
            }
        }
    };
    int pend_pi[2] = {-1, -1}, pend_tg[2] = {0, 0};  // this workgroup's pieces, by side
    // the first and last chunk of each piece's tile group (kept from when the
    // piece was stored, so that counting in needs no load of the problem)
    int pend_first[2] = {0, 0}, pend_end[2] = {0, 0};
    // Side 0 (a tile group that ends in this range, begun in an earlier one)
    // is counted in at the chunk boundary after its piece was stored, so the
    // end of the range does not wait for that round trip: 0 nothing to count,
    // 1 piece stored, 2 counted in (old0: the count before this arrival).
    int s0_state = 0;
    uint32_t old0 = 0u;

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- prologue: the first chunk's activations and scales, the first
    // round of weights.  The first chunk's problem record and the next
    // problem's are read by value, in one round of loads.
    int it = ib;
    int pi0;
    if (count <= kPreloadFirst + 1) {
        const int first[kPreloadFirst] = {i1, i2, i3, i4, i5, i6, i7, i8};
        pi0 = 0;
#pragma unroll
        for (int q = 1; q <= kPreloadFirst; ++q)
            pi0 += (q < count && it >= first[q - 1]) ? 1 : 0;
    } else {
        int item0[kGroupPerLaunch];
#pragma unroll
        for (int q = 0; q < kGroupPerLaunch; ++q)
            item0[q] = grp.item0[q];
        pi0 = find_problem(item0, count, it);
    }
    const KProblem P0 = grp.p[pi0], P1 = grp.p[min(pi0 + 1, count - 1)];
    __builtin_amdgcn_sched_barrier(0);
    ChunkRef cref = chunk_in(P0, pi0, it);
    ChunkRef nref = next_chunk(count, P0, cref);
    const KProblem PN = nref.pi == pi0 ? P0 : P1;
    Src cur = make_src(cref, P0, true);
    Src nxt = make_src(nref, PN, it + 1 < ie);
    act_for(cref, P0, true, 0);
    scales_for(cref, P0, true, 0);
    static_for<PF>([&](auto U) { issue(U, cur, U.value); });
    wait_vmcnt<kIssueLoads>();  // the first chunk's activations and scales have landed
    lds_barrier();

    int par = 0;
    const uint8_t *row = lds + j * kActPitch;
    // The range's last chunk may begin a tile group that the next range
    // finishes at its own start; that range's count is normally in before
    // this one ends.  The counter is read during the second-to-last chunk
    // and looked at after that chunk's boundary wait (which already covers
    // it); if the other part has arrived it is loaded then, lands during the
    // last chunk, and the tile group is finished here, without storing this
    // part, counting in and reading it back.  (Reading the counter within
    // the chunk that uses it made the compiler wait for every older load at
    // that point in every chunk: the register it lands in was reused.)
    bool want1 = false, early1 = false;
    uint32_t cnt1 = 0u;
    f32x4 p1[T];
    for (;;) {
        // The next chunk's activations and scales go into the other buffers
        // (free: every wave passed the barrier after the chunk that used
        // them).  Issued before this chunk's math, after its first round of
        // weights, on every path: the compiler's waits for those weights
        // then never include the staging.
        act_for(nref, grp.p[nref.pi], it + 1 < ie, par ^ 1);
        if constexpr (PANEL && !FP8)  // nref's scale rows, through the resource nxt already holds for its record
            bload16_lds<kAuxStream>(nxt.rw, sc_wave + (par ^ 1) * kScBuf, kPanelCodeBytes + wave * 1024 + 16 * lane);
        else
            scales_for(nref, grp.p[nref.pi], it + 1 < ie, par ^ 1);
        const KProblem &ca = grp.p[cref.pi];
        const uint8_t *abuf = row + par * kActBuf;
        const uint16_t *sc0 = reinterpret_cast<const uint16_t *>(sc_wave + par * kScBuf) + j * scrow;
        if (it + 2 == ie) {  // the last chunk is nref
            const KProblem &na = grp.p[nref.pi];
            const int first = na.item0 + nref.tg * na.cpt;
            want1 = first >= ib && first + na.cpt > ie && range_owner(grp, first + na.cpt - 1, G) == b + 1;
            if (want1 && lane == 0)
                cnt1 = __hip_atomic_load(grp.cnt + b * W + wave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int rd = 0; rd < CH / PF; ++rd) {
            // this round's loads fetch the next round of this chunk, or the
            // first round of the next chunk
            const bool to_next = rd == CH / PF - 1;
            const Src &src = to_next ? nxt : cur;
            const int st0 = to_next ? 0 : (rd + 1) * PF;
            static_for<PF>([&](auto U) {
                const int st = rd * PF + U.value;
                step_math<ACT, FP8, T, WB, PANEL>(abuf, st * (2 * kStepK), g, sc0 + 4 * st, scrow, wb[U.value],
                                                  tsb[U.value], acc);
                __builtin_amdgcn_sched_barrier(0);
                issue(U, src, st0 + U.value);
                __builtin_amdgcn_sched_barrier(0);
            });
        }

        // ---- chunk boundary.  Everything but the newest round of weights is
        // complete after this wait: the next chunk's activations and this
        // wave's scales for it have landed.
        wait_vmcnt<kIssueLoads>();
        const bool last = it + 1 >= ie;
        if (s0_state == 1) {
            // the side-0 piece, stored at an earlier boundary, is complete
            // (older than the newest round): count in now
            const int b0 = range_owner(grp, pend_first[0], G);
            if (lane == 0)
                old0 = __hip_atomic_fetch_add(grp.cnt + b0 * W + wave, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s0_state = 2;
        }
        if (cref.c == ca.cpt - 1 || last) {  // this workgroup's part of the tile group is done
            const int first = ca.item0 + cref.tg * ca.cpt;
            if (first >= ib && first + ca.cpt <= ie) {
                store_tiles(ca, cref.tg, acc);
            } else if (early1) {
                // both parts in registers: added in range order (this part
                // first), as the last arrival would; the counter is left at zero
#pragma unroll
                for (int t = 0; t < T; ++t)
                    p1[t] = acc[t] + p1[t];
                store_tiles(ca, cref.tg, p1);
                if (lane == 0)
                    __hip_atomic_store(grp.cnt + b * W + wave, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                const int side = first + ca.cpt > ie ? 1 : 0;  // 1: the tile group goes on past this range
#pragma unroll
                for (int t = 0; t < T; ++t)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[t]), rp,
                                                           slot_off(b, side, t), 0, kCoherent);
                pend_pi[side] = cref.pi;
                pend_tg[side] = cref.tg;
                pend_first[side] = first;
                pend_end[side] = first + ca.cpt - 1;
                if (side == 0)
                    s0_state = 1;
            }
#pragma unroll
            for (int t = 0; t < T; ++t)
                acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (last)
            break;
        if (want1 && it + 2 == ie) {
            // the count (complete after the boundary wait); the other part is
            // read only after its arrival was seen
            early1 = __builtin_amdgcn_readfirstlane(cnt1) == 1u;
            if (early1) {
#pragma unroll
                for (int t = 0; t < T; ++t)
                    p1[t] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, slot_off(b + 1, 0, t), 0, kCoherent));
            }
        }
        lds_barrier();  // every wave is done with buffer `par`, and sees the next chunk's activations
        ++it;
        cref = nref;
        nref = next_chunk(count, grp.p[nref.pi], nref);
        cur = nxt;
        nxt = make_src(nref, grp.p[nref.pi], it + 1 < ie);
        par ^= 1;
    }

    // ---- pieces: count in (per wave: each wave owns its T tiles), and the
    // last arrival adds the pieces in range order.  The pieces were written
    // with agent-coherent stores that are complete after this wait.
    // Both sides' arrivals go out before either count is looked at: one
    // round trip to the coherence point instead of two.
    wait_vmcnt<0>();
    int b0s[2] = {0, 0}, b1s[2] = {0, 0};
    uint32_t old[2] = {0u, 0u};
#pragma unroll
    for (int side = 0; side < 2; ++side) {
        if (pend_pi[side] < 0)
            continue;
        b0s[side] = range_owner(grp, pend_first[side], G);
        b1s[side] = range_owner(grp, pend_end[side], G);
        if (side == 0 && s0_state == 2)
            old[0] = old0;  // counted in during the walk
        else if (lane == 0)
            old[side] = __hip_atomic_fetch_add(grp.cnt + b0s[side] * W + wave, 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int side = 0; side < 2; ++side) {
        if (pend_pi[side] < 0)
            continue;
        const KProblem &a = grp.p[pend_pi[side]];
        const int b0 = b0s[side], b1 = b1s[side];
        if (__builtin_amdgcn_readfirstlane(old[side]) != (uint32_t)(b1 - b0))
            continue;
        if (lane == 0)  // every piece has arrived: leave the counter at zero for the next call
            __hip_atomic_store(grp.cnt + b0 * W + wave, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // The pieces' loads go out kSumBatch workgroups at a time (one round
        // trip for the usual two to four pieces); the adds keep range order.
        // The explicit wait before the stores matters: without it every
        // output store waits for the one before it to complete.
        constexpr int kSumBatch = 4;
        f32x4 sum[T];
        for (int wg0 = b0; wg0 <= b1; wg0 += kSumBatch) {
            f32x4 v[kSumBatch][T];
#pragma unroll
            for (int u = 0; u < kSumBatch; ++u) {
                const int wg = wg0 + u;
#pragma unroll
                for (int t = 0; t < T; ++t)
                    v[u][t] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   rp, wg <= b1 ? slot_off(wg, wg < b1 ? 1 : 0, t) : kOut, 0, kCoherent));
            }
            wait_vmcnt<0>();
#pragma unroll
            for (int u = 0; u < kSumBatch; ++u) {
                if (wg0 + u > b1)
                    break;
#pragma unroll
                for (int t = 0; t < T; ++t)
                    sum[t] = wg0 + u == b0 ? v[u][t] : sum[t] + v[u][t];
            }
        }
        store_tiles(a, pend_tg[side], sum);
    }
}

// ---------------------------------------------------------------------------
// Q4_0 panel layout.  A panel is 256 consecutive features (16 tiles of 16), a
// chunk 4 steps of 128 k; record (panel p, chunk c) of a matrix with C chunks
// per panel starts at byte (p * C + c) * kPanelRecordBytes and holds
//   codes:  for step s, tile t, lane l = 16 g + j, at 16 KiB * s + 1 KiB * t +
//           16 l: dword q (q = 0..3) is dword g (bytes 4g..4g+3) of block
//           4 (4c + s) + q of feature 256p + 16t + j -- what the lane would
//           hold after loading block 4 (4c + s) + g and the lane-group
//           transpose;
//   scales: at 64 KiB + 512 B * t: the fp16 scales of the tile's 16 features,
//           feature-major, 16 blocks (16c .. 16c + 15) each.
// Features past M and blocks past K/32 are zeros.  A workgroup of 8 waves (2
// tiles each) reads one record per chunk front to back: 16 KiB per step, then
// the scales; each staged activation chunk (16 rows x 512 k) serves 256
// features.  The repack runs once per matrix; every thread writes one 16-byte
// piece.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void panel_pack_kernel(const uint32_t *codes, const uint16_t *scales, int M,
                                                         int K, int chunks, int64_t pieces, u32x4 *panel) {
    constexpr int kPieces = kPanelRecordBytes / 16, kCodePieces = kPanelCodeBytes / 16;
    const int NB = K >> 5;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pieces; i += (int64_t)gridDim.x * 256) {
        const int64_t rec = i / kPieces;
        const int in = (int)(i - rec * kPieces);
        const int p = (int)(rec / chunks), c = (int)(rec - (int64_t)p * chunks);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (in < kCodePieces) {
            const int s = in / (kPanelTiles * 64), t = (in >> 6) % kPanelTiles, l = in & 63, g = l >> 4, j = l & 15;
            const int m = kPanelFeatures * p + 16 * t + j;
            if (m < M) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int blk = 4 * (kPanelSteps * c + s) + q;
                    if (blk < NB)
                        v[q] = codes[(size_t)m * (K >> 3) + 4 * blk + g];
                }
            }
        } else {
            constexpr int kTilePieces = kPanelTileScaleBytes / 16, kFeatPieces = kTilePieces / 16;
            const int t = (in - kCodePieces) / kTilePieces, l = (in - kCodePieces) % kTilePieces;
            const int m = kPanelFeatures * p + 16 * t + l / kFeatPieces,
                      b0 = 4 * kPanelSteps * c + 8 * (l % kFeatPieces);
            if (m < M) {
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    h[e] = b0 + e < NB ? scales[(size_t)m * NB + b0 + e] : 0u;
                v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
            }
        }
        panel[i] = v;
    }
}

// ---------------------------------------------------------------------------
// FP8 panel layout: record (p, c) of a matrix with C records per panel (128
// features x 8 steps of 128 k) starts at byte (p * C + c) * kFp8RecordBytes;
// at 16 KiB * s + 2 KiB * w + 1 KiB * h + 16 l it holds the 16 bytes
// [128 (8c + s) + 32 g + 16 h, +16) of feature 128 p + 16 w + j (g = l / 16,
// j = l % 16): what lane l of wave w loads for half h of step s when it reads
// the row-major matrix.  Features past M and steps past K are zeros.  Every
// thread writes one 16-byte piece.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8_panel_pack_kernel(const u32x4 *w, int M, int K, int chunks,
                                                             int64_t pieces, u32x4 *panel) {
    constexpr int kPieces = kFp8RecordBytes / 16;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pieces; i += (int64_t)gridDim.x * 256) {
        const int64_t rec = i / kPieces;
        const int in = (int)(i - rec * kPieces);
        const int p = (int)(rec / chunks), c = (int)(rec - (int64_t)p * chunks);
        const int s = in >> 10, wv = (in >> 7) & 7, h = (in >> 6) & 1, l = in & 63;
        const int m = kFp8PanelFeatures * p + 16 * wv + (l & 15);
        const int k0 = 128 * (kFp8PanelSteps * c + s) + 32 * (l >> 4) + 16 * h;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (m < M && k0 < K)
            v = w[((size_t)m * K + k0) >> 4];
        panel[i] = v;
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
namespace {

int device_cus() {
    static std::atomic<int> cus{0};
    int v = cus.load(std::memory_order_relaxed);
    if (v == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cus.store(v, std::memory_order_relaxed);
    }
    return v;
}

template <typename Kern>
int resident_groups(Kern kern, int threads, size_t shm) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(kern), threads, shm) !=
            hipSuccess ||
        n <= 0)
        n = 1;
    return n * device_cus();
}

// Walk-kernel pipeline depth: steps of weight loads in flight per wave (one
// workgroup per CU; 4 steps of 1-2 tiles or 2 steps of wider ones; FP8 with
// one tile per wave, 32 bytes per lane and step, 8 steps: measured +3% on
// the FP8 stream, while Q4_0 row-major gained nothing from 8).
__host__ __device__ constexpr int walk_depth(bool fp8, int T) {
    return fp8 && T == 1 ? 8 : (fp8 ? 2 * T : T) >= 4 ? 2 : 4;
}

template <int ACT, bool FP8, int T, int W, bool PANEL = false>
hipError_t launch_tw(const VerifyLaunch &l) {
    constexpr int TG = T * W;
    const VerifyPlan &pl = l.probs[0].plan;
    const bool walk = pl.walk;
    const size_t shm = verify_lds_bytes(FP8, T, W, walk);
    const auto wkern = walk_kernel<ACT, FP8, T, W, walk_depth(FP8, T), PANEL>;
    void (*okern)(KGroup) = nullptr;
    if constexpr (W <= 8 && !PANEL) {  // the one-shot kernel takes 2, 4 or 8 waves
        okern = oneshot_kernel<ACT, FP8, T, W, pipeline_depth(FP8, T)>;
    } else if (!walk) {
        return hipErrorInvalidValue;
    }
    const void *kern = walk ? reinterpret_cast<const void *>(wkern) : reinterpret_cast<const void *>(okern);
    if (shm > 64 * 1024 && hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm) != hipSuccess)
        return hipErrorInvalidValue;
    KGroup grp{};
    grp.count = l.count;
    grp.out_dtype = l.out_dtype;
    grp.alpha = l.alpha;
    int64_t items = 0;
    for (int i = 0; i < l.count; ++i) {
        const VerifyProblem &q = l.probs[i];
        KProblem &k = grp.p[i];
        k.w = static_cast<const uint8_t *>(q.w);
        k.scales = q.scales;
        k.M = q.M;
        k.K = q.K;
        k.chunk = q.plan.chunk;
        k.ntg = verify_tile_groups(q.M, TG);
        constexpr int kChunk = (PANEL && !FP8) ? kPanelSteps : kWalkSteps;
        k.cpt = (verify_steps(FP8, q.K) + kChunk - 1) / kChunk;
        k.item0 = (int)items;
        items += walk ? (int64_t)k.ntg * k.cpt : k.ntg;
    }
    if (items >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    grp.items = (int)items;
    int grid = (int)items;  // the walk kernel relies on grid <= items: every range holds a chunk
    if (walk) {
        grid = std::min(grid, resident_groups(kern, 64 * W, shm));
        grid = std::min(grid, pl.groups > 0 ? std::min(pl.groups, kMaxWalkGroups) : kMaxWalkGroups);
        grp.cnt = static_cast<uint32_t *>(l.workspace);
        grp.part = reinterpret_cast<float *>(static_cast<char *>(l.workspace) + kWalkCounterBytes);
        if (grid < 1 || grid > items)  // the kernel does not check for an empty range
            return hipErrorInvalidValue;
        grp.share = (int)(items / grid);
        grp.extra = (int)(items % grid);  // below grid <= 1024: b * extra stays in 32 bits
    }
    if (l.used) {
        *l.used = walk ? kWalkCounterBytes + (size_t)grid * 2 * TG * 1024 : 0;
        return hipSuccess;
    }
    for (int i = 0; i < l.count; ++i)
        grp.item0[i] = grp.p[i].item0;
    // Row groups of 16 run one after another: they share the workspace and
    // are independent otherwise.
    const int groups = (l.N + 15) / 16;
    for (int g0 = 0; g0 < groups; ++g0) {
        grp.N = std::min(16, l.N - g0 * 16);
        for (int i = 0; i < l.count; ++i) {
            const VerifyProblem &q = l.probs[i];
            grp.p[i].act = static_cast<const uint16_t *>(q.act) + (size_t)g0 * 16 * q.K;
            grp.p[i].out = static_cast<char *>(q.out) + (size_t)g0 * 16 * q.M * out_elem_bytes(l.out_dtype);
        }
        if (walk) {
            int first[kPreloadFirst];  // problems past the launch's count are never compared
            for (int q = 1; q <= kPreloadFirst; ++q)
                first[q - 1] = q < l.count ? grp.item0[q] : 0x7FFFFFFF;
            hipLaunchKernelGGL(wkern, dim3(grid), dim3(64 * W), shm, l.stream, grid, grp.share, grp.extra, grp.count,
                               grp.N, first[0], first[1], first[2], first[3], first[4], first[5], first[6], first[7],
                               grp);
        } else {
            hipLaunchKernelGGL(okern, dim3(grid), dim3(64 * W), shm, l.stream, grp);
        }
    }
    return hipGetLastError();
}

template <int ACT, bool FP8, int T>
hipError_t dispatch_w(const VerifyLaunch &l) {
    switch (l.waves) {
    case 2: return launch_tw<ACT, FP8, T, 2>(l);
    case 4: return launch_tw<ACT, FP8, T, 4>(l);
    case 8: return launch_tw<ACT, FP8, T, 8>(l);
    case 12: return T == 1 ? launch_tw<ACT, FP8, 1, 12>(l) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int ACT, bool FP8>
hipError_t dispatch_t(const VerifyLaunch &l) {
    switch (l.tiles) {
    case 1: return dispatch_w<ACT, FP8, 1>(l);
    case 2: return dispatch_w<ACT, FP8, 2>(l);
    case 4: return dispatch_w<ACT, FP8, 4>(l);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int64_t panel_chunks(int K) { return ((int64_t)verify_steps(false, K) + kPanelSteps - 1) / kPanelSteps; }

size_t panel_bytes(int M, int K) {
    return (size_t)((M + kPanelFeatures - 1) / kPanelFeatures) * (size_t)panel_chunks(K) * kPanelRecordBytes;
}

size_t fp8_panel_bytes(int M, int K) {
    const int64_t chunks = ((int64_t)verify_steps(true, K) + kFp8PanelSteps - 1) / kFp8PanelSteps;
    return (size_t)((M + kFp8PanelFeatures - 1) / kFp8PanelFeatures) * (size_t)chunks * kFp8RecordBytes;
}

hipError_t launch_fp8_panel_pack(const void *w, int M, int K, void *panel, hipStream_t stream) {
    const int chunks = (verify_steps(true, K) + kFp8PanelSteps - 1) / kFp8PanelSteps;
    const int64_t pieces = (int64_t)(fp8_panel_bytes(M, K) / 16);
    const int64_t blocks = std::min<int64_t>((pieces + 255) / 256, 65536);
    hipLaunchKernelGGL(fp8_panel_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(w), M, K, chunks, pieces, static_cast<u32x4 *>(panel));
    return hipGetLastError();
}

hipError_t launch_panel_pack(const void *codes, const void *scales, int M, int K, void *panel,
                             hipStream_t stream) {
    const int64_t pieces = (int64_t)(panel_bytes(M, K) / 16);
    const int64_t blocks = std::min<int64_t>((pieces + 255) / 256, 65536);
    hipLaunchKernelGGL(panel_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint32_t *>(codes), static_cast<const uint16_t *>(scales), M, K,
                       (int)panel_chunks(K), pieces, static_cast<u32x4 *>(panel));
    return hipGetLastError();
}

int verify_steps(bool fp8, int K) { return fp8 ? K / 128 : (K / 32 + 3) / 4; }

int verify_tile_groups(int M, int tiles_per_group) { return verify_tile_groups_dev(M, tiles_per_group); }

int64_t verify_chunks(bool fp8, const VerifyPlan &pl, int M, int K) {
    const int chunk = (pl.panel && !fp8) ? kPanelSteps : kWalkSteps;
    return (int64_t)verify_tile_groups(M, pl.tiles * pl.waves) * ((verify_steps(fp8, K) + chunk - 1) / chunk);
}

size_t verify_lds_bytes(bool fp8, int tiles, int waves, bool walk) {
    if (walk)  // two activation buffers; Q4_0: two scale buffers per wave
        return 2 * (size_t)kActBuf + (fp8 ? 0 : (size_t)waves * 2 * tiles * 1024);
    if (fp8)
        return kActLdsBytes;
    const int tg_insts = scale_insts(tiles * waves, waves);
    return kActLdsBytes + (size_t)((tg_insts + waves - 1) / waves) * waves * 1024;
}

size_t verify_walk_workspace(const VerifyPlan &pl, int64_t chunks) {
    if (!pl.walk || chunks <= 0)
        return 0;
    const int64_t cap = pl.groups > 0 ? std::min(pl.groups, kMaxWalkGroups) : kMaxWalkGroups;
    return kWalkCounterBytes + (size_t)std::min(chunks, cap) * 2 * pl.tiles * pl.waves * 1024;
}

// Completes and checks a plan whose tiles, waves and form are set: tiles in
// {1, 2, 4}, waves in {2, 4, 8}, groups >= 0.  The walk kernel's Q4_0 scales
// move in 16-byte pieces, so it needs K % 256 == 0 for row-major weights.
// Panel weights walk with one tile per wave and one panel per workgroup, at
// any K.  The LDS must fit.
bool verify_plan_finish(bool fp8, int M, int K, VerifyPlan &pl) {
    (void)M;
    if (pl.panel) {
        if (!pl.walk || pl.groups < 0)
            return false;
        if (fp8 ? (pl.tiles != 1 || pl.waves * 16 != kFp8PanelFeatures)
                : (pl.tiles != kPanelWaveTiles || pl.waves != kPanelWaves))
            return false;
        pl.chunk = fp8 ? kFp8PanelSteps : kPanelSteps;
        return true;
    }
    if (!(pl.tiles == 1 || pl.tiles == 2 || pl.tiles == 4) || !(pl.waves == 2 || pl.waves == 4 || pl.waves == 8 ||
                                                                 (pl.waves == 12 && pl.tiles == 1 && pl.walk)) ||
        pl.groups < 0)
        return false;
    if (pl.walk) {
        if (!fp8 && K % 256 != 0)
            return false;
        pl.chunk = kWalkSteps;
    } else {
        pl.groups = 0;
        pl.chunk = max_chunk_steps(pl.waves);
    }
    return verify_lds_bytes(fp8, pl.tiles, pl.waves, pl.walk) <= kMaxLdsBytes;
}

hipError_t launch_verify(const VerifyLaunch &l) {
    if (l.count < 1 || l.count > kGroupPerLaunch)
        return hipErrorInvalidValue;
    if (l.probs[0].plan.panel) {
        if (!l.probs[0].plan.walk)
            return hipErrorInvalidValue;
        if (l.fp8) {
            constexpr int kW = kFp8PanelFeatures / 16;
            if (l.tiles != 1 || l.waves != kW)
                return hipErrorInvalidValue;
            return l.act_dtype == VQ_DTYPE_BF16 ? launch_tw<VQ_DTYPE_BF16, true, 1, kW, true>(l)
                                                : launch_tw<VQ_DTYPE_F16, true, 1, kW, true>(l);
        }
        if (l.tiles != kPanelWaveTiles || l.waves != kPanelWaves)
            return hipErrorInvalidValue;
        return l.act_dtype == VQ_DTYPE_BF16
                   ? launch_tw<VQ_DTYPE_BF16, false, kPanelWaveTiles, kPanelWaves, true>(l)
                   : launch_tw<VQ_DTYPE_F16, false, kPanelWaveTiles, kPanelWaves, true>(l);
    }
    if (l.act_dtype == VQ_DTYPE_BF16)
        return l.fp8 ? dispatch_t<VQ_DTYPE_BF16, true>(l) : dispatch_t<VQ_DTYPE_BF16, false>(l);
    return l.fp8 ? dispatch_t<VQ_DTYPE_F16, true>(l) : dispatch_t<VQ_DTYPE_F16, false>(l);
}

}  // namespace vq
