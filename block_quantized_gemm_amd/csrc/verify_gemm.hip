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
// Work decomposition (the kernel is bound by HBM and by what reaches the CUs):
//  * A workgroup is W waves; each wave owns T tiles of 16 features, so the
//    workgroup covers TG = T * W tiles.  K is cut into S slices of `sl` steps
//    of 128; workgroup (tile group, slice) computes its TG tiles over its
//    slice.  The grid is sized so that all workgroups are resident at once
//    and every wave has the same work.
//  * The slice's 16 activation rows (and, for Q4_0, the workgroup's block
//    scales) are staged into LDS in MFMA operand order with whole-line loads;
//    afterwards the waves only read LDS (no barrier inside a chunk).  Each
//    staged activation element serves TG tiles, so activation traffic is
//    1/TG of what a per-tile read would cost.
//  * Weight bytes are streamed with 16-byte raw buffer loads (rows past M read
//    as zeros) PF steps ahead of the compute in a register pipeline.
//  * Slices of one tile group are combined through a caller workspace: each
//    workgroup writes its fp32 partial tiles, then counts itself in; the last
//    to arrive adds the S partials in the fixed order 0, 1, ..., S-1 and
//    stores the output.  No value is combined by atomics, so the result is
//    the same on every run and whichever workgroup finishes last.
//  * A slice longer than one LDS chunk (always the case without a workspace,
//    S = 1) is walked chunk by chunk, re-staging the activations.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

constexpr int kStepK = 128;                    // k per step: 4 Q4_0 blocks or one FP8 chunk
constexpr int kActStepBytes = 16 * kStepK * 2;  // one step of 16 activation rows (bf16/fp16)

// One problem of a launch (kernel arguments, by value).
struct KProblem {
    const uint8_t *w;     // Q4_0 codes [M][K/2] or E4M3 bytes [M][K]
    const void *scales;   // Q4_0 f16 [M][K/32] or FP8 f32 [ceil(M/128)][K/128]
    const uint16_t *act;  // this row group's [<=16][K] activations
    void *out;            // this row group's [<=16][M] outputs
    float *part;          // split: fp32 partial tiles [tile groups][S][TG][64 lanes][4]
    uint32_t *cnt;        // split: arrival counters [tile groups], zero between calls
    int M, K;
    int S, sl, chunk;     // slices, steps per slice, steps per LDS chunk
    int item0;            // first workgroup of this problem in the launch
};

// A launch: up to kGroupPerLaunch problems sharing the launch shape, the row
// count (<= 16), the output dtype and alpha; `items` workgroups in all.  Item
// i belongs to the last problem whose item0 <= i.
struct KGroup {
    KProblem p[kGroupPerLaunch];
    int count, items, N, out_dtype;
    float alpha;
};

// LDS position of activation piece p (k = 8p .. 8p+7 of the step) of row r, in
// the operand layout [32-k group q][lane = 16 g + r][16 bytes]:
//  Q4_0: lane (r, g)'s operand for block q is x[4g .. 4g+3] (first 8 bytes)
//        and x[16+4g .. 16+4g+3] (last 8 bytes) of that block, the order in
//        which q4_operand lays out the codes.  A piece splits over two lanes.
//  FP8:  lane (r, g)'s operand for MFMA u is x[32g + 8u .. +8]: piece p is one
//        whole operand (g = p / 4, u = p % 4).
template <bool FP8>
__device__ __forceinline__ void act_piece_to_lds(uint8_t *tile, int r, int p, u32x4 v) {
    if constexpr (FP8) {
        *reinterpret_cast<u32x4 *>(tile + ((p & 3) * 64 + 16 * (p >> 2) + r) * 16) = v;
    } else {
        const int blk = p >> 2, q = p & 3;
        const int g0 = 2 * (q & 1), half = q >> 1;
        uint8_t *base = tile + blk * 1024 + half * 8;
        *reinterpret_cast<u32x2 *>(base + (16 * g0 + r) * 16) = u32x2{v[0], v[1]};
        *reinterpret_cast<u32x2 *>(base + (16 * (g0 + 1) + r) * 16) = u32x2{v[2], v[3]};
    }
}

// Most steps per LDS chunk for a workgroup of W waves: bounded so that all
// staging loads of a chunk (<= 8 per thread for activations, 2 T for scales)
// can be in flight at once.
__host__ __device__ constexpr int max_chunk_steps(int W) { return W >= 4 ? 8 : 4; }

__host__ __device__ inline int verify_tile_groups_dev(int M, int tg) { return ((M + 15) / 16 + tg - 1) / tg; }

// Pipeline depth: stages of weight loads in flight per wave.
__host__ __device__ constexpr int pipeline_depth(bool fp8, int T) { return ((fp8 ? 2 * T : T) >= 4) ? 2 : 4; }

template <int ACT, bool FP8, int T, int W, int PF>
__global__ __launch_bounds__(64 * W) void verify_kernel(const KGroup grp) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    using A16 = Act16<ACT>;
    constexpr int TG = T * W;                   // tiles per workgroup
    constexpr int NT = 64 * W;                  // threads per workgroup
    constexpr int WB = FP8 ? 2 : 1;             // 16-byte weight loads per lane, tile and step
    constexpr int kStepBytes = FP8 ? 128 : 64;  // weight bytes per feature row per step
    constexpr int CH = max_chunk_steps(W);
    constexpr int kOut = 0x7FFFFFF0;            // an offset past every buffer: the load returns zeros
    static_assert(CH % PF == 0, "chunks hold whole pipeline rounds");

    // ---- this workgroup's item and problem (wave-uniform scalar work).
    // Workgroups are handed to the 8 XCDs in turn (b % 8); each XCD is given
    // one contiguous range of items, so the slices and tile groups that share
    // an activation slice run on one XCD close together in time and find it
    // in that XCD's L2.  (A bijection on [0, items): the result does not
    // depend on where an item runs, only the cache behaviour does.)
    const int b = (int)blockIdx.x;
    const int nq = grp.items >> 3, nr = grp.items & 7;
    const int xcd = b & 7, loc = b >> 3;
    const int it_all = xcd < nr ? xcd * (nq + 1) + loc : nr * (nq + 1) + (xcd - nr) * nq + loc;
    int pi = 0;
    for (int q = 1; q < grp.count; ++q)
        if (it_all >= grp.p[q].item0)
            pi = q;
    const KProblem &a = grp.p[pi];
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int j = lane & 15;
    const int g = lane >> 4;
    const int M = a.M, K = a.K, S = a.S;
    const int NB = K >> 5;
    const int steps = FP8 ? (K >> 7) : ((NB + 3) >> 2);  // the last Q4_0 step may be partial
    const int item = it_all - a.item0;
    const int tg = item / S;
    const int sidx = item - tg * S;
    const int s0 = sidx * a.sl;
    const int ns = min(a.sl, steps - s0);  // >= 1: the host never makes an empty slice
    const int nrows = grp.N;               // <= 16
    const int fwg = tg * TG * 16;          // first feature of the workgroup
    const int fwv = fwg + wave * T * 16;   // first feature of this wave
    const int wrow = FP8 ? K : (K >> 1);   // weight bytes per feature row
    const int chunk = a.chunk;             // <= CH, a multiple of PF

    uint8_t *act_lds = lds;
    uint16_t *sc_lds = reinterpret_cast<uint16_t *>(lds + (size_t)chunk * kActStepBytes);
    const int scrow = 4 * chunk;  // staged scales per feature

    // ---- weights of this wave's T tiles; rows past M read as zeros
    const int wfeat = max(0, min(M - fwv, T * 16));
    const rsrc_t rw = make_rsrc(a.w + (size_t)min(fwv, M) * wrow, (uint32_t)wfeat * (uint32_t)wrow);
    const int vw = j * wrow + (FP8 ? 32 : 16) * g;
    const float *tsrow[T];
    if constexpr (FP8) {
#pragma unroll
        for (int t = 0; t < T; ++t)
            tsrow[t] = static_cast<const float *>(a.scales) + (size_t)(min(fwv + 16 * t, M - 1) >> 7) * steps + s0;
    }

    u32x4 wb[PF][T][WB];
    float tsb[PF][T];
    // The step offset goes into the per-lane offset, which the buffer range
    // check covers: the partial last Q4_0 step of the last row then reads zeros
    // instead of bytes past the end of the array.
    auto issue = [&](auto U, int st) {
        const int koff = vw + kStepBytes * (s0 + st);
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
            for (int h = 0; h < WB; ++h)
                wb[U.value][t][h] = bload16<kAuxCached>(rw, koff + t * 16 * wrow + 16 * h, 0);
            if constexpr (FP8)
                tsb[U.value][t] = tsrow[t][st];
        }
    };

    // ---- staging of one chunk of the slice: activations (and Q4_0 scales).
    // Loads and LDS stores are separate steps so that the loads can be issued
    // before the first weight loads: the wait for them then leaves the weight
    // loads in flight.  Every load is issued (out-of-range ones read zeros),
    // which keeps the compiler's wait counts exact.
    constexpr int LR = NT / 16;                        // threads per activation row
    constexpr int APT = (16 * CH + LR - 1) / LR;       // 16-byte pieces per thread
    constexpr int SPT = FP8 ? 1 : (TG * 16 * 8 + NT - 1) / NT;  // scale loads per thread
    const rsrc_t ra = make_rsrc(a.act, (uint32_t)nrows * (uint32_t)K * 2u);
    const int wgfeat = max(0, min(M - fwg, TG * 16));
    const uint8_t *sbase = FP8 ? nullptr : static_cast<const uint8_t *>(a.scales) + (size_t)min(fwg, M) * NB * 2;
    const rsrc_t rs = make_rsrc(sbase, FP8 ? 0u : (uint32_t)wgfeat * (uint32_t)NB * 2u);
    const int ar = threadIdx.x / LR;  // activation row staged by this thread
    const int alt = threadIdx.x % LR;
    u32x4 sa[APT];
    u32x2 ss[SPT];
    auto stage_load = [&](int c0, int nc) {
        // row ar: consecutive 16-byte pieces (whole cache lines) of the row's
        // nc * 256 contiguous bytes; pieces past K are zeros, rows past N read
        // as zeros
        const int kb = (s0 + c0) * kStepK;
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int p = alt + LR * i;
            const bool ok = p < 16 * nc && kb + 8 * p < K;
            sa[i] = bload16<kAuxCached>(ra, ok ? ar * K * 2 + 2 * kb + 16 * p : kOut, 0);
        }
        if constexpr (!FP8) {
            // scales: 8 threads per feature row, one step (4 blocks) each
            const bool vec = (NB & 3) == 0;
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                const int e = threadIdx.x + NT * i;
                const int fi = e >> 3, st = e & 7;
                const int blk = 4 * (s0 + c0 + st);
                const bool ok = st < nc && fi < TG * 16;
                const int off = (fi * NB + blk) * 2;
                if (vec) {
                    ss[i] = bload8<kAuxCached>(rs, ok ? off : kOut, 0);
                } else {
                    uint32_t h[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        h[b] = bload2<kAuxCached>(rs, ok && blk + b < NB ? off + 2 * b : kOut, 0);
                    ss[i] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
                }
            }
        }
    };
    auto stage_store = [&](int nc) {
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int p = alt + LR * i;
            if (p < 16 * nc)
                act_piece_to_lds<FP8>(act_lds + (p >> 4) * kActStepBytes, ar, p & 15, sa[i]);
        }
        if constexpr (!FP8) {
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                const int e = threadIdx.x + NT * i;
                const int fi = e >> 3, st = e & 7;
                if (st < nc && fi < TG * 16)
                    *reinterpret_cast<u32x2 *>(sc_lds + fi * scrow + 4 * st) = ss[i];
            }
        }
    };

    // ---- the math of one step (st counted from the slice start, c0 = its chunk's start)
    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](auto U, int st, int c0) {
        const uint8_t *tp = act_lds + (st - c0) * kActStepBytes;
        u32x4 av[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            av[q] = *reinterpret_cast<const u32x4 *>(tp + (q * 64 + lane) * 16);
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FP8) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                f32x4 part = zero4;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const u32x4 src = wb[U.value][t][u >> 1];
                    const uint32_t e0 = src[2 * (u & 1)], e1 = src[2 * (u & 1) + 1];
                    const u32x4 bop = {A16::template fp8x2<false>(e0), A16::template fp8x2<true>(e0),
                                       A16::template fp8x2<false>(e1), A16::template fp8x2<true>(e1)};
                    part = A16::mfma(av[u], bop, part);
                }
                const float ts = tsb[U.value][t];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[t][r] = __builtin_fmaf(ts, part[r], acc[t][r]);
            }
        } else {
            const u32x4 negc = {A16::kNegOffset, A16::kNegOffset, A16::kNegOffset, A16::kNegOffset};
            f32x4 corr[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                corr[q] = A16::mfma(av[q], negc, zero4);  // -(MAGIC + 8) * sum x, per row
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const u32x2 scp =
                    *reinterpret_cast<const u32x2 *>(sc_lds + ((wave * T + t) * 16 + j) * scrow + 4 * (st - c0));
                uint32_t d[4] = {wb[U.value][t][0][0], wb[U.value][t][0][1], wb[U.value][t][0][2],
                                 wb[U.value][t][0][3]};
                transpose_lane_groups(d[0], d[1], d[2], d[3]);  // lane group g: dword g of blocks 0..3
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 dot = A16::mfma(av[q], q4_operand<A16::kMagicByte>(d[q]), corr[q]);
                    const float s = h2f((q & 1) ? (scp[q >> 1] >> 16) : (scp[q >> 1] & 0xFFFFu));
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[t][r] = __builtin_fmaf(s, dot[r], acc[t][r]);
                }
            }
        }
    };

    // ---- prologue: staging loads of the first chunk, the first PF steps of
    // weights, then the staged chunk into LDS
    const int nc0 = min(chunk, ns);
    stage_load(0, nc0);
    if (ns >= PF) {
        static_for<PF>([&](auto U) { issue(U, U.value); });
    } else {
        static_for<PF>([&](auto U) {
            if (U.value < ns)
                issue(U, U.value);
        });
    }
    stage_store(nc0);
    __syncthreads();

    // ---- chunks of the slice; weight loads run PF steps ahead across chunks
    for (int c0 = 0; c0 < ns; c0 += chunk) {
        const int c1 = min(ns, c0 + chunk);
        if (c0 > 0) {
            __syncthreads();
            stage_load(c0, c1 - c0);
            stage_store(c1 - c0);
            __syncthreads();
        }
        int i = c0;
        // steady state: every load unconditional, so the compiler counts them
        // and waits only for the stage it is about to use
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
                if (st + PF < ns)
                    issue(std::integral_constant<int, U>{}, st + PF);
            }
        });
    }

    // ---- epilogue
    auto store_tile = [&](int t, f32x4 v) {
        const int feat = fwv + t * 16 + j;
        if (feat < M) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * g + r;
                if (row < nrows)
                    store_out(a.out, grp.out_dtype, (size_t)row * M + feat, grp.alpha * v[r]);
            }
        }
    };
    if (S == 1) {
#pragma unroll
        for (int t = 0; t < T; ++t)
            store_tile(t, acc[t]);
        return;
    }
    // Split K: publish this slice's partial tiles, count in, and let the last
    // workgroup of the tile group add the slices in order.  The partial tiles
    // are written and read with agent-coherent (sc1) accesses, which go
    // through to memory rather than stopping in one die's L2, so no cache
    // writeback or invalidation is needed; the wait before the barrier makes
    // every store complete before the count is taken.
    constexpr int kCoherent = 0x10;  // sc1
    const int ntg = verify_tile_groups_dev(M, TG);
    const rsrc_t rp = make_rsrc(a.part, (uint32_t)ntg * (uint32_t)S * TG * 1024u);
    const int mine = ((tg * S + sidx) * TG + wave * T) * 1024 + lane * 16;
#pragma unroll
    for (int t = 0; t < T; ++t)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[t]), rp, mine + t * 1024, 0, kCoherent);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int *flag = reinterpret_cast<int *>(lds);  // the activation tiles are no longer read
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(a.cnt + tg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == (uint32_t)(S - 1);
        if (last)  // every slice has arrived: leave the counter at zero for the next call
            __hip_atomic_store(a.cnt + tg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
    }
    __syncthreads();
    if (*flag == 0)
        return;
    const int base = (tg * S * TG + wave * T) * 1024 + lane * 16;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
        for (int s8 = 0; s8 < S; s8 += 8) {
            f32x4 v[8];  // eight slices' loads in flight at once
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rp, s8 + u < S ? base + (s8 + u) * TG * 1024 + t * 1024 : kOut, 0,
                                                     kCoherent));
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s2 = s8 + u;
                if (s2 < S) {
                    const f32x4 w = s2 == sidx ? acc[t] : v[u];
                    sum = s2 == 0 ? w : sum + w;
                }
            }
        }
        store_tile(t, sum);
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
namespace {

template <int ACT, bool FP8, int T, int W>
hipError_t launch_tw(const VerifyLaunch &l) {
    constexpr int PF = pipeline_depth(FP8, T);
    auto kern = verify_kernel<ACT, FP8, T, W, PF>;
    size_t shm = 0;
    for (int i = 0; i < l.count; ++i)
        shm = std::max(shm, verify_lds_bytes(FP8, T, W, l.probs[i].plan.chunk));
    if (shm > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)shm) != hipSuccess)
        return hipErrorInvalidValue;
    KGroup grp{};
    grp.count = l.count;
    grp.out_dtype = l.out_dtype;
    grp.alpha = l.alpha;
    int items = 0;
    size_t cnt_off = 0, part_off = verify_counter_bytes();
    for (int i = 0; i < l.count; ++i) {
        const VerifyProblem &q = l.probs[i];
        KProblem &k = grp.p[i];
        const int ntg = verify_tile_groups(q.M, T * W);
        k.w = static_cast<const uint8_t *>(q.w);
        k.scales = q.scales;
        k.M = q.M;
        k.K = q.K;
        k.S = q.plan.slices;
        k.sl = q.plan.sl;
        k.chunk = q.plan.chunk;
        k.item0 = items;
        items += ntg * q.plan.slices;
        if (q.plan.slices > 1) {
            k.cnt = reinterpret_cast<uint32_t *>(static_cast<char *>(l.workspace) + cnt_off);
            k.part = reinterpret_cast<float *>(static_cast<char *>(l.workspace) + part_off);
            cnt_off += (size_t)ntg * 4;
            part_off += verify_partial_bytes(q.plan, q.M);
        }
    }
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
        grp.items = items;
        hipLaunchKernelGGL(kern, dim3(items), dim3(64 * W), shm, l.stream, grp);
    }
    return hipGetLastError();
}

template <int ACT, bool FP8, int T>
hipError_t dispatch_w(const VerifyLaunch &l) {
    switch (l.waves) {
    case 2: return launch_tw<ACT, FP8, T, 2>(l);
    case 4: return launch_tw<ACT, FP8, T, 4>(l);
    case 8: return launch_tw<ACT, FP8, T, 8>(l);
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

int verify_steps(bool fp8, int K) { return fp8 ? K / 128 : (K / 32 + 3) / 4; }

int verify_tile_groups(int M, int tiles_per_group) { return verify_tile_groups_dev(M, tiles_per_group); }

int pipeline_depth_of(bool fp8, int tiles) { return pipeline_depth(fp8, tiles); }

int verify_max_chunk(int waves) { return max_chunk_steps(waves); }

size_t verify_counter_bytes() { return (size_t)kMaxSplitTileGroups * 4; }

size_t verify_lds_bytes(bool fp8, int tiles, int waves, int chunk) {
    const size_t act_b = (size_t)chunk * kActStepBytes;
    const size_t sc_b = fp8 ? 0 : (size_t)tiles * waves * 16 * 4 * chunk * 2;
    return act_b + sc_b;
}

size_t verify_partial_bytes(const VerifyPlan &pl, int M) {
    if (pl.slices <= 1)
        return 0;
    return (size_t)verify_tile_groups(M, pl.tiles * pl.waves) * pl.slices * pl.tiles * pl.waves * 1024;
}

size_t verify_workspace_bytes(const VerifyPlan &pl, int M) {
    const size_t part = verify_partial_bytes(pl, M);
    return part ? verify_counter_bytes() + part : 0;
}

// Completes and checks a plan whose tiles, waves and requested slices are
// set: tiles in {1, 2, 4}, waves in {2, 4, 8}, 1 <= slices <= steps, and a
// split only with at most kMaxSplitTileGroups tile groups and partial tiles
// addressable in 32 bits.  The slice count becomes the number of non-empty
// slices of ceil(steps / slices) steps; the LDS chunk is the slice rounded up
// to whole pipeline rounds, capped by the staging bound.
bool verify_plan_finish(bool fp8, int M, int K, VerifyPlan &pl) {
    if (!(pl.tiles == 1 || pl.tiles == 2 || pl.tiles == 4) || !(pl.waves == 2 || pl.waves == 4 || pl.waves == 8))
        return false;
    const int steps = verify_steps(fp8, K);
    if (pl.slices < 1 || pl.slices > steps)
        return false;
    pl.sl = (steps + pl.slices - 1) / pl.slices;
    pl.slices = (steps + pl.sl - 1) / pl.sl;
    if (pl.slices > 1 && (verify_tile_groups(M, pl.tiles * pl.waves) > kMaxSplitTileGroups ||
                          verify_partial_bytes(pl, M) >= ((size_t)1 << 31)))
        return false;
    const int pf = pipeline_depth(fp8, pl.tiles);
    pl.chunk = std::min(max_chunk_steps(pl.waves), (pl.sl + pf - 1) / pf * pf);
    return verify_lds_bytes(fp8, pl.tiles, pl.waves, pl.chunk) <= kMaxLdsBytes;
}

hipError_t launch_verify(const VerifyLaunch &l) {
    if (l.count < 1 || l.count > kGroupPerLaunch)
        return hipErrorInvalidValue;
    if (l.act_dtype == VQ_DTYPE_BF16)
        return l.fp8 ? dispatch_t<VQ_DTYPE_BF16, true>(l) : dispatch_t<VQ_DTYPE_BF16, false>(l);
    return l.fp8 ? dispatch_t<VQ_DTYPE_F16, true>(l) : dispatch_t<VQ_DTYPE_F16, false>(l);
}

}  // namespace vq
