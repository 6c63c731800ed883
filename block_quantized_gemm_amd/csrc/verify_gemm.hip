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
//    the constant -(MAGIC + 8) forms the per-row offset term, which enters the
//    block MFMA as its accumulator, so the MFMA returns the exact block sum
//    (q - 8) x in fp32.  The fp16 block scale is one fp32 FMA per output.
//  * FP8: 32 contiguous bytes per lane per 128-wide chunk, hardware E4M3 ->
//    16-bit conversion (exact), 4 MFMAs per chunk, one FMA with the fp32 tile
//    scale.
//
// Data movement (the kernel is bound by what reaches the CUs):
//  * A workgroup is FG x KW waves.  The FG waves of one K-group work on FG
//    different 16-feature tiles at the same K step; the KW K-groups split K
//    into contiguous ranges.  Per 128-wide step, a K-group's 16 x 128
//    activation tile is read from memory once (one contiguous 16-byte load per
//    lane and piece, whole cache lines), scattered into LDS in MFMA operand
//    order and read back by all FG waves, so activation traffic per weight
//    byte falls by FG.  With FG = 1 the tile is private to its wave and needs
//    no barrier; with FG > 1 it is double-buffered with one barrier per step.
//  * The workgroup's Q4_0 block scales are staged into LDS once.
//  * Weight bytes are streamed with 16-byte raw buffer loads (rows past M read
//    as zeros) PF steps ahead of the compute in a register pipeline.
//  * K-group partial sums are combined through LDS in the fixed order
//    0, 1, ..., KW-1: no atomics, the same result on every run.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

constexpr int kStepK = 128;                      // k per step: 4 Q4_0 blocks or one FP8 chunk
constexpr int kActTileBytes = 16 * kStepK * 2;   // one step of 16 activation rows (bf16/fp16)

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

template <bool FP8>
struct WStage;
template <>
struct WStage<false> {
    u32x4 c;  // 16 code bytes: block 4s + g of the lane's feature
};
template <>
struct WStage<true> {
    u32x4 w0, w1;  // 32 E4M3 bytes: k = 32g .. 32g + 31 of the step
};

// One Q4_0 step (4 blocks) for one 16-feature tile.
template <int ACT, bool FULL>
__device__ __forceinline__ void q4_step(u32x4 c, const u32x4 (&a)[4], const uint32_t (&sc)[4], int nblk,
                                        f32x4 &acc) {
    using A16 = Act16<ACT>;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const u32x4 negc = {A16::kNegOffset, A16::kNegOffset, A16::kNegOffset, A16::kNegOffset};
    uint32_t d[4] = {c[0], c[1], c[2], c[3]};
    transpose_lane_groups(d[0], d[1], d[2], d[3]);  // lane group g: dword g of blocks 0..3
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        if (FULL || tb < nblk) {
            const f32x4 corr = A16::mfma(a[tb], negc, zero4);  // -(MAGIC + 8) * sum x, per row
            const f32x4 dot = A16::mfma(a[tb], q4_operand<A16::kMagicByte>(d[tb]), corr);
            const float s = h2f(sc[tb]);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r] = __builtin_fmaf(s, dot[r], acc[r]);
        }
    }
}

// One FP8 chunk (128 k) for one 16-feature tile.
template <int ACT>
__device__ __forceinline__ void fp8_step(const WStage<true> &w, const u32x4 (&a)[4], float ts, f32x4 &acc) {
    using A16 = Act16<ACT>;
    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const u32x4 src = u < 2 ? w.w0 : w.w1;
        const uint32_t e0 = src[2 * (u & 1)], e1 = src[2 * (u & 1) + 1];
        const u32x4 bop = {A16::template fp8x2<false>(e0), A16::template fp8x2<true>(e0),
                           A16::template fp8x2<false>(e1), A16::template fp8x2<true>(e1)};
        part = A16::mfma(a[u], bop, part);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        acc[r] = __builtin_fmaf(ts, part[r], acc[r]);
}

// ---------------------------------------------------------------------------
// The verify kernel.  grid = (ceil(tiles / FG), groups of 16 rows), block =
// 64 * FG * KW.  Dynamic LDS: the K-groups' activation tiles (two buffers
// each when FG > 1, one otherwise), then the Q4_0 block scales of the
// workgroup's FG * 16 feature rows.
// ---------------------------------------------------------------------------
template <int ACT, bool FP8, int FG, int KW, int PF, bool SVEC>
__global__ __launch_bounds__(64 * FG * KW) void verify_kernel(
    const uint8_t *__restrict__ wts, const void *__restrict__ scales, const uint16_t *__restrict__ act,
    void *__restrict__ out, int out_dtype, int N, int M, int K, float alpha) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    static_assert(FG == 1 || FG == 2 || FG == 4, "FG");
    constexpr int NW = FG * KW;
    constexpr int AP = 4 / FG;          // 16-byte activation pieces per lane per step
    constexpr bool SHARED = FG > 1;     // tile shared across waves: double buffer + barriers
    constexpr int NBUF = SHARED ? 2 : 1;

    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int fw = wave % FG;  // this wave's feature tile in the workgroup
    const int kg = wave / FG;  // this wave's K-group
    const int j = lane & 15;
    const int g = lane >> 4;

    const int NB = K >> 5;
    const int S = FP8 ? (K >> 7) : (NB + 3) >> 2;  // steps; the last Q4_0 step may be partial
    // K-group kg takes steps kg, kg + KW, kg + 2 KW, ...: the KW waves of a tile
    // read neighbouring 64-byte pieces of each weight row, so the workgroup
    // sweeps every row in 64 KW-byte runs (DRAM pages are visited once, not
    // once per piece).  Group sizes differ by at most one, so only a group's
    // final iteration can be empty and only the final step of K can be
    // partial; the steady-state loop reaches neither.
    const int n_iter = (S + KW - 1) / KW;
    const int n_mine = (S - kg + KW - 1) / KW;
    auto step_of = [&](int it) { return kg + it * KW; };
    const int feat0 = blockIdx.x * FG * 16;
    const int frows = min(M - feat0, FG * 16);
    const int row0 = blockIdx.y * 16;
    const int nrows = min(16, N - row0);

    // Buffer resources sized to the workgroup's rows: reads past them return 0.
    const int wrow = FP8 ? K : (K >> 1);  // weight bytes per feature row
    const rsrc_t rw = make_rsrc(wts + (size_t)feat0 * wrow, (uint32_t)frows * (uint32_t)wrow);
    const rsrc_t ra = make_rsrc(act + (size_t)row0 * K, (uint32_t)nrows * (uint32_t)K * 2u);
    const int vw = (fw * 16 + j) * wrow + (FP8 ? 32 : 16) * g;
    const int wstep = FP8 ? 128 : 64;  // weight bytes per row per step

    // Activation pieces this lane stages: piece c = fw * 64 + lane + FG * 64 * a
    // of its K-group's tile; row c / 16, 16-byte piece c % 16 of that row.
    int va[AP], ar[AP], ap[AP];
#pragma unroll
    for (int a = 0; a < AP; ++a) {
        const int c = fw * 64 + lane + FG * 64 * a;
        ar[a] = c >> 4;
        ap[a] = c & 15;
        va[a] = ar[a] * K * 2 + 16 * ap[a];
    }
    auto tile_ptr = [&](int buf) { return lds + (size_t)(kg * NBUF + buf) * kActTileBytes; };

    const uint16_t *sc_lds = reinterpret_cast<const uint16_t *>(lds + (size_t)KW * NBUF * kActTileBytes);
    const uint16_t *my_sc = sc_lds + (fw * 16 + j) * NB;
    const float *tsrow = nullptr;
    if constexpr (FP8)
        tsrow = static_cast<const float *>(scales) + (size_t)(min(feat0 + fw * 16, M - 1) >> 7) * S;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};

    // ---- register pipeline: PF steps of weights and activation pieces in flight
    WStage<FP8> ws[PF];
    u32x4 ax[PF][AP];
    auto issue = [&](auto U, int i) {
        const int s = step_of(i);
        if constexpr (FP8) {
            ws[U.value].w0 = bload16<kAuxCached>(rw, vw, wstep * s);
            ws[U.value].w1 = bload16<kAuxCached>(rw, vw + 16, wstep * s);
        } else {
            ws[U.value].c = bload16<kAuxCached>(rw, vw, wstep * s);
        }
#pragma unroll
        for (int a = 0; a < AP; ++a)
            ax[U.value][a] = bload16<kAuxCached>(ra, va[a], 256 * s);
    };
    auto stage_act = [&](auto U, int buf) {
        uint8_t *tp = tile_ptr(buf);
#pragma unroll
        for (int a = 0; a < AP; ++a)
            act_piece_to_lds<FP8>(tp, ar[a], ap[a], ax[U.value][a]);
    };
    // One iteration: read this step's operands from LDS, stage the next step's
    // activations, then the math (the reads come first: with one buffer the
    // next step overwrites the tile).  FULL: a whole step of K inside this
    // K-group's range, no runtime checks at all.
    auto iterate = [&](auto U, int it, bool stage_next, auto Full) {
        constexpr bool FULL = decltype(Full)::value;
        constexpr int NEXT = (decltype(U)::value + 1) % PF;
        const int s = step_of(it);
        const uint8_t *tp = tile_ptr(it % NBUF);
        u32x4 a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            a[q] = *reinterpret_cast<const u32x4 *>(tp + (q * 64 + lane) * 16);
        uint32_t sc[4] = {0u, 0u, 0u, 0u};
        int nblk = 4;
        if constexpr (!FP8) {
            if constexpr (!FULL)
                nblk = it < n_mine ? min(4, NB - 4 * s) : 0;
            if (FULL || nblk == 4) {
                if constexpr (SVEC) {
                    const u32x2 p = *reinterpret_cast<const u32x2 *>(my_sc + 4 * s);
                    sc[0] = p[0] & 0xFFFFu; sc[1] = p[0] >> 16; sc[2] = p[1] & 0xFFFFu; sc[3] = p[1] >> 16;
                } else {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb)
                        sc[tb] = my_sc[4 * s + tb];
                }
            } else {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    sc[tb] = tb < nblk ? (uint32_t)my_sc[4 * s + tb] : 0u;
            }
        }
        if (stage_next)
            stage_act(std::integral_constant<int, NEXT>{}, (it + 1) % NBUF);
        if constexpr (FULL) {
            if constexpr (FP8)
                fp8_step<ACT>(ws[U.value], a, tsrow[s], acc);
            else
                q4_step<ACT, true>(ws[U.value].c, a, sc, 4, acc);
        } else if (it < n_mine) {
            if constexpr (FP8)
                fp8_step<ACT>(ws[U.value], a, tsrow[s], acc);
            else if (nblk == 4)
                q4_step<ACT, true>(ws[U.value].c, a, sc, 4, acc);
            else
                q4_step<ACT, false>(ws[U.value].c, a, sc, nblk, acc);
        }
    };
    using Full = std::true_type;
    using Guarded = std::false_type;

    // ---- prologue: first PF steps in flight, then the scales, then tile 0
    const bool steady = n_iter - 1 >= 2 * PF;
    if (steady) {
        static_for<PF>([&](auto U) { issue(U, U.value); });
    } else {
        static_for<PF>([&](auto U) {
            if (U.value < n_iter)
                issue(U, U.value);
        });
    }
    if constexpr (!FP8) {
        // the workgroup's scale rows are contiguous in memory
        const uint32_t sbytes = (uint32_t)frows * (uint32_t)NB * 2u;
        const rsrc_t rs = make_rsrc(static_cast<const uint16_t *>(scales) + (size_t)feat0 * NB, sbytes);
        uint8_t *dst = lds + (size_t)KW * NBUF * kActTileBytes;
        // whole 16-byte chunks, then the remainder one scale at a time: the
        // buffer range check works per dword, so a load ending mid-dword past
        // the resource would read that dword as 0
        const uint32_t full = sbytes & ~15u;
        for (uint32_t o = threadIdx.x * 16u; o < full; o += 64u * NW * 16u)
            *reinterpret_cast<u32x4 *>(dst + o) = bload16<kAuxCached>(rs, (int)o, 0);
        for (uint32_t o = full + threadIdx.x * 2u; o < sbytes; o += 64u * NW * 2u)
            *reinterpret_cast<uint16_t *>(dst + o) = (uint16_t)bload2<kAuxCached>(rs, (int)o, 0);
    }
    if (n_iter > 0)
        stage_act(std::integral_constant<int, 0>{}, 0);
    __syncthreads();

    // ---- steady state: loads issued unconditionally, so the compiler counts
    // them and waits only for the slot it is about to use
    int i = 0;
    if (steady) {
        do {
            static_for<PF>([&](auto U) {
                const int it = i + U.value;
                iterate(U, it, true, Full{});
                __builtin_amdgcn_sched_barrier(0);
                issue(U, it + PF);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (SHARED)
                    __syncthreads();
            });
            i += PF;
        } while (i + 2 * PF <= n_iter - 1);
    }
    // ---- tail: the last n_iter - i (<= 2 PF) iterations
    static_for<2 * PF + 1>([&](auto V) {
        constexpr int U = V.value % PF;
        const int it = i + V.value;
        if (it < n_iter) {
            iterate(std::integral_constant<int, U>{}, it, it + 1 < n_iter, Guarded{});
            if (it + PF < n_iter)
                issue(std::integral_constant<int, U>{}, it + PF);
        }
        if constexpr (SHARED)
            __syncthreads();
    });
    if constexpr (!SHARED)
        __syncthreads();

    // ---- combine the K-groups in fixed order, scale, round, store
    float *red = reinterpret_cast<float *>(lds);  // reuses the activation tiles
#pragma unroll
    for (int r = 0; r < 4; ++r)
        red[((kg * FG + fw) * 4 + r) * 64 + lane] = acc[r];
    __syncthreads();
    for (int o = threadIdx.x; o < FG * 4 * 64; o += NW * 64) {
        float s = red[o];
#pragma unroll
        for (int w = 1; w < KW; ++w)
            s += red[w * FG * 4 * 64 + o];
        const int ln = o & 63, r = (o >> 6) & 3, f = o >> 8;
        const int feat = feat0 + f * 16 + (ln & 15);
        const int row = 4 * (ln >> 4) + r;
        if (row < nrows && feat < M)
            store_out(out, out_dtype, (size_t)(row0 + row) * M + feat, alpha * s);
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
namespace {

constexpr int kMaxGridY = 65535;

template <bool FP8, int FG>
constexpr int pipeline_depth() {
    return FP8 ? (FG == 1 ? 3 : 4) : (FG == 1 ? 4 : 6);
}

template <int ACT, bool FP8, int FG, int KW>
hipError_t launch_one(const VerifyArgs &p) {
    constexpr int PF = pipeline_depth<FP8, FG>();
    const int tiles = (p.M + 15) / 16;
    const int gx = (tiles + FG - 1) / FG;
    const int groups = (p.N + 15) / 16;
    const size_t shm = verify_lds_bytes(FP8, FG, KW, p.K);
    auto kern = (FP8 || (p.K / 32) % 4 == 0) ? verify_kernel<ACT, FP8, FG, KW, PF, true>
                                              : verify_kernel<ACT, FP8, FG, KW, PF, false>;
    if (shm > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)shm) != hipSuccess)
        return hipErrorInvalidValue;
    for (int g0 = 0; g0 < groups; g0 += kMaxGridY) {
        const int gy = std::min(kMaxGridY, groups - g0);
        const uint16_t *act = reinterpret_cast<const uint16_t *>(p.act) + (size_t)g0 * 16 * p.K;
        void *out = static_cast<char *>(p.out) + (size_t)g0 * 16 * p.M * out_elem_bytes(p.out_dtype);
        const int n = std::min(p.N - g0 * 16, gy * 16);
        hipLaunchKernelGGL(kern, dim3(gx, gy), dim3(64 * FG * KW), shm, p.stream,
                           reinterpret_cast<const uint8_t *>(p.w), p.scales, act, out, p.out_dtype, n, p.M, p.K,
                           p.alpha);
    }
    return hipGetLastError();
}

template <int ACT, bool FP8, int FG>
hipError_t dispatch_kw(const VerifyArgs &p) {
    switch (p.waves_k) {
    case 1: return launch_one<ACT, FP8, FG, 1>(p);
    case 2: return launch_one<ACT, FP8, FG, 2>(p);
    case 4: return launch_one<ACT, FP8, FG, 4>(p);
    case 8:
        if constexpr (FG <= 2)
            return launch_one<ACT, FP8, FG, 8>(p);
        return hipErrorInvalidValue;
    case 16:
        if constexpr (FG == 1)
            return launch_one<ACT, FP8, FG, 16>(p);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int ACT, bool FP8>
hipError_t dispatch_fg(const VerifyArgs &p) {
    switch (p.tiles_per_wg) {
    case 1: return dispatch_kw<ACT, FP8, 1>(p);
    case 2: return dispatch_kw<ACT, FP8, 2>(p);
    case 4: return dispatch_kw<ACT, FP8, 4>(p);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t verify_lds_bytes(bool fp8, int fg, int kw, int K) {
    const size_t nbuf = fg > 1 ? 2 : 1;
    const size_t act_b = (size_t)kw * nbuf * kActTileBytes;
    const size_t sc_b = fp8 ? 0 : ((((size_t)fg * 16 * (K / 32) * 2) + 15) & ~(size_t)15);
    return act_b + sc_b;  // the final reduction (kw * fg KB) fits in act_b
}

bool verify_shape_ok(bool fp8, int fg, int kw, int K) {
    if (!(fg == 1 || fg == 2 || fg == 4) || !(kw == 1 || kw == 2 || kw == 4 || kw == 8 || kw == 16))
        return false;
    if (fg * kw > 16)
        return false;
    return verify_lds_bytes(fp8, fg, kw, K) <= kMaxLdsBytes;
}

hipError_t launch_verify(const VerifyArgs &p, bool fp8) {
    if (p.act_dtype == VQ_DTYPE_BF16)
        return fp8 ? dispatch_fg<VQ_DTYPE_BF16, true>(p) : dispatch_fg<VQ_DTYPE_BF16, false>(p);
    return fp8 ? dispatch_fg<VQ_DTYPE_F16, true>(p) : dispatch_fg<VQ_DTYPE_F16, false>(p);
}

}  // namespace vq
