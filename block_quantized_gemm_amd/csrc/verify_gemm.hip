// verify_gemm.hip -- the verification matmul for a draft block of <= 16 rows.
//
// "Qwen3.8-27B on the AMD R9700: up to 227 tok/s", section "A block-diffusion
// drafter, verified exactly": the target checks a whole draft block in one
// batched forward that reads the weights once, so 16 rows cost about what one
// row costs.  This file is that product for two weight formats:
//   Q4_0   -- "Qwen3.8-27B at 45.7 tok/s ...", section "Prompt processing":
//             4-bit codes, offset 8, blocks of 32, one fp16 scale per block;
//   FP8    -- "r9k: a from-scratch inference engine ...", opening paragraph:
//             E4M3 weights with one scale per 128 x 128 tile.
//
// Design (gfx950, wave64):
//  * One MFMA 16x16x32 (bf16 or fp16) per (16 output features x 32 k).  The
//    A operand is the activation block (rows zero-padded to 16), the B operand
//    the dequantised weights.  The same instruction sequence runs for every
//    N <= 16, so an output row's arithmetic never depends on N (the pages
//    compare outputs byte for byte across block widths; "What 'lossless' means
//    here, precisely").
//  * Q4_0: each lane streams one whole 16-byte block of one feature with a
//    128-bit load; a 4x4 lane-group transpose (permlane swaps) hands every
//    lane its 4-byte slice of each block.  Codes become the exact 16-bit
//    values MAGIC + q; an extra MFMA with constant -(MAGIC + 8) computes the
//    per-row offset term, which enters the block MFMA as its accumulator, so
//    the MFMA result is the exact block dot sum (q - 8) x in fp32.  The fp16
//    block scale is then applied with one fp32 FMA per output.
//  * FP8: 32 contiguous bytes per lane per 128-wide chunk, hardware E4M3 ->
//    16-bit conversion (exact), 4 MFMAs per chunk accumulated from zero, then
//    one FMA with the chunk's fp32 tile scale.
//  * A workgroup is `KW` waves that split K (wave w takes steps w, w+KW, ...)
//    over the same `T` feature tiles; partial sums are combined through LDS in
//    the fixed order w = 0, 1, ..., KW-1.  No atomics: results are the same on
//    every run.
//  * Loads are raw buffer loads against resources sized to the workgroup's
//    rows, so rows past M (weights) or N (activations) read as zeros without
//    any divergent branch, and the step offset is a wave-uniform SGPR.  Each
//    wave keeps PF steps of loads in flight ahead of the one it computes:
//    HBM latency is hidden by memory-level parallelism, not by occupancy.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

// --------------------------------------------------------------------------
// Shared epilogue: fixed-order cross-wave reduction, alpha, rounding, store.
// acc[t][r] of lane (j = lane & 15, g = lane >> 4) is output row 4g + r of
// feature 16 * (tile0 + t) + j.
// --------------------------------------------------------------------------
template <int T, int KW>
__device__ __forceinline__ void reduce_store(f32x4 (&acc)[T], void *__restrict__ out, int out_dtype,
                                             int M, int row0, int nrows, int tile0, float alpha) {
    const int lane = threadIdx.x & 63;
    if constexpr (KW == 1) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int f = (tile0 + t) * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * (lane >> 4) + r;
                if (row < nrows && f < M)
                    store_out(out, out_dtype, (size_t)(row0 + row) * M + f, alpha * acc[t][r]);
            }
        }
    } else {
        __shared__ float red[KW][T * 4 * kWave];
        const int wave = threadIdx.x >> 6;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[wave][(t * 4 + r) * kWave + lane] = acc[t][r];
        __syncthreads();
        for (int o = threadIdx.x; o < T * 4 * kWave; o += KW * kWave) {
            float s = red[0][o];
#pragma unroll
            for (int w = 1; w < KW; ++w)
                s += red[w][o];
            const int ln = o & 63;
            const int tr = o >> 6;
            const int t = tr >> 2, r = tr & 3;
            const int f = (tile0 + t) * 16 + (ln & 15);
            const int row = 4 * (ln >> 4) + r;
            if (row < nrows && f < M)
                store_out(out, out_dtype, (size_t)(row0 + row) * M + f, alpha * s);
        }
    }
}

// --------------------------------------------------------------------------
// Q4_0 verify kernel.  grid = (ceil(tiles / T), row groups), block = 64 * KW.
//
// One "step" is 4 consecutive 32-blocks (128 k).  Wave w of the workgroup
// takes steps w, w + KW, w + 2 KW, ...; PF steps of loads are kept in flight
// ahead of the step being computed (software pipeline).
// --------------------------------------------------------------------------
template <int T>
struct Q4Stage {
    uint32_t c[T][4];   // codes: lane group g holds block 4s+g, 16 bytes
    uint32_t sc[T][4];  // the lane's 4 block scales of the step: fp16 pairs in [0], [1]
                        // (8-byte path) or one fp16 per entry (2-byte path)
    u32x4 a[4];         // activation operand of each of the 4 blocks
};

template <int T, bool SVEC>
__device__ __forceinline__ void q4_load(Q4Stage<T> &st, int s, rsrc_t rc, rsrc_t rs, rsrc_t ra, int vc, int vs,
                                        int va, int tile_cbytes, int tile_sbytes) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const u32x4 v = bload16<kAuxStream>(rc, vc, 64 * s + t * tile_cbytes);
        st.c[t][0] = v[0]; st.c[t][1] = v[1]; st.c[t][2] = v[2]; st.c[t][3] = v[3];
        if constexpr (SVEC) {
            const u32x2 w = bload8<kAuxStream>(rs, vs, 8 * s + t * tile_sbytes);
            st.sc[t][0] = w[0]; st.sc[t][1] = w[1];
        } else {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                st.sc[t][tb] = bload2<kAuxStream>(rs, vs + 2 * tb, 8 * s + t * tile_sbytes);
        }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const u32x2 lo = bload8<kAuxCached>(ra, va + 64 * tb, 256 * s);
        const u32x2 hi = bload8<kAuxCached>(ra, va + 64 * tb + 32, 256 * s);
        st.a[tb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
}

template <int ACT, int T, bool SVEC, bool FULL>
__device__ __forceinline__ void q4_compute(Q4Stage<T> &st, int nblk, f32x4 (&acc)[T]) {
    using A16 = Act16<ACT>;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const u32x4 negc = {A16::kNegOffset, A16::kNegOffset, A16::kNegOffset, A16::kNegOffset};
    // lane group g gets dword g of each of the 4 blocks
#pragma unroll
    for (int t = 0; t < T; ++t)
        transpose_lane_groups(st.c[t][0], st.c[t][1], st.c[t][2], st.c[t][3]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        if (FULL || tb < nblk) {  // wave-uniform: only the last step of a ragged K is partial
            // -(MAGIC + 8) * (sum of the block's activations), per row
            const f32x4 corr = A16::mfma(st.a[tb], negc, zero4);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const u32x4 bop = q4_operand<A16::kMagicByte>(st.c[t][tb]);
                const f32x4 d = A16::mfma(st.a[tb], bop, corr);  // exact sum (q - 8) x
                float dsc;
                if constexpr (SVEC) {
                    const uint32_t pair = st.sc[t][tb >> 1];
                    dsc = h2f((tb & 1) ? (pair >> 16) : (pair & 0xFFFFu));
                } else {
                    dsc = h2f(st.sc[t][tb]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[t][r] = __builtin_fmaf(dsc, d[r], acc[t][r]);
            }
        }
    }
}

template <int ACT, int T, int KW, int PF, bool SVEC>
__global__ __launch_bounds__(64 * KW) void q4_0_verify_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ act, void *__restrict__ out, int out_dtype, int N, int M, int K,
    float alpha) {
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int j = lane & 15;  // A row (activation row) and B/D column (feature)
    const int g = lane >> 4;  // k-slot group
    const int NB = K >> 5;    // 32-blocks per row
    const int S = (NB + 3) >> 2;
    const int tile0 = blockIdx.x * T;
    const int row0 = blockIdx.y * 16;
    const int nrows = min(16, N - row0);
    const int frows = min(M - tile0 * 16, T * 16);  // feature rows owned by this workgroup

    // buffer resources sized to this workgroup's rows: anything past them reads as 0
    const rsrc_t rc = make_rsrc(codes + (size_t)tile0 * 16 * (size_t)(K >> 1), (uint32_t)frows * (uint32_t)(K >> 1));
    const rsrc_t rs = make_rsrc(scales + (size_t)tile0 * 16 * NB, (uint32_t)frows * (uint32_t)NB * 2u);
    const rsrc_t ra = make_rsrc(act + (size_t)row0 * K, (uint32_t)nrows * (uint32_t)K * 2u);
    const int vc = j * (K >> 1) + 16 * g;
    const int vs = j * NB * 2;
    const int va = j * K * 2 + 8 * g;
    const int tile_cbytes = 16 * (K >> 1);
    const int tile_sbytes = 16 * NB * 2;

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Steps of this wave: wave, wave + KW, ...; only the very last step of K can
    // be partial, and the pipeline's steady state never computes it.
    // When every step is full (K % 128 == 0), workgroup b walks its steps in an
    // order rotated by b, so the thousands of concurrently running waves read
    // different activation lines instead of all hitting the same ones.  The
    // order is a function of the launch shape only, never of N.
    const int ns = (S - wave + KW - 1) / KW;
    const int rot = (SVEC && ns > 0) ? (int)(blockIdx.x % (unsigned)ns) : 0;
    auto step_of = [&](int i) {
        int r = i + rot;
        r = r >= ns ? r - ns : r;
        return wave + r * KW;
    };
    Q4Stage<T> st[PF];
    pipeline<PF>(
        ns,
        [&](auto U, int i) {
            q4_load<T, SVEC>(st[U.value], step_of(i), rc, rs, ra, vc, vs, va, tile_cbytes, tile_sbytes);
        },
        [&](auto U, int i, bool full) {
            if (full)
                q4_compute<ACT, T, SVEC, true>(st[U.value], 4, acc);
            else
                q4_compute<ACT, T, SVEC, false>(st[U.value], min(4, NB - 4 * step_of(i)), acc);
        });
    reduce_store<T, KW>(acc, out, out_dtype, M, row0, nrows, tile0, alpha);
}

// --------------------------------------------------------------------------
// FP8 E4M3 + 128x128 fp32 tile scales.  K % 128 == 0.  One "chunk" = 128 k.
// --------------------------------------------------------------------------
template <int T>
struct F8Stage {
    u32x4 w[T][2];  // 32 weight bytes per lane per tile
    u32x4 a[4];     // 4 activation operands (8 values each)
};

template <int T>
__device__ __forceinline__ void f8_load(F8Stage<T> &st, int c, rsrc_t rw, rsrc_t ra, int vw, int va,
                                        int tile_bytes) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
        st.w[t][0] = bload16<kAuxStream>(rw, vw, 128 * c + t * tile_bytes);
        st.w[t][1] = bload16<kAuxStream>(rw, vw + 16, 128 * c + t * tile_bytes);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
        st.a[u] = bload16<kAuxCached>(ra, va + 16 * u, 256 * c);
}

template <int ACT, int T>
__device__ __forceinline__ void f8_compute(F8Stage<T> &st, int c, const float *const (&srow)[T],
                                           f32x4 (&acc)[T]) {
    using A16 = Act16<ACT>;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t d0 = st.w[t][q >> 1][2 * (q & 1)];
            const uint32_t d1 = st.w[t][q >> 1][2 * (q & 1) + 1];
            const u32x4 bop = {A16::template fp8x2<false>(d0), A16::template fp8x2<true>(d0),
                               A16::template fp8x2<false>(d1), A16::template fp8x2<true>(d1)};
            part = A16::mfma(st.a[q], bop, part);
        }
        const float ts = srow[t][c];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc[t][r] = __builtin_fmaf(ts, part[r], acc[t][r]);
    }
}

template <int ACT, int T, int KW, int PF>
__global__ __launch_bounds__(64 * KW) void fp8_verify_kernel(
    const uint8_t *__restrict__ w, const float *__restrict__ tscales,
    const uint16_t *__restrict__ act, void *__restrict__ out, int out_dtype, int N, int M, int K) {
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int j = lane & 15;
    const int g = lane >> 4;
    const int C = K >> 7;  // 128-wide chunks
    const int tile0 = blockIdx.x * T;
    const int row0 = blockIdx.y * 16;
    const int nrows = min(16, N - row0);
    const int frows = min(M - tile0 * 16, T * 16);

    const rsrc_t rw = make_rsrc(w + (size_t)tile0 * 16 * (size_t)K, (uint32_t)frows * (uint32_t)K);
    const rsrc_t ra = make_rsrc(act + (size_t)row0 * K, (uint32_t)nrows * (uint32_t)K * 2u);
    const int vw = j * K + 32 * g;
    const int va = j * K * 2 + 64 * g;
    const int tile_bytes = 16 * K;

    // all 16 features of a tile share one 128-row scale group
    const float *srow[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        srow[t] = tscales + (size_t)(min((tile0 + t) * 16, M - 1) >> 7) * C;

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ns = (C - wave + KW - 1) / KW;
    const int rot = ns > 0 ? (int)(blockIdx.x % (unsigned)ns) : 0;  // see the Q4_0 kernel
    auto chunk_of = [&](int i) {
        int r = i + rot;
        r = r >= ns ? r - ns : r;
        return wave + r * KW;
    };
    F8Stage<T> st[PF];
    pipeline<PF>(
        ns, [&](auto U, int i) { f8_load<T>(st[U.value], chunk_of(i), rw, ra, vw, va, tile_bytes); },
        [&](auto U, int i, bool) { f8_compute<ACT, T>(st[U.value], chunk_of(i), srow, acc); });
    reduce_store<T, KW>(acc, out, out_dtype, M, row0, nrows, tile0, 1.0f);
}

// --------------------------------------------------------------------------
// Host-side launchers.
// --------------------------------------------------------------------------
namespace {

constexpr int kMaxGridY = 65535;

template <int ACT, int T, int KW>
hipError_t launch_q4(const VerifyArgs &p) {
    const int tiles = (p.M + 15) / 16;
    const int gx = (tiles + T - 1) / T;
    const int groups = (p.N + 15) / 16;
    for (int g0 = 0; g0 < groups; g0 += kMaxGridY) {
        const int gy = std::min(kMaxGridY, groups - g0);
        const uint16_t *act = reinterpret_cast<const uint16_t *>(p.act) + (size_t)g0 * 16 * p.K;
        void *out = static_cast<char *>(p.out) + (size_t)g0 * 16 * p.M * out_elem_bytes(p.out_dtype);
        const int n = std::min(p.N - g0 * 16, gy * 16);
        constexpr int PF = T == 1 ? 4 : (T == 2 ? 3 : 2);
        if ((p.K / 32) % 4 == 0)
            hipLaunchKernelGGL((q4_0_verify_kernel<ACT, T, KW, PF, true>), dim3(gx, gy), dim3(64 * KW), 0,
                               p.stream, reinterpret_cast<const uint8_t *>(p.w),
                               reinterpret_cast<const uint16_t *>(p.scales), act, out, p.out_dtype, n, p.M,
                               p.K, p.alpha);
        else
            hipLaunchKernelGGL((q4_0_verify_kernel<ACT, T, KW, PF, false>), dim3(gx, gy), dim3(64 * KW), 0,
                               p.stream, reinterpret_cast<const uint8_t *>(p.w),
                               reinterpret_cast<const uint16_t *>(p.scales), act, out, p.out_dtype, n, p.M,
                               p.K, p.alpha);
    }
    return hipGetLastError();
}

template <int ACT, int T, int KW>
hipError_t launch_fp8(const VerifyArgs &p) {
    const int tiles = (p.M + 15) / 16;
    const int gx = (tiles + T - 1) / T;
    const int groups = (p.N + 15) / 16;
    for (int g0 = 0; g0 < groups; g0 += kMaxGridY) {
        const int gy = std::min(kMaxGridY, groups - g0);
        const uint16_t *act = reinterpret_cast<const uint16_t *>(p.act) + (size_t)g0 * 16 * p.K;
        void *out = static_cast<char *>(p.out) + (size_t)g0 * 16 * p.M * out_elem_bytes(p.out_dtype);
        const int n = std::min(p.N - g0 * 16, gy * 16);
        constexpr int PF = T == 1 ? 4 : (T == 2 ? 3 : 2);
        hipLaunchKernelGGL((fp8_verify_kernel<ACT, T, KW, PF>), dim3(gx, gy), dim3(64 * KW), 0, p.stream,
                           reinterpret_cast<const uint8_t *>(p.w), reinterpret_cast<const float *>(p.scales),
                           act, out, p.out_dtype, n, p.M, p.K);
    }
    return hipGetLastError();
}

template <int ACT, int T>
hipError_t dispatch_kw(const VerifyArgs &p, int kw, bool fp8) {
    switch (kw) {
    case 1: return fp8 ? launch_fp8<ACT, T, 1>(p) : launch_q4<ACT, T, 1>(p);
    case 2: return fp8 ? launch_fp8<ACT, T, 2>(p) : launch_q4<ACT, T, 2>(p);
    case 4: return fp8 ? launch_fp8<ACT, T, 4>(p) : launch_q4<ACT, T, 4>(p);
    case 8: return fp8 ? launch_fp8<ACT, T, 8>(p) : launch_q4<ACT, T, 8>(p);
    case 16: return fp8 ? launch_fp8<ACT, T, 16>(p) : launch_q4<ACT, T, 16>(p);
    default: return hipErrorInvalidValue;
    }
}

template <int ACT>
hipError_t dispatch_t(const VerifyArgs &p, int t, int kw, bool fp8) {
    switch (t) {
    case 1: return dispatch_kw<ACT, 1>(p, kw, fp8);
    case 2: return dispatch_kw<ACT, 2>(p, kw, fp8);
    case 4: return dispatch_kw<ACT, 4>(p, kw, fp8);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_verify(const VerifyArgs &p, bool fp8) {
    if (p.act_dtype == VQ_DTYPE_BF16)
        return dispatch_t<VQ_DTYPE_BF16>(p, p.tiles_per_wave, p.waves_k, fp8);
    return dispatch_t<VQ_DTYPE_F16>(p, p.tiles_per_wave, p.waves_k, fp8);
}

}  // namespace vq
