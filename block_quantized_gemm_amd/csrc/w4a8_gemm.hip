// w4a8_gemm.hip -- Q4_0 weights x int8 activations with fp16 per-32-block
// scales (the prefill-sized "exact int8 path").
//
// "Qwen3.8-27B at 45.7 tok/s: DFlash2 in 1bit serve, and 4-bit activations
// with a Hadamard rotation", section "Prompt processing: 4-bit activations,
// rotated first": every 32-block contributes d_w * d_x * D_b to an output,
// where D_b is the exact integer dot of the block's weight values (q - 8) and
// activation codes.
//
// The integer dot runs on the 16-bit MFMA with integer-valued operands: an
// activation code x (|x| <= 127) and a Q4_0 value are exact in fp16, every
// product and partial sum is an integer below 2^24, so the fp32 result is the
// exact dot -- with no int -> float conversion per output and block, which is
// what bounds this GEMM (the 16x16x32 int8 MFMA takes the same 16 cycles per
// 32-block as the 16-bit one, so nothing is given up on the matrix side).
// Operands: x becomes fp16 x exactly (byte permute under the exponent byte of
// 1024, one packed subtract); a code q becomes fp16 1024 + q (permute only),
// and the offset is removed through the accumulator input: an MFMA of the
// activations with the constant -1032 yields -1032 * sum(x) per row and block,
// so D = sum x (1024 + q) - 1032 sum x = sum x (q - 8).  Epilogue per output
// and block: one fp32 product of the two fp16 scales (exact) and one FMA.
//
// Tiling: a workgroup of 8 waves computes 128 rows x 288 features (288 = 18
// MFMA tiles: 17408 features make 61 columns, so a 512-row prefill is one
// round of 244 workgroups on 256 CUs).  Wave (fg, rg, kh) takes features
// 144 fg .. +144, rows 64 rg .. +64 and blocks 2 kh, 2 kh + 1 of every 4-block
// chunk of K; the two k halves are added at the end (kh 0 + kh 1, fixed
// order), so each row's arithmetic is independent of N.  Chunks are loaded
// straight into LDS (16 B per lane, no registers) one chunk ahead, into the
// other of two stages; 16-byte pieces are XOR-swizzled by row (activations)
// and by feature (codes) so that the operand reads are free of bank
// conflicts.  Scales are converted to fp32 on the way into LDS.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kW4Rows = 128, kW4Feats = 288;  // per workgroup
constexpr int kW4Blocks = 4;                  // 32-blocks per K chunk
constexpr int kW4Threads = 512;
constexpr int kW4FeatTiles = kW4Feats / 2 / 16;            // 9 tiles per wave
constexpr int kAStage = kW4Rows * 128;                     // int8 codes, 128 B per row
constexpr int kBStage = kW4Feats * 64;                     // Q4_0 codes, 64 B per feature
constexpr int kSxStage = kW4Blocks * kW4Rows * 4;          // fp32 [block][row]
constexpr int kSwStage = kW4Blocks * kW4Feats * 4;         // fp32 [block][feature]
constexpr int kStage = kAStage + kBStage + kSxStage + kSwStage;
constexpr int kW4Lds = 2 * kStage;
constexpr int kTileBytes = 64 * kW4Feats * 4;  // k-half exchange and half of the output tile (fp32)
static_assert(kTileBytes <= kW4Lds, "epilogue area");
constexpr int kOutOfRange = 0x7FFFFFF0;  // past every range below: the load returns zeros
constexpr uint32_t kF16Magic = 0x64646464u;  // fp16 1024 + byte
constexpr uint32_t kF16Neg1152 = 0xE480E480u;
constexpr uint32_t kF16Neg1032 = 0xE408E408u;

__device__ __forceinline__ uint32_t pk_add_f16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) + __builtin_bit_cast(f16x2, b));
}

// Activation codes at k = 4g..4g+3 (lo) and 16+4g..16+4g+3 (hi) -> the exact
// fp16 MFMA operand in the k order of q4_operand.  x XOR 0x80 is x + 128 as an
// unsigned byte; under the exponent byte of 1024 it reads 1152 + x, exact, and
// the packed subtract leaves x.
__device__ __forceinline__ u32x4 i8_operand(uint32_t lo, uint32_t hi) {
    const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
    u32x4 r;
    r[0] = pk_add_f16(__builtin_amdgcn_perm(kF16Magic, a, 0x04010400u), kF16Neg1152);
    r[1] = pk_add_f16(__builtin_amdgcn_perm(kF16Magic, a, 0x04030402u), kF16Neg1152);
    r[2] = pk_add_f16(__builtin_amdgcn_perm(kF16Magic, b, 0x04010400u), kF16Neg1152);
    r[3] = pk_add_f16(__builtin_amdgcn_perm(kF16Magic, b, 0x04030402u), kF16Neg1152);
    return r;
}

__global__ __launch_bounds__(kW4Threads) void w4a8_kernel(const uint8_t *__restrict__ codes,
                                                          const uint16_t *__restrict__ wscales,
                                                          const int8_t *__restrict__ qx,
                                                          const uint16_t *__restrict__ xscales,
                                                          void *__restrict__ out, int out_dtype, int N, int M,
                                                          int K, float alpha, int row_groups) {
    using F16 = Act16<VQ_DTYPE_F16>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = threadIdx.x, lane = t & 63, wave = wave_id(), j = lane & 15, g = lane >> 4;
    const int fg = wave & 1, rg = (wave >> 1) & 1, kh = wave >> 2;
    // tiles in column order (the row groups of one feature column are
    // consecutive), numbered so that each XCD holds a run of whole columns
    const int tile = xcd_run_index((int)blockIdx.x, (int)gridDim.x);
    const int fb = tile / row_groups * kW4Feats, rb = tile % row_groups * kW4Rows;
    const int NB = K >> 5, KH = K >> 1;
    const int nch = (NB + kW4Blocks - 1) / kW4Blocks;
    const int rows = min(kW4Rows, N - rb), feats = min(kW4Feats, M - fb);

    // Loads of one chunk.  Activations: 16 wave loads of 8 rows x 128 B (this
    // wave: pieces wave and wave + 8); codes: 18 wave loads of 16 features x
    // 64 B (wave, wave + 8, wave + 16 < 18).  Each range covers only its own
    // rows or features, so rows past N and features past M read zeros.
    rsrc_t ra[2], rw[3];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = wave + 8 * i;
        ra[i] = make_rsrc(qx + (size_t)(rb + 8 * p) * K, (uint32_t)max(0, min(8, rows - 8 * p)) * (uint32_t)K);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int p = wave + 8 * i;
        rw[i] = make_rsrc(codes + (size_t)(fb + 16 * p) * KH,
                          p < 18 ? (uint32_t)max(0, min(16, feats - 16 * p)) * (uint32_t)KH : 0u);
    }
    const rsrc_t rsx = make_rsrc(xscales + (size_t)rb * NB, (uint32_t)rows * (uint32_t)NB * 2u);
    const rsrc_t rsw = make_rsrc(wscales + (size_t)fb * NB, (uint32_t)feats * (uint32_t)NB * 2u);
    // lane roles in the loads: activation row piece (8 rows x 8 slots), code
    // feature piece (16 features x 4 slots)
    const int a_row = lane >> 3, a_slot = lane & 7;
    const int b_feat = lane >> 2, b_slot = lane & 3;

    uint32_t gs[kW4Blocks];  // this thread's 4 scales of the next chunk (fp16 bits)
    auto issue = [&](int c, int stage) {
        uint8_t *st = lds + stage * kStage;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = wave + 8 * i, row = 8 * p + a_row;
            const int kb = 128 * c + 16 * (a_slot ^ ((row >> 1) & 7));
            bload16_lds(ra[i], st + 1024 * p, kb < K ? a_row * K + kb : kOutOfRange);
        }
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int p = wave + 8 * i, f = 16 * p + b_feat;
            const int kb = 64 * c + 16 * (b_slot ^ ((f >> 2) & 3));
            if (p < 18)
                bload16_lds(rw[i], st + kAStage + 1024 * p, kb < KH ? b_feat * KH + kb : kOutOfRange);
        }
        // waves 0, 1: the activation scales of rows t; waves 2..6: the weight
        // scales of features t - 128 (lanes past the 288th feature read zeros)
        if (wave < 7) {
            const rsrc_t rs = wave < 2 ? rsx : rsw;
            const int who = wave < 2 ? t : t - kW4Rows;
#pragma unroll
            for (int q = 0; q < kW4Blocks; ++q) {
                const int blk = kW4Blocks * c + q;
                gs[q] = bload2<kAuxCached>(rs, blk < NB && who < kW4Feats ? (who * NB + blk) * 2 : kOutOfRange, 0);
            }
        }
    };
    auto store_scales = [&](int stage) {
        float *sx = reinterpret_cast<float *>(lds + stage * kStage + kAStage + kBStage);
        float *sw = sx + kW4Blocks * kW4Rows;
        if (t < kW4Rows) {
#pragma unroll
            for (int q = 0; q < kW4Blocks; ++q)
                sx[q * kW4Rows + t] = h2f(gs[q]);
        } else if (t < kW4Rows + kW4Feats) {
#pragma unroll
            for (int q = 0; q < kW4Blocks; ++q)
                sw[q * kW4Feats + t - kW4Rows] = h2f(gs[q]);
        }
    };

    f32x4 acc[4][kW4FeatTiles];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ft = 0; ft < kW4FeatTiles; ++ft)
            acc[rt][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const u32x4 neg1032 = {kF16Neg1032, kF16Neg1032, kF16Neg1032, kF16Neg1032};
    // swizzle of this lane's operand rows and features (their low 4 bits are j)
    const int a_sw = (j >> 1) & 7, b_sw = (j >> 2) & 3;

    issue(0, 0);
    wait_vmcnt<0>();
    store_scales(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch)
            issue(c + 1, (c + 1) & 1);
        const uint8_t *st = lds + (c & 1) * kStage;
        const uint8_t *as = st + (rg * 64 + j) * 128 + 4 * g;
        const uint8_t *bs = st + kAStage + (fg * 144 + j) * 64 + 4 * g;
        const float *sx = reinterpret_cast<const float *>(st + kAStage + kBStage) + rg * 64 + 4 * g;
        const float *sw = reinterpret_cast<const float *>(st + kAStage + kBStage + kSxStage) + fg * 144 + j;
#pragma unroll 1
        for (int qq = 0; qq < 2; ++qq) {
            const int q = 2 * kh + qq;
            u32x4 a[4];
            f32x4 z[4], dx[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const uint8_t *ar = as + rt * 16 * 128;
                const uint32_t lo = *reinterpret_cast<const uint32_t *>(ar + 16 * ((2 * q) ^ a_sw));
                const uint32_t hi = *reinterpret_cast<const uint32_t *>(ar + 16 * ((2 * q + 1) ^ a_sw));
                a[rt] = i8_operand(lo, hi);
                z[rt] = F16::mfma(a[rt], neg1032, zero4);
                dx[rt] = *reinterpret_cast<const f32x4 *>(sx + q * kW4Rows + rt * 16);
            }
#pragma unroll
            for (int ft = 0; ft < kW4FeatTiles; ++ft) {
                const uint32_t wv = *reinterpret_cast<const uint32_t *>(bs + ft * 16 * 64 + 16 * (q ^ b_sw));
                const u32x4 b = q4_operand<kF16Magic>(wv);
                const float dw = sw[q * kW4Feats + ft * 16];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const f32x4 d = F16::mfma(a[rt], b, z[rt]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[rt][ft][r] = __builtin_fmaf(dw * dx[rt][r], d[r], acc[rt][ft][r]);
                }
            }
        }
        if (c + 1 < nch) {
            wait_vmcnt<0>();
            store_scales((c + 1) & 1);
        }
        __syncthreads();
    }

    // k halves added in a fixed order (kh 0 + kh 1), times alpha, and the
    // tile stored as whole rows
    prefill_store_tile<kW4FeatTiles>(acc, lds, lane, fg, rg, kh, out, out_dtype, N, M, rb, fb, alpha);
}

}  // namespace

hipError_t launch_w4a8(const W4A8Args &p) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(w4a8_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kW4Lds) != hipSuccess)
        return hipErrorInvalidValue;
    const int gx = (p.M + kW4Feats - 1) / kW4Feats;
    const int groups = (p.N + kW4Rows - 1) / kW4Rows;
    const int per_launch = std::max(1, (1 << 30) / gx);  // row groups per launch (grid below 2^30)
    for (int g0 = 0; g0 < groups; g0 += per_launch) {
        const int gy = std::min(per_launch, groups - g0);
        const int8_t *qx = reinterpret_cast<const int8_t *>(p.qx) + (size_t)g0 * kW4Rows * p.K;
        const uint16_t *xs = reinterpret_cast<const uint16_t *>(p.xscales) + (size_t)g0 * kW4Rows * (p.K / 32);
        void *out = static_cast<char *>(p.out) + (size_t)g0 * kW4Rows * p.M * out_elem_bytes(p.out_dtype);
        const int n = std::min(p.N - g0 * kW4Rows, gy * kW4Rows);
        hipLaunchKernelGGL(w4a8_kernel, dim3(gx * gy), dim3(kW4Threads), kW4Lds, p.stream,
                           reinterpret_cast<const uint8_t *>(p.codes), reinterpret_cast<const uint16_t *>(p.wscales),
                           qx, xs, out, p.out_dtype, n, p.M, p.K, p.alpha, gy);
    }
    return hipGetLastError();
}

}  // namespace vq
