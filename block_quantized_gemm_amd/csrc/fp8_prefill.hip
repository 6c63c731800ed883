// fp8_prefill.hip -- FP8 block-scaled weights times many 16-bit activation
// rows (prompt-sized batches), on the 16-bit MFMA.
//
// "r9k: a from-scratch inference engine for Qwen3.8-27B on two Radeon AI PRO
// R9700", opening paragraph: FP8 E4M3 weights with one scale per 128 x 128
// tile, a custom block-scaled FP8 GEMM.  The verify kernels serve a draft
// block of <= 16 rows by streaming the weights once; a prompt of hundreds of
// rows is compute-bound instead, and this kernel tiles it for the MFMA.
//
// Arithmetic: every E4M3 code converts exactly to bf16 / fp16 (hardware
// conversion); the MFMA 16x16x32 multiplies it by the activations exactly and
// sums in fp32.  A 16-feature tile and the 128 k of one chunk lie in one
// scale tile, so MFMA steps within a chunk accumulate a partial that is added
// to the output with one fp32 FMA with that tile's scale.
//
// Tiling: a workgroup of 8 waves computes 128 rows x 288 features (18 MFMA
// tiles; 17408 features make 61 columns, so a 512-row prompt is one round of
// 244 workgroups on 256 CUs).  Wave (fg, rg, kh) takes features 144 fg ..
// +144, rows 64 rg .. +64, and the MFMA steps 2 kh, 2 kh + 1 of every 128-k
// chunk: for each output tile it sums its two steps on the MFMA and adds that
// partial, times the chunk's tile scale, with one fp32 FMA; the two k halves
// are added at the end (kh 0 + kh 1, fixed order), so each row's arithmetic
// is independent of N.  Chunks (activations 128 rows x 256 B, codes 288
// features x 128 B) are loaded straight into LDS (16 B per lane, no
// registers) one chunk ahead, into the other of two stages; 16-byte pieces
// are XOR-swizzled by row and by feature so that the operand reads are free
// of bank conflicts.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

namespace {

constexpr int kPfRows = 128, kPfFeats = 288, kPfK = 128;  // per workgroup and chunk
constexpr int kPfThreads = 512;
constexpr int kPfFeatTiles = kPfFeats / 2 / 16;  // 9 tiles per wave
constexpr int kPfAStage = kPfRows * 2 * kPfK;    // 16-bit rows, 256 B each
constexpr int kPfBStage = kPfFeats * kPfK;       // E4M3 codes, 128 B per feature
constexpr int kPfStage = kPfAStage + kPfBStage;
constexpr int kPfLds = 2 * kPfStage;
constexpr int kPfTileBytes = 64 * kPfFeats * 4;  // k-half exchange and half of the output tile (fp32)
static_assert(kPfTileBytes <= kPfLds, "epilogue area");
constexpr int kPfOut = 0x7FFFFFF0;  // past every range below: the load returns zeros

template <int ACT>
__global__ __launch_bounds__(kPfThreads) void fp8_prefill_kernel(const uint8_t *__restrict__ w,
                                                                 const float *__restrict__ ts,
                                                                 const uint16_t *__restrict__ x,
                                                                 void *__restrict__ out, int out_dtype, int N, int M,
                                                                 int K, int row_groups) {
    using A16 = Act16<ACT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63, wave = wave_id(), j = lane & 15, g = lane >> 4;
    const int fg = wave & 1, rg = (wave >> 1) & 1, kh = wave >> 2;
    // tiles in column order (the row groups of one feature column are
    // consecutive), numbered so that each XCD holds a run of whole columns
    const int tile = xcd_run_index((int)blockIdx.x, (int)gridDim.x);
    const int fb = tile / row_groups * kPfFeats, rb = tile % row_groups * kPfRows;
    const int nch = K / kPfK, nft = (M + 127) / 128;
    const int rows = min(kPfRows, N - rb), feats = min(kPfFeats, M - fb);

    // Ranges: activation rows in groups of 32, codes in groups of 64
    // features (each below 2^30 bytes); rows past N and features past M read
    // zeros.  A wave load covers 4 rows x 256 B or 8 features x 128 B.
    rsrc_t ra[4], rw[5];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        ra[m] = make_rsrc(x + (size_t)(rb + 32 * m) * K, (uint32_t)max(0, min(32, rows - 32 * m)) * (uint32_t)K * 2u);
#pragma unroll
    for (int m = 0; m < 5; ++m)
        rw[m] = make_rsrc(w + (size_t)(fb + 64 * m) * K, (uint32_t)max(0, min(64, feats - 64 * m)) * (uint32_t)K);
    // Lane offsets of the chunk loads (the chunk's k offset goes in the
    // wave-uniform part).  Activation load i = wave + 8 m covers rows 4 i ..
    // 4 i + 3 of range m (row 4 wave + lane / 16 there); code load i = wave +
    // 8 m (< 36) covers features 8 i .. 8 i + 7 of range m (8 wave + lane / 8).
    // The swizzle terms depend on the row or feature mod 16 only, the same
    // for every m.
    const int a_row = 4 * wave + (lane >> 4), b_feat = 8 * wave + (lane >> 3);
    const int a_voff = a_row * K * 2 + 16 * ((lane & 15) ^ (a_row & 15));
    const int b_voff = b_feat * K + 16 * ((lane & 7) ^ ((b_feat >> 1) & 7));
    auto issue = [&](int c, int stage) {
        uint8_t *st = lds + stage * kPfStage;
        const int k0 = c * kPfK;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            bload16_lds(ra[m], st + 1024 * (wave + 8 * m), a_voff, 2 * k0);
#pragma unroll
        for (int m = 0; m < 5; ++m)
            if (wave + 8 * m < 36)
                bload16_lds(rw[m], st + kPfAStage + 1024 * (wave + 8 * m), b_voff, k0);
    };

    f32x4 acc[4][kPfFeatTiles];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ft = 0; ft < kPfFeatTiles; ++ft)
            acc[rt][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // Tile scales: lane ft (< 9) of each wave loads the chunk's scale of the
    // wave's feature tile ft (its 128-feature scale tile, clamped: tiles past
    // M multiply zeros), one chunk ahead like the operands; the FMAs read it
    // back with a lane read.  (A scalar load here would share its wait
    // counter with the LDS reads and stall every one of them.)
    const rsrc_t rts = make_rsrc(ts, (uint32_t)nft * (uint32_t)nch * 4u);
    const int ts_off = lane < kPfFeatTiles ? min((fb + fg * 144 + lane * 16) >> 7, nft - 1) * nch * 4 : kPfOut;
    const int b_sw = (j >> 1) & 7;

    issue(0, 0);
    uint32_t scale_next = bload4<kAuxCached>(rts, ts_off, 0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const uint32_t scale_bits = scale_next;
        if (c + 1 < nch) {
            issue(c + 1, (c + 1) & 1);
            scale_next = bload4<kAuxCached>(rts, ts_off, 4 * (c + 1));
        }
        const uint8_t *st = lds + (c & 1) * kPfStage;
        const uint8_t *as = st + (rg * 64 + j) * 256;
        const uint8_t *bs = st + kPfAStage + (fg * 144 + j) * 128 + 8 * (g & 1);
        u32x4 a[4][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)  // step 2 kh + s2: bytes 64 step + 16 g
                a[rt][s2] = *reinterpret_cast<const u32x4 *>(as + rt * 16 * 256 + 16 * ((4 * (2 * kh + s2) + g) ^ j));
        float sc[kPfFeatTiles];  // the chunk's tile scale of each feature tile
#pragma unroll
        for (int ft = 0; ft < kPfFeatTiles; ++ft)
            sc[ft] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(scale_bits, ft));
#pragma unroll
        for (int ft = 0; ft < kPfFeatTiles; ++ft) {
            u32x4 b[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {  // bytes 32 step + 8 g
                const u32x2 wv = *reinterpret_cast<const u32x2 *>(bs + ft * 16 * 128 +
                                                                  16 * ((2 * (2 * kh + s2) + (g >> 1)) ^ b_sw));
                b[s2] = u32x4{A16::template fp8x2<false>(wv[0]), A16::template fp8x2<true>(wv[0]),
                              A16::template fp8x2<false>(wv[1]), A16::template fp8x2<true>(wv[1])};
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const f32x4 part = A16::mfma(a[rt][1], b[1], A16::mfma(a[rt][0], b[0], zero4));
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[rt][ft][r] = __builtin_fmaf(sc[ft], part[r], acc[rt][ft][r]);
            }
        }
        // unconditional (nothing is outstanding after the last chunk): a
        // branch here let the compiler sink the scale FMAs past it, keeping
        // every partial tile live at once
        wait_vmcnt<0>();
        __syncthreads();
    }

    // k halves added in a fixed order (kh 0 + kh 1) and the tile stored as
    // whole rows
    prefill_store_tile<kPfFeatTiles>(acc, lds, lane, fg, rg, kh, out, out_dtype, N, M, rb, fb, 1.0f);
}

template <int ACT>
hipError_t launch_act(const Fp8PrefillArgs &p) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(fp8_prefill_kernel<ACT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kPfLds) != hipSuccess)
        return hipErrorInvalidValue;
    const int gx = (p.M + kPfFeats - 1) / kPfFeats;
    const int groups = (p.N + kPfRows - 1) / kPfRows;
    const int per_launch = std::max(1, (1 << 30) / gx);  // row groups per launch (grid below 2^30)
    for (int g0 = 0; g0 < groups; g0 += per_launch) {
        const int gy = std::min(per_launch, groups - g0);
        const uint16_t *x = static_cast<const uint16_t *>(p.act) + (size_t)g0 * kPfRows * p.K;
        void *out = static_cast<char *>(p.out) + (size_t)g0 * kPfRows * p.M * out_elem_bytes(p.out_dtype);
        const int n = std::min(p.N - g0 * kPfRows, gy * kPfRows);
        hipLaunchKernelGGL(fp8_prefill_kernel<ACT>, dim3(gx * gy), dim3(kPfThreads), kPfLds, p.stream,
                           static_cast<const uint8_t *>(p.w), p.tile_scales, x, out, p.out_dtype, n, p.M, p.K, gy);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_prefill(const Fp8PrefillArgs &p) {
    return p.act_dtype == VQ_DTYPE_BF16 ? launch_act<VQ_DTYPE_BF16>(p) : launch_act<VQ_DTYPE_F16>(p);
}

}  // namespace vq
