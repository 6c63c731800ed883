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
// scale tile, so the four MFMA steps of a chunk accumulate a partial (from
// zero) that is added to the output with one fp32 FMA with that tile's
// scale; each row's arithmetic is independent of N.
//
// Tiling: a workgroup of 8 waves computes 128 rows x 320 features (20 MFMA
// tiles; 17408 features make 55 columns, so a 512-row prompt is one round of
// 220 workgroups on 256 CUs).  Wave (rg, fg) takes rows 64 rg .. +64 and
// features 80 fg .. +80 over all of K: per chunk 4 row tiles x 5 feature
// tiles x 4 steps = 80 MFMAs, each converted weight operand serving the 4
// row tiles, and one scale FMA per output.  A lane reads 16 codes of a
// feature (two MFMA steps) with one 16-byte LDS read.  (A 128 x 288 tiling with the
// chunk's steps split between two waves took two scale FMAs per output and
// chunk and was about 3% slower.)  Chunks (activations 128 rows x 256 B,
// codes 320 features x 128 B) are loaded straight into LDS (16 B per lane,
// no registers) one chunk ahead, into the other of two stages; 16-byte pieces
// are XOR-swizzled by row and by feature so that the operand reads are free
// of bank conflicts.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

namespace {

constexpr int kPfRows = 128, kPfFeats = 320, kPfK = 128;  // per workgroup and chunk
constexpr int kPfThreads = 512;
constexpr int kPfFeatTiles = kPfFeats / 4 / 16;  // 5 tiles per wave
constexpr int kPfAStage = kPfRows * 2 * kPfK;    // 16-bit rows, 256 B each
constexpr int kPfBStage = kPfFeats * kPfK;       // E4M3 codes, 128 B per feature
constexpr int kPfStage = kPfAStage + kPfBStage;
constexpr int kPfLds = 2 * kPfStage;
constexpr int kPfOut = 0x7FFFFFF0;  // past every range below: the load returns zeros
constexpr int kPfEpiBytes = 64 * kPfFeats * 4;  // half of the output tile (fp32), staged for the stores
static_assert(kPfEpiBytes <= kPfLds, "epilogue area");

// The output tile, half of the rows at a time: the waves of row group h round
// their results to the output type into LDS, then all waves store 16-byte
// pieces of whole output rows (one element at a time at a ragged right edge,
// or where rows are not 16-byte aligned).  The stages are free by then.
template <int OD>
__device__ __forceinline__ void store_tile(f32x4 (&acc)[4][kPfFeatTiles], uint8_t *lds, int lane, int fg, int rg,
                                               void *out, int N, int M, int rb, int fb) {
    constexpr int esz = OD == VQ_DTYPE_F32 ? 4 : 2;
    constexpr int rowb = kPfFeats * esz, row_pieces = rowb / 16, per = 16 / esz;
    const int j = lane & 15, g = lane >> 4;
    const bool vec = ((size_t)M * (size_t)esz) % 16 == 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (rg == h) {
            // local row 16 rt + 4 g + r, local feature 80 fg + 16 ft + j
            uint8_t *base = lds + (4 * g) * rowb + (80 * fg + j) * esz;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ft = 0; ft < kPfFeatTiles; ++ft)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        uint8_t *dst = base + (rt * 16 + r) * rowb + 16 * ft * esz;
                        const float v = acc[rt][ft][r];
                        if constexpr (OD == VQ_DTYPE_F32)
                            *reinterpret_cast<float *>(dst) = v;
                        else if constexpr (OD == VQ_DTYPE_BF16)
                            *reinterpret_cast<__bf16 *>(dst) = static_cast<__bf16>(v);
                        else
                            *reinterpret_cast<_Float16 *>(dst) = static_cast<_Float16>(v);
                    }
        }
        __syncthreads();
        for (int i = (int)threadIdx.x; i < 64 * row_pieces; i += (int)blockDim.x) {
            const int lr = i / row_pieces, q = i - lr * row_pieces;
            const int row = rb + 64 * h + lr;
            const int f0 = fb + q * per;
            if (row >= N || f0 >= M)
                continue;
            const uint8_t *src = lds + lr * rowb + q * 16;
            uint8_t *dst = static_cast<uint8_t *>(out) + ((size_t)row * (size_t)M + (size_t)f0) * esz;
            if (vec && f0 + per <= M) {
                *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(src);
            } else {
                for (int e = 0; e < per && f0 + e < M; ++e) {
                    if constexpr (esz == 4)
                        reinterpret_cast<uint32_t *>(dst)[e] = reinterpret_cast<const uint32_t *>(src)[e];
                    else
                        reinterpret_cast<uint16_t *>(dst)[e] = reinterpret_cast<const uint16_t *>(src)[e];
                }
            }
        }
        __syncthreads();
    }
}

template <int ACT>
__global__ __launch_bounds__(kPfThreads) void fp8_prefill_kernel(const uint8_t *__restrict__ w,
                                                                 const float *__restrict__ ts,
                                                                 const uint16_t *__restrict__ x,
                                                                 void *__restrict__ out, int out_dtype, int N, int M,
                                                                 int K, int row_groups) {
    using A16 = Act16<ACT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63, wave = wave_id(), j = lane & 15, g = lane >> 4;
    const int rg = wave & 1, fg = wave >> 1;
    const int tile = xcd_run_index((int)blockIdx.x, (int)gridDim.x);
    const int fb = tile / row_groups * kPfFeats, rb = tile % row_groups * kPfRows;
    const int nch = K / kPfK, nft = (M + 127) / 128;
    const int rows = min(kPfRows, N - rb), feats = min(kPfFeats, M - fb);

    // Ranges: activation rows in groups of 32, codes in groups of 64
    // features (each below 2^30 bytes); rows past N and features past M read
    // zeros.  A wave load covers 4 rows x 256 B or 8 features x 128 B:
    // activation load i = wave + 8 m covers rows 4 i .. 4 i + 3 (row 4 wave +
    // lane / 16 of range m), code load i = wave + 8 m features 8 i .. 8 i + 7
    // (8 wave + lane / 8 of range m).  The swizzle terms depend on the row or
    // feature mod 16 only, the same for every m.
    rsrc_t ra[4], rw[5];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        ra[m] = make_rsrc(x + (size_t)(rb + 32 * m) * K, (uint32_t)max(0, min(32, rows - 32 * m)) * (uint32_t)K * 2u);
#pragma unroll
    for (int m = 0; m < 5; ++m)
        rw[m] = make_rsrc(w + (size_t)(fb + 64 * m) * K, (uint32_t)max(0, min(64, feats - 64 * m)) * (uint32_t)K);
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
            bload16_lds(rw[m], st + kPfAStage + 1024 * (wave + 8 * m), b_voff, k0);
    };

    f32x4 acc[4][kPfFeatTiles];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ft = 0; ft < kPfFeatTiles; ++ft)
            acc[rt][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // Tile scales: lane ft (< 5) of each wave loads the chunk's scale of the
    // wave's feature tile ft (its 128-feature scale tile, clamped: tiles past
    // M multiply zeros), one chunk ahead like the operands; the FMAs read it
    // back with a lane read.  (A scalar load here would share its wait
    // counter with the LDS reads and stall every one of them.)
    const rsrc_t rts = make_rsrc(ts, (uint32_t)nft * (uint32_t)nch * 4u);
    const int ts_off = lane < kPfFeatTiles ? min((fb + fg * 80 + lane * 16) >> 7, nft - 1) * nch * 4 : kPfOut;
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
        const uint8_t *bs = st + kPfAStage + (fg * 80 + j) * 128;
        // The k order of the MFMA steps: lane group g of step s takes k = 16 (4
        // (s / 2) + g) + 8 (s % 2) .. +8, so that one 16-byte read of a
        // feature's codes (k = 16 (4 pr + g) .. +16) feeds steps 2 pr and
        // 2 pr + 1; the activations follow the same order (the MFMA sums its
        // 32 products in any k order both operands share).
        u32x4 a[4][4];  // the wave's 4 row tiles, 4 steps
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int s = 0; s < 4; ++s)  // 16-byte piece 8 (s / 2) + 2 g + s % 2 of the row
                a[rt][s] = *reinterpret_cast<const u32x4 *>(
                    as + rt * 16 * 256 + 16 * ((8 * (s >> 1) + 2 * g + (s & 1)) ^ j));
        float sc[kPfFeatTiles];
#pragma unroll
        for (int ft = 0; ft < kPfFeatTiles; ++ft)
            sc[ft] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(scale_bits, ft));
#pragma unroll
        for (int ft = 0; ft < kPfFeatTiles; ++ft) {
            f32x4 part[4] = {zero4, zero4, zero4, zero4};  // this chunk's partial, from zero
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {  // codes k = 16 (4 pr + g) .. +16: steps 2 pr, 2 pr + 1
                const u32x4 wv =
                    *reinterpret_cast<const u32x4 *>(bs + ft * 16 * 128 + 16 * ((4 * pr + g) ^ b_sw));
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4 b = u32x4{A16::template fp8x2<false>(wv[2 * h]), A16::template fp8x2<true>(wv[2 * h]),
                                          A16::template fp8x2<false>(wv[2 * h + 1]),
                                          A16::template fp8x2<true>(wv[2 * h + 1])};
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
                        part[rt] = A16::mfma(a[rt][2 * pr + h], b, part[rt]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[rt][ft][r] = __builtin_fmaf(sc[ft], part[rt][r], acc[rt][ft][r]);
        }
        // unconditional (nothing is outstanding after the last chunk): a
        // branch here let the compiler sink the scale FMAs past it
        wait_vmcnt<0>();
        __syncthreads();
    }

    if (out_dtype == VQ_DTYPE_F32)
        store_tile<VQ_DTYPE_F32>(acc, lds, lane, fg, rg, out, N, M, rb, fb);
    else if (out_dtype == VQ_DTYPE_BF16)
        store_tile<VQ_DTYPE_BF16>(acc, lds, lane, fg, rg, out, N, M, rb, fb);
    else
        store_tile<VQ_DTYPE_F16>(acc, lds, lane, fg, rg, out, N, M, rb, fb);
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
