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
// sums in fp32.  Features [128 i, 128 i + 128) of a workgroup and the 128 k
// of one chunk lie in one scale tile, so a chunk's four MFMA steps accumulate
// a partial that is added to the output with one fp32 FMA with that tile's
// scale -- the order the verify kernels use for each output too.
//
// Tiling: a workgroup of 4 waves computes 128 rows x 128 features; wave
// (wr, wf) takes rows 64 wr .. +64 and features 64 wf .. +64 as 4 x 4 MFMA
// tiles.  K moves in chunks of 128: the chunk's activations (128 rows x 256 B)
// and weights (128 features x 128 B) are loaded into registers while the
// previous chunk is computed from LDS, then written to the other of two LDS
// buffers (rows padded by 16 bytes against bank conflicts).  k-slot group g of
// the MFMA covers k = 32 s + 8 g .. +7 of step s for both operands.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

namespace {

constexpr int kPfRows = 128, kPfFeats = 128, kPfK = 128;  // per workgroup and chunk
constexpr int kPfAPitch = 2 * kPfK + 16;                  // activation bytes per row in LDS
constexpr int kPfBPitch = kPfK + 16;                      // weight bytes per feature in LDS
constexpr int kPfABytes = kPfRows * kPfAPitch;
constexpr int kPfBBytes = kPfFeats * kPfBPitch;
constexpr int kPfBuf = kPfABytes + kPfBBytes;
constexpr int kPfOut = 0x7FFFFFF0;  // past every range below: the load returns zeros

template <int ACT>
__global__ __launch_bounds__(256) void fp8_prefill_kernel(const uint8_t *__restrict__ w, const float *__restrict__ ts,
                                                          const uint16_t *__restrict__ x, void *__restrict__ out,
                                                          int out_dtype, int N, int M, int K) {
    using A16 = Act16<ACT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = threadIdx.x, lane = t & 63, wave = wave_id(), j = lane & 15, g = lane >> 4;
    const int wr = wave >> 1, wf = wave & 1;
    const int fb = blockIdx.x * kPfFeats, rb = blockIdx.y * kPfRows;
    const int nch = K / kPfK;
    const int rows = min(kPfRows, N - rb), feats = min(kPfFeats, M - fb);
    const float *trow = ts + (size_t)(fb / 128) * nch;  // this workgroup's scale tiles, one per chunk

    // Activation rows in two halves of 64 (each range below 2^31 bytes), the
    // weights of this workgroup's features; loads past them read zeros.
    const rsrc_t ra0 = make_rsrc(x + (size_t)rb * K, (uint32_t)min(rows, 64) * (uint32_t)K * 2u);
    const rsrc_t ra1 = make_rsrc(x + (size_t)(rb + 64) * K * (rows > 64), (uint32_t)max(rows - 64, 0) * (uint32_t)K * 2u);
    const rsrc_t rw = make_rsrc(w + (size_t)fb * K, (uint32_t)feats * (uint32_t)K);

    // one chunk: 8 activation pieces and 4 weight pieces of 16 bytes per thread
    u32x4 ga[8], gb[4];
    auto load_chunk = [&](int c) {
        const int k0 = c * kPfK;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int p = t + 256 * i, row = p >> 4, col = 2 * k0 + 16 * (p & 15);  // bytes
            ga[i] = bload16<kAuxCached>(i < 4 ? ra0 : ra1, (row & 63) * K * 2 + col, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = t + 256 * i, f = p >> 3, col = k0 + 16 * (p & 7);
            gb[i] = bload16<kAuxCached>(rw, f * K + col, 0);
        }
    };
    auto store_chunk = [&](int buf) {
        uint8_t *base = lds + buf * kPfBuf;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int p = t + 256 * i;
            *reinterpret_cast<u32x4 *>(base + (p >> 4) * kPfAPitch + 16 * (p & 15)) = ga[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = t + 256 * i;
            *reinterpret_cast<u32x4 *>(base + kPfABytes + (p >> 3) * kPfBPitch + 16 * (p & 7)) = gb[i];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ft = 0; ft < 4; ++ft)
            acc[rt][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    load_chunk(0);
    wait_vmcnt<0>();
    store_chunk(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch)
            load_chunk(c + 1);
        const uint8_t *base = lds + (c & 1) * kPfBuf;
        const uint8_t *abase = base + (wr * 64 + j) * kPfAPitch + 16 * g;
        const uint8_t *bbase = base + kPfABytes + (wf * 64 + j) * kPfBPitch + 8 * g;
        const float s = trow[c];
        f32x4 part[4][4];
#pragma unroll
        for (int st = 0; st < kPfK / 32; ++st) {
            u32x4 bop[4];
#pragma unroll
            for (int ft = 0; ft < 4; ++ft) {
                const u32x2 wv = *reinterpret_cast<const u32x2 *>(bbase + ft * 16 * kPfBPitch + 32 * st);
                bop[ft] = u32x4{A16::template fp8x2<false>(wv[0]), A16::template fp8x2<true>(wv[0]),
                                A16::template fp8x2<false>(wv[1]), A16::template fp8x2<true>(wv[1])};
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const u32x4 aop = *reinterpret_cast<const u32x4 *>(abase + rt * 16 * kPfAPitch + 64 * st);
#pragma unroll
                for (int ft = 0; ft < 4; ++ft)
                    part[rt][ft] = A16::mfma(aop, bop[ft], st == 0 ? zero4 : part[rt][ft]);
            }
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ft = 0; ft < 4; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[rt][ft][r] = __builtin_fmaf(s, part[rt][ft][r], acc[rt][ft][r]);
        if (c + 1 < nch) {
            wait_vmcnt<0>();
            store_chunk((c + 1) & 1);
        }
        __syncthreads();
    }

#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ft = 0; ft < 4; ++ft) {
            const int f = fb + wf * 64 + ft * 16 + j;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rb + wr * 64 + rt * 16 + 4 * g + r;
                if (row < N && f < M)
                    store_out(out, out_dtype, (size_t)row * M + f, acc[rt][ft][r]);
            }
        }
}

template <int ACT>
hipError_t launch_act(const Fp8PrefillArgs &p) {
    const size_t shm = 2 * (size_t)kPfBuf;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(fp8_prefill_kernel<ACT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm) != hipSuccess)
        return hipErrorInvalidValue;
    const int gx = (p.M + kPfFeats - 1) / kPfFeats;
    const int groups = (p.N + kPfRows - 1) / kPfRows;
    constexpr int kMaxGridY = 65535;
    for (int g0 = 0; g0 < groups; g0 += kMaxGridY) {
        const int gy = std::min(kMaxGridY, groups - g0);
        const uint16_t *x = static_cast<const uint16_t *>(p.act) + (size_t)g0 * kPfRows * p.K;
        void *out = static_cast<char *>(p.out) + (size_t)g0 * kPfRows * p.M * out_elem_bytes(p.out_dtype);
        const int n = std::min(p.N - g0 * kPfRows, gy * kPfRows);
        hipLaunchKernelGGL(fp8_prefill_kernel<ACT>, dim3(gx, gy), dim3(256), shm, p.stream,
                           static_cast<const uint8_t *>(p.w), p.tile_scales, x, out, p.out_dtype, n, p.M, p.K);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_prefill(const Fp8PrefillArgs &p) {
    return p.act_dtype == VQ_DTYPE_BF16 ? launch_act<VQ_DTYPE_BF16>(p) : launch_act<VQ_DTYPE_F16>(p);
}

}  // namespace vq
