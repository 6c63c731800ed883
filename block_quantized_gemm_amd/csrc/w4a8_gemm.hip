// w4a8_gemm.hip -- Q4_0 weights x int8 activations with fp16 per-32-block
// scales, on the int8 MFMA (the prefill-sized "exact int8 path").
//
// "Qwen3.8-27B at 45.7 tok/s: DFlash2 in 1bit serve, and 4-bit activations
// with a Hadamard rotation", section "Prompt processing: 4-bit activations,
// rotated first": a Q4_0 code is a 4-bit value with offset 8, and flipping its
// top bit gives the same value in two's complement.  Here (q XOR 8) is placed
// in the HIGH nibble of an int8, which makes the byte exactly 16 * (q - 8);
// the factor 16 is folded into the (power-of-two exact) weight scale.
//
// Per 32-block b: D_b = sum_j 16 (q - 8) q_x on a 16x16x32 int8 MFMA (exact
// int32), then out += (d_w / 16) * d_x * D_b in fp32.  The per-block scale
// epilogue (int->float, scale product, FMA for every output and block) is the
// bound of this kernel: the MFMA itself needs only a fraction of the time.
//
// Mapping: 4 waves per workgroup, each wave one 16-feature tile and RT row
// tiles of 16 rows (all waves share the rows).  k-slot group g of the MFMA
// covers k = 32b + 8g .. 8g+7: lanes with g < 2 take the low nibbles of block
// bytes 8g..8g+7, lanes with g >= 2 the high nibbles of bytes 8(g-2)..+7.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

constexpr int kW4A8RowTiles = 4;

template <int RT>
__global__ __launch_bounds__(256) void w4a8_kernel(const uint8_t *__restrict__ codes,
                                                    const uint16_t *__restrict__ wscales,
                                                    const int8_t *__restrict__ qx,
                                                    const uint16_t *__restrict__ xscales,
                                                    void *__restrict__ out, int out_dtype, int N,
                                                    int M, int K, float alpha) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int g = lane >> 4;
    const int NB = K >> 5;
    const int f = (blockIdx.x * 4 + wave) * 16 + j;
    const bool fvalid = f < M;
    const uint8_t *crow = codes + (size_t)(fvalid ? f : 0) * (size_t)(K >> 1) + 8 * (g & 1);
    const uint16_t *wsrow = wscales + (size_t)(fvalid ? f : 0) * NB;
    const int shift = g < 2 ? 4 : 0;
    const int rowbase = blockIdx.y * 16 * RT;

    const int8_t *arow[RT];
    bool avalid[RT];
    const uint16_t *xsrow[RT][4];
    bool ovalid[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int ar = rowbase + 16 * rt + j;
        avalid[rt] = ar < N;
        arow[rt] = qx + (size_t)(avalid[rt] ? ar : 0) * K + 8 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int orow = rowbase + 16 * rt + 4 * g + r;
            ovalid[rt][r] = orow < N;
            xsrow[rt][r] = xscales + (size_t)(ovalid[rt][r] ? orow : 0) * NB;
        }
    }

    f32x4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const i32x4 izero = {0, 0, 0, 0};

    for (int b = 0; b < NB; ++b) {
        u32x2 wv = {0u, 0u};
        float dw = 0.f;
        if (fvalid) {
            wv = ld8(crow + 16 * b);
            dw = h2f(wsrow[b]) * 0.0625f;  // exact: removes the operand's factor 16
        }
        const uint32_t t0 = wv[0] ^ 0x88888888u, t1 = wv[1] ^ 0x88888888u;
        const uint64_t bop = (uint64_t)((t0 << shift) & 0xF0F0F0F0u) |
                             ((uint64_t)((t1 << shift) & 0xF0F0F0F0u) << 32);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const u32x2 av = avalid[rt] ? ld8(arow[rt] + 32 * b) : u32x2{0u, 0u};
            const uint64_t aop = (uint64_t)av[0] | ((uint64_t)av[1] << 32);
            const i32x4 dot = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)aop, (long)bop, izero, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float dx = ovalid[rt][r] ? h2f(xsrow[rt][r][b]) : 0.f;
                acc[rt][r] = __builtin_fmaf(dw * dx, (float)dot[r], acc[rt][r]);
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (ovalid[rt][r] && fvalid)
                store_out(out, out_dtype, (size_t)(rowbase + 16 * rt + 4 * g + r) * M + f,
                          alpha * acc[rt][r]);
}

hipError_t launch_w4a8(const W4A8Args &p) {
    constexpr int RT = kW4A8RowTiles;
    const int tiles = (p.M + 15) / 16;
    const int gx = (tiles + 3) / 4;
    const int rows_per_wg = 16 * RT;
    const int groups = (p.N + rows_per_wg - 1) / rows_per_wg;
    constexpr int kMaxGridY = 65535;
    for (int g0 = 0; g0 < groups; g0 += kMaxGridY) {
        const int gy = std::min(kMaxGridY, groups - g0);
        const int8_t *qx = reinterpret_cast<const int8_t *>(p.qx) + (size_t)g0 * rows_per_wg * p.K;
        const uint16_t *xs = reinterpret_cast<const uint16_t *>(p.xscales) + (size_t)g0 * rows_per_wg * (p.K / 32);
        void *out = static_cast<char *>(p.out) + (size_t)g0 * rows_per_wg * p.M * out_elem_bytes(p.out_dtype);
        const int n = std::min(p.N - g0 * rows_per_wg, gy * rows_per_wg);
        hipLaunchKernelGGL(w4a8_kernel<RT>, dim3(gx, gy), dim3(256), 0, p.stream,
                           reinterpret_cast<const uint8_t *>(p.codes),
                           reinterpret_cast<const uint16_t *>(p.wscales), qx, xs, out, p.out_dtype, n,
                           p.M, p.K, p.alpha);
    }
    return hipGetLastError();
}

}  // namespace vq
