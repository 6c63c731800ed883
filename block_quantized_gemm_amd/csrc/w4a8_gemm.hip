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
// bound of this kernel: three fp32 VALU operations per output per 32 MACs,
// against which the MFMA itself needs only a fraction of the time.
//
// Tiling: a workgroup of 4 waves computes 128 rows x 128 features; wave
// (wr, wf) takes rows 64 wr .. +64 and features 64 wf .. +64 as 4 x 4 MFMA
// tiles.  K moves in chunks of 4 blocks (128 k): the chunk's activation codes
// (128 x 128 B), weight codes (128 x 64 B) and both scale sets are loaded into
// registers while the previous chunk is computed from LDS, then written to
// the other of two LDS buffers.  k-slot group g of the MFMA covers k = 32b +
// 8g .. 8g+7: lanes with g < 2 take the low nibbles of block bytes 8g..8g+7,
// lanes with g >= 2 the high nibbles of bytes 8(g-2)..+7.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

constexpr int kW4Rows = 128, kW4Feats = 128;  // per workgroup
constexpr int kW4Blocks = 4;                  // 32-blocks per chunk
constexpr int kAPitch = 128 + 16;             // activation codes: bytes per row in LDS
constexpr int kBPitch = 64 + 16;              // weight codes: bytes per feature in LDS
constexpr int kABytes = kW4Rows * kAPitch;
constexpr int kBBytes = kW4Feats * kBPitch;
constexpr int kSBytes = kW4Blocks * kW4Rows * 4;  // one scale set: [block][row] fp32
constexpr int kW4Buf = kABytes + kBBytes + 2 * kSBytes;
constexpr int kOutOfRange = 0x7FFFFFF0;  // past every range below: the load returns zeros

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void w4a8_kernel(const uint8_t *__restrict__ codes,
                                                  const uint16_t *__restrict__ wscales,
                                                  const int8_t *__restrict__ qx,
                                                  const uint16_t *__restrict__ xscales,
                                                  void *__restrict__ out, int out_dtype, int N, int M,
                                                  int K, float alpha) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kW4Buf];
    const int t = threadIdx.x, lane = t & 63, wave = wave_id(), j = lane & 15, g = lane >> 4;
    const int wr = wave >> 1, wf = wave & 1;
    const int fb = blockIdx.x * kW4Feats, rb = blockIdx.y * kW4Rows;
    const int NB = K >> 5, KH = K >> 1;
    const int nch = (NB + kW4Blocks - 1) / kW4Blocks;
    const int rows = min(kW4Rows, N - rb), feats = min(kW4Feats, M - fb);

    // Ranges: activation rows in two halves of 64 (each below 2^30 bytes),
    // weight codes, and the two scale arrays; loads past them read zeros.
    const rsrc_t ra0 = make_rsrc(qx + (size_t)rb * K, (uint32_t)min(rows, 64) * (uint32_t)K);
    const rsrc_t ra1 = make_rsrc(qx + (size_t)(rb + 64) * K * (rows > 64), (uint32_t)max(rows - 64, 0) * (uint32_t)K);
    const rsrc_t rw = make_rsrc(codes + (size_t)fb * KH, (uint32_t)feats * (uint32_t)KH);
    const rsrc_t rsx = make_rsrc(xscales + (size_t)rb * NB, (uint32_t)rows * (uint32_t)NB * 2u);
    const rsrc_t rsw = make_rsrc(wscales + (size_t)fb * NB, (uint32_t)feats * (uint32_t)NB * 2u);

    // ---- one chunk's global -> register loads (each thread: 4 activation
    // pieces, 2 weight pieces of 16 bytes, 4 scales)
    u32x4 ga[4], gb[2];
    uint32_t gs[4];
    auto load_chunk = [&](int c) {
        const int k0 = c * kW4Blocks * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = t + 256 * i, row = p >> 3, col = k0 + 16 * (p & 7);
            const int off = col < K ? (row & 63) * K + col : kOutOfRange;
            ga[i] = bload16<kAuxCached>(i < 2 ? ra0 : ra1, off, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = t + 256 * i, f = p >> 2, col = (k0 >> 1) + 16 * (p & 3);
            gb[i] = bload16<kAuxCached>(rw, col < KH ? f * KH + col : kOutOfRange, 0);
        }
        const int rf = t & 127;  // waves 0, 1: activation scales of row rf; waves 2, 3: weight scales of feature rf
        const rsrc_t rs = wave < 2 ? rsx : rsw;
#pragma unroll
        for (int q = 0; q < kW4Blocks; ++q) {
            const int blk = c * kW4Blocks + q;
            gs[q] = bload2<kAuxCached>(rs, blk < NB ? (rf * NB + blk) * 2 : kOutOfRange, 0);
        }
    };
    auto store_chunk = [&](int buf) {
        uint8_t *base = lds + buf * kW4Buf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = t + 256 * i;
            *reinterpret_cast<u32x4 *>(base + (p >> 3) * kAPitch + 16 * (p & 7)) = ga[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = t + 256 * i;
            *reinterpret_cast<u32x4 *>(base + kABytes + (p >> 2) * kBPitch + 16 * (p & 3)) = gb[i];
        }
        float *sc = reinterpret_cast<float *>(base + kABytes + kBBytes + (wave < 2 ? 0 : kSBytes));
#pragma unroll
        for (int q = 0; q < kW4Blocks; ++q)  // the weight scales carry the operand's 1/16 (exact)
            sc[q * kW4Rows + (t & 127)] = wave < 2 ? h2f(gs[q]) : h2f(gs[q]) * 0.0625f;
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ft = 0; ft < 4; ++ft)
            acc[rt][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    const i32x4 izero = {0, 0, 0, 0};
    const int shift = g < 2 ? 4 : 0;

    load_chunk(0);
    wait_vmcnt<0>();
    store_chunk(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch)
            load_chunk(c + 1);
        const uint8_t *base = lds + (c & 1) * kW4Buf;
        const uint8_t *abase = base + (wr * 64 + j) * kAPitch + 8 * g;
        const uint8_t *bbase = base + kABytes + (wf * 64 + j) * kBPitch + 8 * (g & 1);
        const float *sx = reinterpret_cast<const float *>(base + kABytes + kBBytes) + wr * 64 + 4 * g;
        const float *sw = reinterpret_cast<const float *>(base + kABytes + kBBytes + kSBytes) + wf * 64 + j;
#pragma unroll 1
        for (int q = 0; q < kW4Blocks; ++q) {
            long bop[4];
            float dw[4];
#pragma unroll
            for (int ft = 0; ft < 4; ++ft) {
                const u32x2 wv = *reinterpret_cast<const u32x2 *>(bbase + ft * 16 * kBPitch + 16 * q);
                const uint32_t b0 = ((wv[0] << shift) & 0xF0F0F0F0u) ^ 0x80808080u;
                const uint32_t b1 = ((wv[1] << shift) & 0xF0F0F0F0u) ^ 0x80808080u;
                bop[ft] = (long)((uint64_t)b0 | ((uint64_t)b1 << 32));
                dw[ft] = sw[q * kW4Rows + ft * 16];
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const u32x2 av = *reinterpret_cast<const u32x2 *>(abase + rt * 16 * kAPitch + 32 * q);
                const long aop = (long)((uint64_t)av[0] | ((uint64_t)av[1] << 32));
                const f32x4 dx = *reinterpret_cast<const f32x4 *>(sx + q * kW4Rows + rt * 16);
#pragma unroll
                for (int ft = 0; ft < 4; ++ft) {
                    const i32x4 dot = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop[ft], izero, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[rt][ft][r] = __builtin_fmaf(dw[ft] * dx[r], (float)dot[r], acc[rt][ft][r]);
                }
            }
        }
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
                    store_out(out, out_dtype, (size_t)row * M + f, alpha * acc[rt][ft][r]);
            }
        }
}

hipError_t launch_w4a8(const W4A8Args &p) {
    const int gx = (p.M + kW4Feats - 1) / kW4Feats;
    const int groups = (p.N + kW4Rows - 1) / kW4Rows;
    constexpr int kMaxGridY = 65535;
    for (int g0 = 0; g0 < groups; g0 += kMaxGridY) {
        const int gy = std::min(kMaxGridY, groups - g0);
        const int8_t *qx = reinterpret_cast<const int8_t *>(p.qx) + (size_t)g0 * kW4Rows * p.K;
        const uint16_t *xs = reinterpret_cast<const uint16_t *>(p.xscales) + (size_t)g0 * kW4Rows * (p.K / 32);
        void *out = static_cast<char *>(p.out) + (size_t)g0 * kW4Rows * p.M * out_elem_bytes(p.out_dtype);
        const int n = std::min(p.N - g0 * kW4Rows, gy * kW4Rows);
        hipLaunchKernelGGL(w4a8_kernel, dim3(gx, gy), dim3(256), 0, p.stream,
                           reinterpret_cast<const uint8_t *>(p.codes), reinterpret_cast<const uint16_t *>(p.wscales),
                           qx, xs, out, p.out_dtype, n, p.M, p.K, p.alpha);
    }
    return hipGetLastError();
}

}  // namespace vq
