// h32_quant.hip -- Walsh-Hadamard-32 rotation fused into the int8 (and
// 4-bit) activation quantizer.
//
// "Qwen3.8-27B at 45.7 tok/s: DFlash2 in 1bit serve, and 4-bit activations
// with a Hadamard rotation", section "Prompt processing: 4-bit activations,
// rotated first": each 32-block of activations is rotated by a 32-point
// Walsh-Hadamard transform before rounding, and the rotation runs inside the
// quantizer as in-register butterflies plus lane shuffles.
//
// Mapping: 8 lanes per (row, 32-block), 4 consecutive elements per lane.
// Butterfly stages h = 1, 2 are in-register, h = 4, 8, 16 exchange with lanes
// p ^ 1, p ^ 2, p ^ 4.  Each stage computes (x_i + x_{i+h}, x_i - x_{i+h})
// with single IEEE fp32 adds, in the fixed order h = 1, 2, 4, 8, 16.  Then
// amax over the block, d = fp16_rne(amax / QMAX) with a correctly rounded
// division, q = clamp(rint(u / d), -QMAX, QMAX): QMAX = 127 for int8 codes,
// 7 for the 4-bit activation codes of the same section (stored one per byte,
// so the same GEMM reads them).  Every operation is one IEEE
// rounding (no FMA contraction is possible: there are no multiplies), so the
// codes and scales are reproducible bit for bit on any IEEE implementation.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

template <int XD>
__device__ __forceinline__ float act_to_f32(uint32_t bits16) {
    if constexpr (XD == VQ_DTYPE_BF16)
        return __builtin_bit_cast(float, bits16 << 16);
    else
        return h2f(bits16);
}

__device__ __forceinline__ float butterfly(float own, int p, int mask) {
    const float other = __shfl_xor(own, mask, 64);
    // lower index of the pair keeps the sum, upper index gets lower - upper
    return (p & mask) ? (other - own) : (own + other);
}

template <int XD, int QMAX>
__global__ __launch_bounds__(256) void h32_quant_kernel(const uint16_t *__restrict__ x,
                                                         int8_t *__restrict__ q,
                                                         uint16_t *__restrict__ d,
                                                         int64_t total_blocks) {
    const int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = gl >> 3;  // (row, block) pair; rows are contiguous, so x offset = 32 * blk
    const int p = (int)(gl & 7);
    const bool valid = blk < total_blocks;

    float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
    if (valid) {
        const u32x2 raw = ld8(x + blk * 32 + 4 * p);
        v0 = act_to_f32<XD>(raw[0] & 0xFFFFu);
        v1 = act_to_f32<XD>(raw[0] >> 16);
        v2 = act_to_f32<XD>(raw[1] & 0xFFFFu);
        v3 = act_to_f32<XD>(raw[1] >> 16);
    }
    // h = 1
    const float a0 = v0 + v1, a1 = v0 - v1, a2 = v2 + v3, a3 = v2 - v3;
    // h = 2
    float u0 = a0 + a2, u2 = a0 - a2, u1 = a1 + a3, u3 = a1 - a3;
    // h = 4, 8, 16 across lanes
#pragma unroll
    for (int mask = 1; mask <= 4; mask <<= 1) {
        u0 = butterfly(u0, p, mask);
        u1 = butterfly(u1, p, mask);
        u2 = butterfly(u2, p, mask);
        u3 = butterfly(u3, p, mask);
    }
    float am = fmaxf(fmaxf(fabsf(u0), fabsf(u1)), fmaxf(fabsf(u2), fabsf(u3)));
    am = fmaxf(am, __shfl_xor(am, 1, 64));
    am = fmaxf(am, __shfl_xor(am, 2, 64));
    am = fmaxf(am, __shfl_xor(am, 4, 64));

    const float d32 = am / (float)QMAX;  // correctly rounded (built with fp32 IEEE division)
    const _Float16 dh = static_cast<_Float16>(d32);
    const float df = static_cast<float>(dh);
    int8_t q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (df != 0.0f) {
        auto code = [df](float u) -> int8_t {
            const float r = rintf(u / df);
            return static_cast<int8_t>(fminf(fmaxf(r, -(float)QMAX), (float)QMAX));
        };
        q0 = code(u0); q1 = code(u1); q2 = code(u2); q3 = code(u3);
    }
    if (valid) {
        const uint32_t packed = (uint32_t)(uint8_t)q0 | ((uint32_t)(uint8_t)q1 << 8) |
                                ((uint32_t)(uint8_t)q2 << 16) | ((uint32_t)(uint8_t)q3 << 24);
        *reinterpret_cast<uint32_t *>(q + blk * 32 + 4 * p) = packed;
        if (p == 0)
            d[blk] = __builtin_bit_cast(uint16_t, dh);
    }
}

// ---------------------------------------------------------------------------
// Offline rotation of Q4_0 weights (same section of the same page: the weights
// are rotated once, offline, by the same transform, so that the rotated
// product divided by 32 is the plain one; the pages' tool turns a plain Q4_0
// file into the rotated one).  Per (row, 32-block), 8 lanes as above: lane p
// holds k = 4p .. 4p + 3, i.e. dword p & 3 of the block's 16 code bytes, low
// nibbles for p < 4 and high nibbles for p >= 4 (byte i holds k = i and
// k = 16 + i).  Dequantize exactly (fp16 scale times q - 8), rotate with the
// butterflies above, then requantize by the Q4_0 rule: m = the value of
// largest magnitude (the first one on ties), d = m / -8, id = d != 0 ? 1 / d
// : 0, q = min(15, trunc(x * id + 8.5)), each step one IEEE fp32 operation
// (contraction into FMAs is off in this kernel), d stored as fp16 with
// round-to-nearest-even.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void q4_rotate_h32_kernel(const uint32_t *__restrict__ codes,
                                                             const uint16_t *__restrict__ scales,
                                                             uint32_t *__restrict__ codes_out,
                                                             uint16_t *__restrict__ scales_out,
                                                             int64_t total_blocks) {
    // every multiply and add below is its own IEEE operation: a fused
    // u * id + 8.5 would round once instead of twice and move some codes
#pragma clang fp contract(off)
    const int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = gl >> 3;  // (row, block); a row's blocks are contiguous in both arrays
    const int p = (int)(gl & 7);
    const bool valid = blk < total_blocks;

    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
        const uint32_t word = codes[blk * 4 + (p & 3)];
        const float d0 = h2f(scales[blk]);
        const uint32_t nib = p < 4 ? word : word >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = d0 * (float)((int)((nib >> (8 * i)) & 0xFu) - 8);  // exact
    }
    // h = 1, 2 in registers, h = 4, 8, 16 across the 8 lanes
    const float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
    float u[4] = {a0 + a2, a1 + a3, a0 - a2, a1 - a3};
#pragma unroll
    for (int mask = 1; mask <= 4; mask <<= 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = butterfly(u[i], p, mask);
    }
    // the value of largest magnitude, the first on ties: max of
    // (|u| bits, 31 - k, sign) over the block
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ub = __builtin_bit_cast(uint32_t, u[i]);
        const uint64_t key = ((uint64_t)(ub & 0x7FFFFFFFu) << 32) | ((uint32_t)(31 - (4 * p + i)) << 1) | (ub >> 31);
        best = key > best ? key : best;
    }
#pragma unroll
    for (int mask = 1; mask <= 4; mask <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)best, mask, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), mask, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        best = o > best ? o : best;
    }
    // a block of zeros has m = +0 (whatever the zeros' signs), so d = -0
    const uint32_t mag = (uint32_t)(best >> 32);
    const float m = mag == 0 ? 0.0f : __builtin_bit_cast(float, mag | ((uint32_t)(best & 1u) << 31));
    const float d = m / -8.0f;
    const float id = d != 0.0f ? 1.0f / d : 0.0f;  // correctly rounded (IEEE fp32 division)
    uint32_t q4 = 0;                                // this lane's 4 codes, one per byte
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float t = u[i] * id;
        const float r = t + 8.5f;
        const int qi = (int)r;                      // r >= 0: truncation is floor
        q4 |= (uint32_t)(qi > 15 ? 15 : qi) << (8 * i);
    }
    const uint32_t hi4 = __shfl_xor(q4, 4, 64);     // lanes p and p + 4 share the code bytes
    if (valid && p < 4) {
        codes_out[blk * 4 + p] = q4 | (hi4 << 4);
        if (p == 0)
            scales_out[blk] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(d));
    }
}

hipError_t launch_q4_rotate_h32(const void *codes, const void *scales, int M, int K, void *codes_out,
                                void *scales_out, hipStream_t stream) {
    const int64_t total_blocks = (int64_t)M * (K / 32);
    const int64_t grid = (total_blocks * 8 + 255) / 256;
    hipLaunchKernelGGL(q4_rotate_h32_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const uint32_t *>(codes), static_cast<const uint16_t *>(scales),
                       static_cast<uint32_t *>(codes_out), static_cast<uint16_t *>(scales_out), total_blocks);
    return hipGetLastError();
}

template <int QMAX>
hipError_t launch_quant_q(const void *x, int x_dtype, int8_t *q, void *d, int64_t total_blocks, int64_t grid,
                          hipStream_t stream) {
    if (x_dtype == VQ_DTYPE_BF16)
        hipLaunchKernelGGL((h32_quant_kernel<VQ_DTYPE_BF16, QMAX>), dim3((unsigned)grid), dim3(256), 0, stream,
                           reinterpret_cast<const uint16_t *>(x), q, reinterpret_cast<uint16_t *>(d), total_blocks);
    else
        hipLaunchKernelGGL((h32_quant_kernel<VQ_DTYPE_F16, QMAX>), dim3((unsigned)grid), dim3(256), 0, stream,
                           reinterpret_cast<const uint16_t *>(x), q, reinterpret_cast<uint16_t *>(d), total_blocks);
    return hipGetLastError();
}

hipError_t launch_h32_quant(const void *x, int x_dtype, int8_t *q, void *d, int N, int K, int qmax,
                            hipStream_t stream) {
    const int64_t total_blocks = (int64_t)N * (K / 32);
    const int64_t lanes = total_blocks * 8;
    const int64_t grid = (lanes + 255) / 256;
    if (qmax == 127)
        return launch_quant_q<127>(x, x_dtype, q, d, total_blocks, grid, stream);
    if (qmax == 7)
        return launch_quant_q<7>(x, x_dtype, q, d, total_blocks, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace vq
