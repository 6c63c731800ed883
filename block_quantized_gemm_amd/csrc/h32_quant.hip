// h32_quant.hip -- Walsh-Hadamard-32 rotation fused into the int8 activation
// quantizer.
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
// amax over the block, d = fp16_rne(amax / 127) with a correctly rounded
// division, q = clamp(rint(u / d), -127, 127).  Every operation is one IEEE
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

template <int XD>
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

    const float d32 = am / 127.0f;  // correctly rounded (built with fp32 IEEE division)
    const _Float16 dh = static_cast<_Float16>(d32);
    const float df = static_cast<float>(dh);
    int8_t q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (df != 0.0f) {
        auto code = [df](float u) -> int8_t {
            const float r = rintf(u / df);
            return static_cast<int8_t>(fminf(fmaxf(r, -127.0f), 127.0f));
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

hipError_t launch_h32_quant(const void *x, int x_dtype, int8_t *q, void *d, int N, int K,
                            hipStream_t stream) {
    const int64_t total_blocks = (int64_t)N * (K / 32);
    const int64_t lanes = total_blocks * 8;
    const int64_t grid = (lanes + 255) / 256;
    if (x_dtype == VQ_DTYPE_BF16)
        hipLaunchKernelGGL(h32_quant_kernel<VQ_DTYPE_BF16>, dim3((unsigned)grid), dim3(256), 0, stream,
                           reinterpret_cast<const uint16_t *>(x), q, reinterpret_cast<uint16_t *>(d),
                           total_blocks);
    else
        hipLaunchKernelGGL(h32_quant_kernel<VQ_DTYPE_F16>, dim3((unsigned)grid), dim3(256), 0, stream,
                           reinterpret_cast<const uint16_t *>(x), q, reinterpret_cast<uint16_t *>(d),
                           total_blocks);
    return hipGetLastError();
}

}  // namespace vq
