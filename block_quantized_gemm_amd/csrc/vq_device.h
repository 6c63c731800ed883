// vq_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Everything here is written for CDNA4 (gfx950) wave64: the 16x16x32 16-bit
// MFMA, the 16x16x32 int8 MFMA, the v_permlane16/32_swap lane exchanges and
// the OCP-FP8 conversion instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "vq.h"

namespace vq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// 16-bit activation formats.  A Q4_0 code q becomes the exact 16-bit value
// MAGIC + q by placing the nibble in the low mantissa bits under a fixed
// exponent byte: bf16 0x43nn = 128 + q, fp16 0x64nn = 1024 + q.  The offset
// (MAGIC + 8) is removed through the MFMA accumulator input (see the verify
// kernel).  Every product x * (MAGIC + q) is exact in fp32, but the block
// MFMA adds 32 terms of size about (MAGIC + 8) |x| onto -(MAGIC + 8) * sum x,
// and these mostly cancel: the fp32 rounding of that sum is up to about
// (MAGIC + 8) / 8 times that of a direct sum of (q - 8) x, i.e. about 17x for
// bf16 activations (136 / 8) and about 130x for fp16 (1032 / 8).  The block
// dot is exact where the partial sums are (integer-valued activations of
// modest size); otherwise it carries that amplified fp32 rounding, which the
// parity tolerance covers (fp16 heavy-tailed rows with outlier channels are
// among the parity cases).
// ---------------------------------------------------------------------------
template <int ACT>
struct Act16;

template <>
struct Act16<VQ_DTYPE_BF16> {
    static constexpr uint32_t kMagicByte = 0x43434343u;  // bf16 128 + q
    static constexpr uint32_t kNegOffset = 0xC308C308u;  // bf16 -136, twice
    static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // two E4M3 codes (a 16-bit word of `w`) -> two exact bf16 values
    template <bool HI>
    static __device__ __forceinline__ uint32_t fp8x2(uint32_t w) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    }
};

template <>
struct Act16<VQ_DTYPE_F16> {
    static constexpr uint32_t kMagicByte = 0x64646464u;  // fp16 1024 + q
    static constexpr uint32_t kNegOffset = 0xE408E408u;  // fp16 -1032, twice
    static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    template <bool HI>
    static __device__ __forceinline__ uint32_t fp8x2(uint32_t w) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
    }
};

// ---------------------------------------------------------------------------
// 4x4 transpose across the four 16-lane groups of a wave.
// On entry lane group G holds in r[t] the dword t of "its" 16-byte record;
// on exit lane group G holds in r[t] the dword G of lane group t's record.
// Two v_permlane32_swap then two v_permlane16_swap: one VALU op per dword.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void transpose_lane_groups(uint32_t &r0, uint32_t &r1, uint32_t &r2,
                                                      uint32_t &r3) {
    auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
    auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
    auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    r0 = c[0];
    r1 = c[1];
    r2 = d[0];
    r3 = d[1];
}

// ---------------------------------------------------------------------------
// One dword of Q4_0 codes (block bytes 4g..4g+3) -> the 8 exact 16-bit
// operands MAGIC + q for k = 4g..4g+3 (low nibbles) and 16+4g..16+4g+3 (high
// nibbles), in that k order, two per register.  2 ANDs, 1 shift, 4 byte
// permutes; the permute puts each masked byte under the exponent byte.
// ---------------------------------------------------------------------------
template <uint32_t MAGIC>
__device__ __forceinline__ u32x4 q4_operand(uint32_t v) {
    const uint32_t lo = v & 0x0F0F0F0Fu;
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
    u32x4 r;
    // __builtin_amdgcn_perm(s0, s1, sel): selector byte 0..3 picks a byte of
    // s1, 4..7 a byte of s0.
    r[0] = __builtin_amdgcn_perm(MAGIC, lo, 0x04010400u);  // (k=4g,   4g+1)
    r[1] = __builtin_amdgcn_perm(MAGIC, lo, 0x04030402u);  // (k=4g+2, 4g+3)
    r[2] = __builtin_amdgcn_perm(MAGIC, hi, 0x04010400u);  // (k=16+4g, 17+4g)
    r[3] = __builtin_amdgcn_perm(MAGIC, hi, 0x04030402u);  // (k=18+4g, 19+4g)
    return r;
}

// ---------------------------------------------------------------------------
// Raw buffer loads.  A buffer resource carries a byte size; the hardware
// returns zeros for any lane whose offset falls outside it, which is how rows
// past M or N are masked without divergent branches.  Offsets: a per-lane
// VGPR part and a wave-uniform SGPR part.  Cache policy (aux): non-temporal
// (2) for a stream read once front to back in whole lines (panel records),
// the default (0) where a load takes half of each 128-byte line and the
// next step takes the other half (row-major Q4_0 and FP8 rows), which L2
// must keep.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kAuxStream = 2;  // nt
constexpr int kAuxCached = 0;

// The base and size must be wave-uniform: they are moved to scalar registers
// here, because a descriptor the compiler cannot prove uniform (say, a size
// computed with a vector min/max) would otherwise turn every load through it
// into a loop over the distinct descriptors of the wave.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    // word 3 = 0x00020000: raw (untyped) dword data format for the gfx9 family
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}
template <int AUX>
__device__ __forceinline__ u32x4 bload16(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}
template <int AUX>
__device__ __forceinline__ u32x2 bload8(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX));
}
template <int AUX>
__device__ __forceinline__ uint32_t bload4(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
}
template <int AUX>
__device__ __forceinline__ uint32_t bload2(rsrc_t r, int voff, int soff) {
    return (uint32_t)__builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, AUX));
}

// 16 bytes per lane from a buffer straight into LDS (no registers): lane l's
// bytes land at lds_dst + 16 l, whatever its source offset (voff + the
// wave-uniform soff); out-of-range offsets deliver zeros.  lds_dst must be wave-uniform.  The load counts in
// vmcnt like any other: wait for it before the LDS is read.  AUX: the cache
// policy, as for bload16.
template <int AUX = kAuxCached>
__device__ __forceinline__ void bload16_lds(rsrc_t r, void *lds_dst, int voff, int soff = 0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_dst, 16, voff, soff, 0,
                                             AUX);
}

// s_waitcnt that waits until at most n vector-memory operations are
// outstanding (n <= 63) and leaves the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Workgroup barrier that leaves vmcnt alone.  __syncthreads' release fence
// waits for every outstanding vector memory operation of the wave (buffer
// loads into LDS count there), which would drain the weight pipeline; callers
// of this barrier first wait for exactly the LDS writes the other waves need.
// Outstanding LDS reads of this wave are waited for (lgkmcnt), and the memory
// clobber keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Software pipeline over a wave's `ns` steps with PF stage buffers.
//   load(U, i)          -- issue the loads of step i into stage buffer U
//   compute(U, i, full) -- consume stage U holding step i (full: no K tail)
// U is a std::integral_constant so buffers are indexed at compile time.
// When the wave has at least 2 PF steps, the prologue and the steady-state
// loop issue every load unconditionally: the compiler's wait-count insertion
// then knows how many newer loads are in flight and waits only for the stage
// it is about to use.  Shorter runs (and the tail) use guarded loads.
// ---------------------------------------------------------------------------
template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, F, I + 1>(static_cast<F &&>(f));
    }
}

template <int PF, typename LoadF, typename ComputeF>
__device__ __forceinline__ void pipeline(int ns, LoadF &&load, ComputeF &&compute) {
    int i = 0;
    if (ns >= 2 * PF) {
        static_for<PF>([&](auto U) { load(U, U.value); });
        do {
            static_for<PF>([&](auto U) {
                compute(U, i + U.value, true);
                // keep the refill of this stage right here: the scheduler would
                // otherwise sink it below later compute and drain the pipeline
                __builtin_amdgcn_sched_barrier(0);
                load(U, i + U.value + PF);
                __builtin_amdgcn_sched_barrier(0);
            });
            i += PF;
        } while (i + 2 * PF <= ns);
    } else {
        static_for<PF>([&](auto U) {
            if (U.value < ns)
                load(U, U.value);
        });
    }
    static_for<PF>([&](auto U) {
        if (i + U.value < ns) {
            compute(U, i + U.value, false);
            if (i + U.value + PF < ns)
                load(U, i + U.value + PF);
        }
    });
    static_for<PF>([&](auto U) {
        if (i + PF + U.value < ns)
            compute(U, i + PF + U.value, false);
    });
}

// Workgroups of a 1-D grid go to the 8 XCDs in turn (workgroup b to XCD
// b % 8).  The index returned numbers them so that the workgroups of one XCD
// hold a contiguous run of indices [0, G): tiles that share operands, given
// consecutive indices, then share that XCD's L2.
__device__ __forceinline__ int xcd_run_index(int b, int G) {
    const int xcd = b & 7, loc = b >> 3, n = G >> 3, extra = G & 7;
    return xcd * n + min(xcd, extra) + loc;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// ---------------------------------------------------------------------------
// Plain global loads (used where a buffer resource does not pay).
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld_stream16(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 ld16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ u32x2 ld8(const void *p) {
    return *reinterpret_cast<const u32x2 *>(p);
}

// fp16 bits -> float (exact)
__device__ __forceinline__ float h2f(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// ---------------------------------------------------------------------------
// Output rounding: fp32 -> out dtype, round to nearest even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_out(void *out, int out_dtype, size_t idx, float v) {
    if (out_dtype == VQ_DTYPE_F32) {
        reinterpret_cast<float *>(out)[idx] = v;
    } else if (out_dtype == VQ_DTYPE_BF16) {
        reinterpret_cast<__bf16 *>(out)[idx] = static_cast<__bf16>(v);
    } else {
        reinterpret_cast<_Float16 *>(out)[idx] = static_cast<_Float16>(v);
    }
}

// ---------------------------------------------------------------------------
// Output tile of a prefill workgroup (128 rows x 2 * FT * 16 features, 8
// waves: wave = fg + 2 rg + 4 kh holds rows 64 rg .. +64 and features
// FT * 16 fg .. of the k half kh, as acc[row tile][feature tile]).  Half of
// the row tiles at a time: kh 1 hands its partials to kh 0 through LDS, kh 0
// adds them (kh 0 + kh 1, the same order for every N), multiplies by alpha
// and rounds to the output type (as store_out), the rounded half tile goes
// through LDS, and all waves store it as 16-byte pieces of whole output rows
// (one element at a time at a ragged right edge, or where rows are not 16-byte
// aligned).  Needs 64 * FT * 16 * 4 * 4 bytes of LDS (every operand stage is
// free by then) and the whole workgroup.  The output type is a template
// argument so that the loops over elements carry no branches.
// ---------------------------------------------------------------------------
template <int FT, int OD>
__device__ __forceinline__ void prefill_store_tile_od(f32x4 (&acc)[4][FT], uint8_t *lds, int lane, int fg, int rg,
                                                      int kh, void *out, int N, int M, int rb, int fb, float alpha) {
    constexpr int kFeats = 2 * FT * 16;
    constexpr int esz = OD == VQ_DTYPE_F32 ? 4 : 2;
    constexpr int rowb = kFeats * esz, row_pieces = rowb / 16, per = 16 / esz;
    const int j = lane & 15, g = lane >> 4, pair = fg + 2 * rg;
    const bool vec = ((size_t)M * (size_t)esz) % 16 == 0;
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (kh == 1) {
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[(((pair * 2 + r2) * FT + ft) * 4 + r) * 64 + lane] = acc[2 * h + r2][ft][r];
        }
        __syncthreads();
        if (kh == 0) {
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[2 * h + r2][ft][r] =
                            alpha * (acc[2 * h + r2][ft][r] + red[(((pair * 2 + r2) * FT + ft) * 4 + r) * 64 + lane]);
        }
        __syncthreads();  // the partials are read: the area takes the rounded tile
        if (kh == 0) {
            // local row rg 32 + r2 16 + 4 g + r of the half, local feature FT 16 fg + 16 ft + j
            uint8_t *base = lds + (rg * 32 + 4 * g) * rowb + (FT * 16 * fg + j) * esz;
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        uint8_t *dst = base + (r2 * 16 + r) * rowb + 16 * ft * esz;
                        const float v = acc[2 * h + r2][ft][r];
                        if constexpr (OD == VQ_DTYPE_F32)
                            *reinterpret_cast<float *>(dst) = v;
                        else if constexpr (OD == VQ_DTYPE_BF16)
                            *reinterpret_cast<__bf16 *>(dst) = static_cast<__bf16>(v);
                        else
                            *reinterpret_cast<_Float16 *>(dst) = static_cast<_Float16>(v);
                    }
        }
        __syncthreads();
        // local row lr is output row rb + 64 (lr / 32) + 16 (2 h + lr / 16 % 2) + lr % 16
        for (int i = (int)threadIdx.x; i < 64 * row_pieces; i += (int)blockDim.x) {
            const int lr = i / row_pieces, q = i - lr * row_pieces;
            const int row = rb + (lr >> 5) * 64 + (2 * h + ((lr >> 4) & 1)) * 16 + (lr & 15);
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
        __syncthreads();  // the area is reused by the next half
    }
}

template <int FT>
__device__ __forceinline__ void prefill_store_tile(f32x4 (&acc)[4][FT], uint8_t *lds, int lane, int fg, int rg,
                                                   int kh, void *out, int out_dtype, int N, int M, int rb, int fb,
                                                   float alpha) {
    if (out_dtype == VQ_DTYPE_F32)
        prefill_store_tile_od<FT, VQ_DTYPE_F32>(acc, lds, lane, fg, rg, kh, out, N, M, rb, fb, alpha);
    else if (out_dtype == VQ_DTYPE_BF16)
        prefill_store_tile_od<FT, VQ_DTYPE_BF16>(acc, lds, lane, fg, rg, kh, out, N, M, rb, fb, alpha);
    else
        prefill_store_tile_od<FT, VQ_DTYPE_F16>(acc, lds, lane, fg, rg, kh, out, N, M, rb, fb, alpha);
}

}  // namespace vq
