// hbm_probe.hip -- a plain HBM read probe: the denominator that the verify
// kernels' streaming rate is compared against on the device at hand.
//
// The verify GEMM is a weight stream: its ideal is to read every byte once at
// the rate HBM delivers to a kernel that does nothing else ("Qwen3.8-27B on the
// AMD R9700: up to 227 tok/s", TL;DR: plain decode streams the weights at a
// fraction of the card's bandwidth).  This kernel reads a buffer once with the
// verify kernels' load instruction (16 bytes per lane, 1 KiB per wave
// instruction, raw buffer loads) and folds the words into one XOR per thread,
// stored only if it equals a value the caller never passes, so that no load
// can be dropped.  Three access patterns:
//   blocks  -- one workgroup per 64 KiB block (as many workgroups as blocks;
//              the hardware keeps several per CU);
//   shares  -- `groups` persistent workgroups, workgroup b reading the b-th of
//              `groups` equal contiguous shares front to back, its waves
//              interleaved 1 KiB apart (the walk kernel's pattern);
//   window  -- `groups` persistent workgroups reading 64 KiB blocks b, b + G,
//              b + 2G, ... (the whole grid sweeps one contiguous window);
//   reread  -- as shares, each share read VQ_PROBE_REREAD_PASSES times over
//              in the launch (after the first pass, from L2 if it fits);
//   lds     -- `groups` workgroups each stage the buffer's first 64 KiB in
//              LDS and read `bytes` from it (16 bytes per lane, consecutive
//              lanes on consecutive 16 bytes): the LDS read rate of a CU,
//              for the prefill GEMMs' budgets.
// Each wave keeps `depth` loads in flight.  The loads use the default cache
// policy or the non-temporal one (a stream read once: on gfx950 the latter
// reaches a higher read rate).
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

namespace {

constexpr int kPiece = 1024;       // one wave instruction: 64 lanes x 16 bytes
constexpr int kBlock = 64 * 1024;  // blocks of the blocks and window patterns

struct ProbeArgs {
    const uint8_t *buf;
    uint32_t bytes;
    int mode;
    uint32_t share;     // shares: bytes per workgroup (a multiple of kPiece)
    uint32_t sentinel;  // never equal to a real XOR in practice
    uint32_t *sink;
};

// RR: the reread pattern, in an instantiation of its own (its offsets wrap
// with a mask, and no other pattern's branches sit in its loop: it measures
// L2 hits, where the cost of issuing a load shows).
template <int W, int D, int AUX, bool RR>
__global__ __launch_bounds__(64 * W) void hbm_probe_kernel(const ProbeArgs a) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int b = (int)blockIdx.x, G = (int)gridDim.x;
    const rsrc_t r = make_rsrc(a.buf, a.bytes);
    const int per = (int)(a.share / kPiece) / W;  // shares: pieces of one share (one pass) per wave
    // byte offset of this wave's j-th piece
    auto piece = [&](int j) -> uint32_t {
        if constexpr (RR) {
            return (uint32_t)b * a.share + (uint32_t)(wave + W * (j & (per - 1))) * kPiece;
        } else {
            if (a.mode == VQ_PROBE_BLOCKS)
                return (uint32_t)b * kBlock + (uint32_t)(wave + W * j) * kPiece;
            if (a.mode == VQ_PROBE_SHARES)
                return (uint32_t)b * a.share + (uint32_t)(wave + W * j) * kPiece;
            constexpr int pb = kBlock / kPiece / W;  // pieces of one block per wave
            const int blk = j / pb, in = j - blk * pb;
            return ((uint32_t)blk * (uint32_t)G + (uint32_t)b) * kBlock + (uint32_t)(wave + W * in) * kPiece;
        }
    };
    int n;  // pieces of this wave
    if (RR)
        n = per * VQ_PROBE_REREAD_PASSES;
    else if (a.mode == VQ_PROBE_BLOCKS)
        n = kBlock / kPiece / W;
    else if (a.mode == VQ_PROBE_SHARES)
        n = per;
    else
        n = (int)((a.bytes / kBlock + G - 1 - b) / G) * (kBlock / kPiece / W);
    u32x4 acc = {0u, 0u, 0u, 0u};
    u32x4 st[D];
    pipeline<D>(
        n, [&](auto U, int j) { st[U.value] = bload16<AUX>(r, (int)(piece(j) + 16u * lane), 0); },
        [&](auto U, int, bool) { acc ^= st[U.value]; });
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == a.sentinel)
        a.sink[0] = x;
}

constexpr int kLdsProbeBytes = 64 * 1024;

// D reads of 1 KiB per wave and iteration, from D distinct rows of the wave's
// 16 KiB window (four windows, each shared by the waves w with the same w % 4).
// Each read's 16 bytes are handed to an empty asm statement and one of its
// words goes into the XOR: one VALU instruction per read, so that the reads,
// not the folding (four XORs per read would take as many VALU cycles per CU
// as the LDS takes to deliver the bytes), set the rate.
template <int W, int D>
__global__ __launch_bounds__(64 * W) void lds_probe_kernel(const ProbeArgs a) {
    static_assert(D % 2 == 0 && D <= 16, "pairs of reads, at most 16 rows");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const rsrc_t r = make_rsrc(a.buf, kLdsProbeBytes);
    for (int i = (int)threadIdx.x; i < kLdsProbeBytes / 16; i += 64 * W)
        *reinterpret_cast<u32x4 *>(lds + 16 * i) = bload16<kAuxCached>(r, 16 * i, 0);
    __syncthreads();
    // every read is below 3 * 16 KiB + 15 KiB + 1 KiB = 64 KiB
    const uint8_t *win = lds + (wave & 3) * 16384 + 16 * lane;
    const int iters = (int)(a.bytes / kPiece) / (W * D);
    u32x4 acc = {0u, 0u, 0u, 0u};  // only acc[0] is used
    int off = 0;
    for (int it = 0; it < iters; ++it) {
        asm volatile("" : "+v"(off));  // off stays 0, but the compiler cannot see the reads repeat
        u32x4 v[D];
#pragma unroll
        for (int q = 0; q < D; ++q)
            v[q] = *reinterpret_cast<const u32x4 *>(win + off + kPiece * q);
#pragma unroll
        for (int q = 0; q < D; ++q) {
            asm volatile("" ::"v"(v[q]));  // all 16 bytes are used: the reads stay 16-byte reads
            acc[0] ^= v[q][q & 3];
        }
    }
    const uint32_t x = acc[0];
    if (x == a.sentinel)
        a.sink[0] = x;
}

template <int W>
hipError_t launch_lds(const ProbeArgs &a, int grid, int depth, hipStream_t s) {
    switch (depth) {
    case 4: hipLaunchKernelGGL((lds_probe_kernel<W, 4>), dim3(grid), dim3(64 * W), kLdsProbeBytes, s, a); break;
    case 8: hipLaunchKernelGGL((lds_probe_kernel<W, 8>), dim3(grid), dim3(64 * W), kLdsProbeBytes, s, a); break;
    case 16: hipLaunchKernelGGL((lds_probe_kernel<W, 16>), dim3(grid), dim3(64 * W), kLdsProbeBytes, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int W, int AUX, bool RR>
hipError_t launch_rr(const ProbeArgs &a, int grid, int depth, hipStream_t s) {
    switch (depth) {
    case 4: hipLaunchKernelGGL((hbm_probe_kernel<W, 4, AUX, RR>), dim3(grid), dim3(64 * W), 0, s, a); break;
    case 8: hipLaunchKernelGGL((hbm_probe_kernel<W, 8, AUX, RR>), dim3(grid), dim3(64 * W), 0, s, a); break;
    case 16: hipLaunchKernelGGL((hbm_probe_kernel<W, 16, AUX, RR>), dim3(grid), dim3(64 * W), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int W, int AUX>
hipError_t launch_w(const ProbeArgs &a, int grid, int depth, hipStream_t s) {
    return a.mode == VQ_PROBE_REREAD ? launch_rr<W, AUX, true>(a, grid, depth, s)
                                     : launch_rr<W, AUX, false>(a, grid, depth, s);
}

template <int AUX>
hipError_t launch_aux(const ProbeArgs &a, int grid, int waves, int depth, hipStream_t s) {
    switch (waves) {
    case 4: return launch_w<4, AUX>(a, grid, depth, s);
    case 8: return launch_w<8, AUX>(a, grid, depth, s);
    case 16: return launch_w<16, AUX>(a, grid, depth, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_hbm_probe(const void *buf, size_t bytes, int mode, int groups, int waves, int depth,
                            bool nontemporal, uint32_t *sink, hipStream_t stream) {
    ProbeArgs a{static_cast<const uint8_t *>(buf), (uint32_t)bytes, mode, 0u, 0x9E3779B9u, sink};
    if (mode == VQ_PROBE_LDS) {
        switch (waves) {
        case 4: return launch_lds<4>(a, groups, depth, stream);
        case 8: return launch_lds<8>(a, groups, depth, stream);
        case 16: return launch_lds<16>(a, groups, depth, stream);
        default: return hipErrorInvalidValue;
        }
    }
    if (mode == VQ_PROBE_SHARES || mode == VQ_PROBE_REREAD)
        a.share = (uint32_t)(bytes / (size_t)groups);
    const int grid = mode == VQ_PROBE_BLOCKS ? (int)(bytes / kBlock) : groups;
    return nontemporal ? launch_aux<kAuxStream>(a, grid, waves, depth, stream)
                       : launch_aux<kAuxCached>(a, grid, waves, depth, stream);
}

}  // namespace vq
