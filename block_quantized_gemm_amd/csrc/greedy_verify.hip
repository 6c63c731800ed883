// greedy_verify.hip -- greedy acceptance of a verified draft block.
//
// "Qwen3.8-27B on the AMD R9700: up to 227 tok/s", sections "A block-diffusion
// drafter, verified exactly" and "What 'lossless' means here, precisely": the
// target scores every position of the draft block in one batched forward, and
// a drafted token is committed only where it equals the target's own greedy
// choice, so the output is what plain greedy decoding produces.  This file
// turns the verify pass's logits [n_rows][vocab] into those choices and the
// number of committed tokens.
//
// The choice of a row is its argmax: the first NaN if the row holds one, else
// the first of its largest values (-0 and +0 equal).  Each element becomes a
// 64-bit key whose unsigned order is exactly that preference -- the value
// mapped to an order-preserving 32-bit integer in the high word, the
// complement of its index in the low word -- so that the argmax is one max
// reduction, the same under any reduction order.
//
// Two kernels: the first splits every row into segments, one workgroup per
// (segment, row), and writes each segment's best key to the workspace; the
// second, one workgroup, reduces the segments of every row, writes the
// choices and counts the committed tokens.  The work is bound by reading the
// logits once from HBM.
#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

namespace {

constexpr int kGvThreads = 256;

// Order-preserving key of a float: larger values give larger keys, NaN the
// largest of all, -0 the key of +0.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if (x != x)
        return 0xFFFFFFFFu;
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int DT>
__device__ __forceinline__ float logit_at(const void *p, int64_t i) {
    if constexpr (DT == VQ_DTYPE_F32) {
        return static_cast<const float *>(p)[i];
    } else if constexpr (DT == VQ_DTYPE_BF16) {
        return __builtin_bit_cast(float, (uint32_t) static_cast<const uint16_t *>(p)[i] << 16);
    } else {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<const uint16_t *>(p)[i]));
    }
}

__device__ __forceinline__ uint64_t key_of(float x, int idx) {
    return ((uint64_t)order_key(x) << 32) | (uint32_t)~(uint32_t)idx;
}

__device__ __forceinline__ uint64_t wave_max(uint64_t k) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)k, off, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        k = o > k ? o : k;
    }
    return k;
}

// Workgroup max of one key per thread (kGvThreads threads); every thread gets it.
__device__ __forceinline__ uint64_t block_max(uint64_t k, uint64_t *red) {
    k = wave_max(k);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0)
        red[wave] = k;
    __syncthreads();
    uint64_t m = red[0];
#pragma unroll
    for (int w = 1; w < kGvThreads / 64; ++w)
        m = red[w] > m ? red[w] : m;
    __syncthreads();
    return m;
}

// Best key of 8 consecutive elements of one 16-byte load (two for fp32),
// indices from v.
template <int DT>
__device__ __forceinline__ uint64_t best_of_8(const void *row, int v) {
    uint64_t best = 0;
    if constexpr (DT == VQ_DTYPE_F32) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(static_cast<const float *>(row) + v);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(static_cast<const float *>(row) + v + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // copy the element out first: a bit_cast of a vector element read
            // element 0 whatever i was, with this compiler
            const uint32_t ai = a[i], bi = b[i];
            const uint64_t ka = key_of(__builtin_bit_cast(float, ai), v + i);
            const uint64_t kb = key_of(__builtin_bit_cast(float, bi), v + 4 + i);
            best = ka > best ? ka : best;
            best = kb > best ? kb : best;
        }
    } else {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(row) + v);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint16_t h = (uint16_t)(a[i >> 1] >> (16 * (i & 1)));
            const float x = DT == VQ_DTYPE_BF16 ? __builtin_bit_cast(float, (uint32_t)h << 16)
                                                : static_cast<float>(__builtin_bit_cast(_Float16, h));
            const uint64_t k = key_of(x, v + i);
            best = k > best ? k : best;
        }
    }
    return best;
}

// One workgroup per (segment, row): the best key of the row's elements
// [seg * seg_len, (seg + 1) * seg_len); seg_len is a multiple of 8, so a
// segment of a row that starts 16-byte aligned is read with 16-byte loads
// (scalar loads for an unaligned row and for the row's last few elements).
template <int DT>
__global__ __launch_bounds__(kGvThreads) void argmax_segments(const void *logits, int vocab, int seg_len,
                                                              uint64_t *part) {
    __shared__ uint64_t red[kGvThreads / 64];
    constexpr int kElem = DT == VQ_DTYPE_F32 ? 4 : 2;
    const int seg = (int)blockIdx.x, row = (int)blockIdx.y;
    const int v0 = seg * seg_len, v1 = min(vocab, v0 + seg_len);
    const char *rowp = static_cast<const char *>(logits) + (int64_t)row * vocab * kElem;
    const bool vec = (reinterpret_cast<uintptr_t>(rowp) & 15) == 0;
    uint64_t best = 0;  // below every element's key: the high word of a key is at least key(-inf) > 0
    for (int v = v0 + 8 * (int)threadIdx.x; v < v1; v += 8 * kGvThreads) {
        if (vec && v + 8 <= v1) {
            const uint64_t k = best_of_8<DT>(rowp, v);
            best = k > best ? k : best;
        } else {
            for (int i = v; i < min(v + 8, v1); ++i) {
                const uint64_t k = key_of(logit_at<DT>(rowp, i), i);
                best = k > best ? k : best;
            }
        }
    }
    best = block_max(best, red);
    if (threadIdx.x == 0)
        part[(int64_t)row * gridDim.x + seg] = best;
}

// One workgroup: every row's choice from its segments (one wave per row at a
// time, the rows in parallel), then the committed count: the leading rows
// whose drafted token equals the choice, plus one.
constexpr int kFinishThreads = 1024;

__global__ __launch_bounds__(kFinishThreads) void greedy_finish(const uint64_t *part, int nseg, int n_rows,
                                                                const int32_t *draft, int32_t *tokens,
                                                                int32_t *count) {
    __shared__ int first_miss;
    const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
    if (threadIdx.x == 0)
        first_miss = n_rows - 1;
    __syncthreads();
    for (int r = wave; r < n_rows; r += kFinishThreads / 64) {
        uint64_t best = 0;
        for (int s = lane; s < nseg; s += 64) {
            const uint64_t k = part[(int64_t)r * nseg + s];
            best = k > best ? k : best;
        }
        best = wave_max(best);
        if (lane == 0) {
            const int32_t choice = (int32_t)~(uint32_t)best;
            tokens[r] = choice;
            if (r < n_rows - 1 && draft[r] != choice)
                atomicMin(&first_miss, r);  // LDS atomic
        }
    }
    __syncthreads();
    if (threadIdx.x == 0)
        *count = first_miss + 1;
}

template <int DT>
hipError_t launch_dt(const void *logits, int n_rows, int vocab, const int32_t *draft, int32_t *tokens,
                     int32_t *count, uint64_t *part, hipStream_t stream) {
    const int nseg = greedy_segments(vocab);
    const int seg_len = ((vocab + nseg - 1) / nseg + 7) & ~7;  // whole 16-byte loads inside a segment
    hipLaunchKernelGGL(argmax_segments<DT>, dim3(nseg, n_rows), dim3(kGvThreads), 0, stream, logits, vocab, seg_len,
                       part);
    hipLaunchKernelGGL(greedy_finish, dim3(1), dim3(kFinishThreads), 0, stream, part, nseg, n_rows, draft, tokens,
                       count);
    return hipGetLastError();
}

}  // namespace

int greedy_segments(int vocab) { return std::max(1, std::min(128, (vocab + 4095) / 4096)); }

size_t greedy_workspace_bytes(int n_rows, int vocab) { return (size_t)n_rows * greedy_segments(vocab) * 8; }

hipError_t launch_greedy_verify(const void *logits, int dtype, int n_rows, int vocab, const int32_t *draft,
                                int32_t *tokens, int32_t *count, void *workspace, hipStream_t stream) {
    uint64_t *part = static_cast<uint64_t *>(workspace);
    if (dtype == VQ_DTYPE_F32)
        return launch_dt<VQ_DTYPE_F32>(logits, n_rows, vocab, draft, tokens, count, part, stream);
    if (dtype == VQ_DTYPE_BF16)
        return launch_dt<VQ_DTYPE_BF16>(logits, n_rows, vocab, draft, tokens, count, part, stream);
    return launch_dt<VQ_DTYPE_F16>(logits, n_rows, vocab, draft, tokens, count, part, stream);
}

}  // namespace vq
