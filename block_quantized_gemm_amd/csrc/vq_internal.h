// vq_internal.h -- host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "vq.h"

namespace vq {

// Arguments of one verify GEMM launch, already validated.
struct VerifyArgs {
    const void *w;       // Q4_0 codes or E4M3 bytes
    const void *scales;  // Q4_0 fp16 block scales or FP8 fp32 tile scales
    const void *act;     // [N][K] 16-bit activations
    void *out;           // [N][M]
    int act_dtype, out_dtype;
    int N, M, K;
    float alpha;
    int tiles_per_wg;  // FG: 16-feature tiles per workgroup sharing each activation tile
    int waves_k;       // KW: K-groups per workgroup
    hipStream_t stream;
};

// Largest dynamic LDS a workgroup may use on gfx950 (160 KiB per CU).
constexpr size_t kMaxLdsBytes = 160 * 1024;

// Arguments of one W4A8 launch (int8 activations with fp16 block scales).
struct W4A8Args {
    const void *codes, *wscales, *qx, *xscales;
    void *out;
    int out_dtype;
    int N, M, K;
    float alpha;
    hipStream_t stream;
};

inline size_t out_elem_bytes(int dtype) { return dtype == VQ_DTYPE_F32 ? 4 : 2; }

hipError_t launch_verify(const VerifyArgs &p, bool fp8);
size_t verify_lds_bytes(bool fp8, int fg, int kw, int K);
bool verify_shape_ok(bool fp8, int fg, int kw, int K);
hipError_t launch_w4a8(const W4A8Args &p);
hipError_t launch_h32_quant(const void *x, int x_dtype, int8_t *q, void *d, int N, int K,
                            hipStream_t stream);

}  // namespace vq
