// vq_api.cpp -- the C ABI: argument validation, launch-shape choice, dispatch.
//
// Every argument is checked before the first HIP call; on any error nothing is
// enqueued.  The launch shape of a verify GEMM is a function of (M, K) only,
// never of N, so an output row is computed by the same instruction sequence
// whatever the draft-block width ("Qwen3.8-27B on the AMD R9700: up to 227
// tok/s", section "What 'lossless' means here, precisely": outputs compared
// byte for byte across widths 8, 12 and 16).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "vq.h"
#include "vq_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return VQ_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int known = g_dev_ok[dev].load(std::memory_order_relaxed);
        if (known == 1)
            return VQ_OK;
        if (known == 2)
            return VQ_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return VQ_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices)
        g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? VQ_OK : VQ_ERR_DEVICE;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool float_act(int d) { return d == VQ_DTYPE_F16 || d == VQ_DTYPE_BF16; }
bool out_ok(int d) { return d == VQ_DTYPE_F16 || d == VQ_DTYPE_BF16 || d == VQ_DTYPE_F32; }
bool dim_ok(int64_t v) { return v >= 1 && v <= VQ_MAX_DIM; }

// Default launch shape for an (M, K) verify GEMM: FG feature tiles per
// workgroup share each staged activation tile (activation traffic per weight
// byte falls by FG) while keeping about one workgroup per CU or more on the
// 256-CU part; then KW K-groups per workgroup for ~2-2.5k waves in flight,
// keeping at least 4 steps of 128 k per K-group.  A function of (M, K) only.
constexpr int64_t kMinWorkgroups = 240;
constexpr int64_t kTargetWaves = 2600;

void default_shape(bool fp8, int64_t m, int64_t k, int *fg_out, int *kw_out) {
    const int64_t tiles = (m + 15) / 16;
    const int64_t steps = fp8 ? k / 128 : (k / 32 + 3) / 4;
    int fg = 1;
    if ((tiles + 3) / 4 >= kMinWorkgroups)
        fg = 4;
    else if ((tiles + 1) / 2 >= kMinWorkgroups)
        fg = 2;
    const int64_t wgs = (tiles + fg - 1) / fg;
    int kw = 1;
    while (fg * kw * 2 <= 16 && wgs * fg * kw * 2 <= kTargetWaves && (steps + kw * 2 - 1) / (kw * 2) >= 4 &&
           vq::verify_shape_ok(fp8, fg, kw * 2, (int)k))
        kw *= 2;
    *fg_out = fg;
    *kw_out = kw;
}

int run_verify(bool fp8, const void *w, const void *scales, const void *act, int act_dtype,
               void *out, int out_dtype, int64_t n, int64_t m, int64_t k, float alpha, int tpw,
               int kw, void *stream) {
    if (!w || !scales || !act || !out)
        return VQ_ERR_NULL_POINTER;
    if (!float_act(act_dtype) || !out_ok(out_dtype))
        return VQ_ERR_BAD_DTYPE;
    if (!dim_ok(n) || !dim_ok(m) || !dim_ok(k) || k % (fp8 ? 128 : 32) != 0)
        return VQ_ERR_BAD_SHAPE;
    if (!aligned16(w) || !aligned16(scales) || !aligned16(act) || !aligned16(out))
        return VQ_ERR_MISALIGNED;
    int dt = 0, dk = 0;
    default_shape(fp8, m, k, &dt, &dk);
    if (tpw == 0)
        tpw = dt;
    if (kw == 0)
        kw = dk;
    if (!vq::verify_shape_ok(fp8, tpw, kw, (int)k))
        return VQ_ERR_BAD_CONFIG;
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    vq::VerifyArgs p{w, scales, act, out, act_dtype, out_dtype, (int)n, (int)m, (int)k,
                     alpha, tpw, kw, static_cast<hipStream_t>(stream)};
    return vq::launch_verify(p, fp8) == hipSuccess ? VQ_OK : VQ_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int vq_gemm_q4_0(const void *w_codes, const void *w_scales, const void *act, int act_dtype,
                 const void *act_scales, void *out, int out_dtype, int64_t n_rows, int64_t m,
                 int64_t k, float alpha, void *stream) {
    if (act_dtype != VQ_DTYPE_I8) {
        if (act_scales != nullptr)
            return VQ_ERR_BAD_DTYPE;  // float activations carry no scales
        return run_verify(false, w_codes, w_scales, act, act_dtype, out, out_dtype, n_rows, m, k,
                          alpha, 0, 0, stream);
    }
    if (!w_codes || !w_scales || !act || !act_scales || !out)
        return VQ_ERR_NULL_POINTER;
    if (!out_ok(out_dtype))
        return VQ_ERR_BAD_DTYPE;
    if (!dim_ok(n_rows) || !dim_ok(m) || !dim_ok(k) || k % 32 != 0)
        return VQ_ERR_BAD_SHAPE;
    if (!aligned16(w_codes) || !aligned16(w_scales) || !aligned16(act) || !aligned16(act_scales) ||
        !aligned16(out))
        return VQ_ERR_MISALIGNED;
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    vq::W4A8Args p{w_codes, w_scales, act, act_scales, out, out_dtype, (int)n_rows, (int)m, (int)k,
                   alpha, static_cast<hipStream_t>(stream)};
    return vq::launch_w4a8(p) == hipSuccess ? VQ_OK : VQ_ERR_LAUNCH;
}

int vq_gemm_q4_0_ex(const void *w_codes, const void *w_scales, const void *act, int act_dtype,
                    void *out, int out_dtype, int64_t n_rows, int64_t m, int64_t k, float alpha,
                    int tiles_per_wave, int waves_k, void *stream) {
    return run_verify(false, w_codes, w_scales, act, act_dtype, out, out_dtype, n_rows, m, k, alpha,
                      tiles_per_wave, waves_k, stream);
}

int vq_gemm_fp8_blk128(const void *w_e4m3, const float *w_tile_scales, const void *act,
                       int act_dtype, void *out, int out_dtype, int64_t n_rows, int64_t m,
                       int64_t k, void *stream) {
    return run_verify(true, w_e4m3, w_tile_scales, act, act_dtype, out, out_dtype, n_rows, m, k,
                      1.0f, 0, 0, stream);
}

int vq_gemm_fp8_blk128_ex(const void *w_e4m3, const float *w_tile_scales, const void *act,
                          int act_dtype, void *out, int out_dtype, int64_t n_rows, int64_t m,
                          int64_t k, int tiles_per_wave, int waves_k, void *stream) {
    return run_verify(true, w_e4m3, w_tile_scales, act, act_dtype, out, out_dtype, n_rows, m, k,
                      1.0f, tiles_per_wave, waves_k, stream);
}

int vq_hadamard32_quant_int8(const void *x, int x_dtype, int8_t *q_out, void *scales_out,
                             int64_t n_rows, int64_t k, void *stream) {
    if (!x || !q_out || !scales_out)
        return VQ_ERR_NULL_POINTER;
    if (!float_act(x_dtype))
        return VQ_ERR_BAD_DTYPE;
    if (!dim_ok(n_rows) || !dim_ok(k) || k % 32 != 0)
        return VQ_ERR_BAD_SHAPE;
    if (!aligned16(x) || !aligned16(q_out) || !aligned16(scales_out))
        return VQ_ERR_MISALIGNED;
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    return vq::launch_h32_quant(x, x_dtype, q_out, scales_out, (int)n_rows, (int)k,
                                static_cast<hipStream_t>(stream)) == hipSuccess
               ? VQ_OK
               : VQ_ERR_LAUNCH;
}

int vq_default_launch_shape(int kind, int64_t m, int64_t k, int *tiles_per_wave, int *waves_k) {
    if (!tiles_per_wave || !waves_k)
        return VQ_ERR_NULL_POINTER;
    if ((kind != 0 && kind != 1) || !dim_ok(m) || !dim_ok(k))
        return VQ_ERR_BAD_SHAPE;
    default_shape(kind == 1, m, k, tiles_per_wave, waves_k);
    return VQ_OK;
}

const char *vq_status_string(int status) {
    switch (status) {
    case VQ_OK: return "ok";
    case VQ_ERR_NULL_POINTER: return "a required pointer is NULL";
    case VQ_ERR_BAD_SHAPE: return "bad shape: sizes out of range or K not a multiple of the block";
    case VQ_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
    case VQ_ERR_BAD_DTYPE: return "dtype code unknown or not allowed for this argument";
    case VQ_ERR_DEVICE: return "current HIP device is not gfx950 (or no device)";
    case VQ_ERR_LAUNCH: return "HIP kernel launch failed";
    case VQ_ERR_BAD_CONFIG: return "unsupported explicit launch shape";
    default: return "unknown status";
    }
}

int vq_version(void) { return 100; }

}  // extern "C"
