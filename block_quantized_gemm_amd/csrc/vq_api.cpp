// vq_api.cpp -- the C ABI: argument validation, launch-shape choice, dispatch.
//
// Every argument is checked before the first HIP call; on any error nothing is
// enqueued.  The launch shape of a verify GEMM is a function of (M, K) and the
// workspace capacity only, never of N, so an output row is computed by the
// same instruction sequence whatever the draft-block width ("Qwen3.8-27B on the AMD R9700: up to 227
// tok/s", section "What 'lossless' means here, precisely": outputs compared
// byte for byte across widths 8, 12 and 16).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <vector>

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

// Default launch shape for an (M, K) verify GEMM.  With room for its
// workspace, the walk form: workgroups of eight single-tile waves (a
// workgroup stages each activation element once for 8 tiles; one workgroup
// per CU, its double-buffered activation rows taking half of the LDS), as
// many persistent workgroups as the device holds, each walking an equal
// share of the chunks.  Small M uses smaller
// workgroups.  Otherwise (no workspace, or a Q4_0 K that is not a multiple of
// 256) the one-shot form: one workgroup of four single-tile waves per tile
// group over all of K.  A function of (M, K, workspace capacity) only, never
// of N.
vq::VerifyPlan walk_plan(int64_t m) {
    vq::VerifyPlan pl;
    const int tiles = (int)((m + 15) / 16);
    pl.tiles = 1;
    pl.waves = tiles >= 8 ? 8 : tiles >= 4 ? 4 : 2;
    pl.walk = true;
    return pl;
}

size_t walk_need(bool fp8, const vq::VerifyPlan &pl, int64_t m, int64_t k) {
    return vq::verify_walk_workspace(pl, vq::verify_chunks(fp8, pl, (int)m, (int)k));
}

vq::VerifyPlan default_plan(bool fp8, int64_t m, int64_t k, size_t ws_bytes) {
    vq::VerifyPlan pl = walk_plan(m);
    if (vq::verify_plan_finish(fp8, (int)m, (int)k, pl) && walk_need(fp8, pl, m, k) <= ws_bytes)
        return pl;
    vq::VerifyPlan fb;
    fb.tiles = 1;
    fb.waves = 4;
    vq::verify_plan_finish(fp8, (int)m, (int)k, fb);
    return fb;
}

// The plan of a panel-layout Q4_0 problem: always the walk form, one
// 256-feature panel per workgroup of 8 waves, 2 tiles per wave.
vq::VerifyPlan panel_plan(int max_groups) {
    vq::VerifyPlan pl;
    pl.tiles = vq::kPanelWaveTiles;
    pl.waves = vq::kPanelWaves;
    pl.walk = true;
    pl.panel = true;
    pl.groups = max_groups;
    vq::verify_plan_finish(false, 1, 32, pl);
    return pl;
}

// The plan of a panel-layout FP8 problem: the walk form, one 128-feature
// record per chunk for a workgroup of 8 waves, one tile per wave.
vq::VerifyPlan fp8_panel_plan(int max_groups) {
    vq::VerifyPlan pl;
    pl.tiles = 1;
    pl.waves = vq::kFp8PanelFeatures / 16;
    pl.walk = true;
    pl.panel = true;
    pl.groups = max_groups;
    vq::verify_plan_finish(true, 1, 128, pl);
    return pl;
}

int check_panel_problem(const void *w, const void *act, void *out, int64_t m, int64_t k) {
    if (!w || !act || !out)
        return VQ_ERR_NULL_POINTER;
    if (!dim_ok(m) || !dim_ok(k) || k % 32 != 0)
        return VQ_ERR_BAD_SHAPE;
    if (!aligned16(w) || !aligned16(act) || !aligned16(out))
        return VQ_ERR_MISALIGNED;
    return VQ_OK;
}

int check_problem(bool fp8, const void *w, const void *scales, const void *act, void *out, int64_t m,
                  int64_t k) {
    if (!w || !scales || !act || !out)
        return VQ_ERR_NULL_POINTER;
    if (!dim_ok(m) || !dim_ok(k) || k % (fp8 ? 128 : 32) != 0)
        return VQ_ERR_BAD_SHAPE;
    if (!aligned16(w) || !aligned16(scales) || !aligned16(act) || !aligned16(out))
        return VQ_ERR_MISALIGNED;
    return VQ_OK;
}

// Launches problems[0 .. count) whose plans are finished: consecutive runs
// with the same form (tiles, waves, walk, groups) share a launch, up to
// kGroupPerLaunch problems each.  Launches run one after another on the
// stream, each using the workspace from its start; *ws_need (when asked for,
// nothing is launched) is the largest workspace one launch uses.
int launch_problems(bool fp8, const vq::VerifyProblem *probs, int count, int act_dtype, int out_dtype,
                    int n, float alpha, void *workspace, hipStream_t stream, size_t *ws_need) {
    size_t need = 0;
    int i = 0;
    while (i < count) {
        const vq::VerifyPlan &p0 = probs[i].plan;
        int e = i;
        int64_t chunks = 0;
        while (e < count && e - i < vq::kGroupPerLaunch && probs[e].plan.tiles == p0.tiles &&
               probs[e].plan.waves == p0.waves && probs[e].plan.walk == p0.walk &&
               probs[e].plan.groups == p0.groups && probs[e].plan.panel == p0.panel) {
            chunks += vq::verify_chunks(fp8, probs[e].plan, probs[e].M, probs[e].K);
            ++e;
        }
        need = std::max(need, vq::verify_walk_workspace(p0, chunks));
        if (!ws_need) {
            vq::VerifyLaunch l{fp8, act_dtype, out_dtype, n, alpha, p0.tiles, p0.waves, probs + i, e - i, workspace,
                               stream};
            if (vq::launch_verify(l) != hipSuccess)
                return VQ_ERR_LAUNCH;
        }
        i = e;
    }
    if (ws_need)
        *ws_need = need;
    return VQ_OK;
}

int run_verify(bool fp8, const void *w, const void *scales, const void *act, int act_dtype,
               void *out, int out_dtype, int64_t n, int64_t m, int64_t k, float alpha, int tiles,
               int waves, int max_groups, void *workspace, size_t ws_bytes, void *stream) {
    const int st = check_problem(fp8, w, scales, act, out, m, k);
    if (st != VQ_OK)
        return st;
    if (!float_act(act_dtype) || !out_ok(out_dtype))
        return VQ_ERR_BAD_DTYPE;
    if (!dim_ok(n))
        return VQ_ERR_BAD_SHAPE;
    if (workspace && !aligned16(workspace))
        return VQ_ERR_MISALIGNED;
    if (!workspace)
        ws_bytes = 0;
    vq::VerifyPlan pl;
    if (tiles == 0 && waves == 0 && max_groups == 0) {
        pl = default_plan(fp8, m, k, ws_bytes);
    } else {
        // An explicit shape walks exactly when a workspace is given.
        const vq::VerifyPlan d = walk_plan(m);
        pl.walk = workspace != nullptr;
        pl.tiles = tiles ? tiles : d.tiles;
        pl.waves = waves ? waves : d.waves;
        pl.groups = max_groups;
        if (!pl.walk && max_groups != 0)
            return VQ_ERR_WORKSPACE;
        if (!vq::verify_plan_finish(fp8, (int)m, (int)k, pl))
            return VQ_ERR_BAD_CONFIG;
        if (walk_need(fp8, pl, m, k) > ws_bytes)
            return VQ_ERR_WORKSPACE;
    }
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    const vq::VerifyProblem prob{w, scales, act, out, (int)m, (int)k, pl};
    return launch_problems(fp8, &prob, 1, act_dtype, out_dtype, (int)n, alpha, workspace,
                           static_cast<hipStream_t>(stream), nullptr);
}

// FP8 panel weights: the panel form of the codes, the tile scales as they are.
int run_fp8_panel(const void *w, const void *scales, const void *act, int act_dtype, void *out, int out_dtype,
                  int64_t n, int64_t m, int64_t k, int max_groups, void *workspace, size_t ws_bytes,
                  void *stream) {
    const int st = check_problem(true, w, scales, act, out, m, k);
    if (st != VQ_OK)
        return st;
    if (!float_act(act_dtype) || !out_ok(out_dtype))
        return VQ_ERR_BAD_DTYPE;
    if (!dim_ok(n))
        return VQ_ERR_BAD_SHAPE;
    if (max_groups < 0)
        return VQ_ERR_BAD_CONFIG;
    if (workspace && !aligned16(workspace))
        return VQ_ERR_MISALIGNED;
    const vq::VerifyPlan pl = fp8_panel_plan(max_groups);
    if (!workspace || walk_need(true, pl, m, k) > ws_bytes)
        return VQ_ERR_WORKSPACE;
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    const vq::VerifyProblem prob{w, scales, act, out, (int)m, (int)k, pl};
    return launch_problems(true, &prob, 1, act_dtype, out_dtype, (int)n, 1.0f, workspace,
                           static_cast<hipStream_t>(stream), nullptr);
}

int run_panel(const void *w, const void *act, int act_dtype, void *out, int out_dtype, int64_t n, int64_t m,
              int64_t k, float alpha, int max_groups, void *workspace, size_t ws_bytes, void *stream) {
    const int st = check_panel_problem(w, act, out, m, k);
    if (st != VQ_OK)
        return st;
    if (!float_act(act_dtype) || !out_ok(out_dtype))
        return VQ_ERR_BAD_DTYPE;
    if (!dim_ok(n))
        return VQ_ERR_BAD_SHAPE;
    if (max_groups < 0)
        return VQ_ERR_BAD_CONFIG;
    if (workspace && !aligned16(workspace))
        return VQ_ERR_MISALIGNED;
    const vq::VerifyPlan pl = panel_plan(max_groups);
    if (!workspace || walk_need(false, pl, m, k) > ws_bytes)
        return VQ_ERR_WORKSPACE;
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    const vq::VerifyProblem prob{w, nullptr, act, out, (int)m, (int)k, pl};
    return launch_problems(false, &prob, 1, act_dtype, out_dtype, (int)n, alpha, workspace,
                           static_cast<hipStream_t>(stream), nullptr);
}

// Plans of a grouped call: the default shape of every problem, the walk form
// where the shape allows when a workspace is given (the call then needs what
// vq_workspace_bytes_grouped reports), one-shot without one.  Panel problems
// always walk.
int plan_group(bool fp8, bool panel, const vq_verify_problem *problems, int count, bool split,
               vq::VerifyProblem *out) {
    for (int i = 0; i < count; ++i) {
        const vq_verify_problem &p = problems[i];
        if (panel && fp8) {
            const int st = check_problem(true, p.w, p.scales, p.act, p.out, p.m, p.k);
            if (st != VQ_OK)
                return st;
            out[i] = vq::VerifyProblem{p.w, p.scales, p.act, p.out, (int)p.m, (int)p.k, fp8_panel_plan(0)};
            continue;
        }
        if (panel) {
            const int st = check_panel_problem(p.w, p.act, p.out, p.m, p.k);
            if (st != VQ_OK)
                return st;
            out[i] = vq::VerifyProblem{p.w, nullptr, p.act, p.out, (int)p.m, (int)p.k, panel_plan(0)};
            continue;
        }
        const int st = check_problem(fp8, p.w, p.scales, p.act, p.out, p.m, p.k);
        if (st != VQ_OK)
            return st;
        out[i] = vq::VerifyProblem{p.w, p.scales, p.act, p.out, (int)p.m, (int)p.k,
                                   default_plan(fp8, p.m, p.k, split ? SIZE_MAX : 0)};
    }
    return VQ_OK;
}

int run_group(bool fp8, bool panel, const vq_verify_problem *problems, int count, int act_dtype, int out_dtype,
              int64_t n, float alpha, void *workspace, size_t ws_bytes, void *stream) {
    if (!problems)
        return VQ_ERR_NULL_POINTER;
    if (count < 1 || count > VQ_MAX_GROUP || !dim_ok(n))
        return VQ_ERR_BAD_SHAPE;
    if (!float_act(act_dtype) || !out_ok(out_dtype))
        return VQ_ERR_BAD_DTYPE;
    if (workspace && !aligned16(workspace))
        return VQ_ERR_MISALIGNED;
    std::vector<vq::VerifyProblem> probs(count);
    int st = plan_group(fp8, panel, problems, count, workspace != nullptr, probs.data());
    if (st != VQ_OK)
        return st;
    size_t need = 0;
    launch_problems(fp8, probs.data(), count, act_dtype, out_dtype, (int)n, alpha, workspace, nullptr, &need);
    if (need > (workspace ? ws_bytes : 0) || (panel && !workspace))
        return VQ_ERR_WORKSPACE;
    st = check_device();
    if (st != VQ_OK)
        return st;
    return launch_problems(fp8, probs.data(), count, act_dtype, out_dtype, (int)n, alpha, workspace,
                           static_cast<hipStream_t>(stream), nullptr);
}

}  // namespace

extern "C" {

int vq_gemm_q4_0(const void *w_codes, const void *w_scales, const void *act, int act_dtype,
                 const void *act_scales, void *out, int out_dtype, int64_t n_rows, int64_t m,
                 int64_t k, float alpha, void *workspace, size_t workspace_bytes, void *stream) {
    if (act_dtype != VQ_DTYPE_I8) {
        if (act_scales != nullptr)
            return VQ_ERR_BAD_DTYPE;  // float activations carry no scales
        return run_verify(false, w_codes, w_scales, act, act_dtype, out, out_dtype, n_rows, m, k,
                          alpha, 0, 0, 0, workspace, workspace_bytes, stream);
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

int vq_gemm_q4_0_noalloc(const void *w_codes, const void *w_scales, const void *act, int act_dtype,
                         const void *act_scales, void *out, int out_dtype, int64_t n_rows, int64_t m, int64_t k,
                         float alpha, void *stream) {
    if (act_dtype == VQ_DTYPE_I8)  // the W4A8 kernel uses no scratch memory
        return vq_gemm_q4_0(w_codes, w_scales, act, act_dtype, act_scales, out, out_dtype, n_rows, m, k, alpha,
                            nullptr, 0, stream);
    if (act_scales != nullptr)
        return VQ_ERR_BAD_DTYPE;
    const int st = check_problem(false, w_codes, w_scales, act, out, m, k);
    if (st != VQ_OK)
        return st;
    if (!float_act(act_dtype) || !out_ok(out_dtype))
        return VQ_ERR_BAD_DTYPE;
    if (!dim_ok(n_rows))
        return VQ_ERR_BAD_SHAPE;
    // the launch vq_gemm_q4_0 makes with an ample workspace, so the results
    // are the same bits
    const vq::VerifyPlan pl = default_plan(false, m, k, SIZE_MAX);
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    const vq::VerifyProblem prob{w_codes, w_scales, act, out, (int)m, (int)k, pl};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    void *scratch = nullptr;
    if (pl.walk) {
        size_t used = 0;
        vq::VerifyLaunch l{false, act_dtype, out_dtype, (int)n_rows, alpha, pl.tiles, pl.waves, &prob, 1,
                           nullptr, s, &used};
        if (vq::launch_verify(l) != hipSuccess)
            return VQ_ERR_LAUNCH;
        if (used > vq::kNoallocScratchBytes)
            return VQ_ERR_SCRATCH;
        if (vq::noalloc_scratch(s, &scratch) != hipSuccess)
            return VQ_ERR_LAUNCH;
    }
    return launch_problems(false, &prob, 1, act_dtype, out_dtype, (int)n_rows, alpha, scratch, s, nullptr);
}

int vq_gemm_q4_0_ex(const void *w_codes, const void *w_scales, const void *act, int act_dtype,
                    void *out, int out_dtype, int64_t n_rows, int64_t m, int64_t k, float alpha,
                    int tiles_per_wave, int waves_per_group, int max_groups, void *workspace,
                    size_t workspace_bytes, void *stream) {
    if (tiles_per_wave < 0 || waves_per_group < 0 || max_groups < 0)
        return VQ_ERR_BAD_CONFIG;
    return run_verify(false, w_codes, w_scales, act, act_dtype, out, out_dtype, n_rows, m, k, alpha,
                      tiles_per_wave, waves_per_group, max_groups, workspace, workspace_bytes, stream);
}

int vq_gemm_fp8_blk128(const void *w_e4m3, const float *w_tile_scales, const void *act,
                       int act_dtype, void *out, int out_dtype, int64_t n_rows, int64_t m,
                       int64_t k, void *workspace, size_t workspace_bytes, void *stream) {
    return run_verify(true, w_e4m3, w_tile_scales, act, act_dtype, out, out_dtype, n_rows, m, k,
                      1.0f, 0, 0, 0, workspace, workspace_bytes, stream);
}

int vq_gemm_fp8_blk128_prefill(const void *w_e4m3, const float *w_tile_scales, const void *act, int act_dtype,
                               void *out, int out_dtype, int64_t n_rows, int64_t m, int64_t k, void *stream) {
    const int st = check_problem(true, w_e4m3, w_tile_scales, act, out, m, k);
    if (st != VQ_OK)
        return st;
    if (!float_act(act_dtype) || !out_ok(out_dtype))
        return VQ_ERR_BAD_DTYPE;
    if (!dim_ok(n_rows))
        return VQ_ERR_BAD_SHAPE;
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    const vq::Fp8PrefillArgs p{w_e4m3, w_tile_scales, act, act_dtype, out, out_dtype, (int)n_rows, (int)m, (int)k,
                               static_cast<hipStream_t>(stream)};
    return vq::launch_fp8_prefill(p) == hipSuccess ? VQ_OK : VQ_ERR_LAUNCH;
}

int vq_gemm_fp8_blk128_ex(const void *w_e4m3, const float *w_tile_scales, const void *act,
                          int act_dtype, void *out, int out_dtype, int64_t n_rows, int64_t m,
                          int64_t k, int tiles_per_wave, int waves_per_group, int max_groups,
                          void *workspace, size_t workspace_bytes, void *stream) {
    if (tiles_per_wave < 0 || waves_per_group < 0 || max_groups < 0)
        return VQ_ERR_BAD_CONFIG;
    return run_verify(true, w_e4m3, w_tile_scales, act, act_dtype, out, out_dtype, n_rows, m, k,
                      1.0f, tiles_per_wave, waves_per_group, max_groups, workspace, workspace_bytes,
                      stream);
}

}  // extern "C"

namespace {

int run_quant(const void *x, int x_dtype, int8_t *q_out, void *scales_out, int64_t n_rows, int64_t k, int qmax,
              void *stream) {
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
    return vq::launch_h32_quant(x, x_dtype, q_out, scales_out, (int)n_rows, (int)k, qmax,
                                static_cast<hipStream_t>(stream)) == hipSuccess
               ? VQ_OK
               : VQ_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int vq_hadamard32_quant_int8(const void *x, int x_dtype, int8_t *q_out, void *scales_out,
                             int64_t n_rows, int64_t k, void *stream) {
    return run_quant(x, x_dtype, q_out, scales_out, n_rows, k, 127, stream);
}

int vq_hadamard32_quant_int4(const void *x, int x_dtype, int8_t *q_out, void *scales_out,
                             int64_t n_rows, int64_t k, void *stream) {
    return run_quant(x, x_dtype, q_out, scales_out, n_rows, k, 7, stream);
}

int vq_q4_0_rotate_h32(const void *w_codes, const void *w_scales, int64_t m, int64_t k, void *codes_out,
                       void *scales_out, void *stream) {
    if (!w_codes || !w_scales || !codes_out || !scales_out)
        return VQ_ERR_NULL_POINTER;
    if (!dim_ok(m) || !dim_ok(k) || k % 32 != 0)
        return VQ_ERR_BAD_SHAPE;
    if (!aligned16(w_codes) || !aligned16(w_scales) || !aligned16(codes_out) || !aligned16(scales_out))
        return VQ_ERR_MISALIGNED;
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    return vq::launch_q4_rotate_h32(w_codes, w_scales, (int)m, (int)k, codes_out, scales_out,
                                    static_cast<hipStream_t>(stream)) == hipSuccess
               ? VQ_OK
               : VQ_ERR_LAUNCH;
}

static bool kind_fp8(int kind) { return kind == VQ_KIND_FP8_BLK128 || kind == VQ_KIND_FP8_PANEL; }
static bool kind_panel(int kind) { return kind == VQ_KIND_Q4_0_PANEL || kind == VQ_KIND_FP8_PANEL; }

static bool query_ok(int kind, int64_t m, int64_t k) {
    return (kind == VQ_KIND_Q4_0 || kind == VQ_KIND_FP8_BLK128 || kind == VQ_KIND_Q4_0_PANEL ||
            kind == VQ_KIND_FP8_PANEL) &&
           dim_ok(m) && dim_ok(k) && k % (kind_fp8(kind) ? 128 : 32) == 0;
}

// The default plan of a query: panel problems have only one.
static vq::VerifyPlan query_plan(int kind, int64_t m, int64_t k, size_t ws_bytes) {
    if (kind == VQ_KIND_Q4_0_PANEL)
        return panel_plan(0);
    if (kind == VQ_KIND_FP8_PANEL)
        return fp8_panel_plan(0);
    return default_plan(kind == VQ_KIND_FP8_BLK128, m, k, ws_bytes);
}

size_t vq_workspace_bytes(int kind, int64_t m, int64_t k) {
    if (!query_ok(kind, m, k))
        return 0;
    const bool fp8 = kind_fp8(kind);
    return walk_need(fp8, query_plan(kind, m, k, SIZE_MAX), m, k);
}

int vq_default_launch_shape(int kind, int64_t m, int64_t k, size_t workspace_bytes, int *tiles_per_wave,
                            int *waves_per_group, int *walk, size_t *workspace_used) {
    if (!tiles_per_wave || !waves_per_group || !walk || !workspace_used)
        return VQ_ERR_NULL_POINTER;
    if (!query_ok(kind, m, k))
        return VQ_ERR_BAD_SHAPE;
    const bool fp8 = kind_fp8(kind);
    const vq::VerifyPlan pl = query_plan(kind, m, k, workspace_bytes);
    *tiles_per_wave = pl.tiles;
    *waves_per_group = pl.waves;
    *walk = pl.walk ? 1 : 0;
    *workspace_used = walk_need(fp8, pl, m, k);
    return VQ_OK;
}

int vq_gemm_q4_0_grouped(const vq_verify_problem *problems, int count, int act_dtype, int out_dtype,
                         int64_t n_rows, float alpha, void *workspace, size_t workspace_bytes, void *stream) {
    return run_group(false, false, problems, count, act_dtype, out_dtype, n_rows, alpha, workspace,
                     workspace_bytes, stream);
}

int vq_gemm_fp8_blk128_grouped(const vq_verify_problem *problems, int count, int act_dtype, int out_dtype,
                               int64_t n_rows, void *workspace, size_t workspace_bytes, void *stream) {
    return run_group(true, false, problems, count, act_dtype, out_dtype, n_rows, 1.0f, workspace,
                     workspace_bytes, stream);
}

int vq_gemm_q4_0_panel_grouped(const vq_verify_problem *problems, int count, int act_dtype, int out_dtype,
                               int64_t n_rows, float alpha, void *workspace, size_t workspace_bytes,
                               void *stream) {
    return run_group(false, true, problems, count, act_dtype, out_dtype, n_rows, alpha, workspace,
                     workspace_bytes, stream);
}

int vq_gemm_fp8_blk128_panel_grouped(const vq_verify_problem *problems, int count, int act_dtype, int out_dtype,
                                     int64_t n_rows, void *workspace, size_t workspace_bytes, void *stream) {
    return run_group(true, true, problems, count, act_dtype, out_dtype, n_rows, 1.0f, workspace,
                     workspace_bytes, stream);
}

size_t vq_fp8_panel_bytes(int64_t m, int64_t k) {
    if (!dim_ok(m) || !dim_ok(k) || k % 128 != 0)
        return 0;
    return vq::fp8_panel_bytes((int)m, (int)k);
}

int vq_fp8_to_panel(const void *w_e4m3, int64_t m, int64_t k, void *w_panel, size_t panel_bytes, void *stream) {
    if (!w_e4m3 || !w_panel)
        return VQ_ERR_NULL_POINTER;
    if (!dim_ok(m) || !dim_ok(k) || k % 128 != 0)
        return VQ_ERR_BAD_SHAPE;
    if (!aligned16(w_e4m3) || !aligned16(w_panel))
        return VQ_ERR_MISALIGNED;
    if (panel_bytes < vq::fp8_panel_bytes((int)m, (int)k))
        return VQ_ERR_BAD_SHAPE;
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    return vq::launch_fp8_panel_pack(w_e4m3, (int)m, (int)k, w_panel, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? VQ_OK
               : VQ_ERR_LAUNCH;
}

int vq_gemm_fp8_blk128_panel(const void *w_panel, const void *w_tile_scales, const void *act, int act_dtype,
                             void *out, int out_dtype, int64_t n_rows, int64_t m, int64_t k, void *workspace,
                             size_t workspace_bytes, void *stream) {
    return run_fp8_panel(w_panel, w_tile_scales, act, act_dtype, out, out_dtype, n_rows, m, k, 0, workspace,
                         workspace_bytes, stream);
}

int vq_gemm_fp8_blk128_panel_ex(const void *w_panel, const void *w_tile_scales, const void *act, int act_dtype,
                                void *out, int out_dtype, int64_t n_rows, int64_t m, int64_t k, int max_groups,
                                void *workspace, size_t workspace_bytes, void *stream) {
    return run_fp8_panel(w_panel, w_tile_scales, act, act_dtype, out, out_dtype, n_rows, m, k, max_groups,
                         workspace, workspace_bytes, stream);
}

size_t vq_q4_0_panel_bytes(int64_t m, int64_t k) {
    if (!dim_ok(m) || !dim_ok(k) || k % 32 != 0)
        return 0;
    return vq::panel_bytes((int)m, (int)k);
}

int vq_q4_0_to_panel(const void *w_codes, const void *w_scales, int64_t m, int64_t k, void *w_panel,
                     size_t panel_bytes, void *stream) {
    if (!w_codes || !w_scales || !w_panel)
        return VQ_ERR_NULL_POINTER;
    if (!dim_ok(m) || !dim_ok(k) || k % 32 != 0)
        return VQ_ERR_BAD_SHAPE;
    if (!aligned16(w_codes) || !aligned16(w_scales) || !aligned16(w_panel))
        return VQ_ERR_MISALIGNED;
    if (panel_bytes < vq::panel_bytes((int)m, (int)k))
        return VQ_ERR_BAD_SHAPE;
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    return vq::launch_panel_pack(w_codes, w_scales, (int)m, (int)k, w_panel, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? VQ_OK
               : VQ_ERR_LAUNCH;
}

int vq_gemm_q4_0_panel(const void *w_panel, const void *act, int act_dtype, void *out, int out_dtype,
                       int64_t n_rows, int64_t m, int64_t k, float alpha, void *workspace, size_t workspace_bytes,
                       void *stream) {
    return run_panel(w_panel, act, act_dtype, out, out_dtype, n_rows, m, k, alpha, 0, workspace, workspace_bytes,
                     stream);
}

int vq_gemm_q4_0_panel_ex(const void *w_panel, const void *act, int act_dtype, void *out, int out_dtype,
                          int64_t n_rows, int64_t m, int64_t k, float alpha, int max_groups, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return run_panel(w_panel, act, act_dtype, out, out_dtype, n_rows, m, k, alpha, max_groups, workspace,
                     workspace_bytes, stream);
}

size_t vq_workspace_bytes_grouped(int kind, const vq_verify_problem *problems, int count) {
    if ((kind != VQ_KIND_Q4_0 && kind != VQ_KIND_FP8_BLK128 && kind != VQ_KIND_Q4_0_PANEL &&
         kind != VQ_KIND_FP8_PANEL) ||
        !problems || count < 1 || count > VQ_MAX_GROUP)
        return 0;
    const bool fp8 = kind_fp8(kind);
    std::vector<vq::VerifyProblem> probs(count);
    if (plan_group(fp8, kind_panel(kind), problems, count, true, probs.data()) != VQ_OK)
        return 0;
    size_t need = 0;
    launch_problems(fp8, probs.data(), count, VQ_DTYPE_BF16, VQ_DTYPE_BF16, 1, 1.0f, nullptr, nullptr, &need);
    return need;
}

size_t vq_greedy_workspace_bytes(int64_t n_rows, int64_t vocab) {
    if (n_rows < 1 || n_rows > VQ_MAX_GREEDY_ROWS || !dim_ok(vocab))
        return 0;
    return vq::greedy_workspace_bytes((int)n_rows, (int)vocab);
}

int vq_greedy_verify(const void *logits, int logits_dtype, int64_t n_rows, int64_t vocab, const int32_t *draft,
                     int32_t *tokens_out, int32_t *count_out, void *workspace, size_t workspace_bytes,
                     void *stream) {
    if (!logits || !tokens_out || !count_out || (n_rows > 1 && !draft))
        return VQ_ERR_NULL_POINTER;
    if (logits_dtype != VQ_DTYPE_F32 && !float_act(logits_dtype))
        return VQ_ERR_BAD_DTYPE;
    if (n_rows < 1 || n_rows > VQ_MAX_GREEDY_ROWS || !dim_ok(vocab))
        return VQ_ERR_BAD_SHAPE;
    if (!aligned16(logits) || !aligned16(tokens_out) || !aligned16(count_out) || (draft && !aligned16(draft)) ||
        (workspace && !aligned16(workspace)))
        return VQ_ERR_MISALIGNED;
    if (!workspace || workspace_bytes < vq::greedy_workspace_bytes((int)n_rows, (int)vocab))
        return VQ_ERR_WORKSPACE;
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    return vq::launch_greedy_verify(logits, logits_dtype, (int)n_rows, (int)vocab, draft, tokens_out, count_out,
                                    workspace, static_cast<hipStream_t>(stream)) == hipSuccess
               ? VQ_OK
               : VQ_ERR_LAUNCH;
}

int vq_hbm_read_probe(const void *buf, size_t bytes, int mode, int groups, int waves_per_group, int depth,
                      int nontemporal, uint32_t *sink, void *stream) {
    if (!buf || !sink)
        return VQ_ERR_NULL_POINTER;
    if (!aligned16(buf) || !aligned16(sink))
        return VQ_ERR_MISALIGNED;
    if (bytes < 65536 || bytes > ((size_t)1 << 31) || bytes % 65536 != 0)
        return VQ_ERR_BAD_SHAPE;
    if (mode != VQ_PROBE_BLOCKS && mode != VQ_PROBE_SHARES && mode != VQ_PROBE_WINDOW && mode != VQ_PROBE_REREAD &&
        mode != VQ_PROBE_LDS)
        return VQ_ERR_BAD_CONFIG;
    if ((waves_per_group != 4 && waves_per_group != 8 && waves_per_group != 16) ||
        (depth != 4 && depth != 8 && depth != 16))
        return VQ_ERR_BAD_CONFIG;
    if (mode == VQ_PROBE_BLOCKS ? groups != 0 : (groups < 1 || groups > 65535))
        return VQ_ERR_BAD_CONFIG;
    if (nontemporal != 0 && nontemporal != 1)
        return VQ_ERR_BAD_CONFIG;
    if (mode == VQ_PROBE_LDS && nontemporal != 0)  // LDS reads have no cache policy
        return VQ_ERR_BAD_CONFIG;
    if (mode == VQ_PROBE_LDS && bytes % ((size_t)waves_per_group * (size_t)depth * 1024) != 0)
        return VQ_ERR_BAD_SHAPE;
    if ((mode == VQ_PROBE_SHARES || mode == VQ_PROBE_REREAD) &&
        bytes % ((size_t)groups * (size_t)waves_per_group * 1024) != 0)
        return VQ_ERR_BAD_SHAPE;
    if (mode == VQ_PROBE_REREAD) {  // pieces per wave and pass: a power of two
        const size_t per = bytes / (size_t)groups / ((size_t)waves_per_group * 1024);
        if ((per & (per - 1)) != 0)
            return VQ_ERR_BAD_SHAPE;
    }
    const int dev = check_device();
    if (dev != VQ_OK)
        return dev;
    return vq::launch_hbm_probe(buf, bytes, mode, groups, waves_per_group, depth, nontemporal != 0, sink,
                                static_cast<hipStream_t>(stream)) == hipSuccess
               ? VQ_OK
               : VQ_ERR_LAUNCH;
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
    case VQ_ERR_WORKSPACE: return "workspace too small for the explicit launch shape";
    case VQ_ERR_SCRATCH: return "the launch needs more scratch memory than the fixed array holds";
    default: return "unknown status";
    }
}

int vq_version(void) { return 400; }

}  // extern "C"
