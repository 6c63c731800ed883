// vq_internal.h -- host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "vq.h"

namespace vq {

// Launch shape of a verify GEMM: `tiles` 16-feature tiles per wave, `waves`
// waves per workgroup.  walk: persistent workgroups walking contiguous ranges
// of chunks (tile group x 8 steps of 128), with the pieces of tile groups cut
// by range boundaries combined through the workspace; `groups` caps the
// workgroups (0: as many as the device holds at once).  Otherwise one-shot:
// one workgroup per tile group over all of K, staged `chunk` steps at a time.
struct VerifyPlan {
    int tiles = 0, waves = 0;
    bool walk = false;
    int groups = 0;
    int chunk = 0;
    bool panel = false;  // weights in the panel layout (walk; Q4_0: 2 tiles x 8 waves, FP8: 1 tile x 8 waves)
};

// Q4_0 panel layout: records of 256 features x 4 steps of 128 k, the codes of
// the 4 steps (16 tiles x 1 KiB each) and then the tiles' scales (512 bytes
// each: 16 features x 16 blocks).  A workgroup of 8 waves walks one record
// per chunk, 2 tiles per wave.
constexpr int kPanelFeatures = 256;
constexpr int kPanelTiles = 16;
constexpr int kPanelWaveTiles = 2;
constexpr int kPanelWaves = kPanelTiles / kPanelWaveTiles;
constexpr int kPanelSteps = 4;
constexpr int kPanelCodeBytes = kPanelSteps * kPanelTiles * 1024;
constexpr int kPanelTileScaleBytes = 16 * 4 * kPanelSteps * 2;
constexpr int kPanelRecordBytes = kPanelCodeBytes + kPanelTiles * kPanelTileScaleBytes;

// FP8 panel layout: records of 128 features x 8 steps of 128 k (128 KiB), in
// the order the walk kernel's 8 waves (one 16-feature tile each) load them:
// for step s, wave (tile) w and half h, the 1 KiB that lane l reads at
// 16 KiB * s + 2 KiB * w + 1 KiB * h + 16 l.  Tile scales stay in their own
// array.
constexpr int kFp8PanelFeatures = 128;
constexpr int kFp8PanelSteps = 8;
constexpr int kFp8RecordBytes = kFp8PanelFeatures * kFp8PanelSteps * 128;

// Workspace of a walk launch: arrival counters (one per workgroup and wave,
// kept at zero between calls) in a fixed region at the start, then two fp32
// piece slots of TG tiles per workgroup.  At most kMaxWalkGroups workgroups.
constexpr int kMaxWalkGroups = 1024;
constexpr size_t kWalkCounterBytes = 64 * 1024;
// The allocation-free entry point's fixed scratch: the counters and 8 MiB of
// pieces (the default row-major shape cuts 16 KiB per workgroup: 512
// workgroups, twice the MI355X's resident count).
constexpr size_t kNoallocScratchBytes = kWalkCounterBytes + ((size_t)8 << 20);

// One verify GEMM of a launch, already validated.
struct VerifyProblem {
    const void *w;       // Q4_0 codes or E4M3 bytes
    const void *scales;  // Q4_0 fp16 block scales or FP8 fp32 tile scales
    const void *act;     // [N][K] 16-bit activations
    void *out;           // [N][M]
    int M, K;
    VerifyPlan plan;     // finished; every problem of a launch has the same tiles and waves
};

// Problems per kernel launch (they travel in the kernel arguments).
constexpr int kGroupPerLaunch = 32;

struct VerifyLaunch {
    bool fp8;
    int act_dtype, out_dtype;
    int N;
    float alpha;
    int tiles, waves;
    const VerifyProblem *probs;
    int count;        // 1 .. kGroupPerLaunch
    void *workspace;  // walk launches: counters and pieces
    hipStream_t stream;
    // When set, nothing is launched: the bytes of workspace the launch would
    // use (counters and the pieces of the workgroups it would run) are
    // written here instead.
    size_t *used = nullptr;
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

int verify_steps(bool fp8, int K);
int verify_tile_groups(int M, int tiles_per_group);
int64_t verify_chunks(bool fp8, const VerifyPlan &plan, int M, int K);
size_t verify_lds_bytes(bool fp8, int tiles, int waves, bool walk);
size_t verify_walk_workspace(const VerifyPlan &plan, int64_t chunks);
bool verify_plan_finish(bool fp8, int M, int K, VerifyPlan &plan);
hipError_t launch_verify(const VerifyLaunch &launch);
int64_t panel_chunks(int K);
size_t panel_bytes(int M, int K);
hipError_t launch_panel_pack(const void *codes, const void *scales, int M, int K, void *panel, hipStream_t stream);
size_t fp8_panel_bytes(int M, int K);
hipError_t launch_fp8_panel_pack(const void *w, int M, int K, void *panel, hipStream_t stream);

// Greedy verification: segments per row of the argmax pass, the workspace
// (one 8-byte key per row and segment) and the launch of both kernels.
int greedy_segments(int vocab);
size_t greedy_workspace_bytes(int n_rows, int vocab);
hipError_t launch_greedy_verify(const void *logits, int dtype, int n_rows, int vocab, const int32_t *draft,
                                int32_t *tokens, int32_t *count, void *workspace, hipStream_t stream);

hipError_t launch_w4a8(const W4A8Args &p);

// Arguments of one FP8 prefill launch (16-bit activations, many rows).
struct Fp8PrefillArgs {
    const void *w;
    const float *tile_scales;
    const void *act;
    int act_dtype;
    void *out;
    int out_dtype;
    int N, M, K;
    hipStream_t stream;
};
hipError_t launch_fp8_prefill(const Fp8PrefillArgs &p);
// qmax: 127 (int8 codes) or 7 (4-bit codes, one per byte)
hipError_t launch_h32_quant(const void *x, int x_dtype, int8_t *q, void *d, int N, int K, int qmax,
                            hipStream_t stream);
hipError_t launch_q4_rotate_h32(const void *codes, const void *scales, int M, int K, void *codes_out,
                                void *scales_out, hipStream_t stream);

// The HBM read probe (one kernel; arguments checked by the caller).
// The fixed scratch of the current device (set up on first use: its address
// looked up, its counters cleared by a kernel on `stream`).
hipError_t noalloc_scratch(hipStream_t stream, void **ptr);

hipError_t launch_hbm_probe(const void *buf, size_t bytes, int mode, int groups, int waves, int depth,
                            bool nontemporal, uint32_t *sink, hipStream_t stream);

}  // namespace vq
