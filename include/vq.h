/*
 * vq.h -- C ABI of the block-quantized verify GEMM library (libvq.so), gfx950.
 *
 * The operation is the speculative-decoding verification matmul: a draft block
 * of N activation rows (normally 1..16) times block-quantized weights, reading
 * every weight byte from HBM once whatever N is.  Sources, by page title and
 * section:
 *   [P1] "Qwen3.8-27B on the AMD R9700: up to 227 tok/s", sections
 *        "A block-diffusion drafter, verified exactly" (one batched target
 *        forward checks the whole draft block and reads the weights once) and
 *        "What 'lossless' means here, precisely" (batched and one-row paths
 *        sum in different orders; outputs are compared byte for byte across
 *        block widths).
 *   [P3] "r9k: a from-scratch inference engine for Qwen3.8-27B on two Radeon AI
 *        PRO R9700", opening paragraph (FP8 E4M3 weights in 128 x 128 scale
 *        blocks) and its list of correctness checks (GEMM rounding depends on
 *        the row count).
 *   [P4] "Qwen3.8-27B at 45.7 tok/s: DFlash2 in 1bit serve, and 4-bit
 *        activations with a Hadamard rotation", section "Prompt processing:
 *        4-bit activations, rotated first" (Q4_0 = 4-bit codes with offset 8 in
 *        blocks of 32; top-bit flip = two's complement; a 32-point
 *        Walsh-Hadamard rotation inside the int8 activation quantizer, weights
 *        rotated the same way offline; an exact int8 matmul path).
 *
 * Conventions shared by every entry point
 *  - All pointers are DEVICE pointers on the current HIP device, owned by the
 *    caller, 16-byte aligned, to contiguous row-major arrays.  The library
 *    never allocates, frees or synchronises and keeps no state between calls
 *    beyond what a caller's workspace holds, so calls from several host
 *    threads are safe (each with its own workspace).  Outputs must not alias
 *    inputs.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *    enqueued on it and the call returns at once.
 *  - Every argument is checked before anything is enqueued.  On any non-zero
 *    return nothing was enqueued.  Faults during execution surface at the
 *    caller's next synchronisation, like any asynchronous HIP call.
 *  - Numerics: fp32 accumulation; outputs rounded to nearest-even.  For a given
 *    (M, K) and launch shape the arithmetic of one output row depends only on
 *    that activation row and the weights: it is bit-identical whatever N is,
 *    whatever the other rows hold, and from run to run.
 */
#ifndef VQ_H
#define VQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (0 = success, negative = error; nothing enqueued on error). */
#define VQ_OK 0
#define VQ_ERR_NULL_POINTER (-1)   /* a required pointer is NULL */
#define VQ_ERR_BAD_SHAPE (-2)      /* a size is out of range or not a multiple of its block */
#define VQ_ERR_MISALIGNED (-3)     /* a pointer is not 16-byte aligned */
#define VQ_ERR_BAD_DTYPE (-4)      /* dtype code unknown or not allowed here */
#define VQ_ERR_DEVICE (-5)         /* current device is not gfx950, or no device */
#define VQ_ERR_LAUNCH (-6)         /* the HIP launch itself reported an error */
#define VQ_ERR_BAD_CONFIG (-7)     /* explicit launch shape not supported */
#define VQ_ERR_WORKSPACE (-8)      /* explicit launch shape needs a larger workspace */
#define VQ_ERR_SCRATCH (-9)        /* the launch needs more than the fixed scratch array */

/* Element type codes. */
#define VQ_DTYPE_F16 1             /* IEEE binary16 */
#define VQ_DTYPE_BF16 2            /* bfloat16 */
#define VQ_DTYPE_F32 3             /* IEEE binary32 */
#define VQ_DTYPE_I8 4              /* int8 */

/* Weight formats, for the query functions. */
#define VQ_KIND_Q4_0 0
#define VQ_KIND_FP8_BLK128 1
#define VQ_KIND_Q4_0_PANEL 2       /* Q4_0 in the panel layout (vq_q4_0_to_panel) */
#define VQ_KIND_FP8_PANEL 3        /* E4M3 codes in the FP8 panel layout (vq_fp8_to_panel) */

/* Largest M, K or N accepted by any entry point (indices stay in 32 bits). */
#define VQ_MAX_DIM (1 << 24)

/*
 * Workspace of the verify GEMMs.  The fast ("walk") form runs persistent
 * workgroups, each walking an equal share of the weight stream: 8 steps of
 * 128 k of one group of feature tiles at a time, whole tile groups
 * accumulated in registers over all of K.  A tile group cut by the boundary
 * between two workgroups' shares is finished through a caller-owned device
 * buffer: each side writes its fp32 partial sums there and the last to
 * arrive adds them in share order (an arrival counter per boundary and wave).
 * Per call: 64 KiB of counters plus 2 x 4 bytes per tile-group feature per 16
 * rows per workgroup, at most about 16 MiB (32 MiB on panel weights, whose
 * tile groups are 256 features wide), see vq_workspace_bytes.
 *  - 16-byte aligned device memory, zero-filled by the caller before its first
 *    use.  Every call leaves it ready for the next one (its counters back at
 *    zero), so it is zeroed once, not per call.
 *  - Calls that share one workspace must not overlap in time: use it from one
 *    stream, or order the streams.
 *  - workspace may be NULL (or smaller than needed): the library then runs the
 *    one-shot form (one workgroup per feature-tile group over all of K), which
 *    is correct but slower.  Q4_0 shapes with K not a multiple of 256 always
 *    run one-shot.
 *  - Output bits are a function of the call, not only of the problem.  Where
 *    a tile group is cut depends on the launch: the problems it holds (their
 *    order and shapes) and its workgroup count, which by default is what the
 *    device holds at once and so follows its CU count (256 on an MI355X).
 *    It never depends on N or on the activation values: for a fixed call on a
 *    fixed device every output bit is the same for any number of rows, any
 *    neighbouring rows and from run to run.  The same problem in another call
 *    (alone, or grouped with others), or on a device with another CU count,
 *    may round differently in the last bits (all within the parity bound);
 *    the _ex calls' workgroup cap, set at or below what every device in use
 *    holds at once, fixes the count across devices.
 */

/*
 * vq_gemm_q4_0 -- out[n][m] = alpha * sum_k x[n][k] * w[m][k], Q4_0 weights.
 *
 * Weights [P4]: w[m][k] = d[m][k/32] * (q[m][k] - 8), q in 0..15.
 *   w_codes  u8  [M][K/2].  Within each 32-weight block (16 bytes) byte j holds
 *            the code of k = 32b + j in its low nibble and of k = 32b + 16 + j
 *            in its high nibble (GGUF Q4_0 in-block order; the pages do not fix
 *            an order, this is the library's reading).
 *   w_scales f16 [M][K/32], the block scales d.
 * Activations:
 *   act_dtype F16 or BF16: x = act, [N][K].  N may exceed 16: rows are then
 *            processed in groups of 16 by the same kernel (weights are re-read
 *            per group), which keeps every row's arithmetic independent of N.
 *            act_scales must be NULL.
 *   act_dtype I8: the W4A8 path [P4, "exact int8 path"].  act is int8 q_x
 *            [N][K] and act_scales is f16 [N][K/32] (as written by
 *            vq_hadamard32_quant_int8, or _int4 for 4-bit codes);
 *            x[n][k] = act_scales[n][k/32] *
 *            q_x[n][k].  Each 32-block dot sum (q - 8) * q_x is formed exactly
 *            (an integer) before the fp32 scale products.  For weights and
 *            activations both rotated by the unnormalised H32, pass
 *            alpha = 1/32 to restore the unrotated product.  The workspace is
 *            not used on this path.
 * Output: out [N][M], out_dtype F16, BF16 or F32.
 * Sizes: 1 <= N, M <= VQ_MAX_DIM; 32 <= K <= VQ_MAX_DIM, K % 32 == 0.
 * Returns VQ_OK or a VQ_ERR_* code.
 */
int vq_gemm_q4_0(const void *w_codes, const void *w_scales,
                 const void *act, int act_dtype, const void *act_scales,
                 void *out, int out_dtype,
                 int64_t n_rows, int64_t m, int64_t k,
                 float alpha, void *workspace, size_t workspace_bytes,
                 void *stream);

/*
 * vq_gemm_q4_0_noalloc -- vq_gemm_q4_0 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, layouts, sizes and results as
 * vq_gemm_q4_0 with an ample workspace (the same launch, so the same bits),
 * but no workspace argument: the walk form's arrival counters and partial
 * sums live in a fixed device array inside the library, 64 KiB + 8 MiB per
 * GPU, held until the process ends and set up on the first call on each
 * device (its counters cleared by a kernel on `stream`).  The call allocates
 * and frees nothing.  Every call on one GPU shares that GPU's array, and
 * every call leaves its counters at zero: calls that overlap in time on one
 * GPU (on unordered streams or from several host threads) race and must not
 * be made.  VQ_ERR_SCRATCH if the launch would need more than the array
 * holds (more than 512 resident workgroups of the default shape; none on an
 * MI355X).  act_dtype I8 takes the W4A8 kernel, which needs no scratch.
 */
int vq_gemm_q4_0_noalloc(const void *w_codes, const void *w_scales,
                         const void *act, int act_dtype, const void *act_scales,
                         void *out, int out_dtype,
                         int64_t n_rows, int64_t m, int64_t k,
                         float alpha, void *stream);

/*
 * vq_gemm_fp8_blk128 -- out[n][m] = sum_k x[n][k] * w[m][k], FP8 weights with
 * one fp32 scale per 128 x 128 tile [P3]:
 *   w_e4m3        u8  [M][K], OCP E4M3FN bit patterns (bias 7, max 448, no
 *                 infinities; the pages say only "FP8 E4M3", the variant is the
 *                 library's reading).  NaN codes (0x7F, 0xFF) are outside the
 *                 contract.
 *   w_tile_scales f32 [ceil(M/128)][K/128]; w[m][k] = e4m3(w_e4m3[m][k]) *
 *                 w_tile_scales[m/128][k/128].
 *   act           [N][K], act_dtype F16 or BF16 (rows in groups of 16 as above).
 *   out           [N][M], out_dtype F16, BF16 or F32.
 * Sizes: 1 <= N, M <= VQ_MAX_DIM; 128 <= K <= VQ_MAX_DIM, K % 128 == 0.
 */
int vq_gemm_fp8_blk128(const void *w_e4m3, const float *w_tile_scales,
                       const void *act, int act_dtype,
                       void *out, int out_dtype,
                       int64_t n_rows, int64_t m, int64_t k,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * vq_gemm_fp8_blk128_prefill -- the product of vq_gemm_fp8_blk128 for
 * prompt-sized row counts [P3: "custom block-scaled FP8 GEMM"]: the verify
 * kernels stream the weights once per 16 rows, this one tiles 128 rows x 128
 * features per workgroup on the 16-bit MFMA (compute-bound at hundreds of
 * rows).  Same arguments, layouts and sizes as vq_gemm_fp8_blk128, no
 * workspace.  Arithmetic: E4M3 converted exactly to the activation type,
 * exact products, fp32 sums over each 128-k tile, then one fp32 FMA with the
 * tile scale per output and tile in ascending k -- a row's outputs depend only
 * on that row and the weights (bit-identical for any N), but they may differ
 * in the last bits from vq_gemm_fp8_blk128's.
 */
int vq_gemm_fp8_blk128_prefill(const void *w_e4m3, const float *w_tile_scales,
                               const void *act, int act_dtype,
                               void *out, int out_dtype,
                               int64_t n_rows, int64_t m, int64_t k, void *stream);

/*
 * vq_hadamard32_quant_int8 -- per (row n, 32-block b) of x [N][K] [P4]:
 *   u   = H32 x_b in fp32, H32 the +-1 Sylvester Walsh-Hadamard matrix applied
 *         as radix-2 butterflies h = 1, 2, 4, 8, 16 in that order
 *         (unnormalised: the matching GEMM takes alpha = 1/32);
 *   d   = fp16_rne(fp32(max_j |u_j|) / 127)          -> scales_out [N][K/32] f16
 *   q_j = clamp(rint_half_even(u_j / d), -127, 127)   -> q_out [N][K] int8
 *   A block of zeros gives d = 0 and q = 0.  A block whose d overflows fp16
 *   gets d = +inf and q = 0 (outside any realistic input).
 * Every division is IEEE fp32, correctly rounded, so codes and scales are
 * reproducible bit for bit.
 * x_dtype F16 or BF16.  Sizes: 1 <= N <= VQ_MAX_DIM, 32 <= K <= VQ_MAX_DIM,
 * K % 32 == 0.
 */
int vq_hadamard32_quant_int8(const void *x, int x_dtype,
                             int8_t *q_out, void *scales_out,
                             int64_t n_rows, int64_t k, void *stream);

/*
 * vq_hadamard32_quant_int4 -- the 4-bit activation quantizer of the same
 * section [P4] (there the activations alone go to 4-bit codes, after the
 * same H32 rotation; the weights keep their Q4_0 form): identical to vq_hadamard32_quant_int8 with 7 in place of
 * 127 (the library's reading: the symmetric 4-bit range),
 *   d   = fp16_rne(fp32(max_j |u_j|) / 7)          -> scales_out [N][K/32] f16
 *   q_j = clamp(rint_half_even(u_j / d), -7, 7)     -> q_out [N][K] int8
 * Codes are stored one per byte, so vq_gemm_q4_0 with act_dtype I8 consumes
 * them unchanged (the W4A4 product; gfx950 has no int4 matrix instruction,
 * so the GEMM is the W4A8 one).  Same sizes, errors and reproducibility as
 * the int8 quantizer.
 */
int vq_hadamard32_quant_int4(const void *x, int x_dtype,
                             int8_t *q_out, void *scales_out,
                             int64_t n_rows, int64_t k, void *stream);

/*
 * vq_q4_0_rotate_h32 -- the offline weight rotation of the W4A8 path [P4]
 * (the weights get the same H32 rotation once, ahead of time, which leaves
 * the product of rotated weights and rotated activations as it was; the
 * pages' tool turns a plain Q4_0 file into the rotated one).
 * For every row and 32-block of the Q4_0 matrix (w_codes, w_scales), in the
 * layout of vq_gemm_q4_0:
 *   x = d * (q - 8) exactly in fp32, then u = H32 x by the butterflies of
 *   vq_hadamard32_quant_int8 (fp32, h = 1, 2, 4, 8, 16);
 *   m = the u of largest magnitude (the first on ties; +0 for a block of
 *   zeros), d' = m / -8, id = d' != 0 ? 1 / d' : 0,
 *   q' = min(15, trunc(u * id + 8.5)) -- the Q4_0 rule of the GGUF files the
 *   pages use (the library's reading); every step one IEEE fp32 operation;
 *   written as Q4_0: codes_out u8 [M][K/2], scales_out f16 [M][K/32] = d'
 *   rounded to nearest even.
 * Then vq_gemm_q4_0 with these weights, int8 activations from
 * vq_hadamard32_quant_int8 and alpha = 1/32 approximates the unrotated
 * product; the rotated weights carry a requantization error of at most one
 * level (half a level inside the range).  Input scales must be finite; a
 * rotated scale beyond the fp16 range is stored as +-inf.  Outputs must not
 * alias inputs.  Sizes: 1 <= M, K <= VQ_MAX_DIM, K % 32 == 0.
 */
int vq_q4_0_rotate_h32(const void *w_codes, const void *w_scales, int64_t m, int64_t k,
                       void *codes_out, void *scales_out, void *stream);

/*
 * Grouped verify GEMMs -- several independent problems in as few kernel
 * launches as possible ([P1]: a block is verified by one batched pass over
 * all the weights; [P3]: the decode step is replayed as one HIP graph).  A
 * decode step's projections that read the same activations (or a benchmark's
 * unchained matrices) are independent; one launch over them pays the kernel
 * start and drain once instead of per matrix, and its workgroups -- equal
 * amounts of weight streaming each, by construction of the default shapes --
 * keep every CU busy across matrix boundaries.
 *   problems  host array of `count` descriptors, read during the call only.
 *             Each problem's outputs match its single call up to fp32
 *             rounding (bit-identical when both run one-shot); for a fixed
 *             problem list they are bit-identical for any n_rows.
 *   act_dtype, out_dtype, n_rows (and alpha): shared by all problems.
 *   workspace needs vq_workspace_bytes_grouped() bytes (VQ_ERR_WORKSPACE if
 *             smaller); NULL runs every problem in the one-shot form.
 * 1 <= count <= VQ_MAX_GROUP.  Float activations only.
 */
#define VQ_MAX_GROUP 4096

typedef struct vq_verify_problem {
    const void *w;       /* Q4_0 codes u8 [M][K/2], or E4M3 bytes u8 [M][K] */
    const void *scales;  /* Q4_0 f16 [M][K/32], or FP8 f32 [ceil(M/128)][K/128] */
    const void *act;     /* [n_rows][K] */
    void *out;           /* [n_rows][M] */
    int64_t m, k;
} vq_verify_problem;

int vq_gemm_q4_0_grouped(const vq_verify_problem *problems, int count,
                         int act_dtype, int out_dtype, int64_t n_rows, float alpha,
                         void *workspace, size_t workspace_bytes, void *stream);
int vq_gemm_fp8_blk128_grouped(const vq_verify_problem *problems, int count,
                               int act_dtype, int out_dtype, int64_t n_rows,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Q4_0 panel layout -- the weights of vq_gemm_q4_0 (codes and fp16 block
 * scales [P4]), rearranged once so that the verify GEMM reads them in long
 * contiguous runs: every HBM byte is still read once, but each workgroup
 * streams one 72 KiB record at a time instead of 16-row strips of 64 bytes,
 * and one staged chunk of activations serves 256 features.  Per output the
 * arithmetic is that of the row-major walk form (per 32-block: the exact
 * integer dot, then one FMA with the block scale, blocks in order); where no
 * tile group is cut between workgroups (one workgroup, say) the panel call
 * returns the same bits as vq_gemm_q4_0 with one tile per wave and eight
 * waves.  Where tile groups are cut, the two forms cut them at different k
 * (1024 k row-major, 512 k here) and may differ in the last bits.
 *   A panel is 256 consecutive features, a chunk 512 consecutive k.  With
 *   P = ceil(M/256) panels and C = ceil(K/512) chunks, record (p, c) starts
 *   at byte (p * C + c) * 73728 and holds:
 *    - bytes [0, 65536): for step s = 0..3 (128 k each), tile t = 0..15 (16
 *      features each) and lane l = 0..63 (g = l / 16, j = l % 16), 16 bytes
 *      at 16384 s + 1024 t + 16 l whose dword q (q = 0..3) is dword g (code
 *      bytes 4g..4g+3) of Q4_0 block 16c + 4s + q of feature 256p + 16t + j;
 *    - bytes [65536, 73728): for tile t at 65536 + 512 t, the fp16 scales of
 *      its 16 features, feature-major, 16 blocks (16c .. 16c + 15) each.
 *   Features past M and blocks past K/32 hold zeros.
 *
 * vq_q4_0_panel_bytes -- size of the panel form of an M x K matrix
 *   (P * C * 73728 bytes; 0 for invalid sizes).
 * vq_q4_0_to_panel -- writes the panel form of w_codes/w_scales (the
 *   vq_gemm_q4_0 layout) into w_panel, which must hold panel_bytes >=
 *   vq_q4_0_panel_bytes(m, k) bytes (VQ_ERR_BAD_SHAPE otherwise).  One kernel
 *   on `stream`; the inputs are only read.
 * vq_gemm_q4_0_panel -- vq_gemm_q4_0 with float activations on panel weights.
 *   The workspace is required (VQ_ERR_WORKSPACE when NULL or smaller than
 *   vq_workspace_bytes(VQ_KIND_Q4_0_PANEL, m, k)); any K % 32 == 0 walks.
 * vq_gemm_q4_0_panel_ex -- the same with at most max_groups persistent
 *   workgroups (0: as many as the device holds; values above 1024 act as
 *   1024); max_groups < 0 gives VQ_ERR_BAD_CONFIG.
 * vq_gemm_q4_0_panel_grouped -- vq_gemm_q4_0_grouped on panel weights:
 *   problem.w is the panel form, problem.scales is ignored.  Needs the
 *   workspace vq_workspace_bytes_grouped(VQ_KIND_Q4_0_PANEL, ...) reports.
 * Sizes and the remaining arguments as for vq_gemm_q4_0.
 */
size_t vq_q4_0_panel_bytes(int64_t m, int64_t k);
int vq_q4_0_to_panel(const void *w_codes, const void *w_scales, int64_t m, int64_t k,
                     void *w_panel, size_t panel_bytes, void *stream);
int vq_gemm_q4_0_panel(const void *w_panel, const void *act, int act_dtype,
                       void *out, int out_dtype, int64_t n_rows, int64_t m, int64_t k,
                       float alpha, void *workspace, size_t workspace_bytes, void *stream);
int vq_gemm_q4_0_panel_ex(const void *w_panel, const void *act, int act_dtype,
                          void *out, int out_dtype, int64_t n_rows, int64_t m, int64_t k,
                          float alpha, int max_groups, void *workspace, size_t workspace_bytes,
                          void *stream);
int vq_gemm_q4_0_panel_grouped(const vq_verify_problem *problems, int count,
                               int act_dtype, int out_dtype, int64_t n_rows, float alpha,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * FP8 panel layout -- the E4M3 codes of vq_gemm_fp8_blk128 [P3], rearranged
 * once so that the verify GEMM reads them front to back, 1 KiB per load
 * instruction, instead of 16 rows x 64 bytes at the row stride; the fp32
 * tile scales stay as they are.  Per output the arithmetic is that of the
 * row-major walk form with one tile per wave and eight waves (the same loads
 * into the same registers, the same order): at the same workgroup cap,
 * vq_gemm_fp8_blk128_ex with tiles_per_wave 1 and waves_per_group 8 cuts tile
 * groups at the same k and returns the same bits.
 *   A panel is 128 consecutive features, a chunk 1024 consecutive k.  With
 *   P = ceil(M/128) panels and C = ceil(K/1024) chunks, record (p, c) starts
 *   at byte (p * C + c) * 131072; for step s = 0..7 (128 k each), tile
 *   w = 0..7 (16 features each), half h = 0..1 and lane l = 0..63 (g = l/16,
 *   j = l % 16) the 16 bytes at 16384 s + 2048 w + 1024 h + 16 l are the
 *   codes of k = 1024 c + 128 s + 32 g + 16 h .. +16 of feature
 *   128 p + 16 w + j.  Features past M and steps past K hold zeros.
 *
 * vq_fp8_panel_bytes -- size of the FP8 panel form of an M x K matrix
 *   (P * C * 131072 bytes; 0 for invalid sizes: K % 128 != 0).
 * vq_fp8_to_panel -- writes the panel form of w_e4m3 ([M][K], the
 *   vq_gemm_fp8_blk128 layout) into w_panel (panel_bytes >= the size above,
 *   else VQ_ERR_BAD_SHAPE).  One kernel on `stream`; the input is only read.
 * vq_gemm_fp8_blk128_panel -- vq_gemm_fp8_blk128 on panel weights: w_panel
 *   the panel form, w_tile_scales the [ceil(M/128)][K/128] fp32 array as for
 *   vq_gemm_fp8_blk128.  The workspace is required (VQ_ERR_WORKSPACE when
 *   NULL or smaller than vq_workspace_bytes(VQ_KIND_FP8_PANEL, m, k)).
 * vq_gemm_fp8_blk128_panel_ex -- the same with at most max_groups persistent
 *   workgroups (0: as many as the device holds); max_groups < 0 gives
 *   VQ_ERR_BAD_CONFIG.
 * vq_gemm_fp8_blk128_panel_grouped -- vq_gemm_fp8_blk128_grouped on panel
 *   weights: problem.w is the panel form, problem.scales the tile scales.
 *   Needs the workspace vq_workspace_bytes_grouped(VQ_KIND_FP8_PANEL, ...)
 *   reports.
 * Sizes and the remaining arguments as for vq_gemm_fp8_blk128.
 */
size_t vq_fp8_panel_bytes(int64_t m, int64_t k);
int vq_fp8_to_panel(const void *w_e4m3, int64_t m, int64_t k, void *w_panel, size_t panel_bytes, void *stream);
int vq_gemm_fp8_blk128_panel(const void *w_panel, const void *w_tile_scales, const void *act, int act_dtype,
                             void *out, int out_dtype, int64_t n_rows, int64_t m, int64_t k,
                             void *workspace, size_t workspace_bytes, void *stream);
int vq_gemm_fp8_blk128_panel_ex(const void *w_panel, const void *w_tile_scales, const void *act, int act_dtype,
                                void *out, int out_dtype, int64_t n_rows, int64_t m, int64_t k,
                                int max_groups, void *workspace, size_t workspace_bytes, void *stream);
int vq_gemm_fp8_blk128_panel_grouped(const vq_verify_problem *problems, int count,
                                     int act_dtype, int out_dtype, int64_t n_rows,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* Workspace a grouped call with these problems needs (0 if invalid). */
size_t vq_workspace_bytes_grouped(int kind, const vq_verify_problem *problems, int count);

/* Workspace bytes the default launch shape of an (M, K) verify GEMM uses
 * (kind VQ_KIND_Q4_0, VQ_KIND_FP8_BLK128, VQ_KIND_Q4_0_PANEL or
 * VQ_KIND_FP8_PANEL; independent of N).  0 for invalid arguments or when the
 * shape only runs one-shot. */
size_t vq_workspace_bytes(int kind, int64_t m, int64_t k);

/*
 * vq_gemm_q4_0_ex / vq_gemm_fp8_blk128_ex -- the same operations with an
 * explicit launch shape, for tuning and testing: `tiles_per_wave` 16-feature
 * tiles per wave (1, 2 or 4), `waves_per_group` waves per workgroup (2, 4 or
 * 8).  With workspace non-NULL the call runs the walk form (Q4_0 needs
 * K % 256 == 0), with at most `max_groups` persistent workgroups (0: as many
 * as the device holds at once; at most 1024); with workspace NULL it runs
 * one-shot and max_groups must be 0.  0 for tiles or waves picks the
 * default.  VQ_ERR_BAD_CONFIG for a shape outside these rules or beyond 160
 * KiB of LDS; VQ_ERR_WORKSPACE if max_groups > 0 without a workspace or the
 * workspace is smaller than the shape needs.  Results are bit-identical
 * across N for a fixed launch shape and form; another shape may round
 * differently.  Float activations only.
 */
int vq_gemm_q4_0_ex(const void *w_codes, const void *w_scales,
                    const void *act, int act_dtype,
                    void *out, int out_dtype,
                    int64_t n_rows, int64_t m, int64_t k, float alpha,
                    int tiles_per_wave, int waves_per_group, int max_groups,
                    void *workspace, size_t workspace_bytes, void *stream);
int vq_gemm_fp8_blk128_ex(const void *w_e4m3, const float *w_tile_scales,
                          const void *act, int act_dtype,
                          void *out, int out_dtype,
                          int64_t n_rows, int64_t m, int64_t k,
                          int tiles_per_wave, int waves_per_group, int max_groups,
                          void *workspace, size_t workspace_bytes, void *stream);

/* The launch shape the library picks for an (M, K) verify GEMM given a
 * workspace of workspace_bytes (SIZE_MAX = unlimited): tiles per wave, waves
 * per workgroup, walk (1) or one-shot (0), and the workspace that shape uses.
 * Writes all four outputs; returns VQ_OK or VQ_ERR_BAD_SHAPE /
 * VQ_ERR_NULL_POINTER. */
int vq_default_launch_shape(int kind, int64_t m, int64_t k, size_t workspace_bytes,
                            int *tiles_per_wave, int *waves_per_group, int *walk,
                            size_t *workspace_used);

/*
 * vq_greedy_verify -- greedy acceptance of a verified draft block [P1]
 * ("A block-diffusion drafter, verified exactly", "What 'lossless' means
 * here, precisely": a drafted token is committed only where the target's own
 * greedy choice is the same token, so the output is plain greedy decoding's).
 *   logits    [n_rows][vocab], logits_dtype F32, F16 or BF16: the target's
 *             scores for the block positions; row 0 follows the last
 *             committed token, row i the drafted token i - 1 (the library's
 *             reading of the block layout).
 *   draft     int32 [n_rows - 1]: the drafted tokens (may be NULL when
 *             n_rows == 1).
 *   tokens_out int32 [n_rows]: the target's choice for every row, the argmax
 *             of the row: its first NaN if it holds one, else the first of its
 *             largest values (-0 and +0 equal).
 *   count_out int32 [1]: a + 1, where a is the number of leading positions
 *             i < n_rows - 1 with draft[i] == tokens_out[i]; the committed
 *             tokens are tokens_out[0 .. a] (the accepted drafts, then the
 *             target's own token at the first disagreement, or the bonus token
 *             after a fully accepted block).
 *   workspace vq_greedy_workspace_bytes(n_rows, vocab) bytes of device memory,
 *             any contents (VQ_ERR_WORKSPACE if NULL or smaller).
 * Sizes: 1 <= n_rows <= VQ_MAX_GREEDY_ROWS, 1 <= vocab <= VQ_MAX_DIM.  Outputs
 * are written on `stream`; they are exact (no rounding is involved).
 */
#define VQ_MAX_GREEDY_ROWS 4096
int vq_greedy_verify(const void *logits, int logits_dtype, int64_t n_rows, int64_t vocab,
                     const int32_t *draft, int32_t *tokens_out, int32_t *count_out,
                     void *workspace, size_t workspace_bytes, void *stream);
size_t vq_greedy_workspace_bytes(int64_t n_rows, int64_t vocab);

/*
 * vq_hbm_read_probe -- a plain read of `bytes` of device memory at `buf`,
 * the bandwidth the verify GEMM's weight stream is measured against ([P1]
 * TL;DR: decode streams the weights at a fraction of the card's bandwidth,
 * so the ceiling on the device at hand is worth knowing).  Every 16-byte
 * piece is loaded once with the verify kernels' load instruction (raw buffer
 * loads, 1 KiB per wave instruction) and folded into an XOR; nothing is
 * written except, in the unlikely case that some thread's XOR equals a fixed
 * 32-bit constant, that value to sink[0].  Patterns (`mode`):
 *   VQ_PROBE_BLOCKS  one workgroup per 64 KiB block (groups must be 0);
 *   VQ_PROBE_SHARES  `groups` workgroups, each reading one of `groups` equal
 *                    contiguous shares front to back (the walk kernel's
 *                    pattern); bytes % (groups * waves_per_group * 1024) == 0;
 *   VQ_PROBE_WINDOW  `groups` workgroups reading 64 KiB blocks b, b + groups,
 *                    b + 2 groups, ...
 *   VQ_PROBE_REREAD  as VQ_PROBE_SHARES, but each workgroup reads its share
 *                    VQ_PROBE_REREAD_PASSES times over within the launch, so
 *                    that after the first pass a share small enough for L2
 *                    is read from L2: the launch reads that many times
 *                    `bytes` (the rate of L2 hits per CU, not of HBM);
 *                    bytes / (groups * waves_per_group * 1024) must be a
 *                    power of two;
 *   VQ_PROBE_LDS     `groups` workgroups each copy the first 64 KiB of `buf`
 *                    into LDS, then read `bytes` from LDS (`depth` reads of
 *                    16 bytes per lane in flight per wave, consecutive lanes
 *                    on consecutive 16 bytes): the launch reads groups *
 *                    bytes from LDS and 64 KiB per workgroup from memory,
 *                    the LDS read rate per CU that the prefill GEMMs'
 *                    budgets use; nontemporal must be 0 and bytes % (1024 *
 *                    waves_per_group * depth) == 0;
 * waves_per_group 4, 8 or 16; depth (loads in flight per wave) 4, 8 or 16;
 * nontemporal 0 (default cache policy) or 1 (non-temporal loads, the policy
 * of a stream read once); 65536 <= bytes <= 2^31, bytes % 65536 == 0;
 * 1 <= groups <= 65535 for the persistent patterns.  sink: 4 bytes of device
 * memory.  One kernel on `stream`; time it with events on that stream.
 */
#define VQ_PROBE_BLOCKS 0
#define VQ_PROBE_SHARES 1
#define VQ_PROBE_WINDOW 2
#define VQ_PROBE_REREAD 3
#define VQ_PROBE_LDS 4
#define VQ_PROBE_REREAD_PASSES 16
int vq_hbm_read_probe(const void *buf, size_t bytes, int mode, int groups, int waves_per_group, int depth,
                      int nontemporal, uint32_t *sink, void *stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char *vq_status_string(int status);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int vq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VQ_H */
