/*
 * tgemm -- tiled GEMM  C = A * B^T  for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one FlyDSL's preshuffle GEMM computes (FlyDSL "Kernel
 * authoring guide", section 11 "Complete example: Preshuffle GEMM"; FlyDSL
 * "Kernel Authoring" skill, section 6 "GEMM Pattern (Preshuffle)"):
 *
 *     C[m][n] = cvt( (sum_k A[m][k] * B[n][k]) * s_a * s_b )
 *
 * products of the input elements summed in fp32, the scale applied in fp32
 * as (acc * s_a) * s_b (the Kernel Authoring skill's section 3 shows that
 * order), then converted to the output type with round-to-nearest-even.
 *
 * Storage (all row-major, leading dimensions implicit):
 *   A  M x K    elements of the input type            (lda = K)
 *   B  N x K    elements of the input type            (ldb = K)
 *              or, for GEMM_LAYOUT_BT_PRESHUFFLED, the N*K-element image
 *              written by gemm_preshuffle_b (see there)
 *   C  M x N    elements of the output type           (ldc = N)
 *
 * GEMM_LAYOUT_BN stores B as K x N row-major (ldb = N), the layout of the
 * pages' naive GEMM template (FlyDSL "Kernel Authoring" skill, section 8
 * "Common Patterns and Recipes", the naive GEMM's (K, N):(N, 1) view of B),
 * so C = A * B with b(n,k) = B[k][n].  The kernel reads it through the
 * gfx950 LDS transpose load (ds_read_b64_tr_b16, the 16-lane copy atom of
 * FlyDSL's "add-target-atom-op" skill, section 1.5.2 "Shape-product
 * invariants"; for 8-bit elements its form ds_read_b64_tr_b8).  bf16, fp8
 * e4m3 or int8 inputs; K * N * elem_bytes < 2^31; no pre-shuffled image
 * (gemm_preshuffle_b rejects such plans); fp8 and int8 plans use 256 x 256
 * tiles.
 *
 * GEMM_LAYOUT_AT and GEMM_LAYOUT_AT_BN store A as K x M row-major (lda = M),
 * so a(m,k) = A[k][m]; B is N x K (AT) or K x N (AT_BN, b(n,k) = B[k][n]).
 * The other operand layout the same skill's naive template and transpose
 * atom describe, read through the same LDS transpose load (16-bit or 8-bit
 * form).  bf16, fp8 e4m3 or int8 inputs; M * elem_bytes % 16 == 0 (16-byte
 * pieces of A's K-rows); K * M * elem_bytes < 2^31; such plans always use
 * 256 x 256 tiles.  B is read as stored; only
 * GEMM_LAYOUT_BT_PRESHUFFLED plans read the pre-shuffled image.
 *
 * Every pointer passed to gemm_preshuffle_b / gemm_run is a DEVICE pointer
 * owned by the caller.  The library allocates no device memory, never
 * synchronises, and launches asynchronously on the given stream; a plan holds
 * only host metadata and may be destroyed as soon as gemm_run returns.
 * Calls on one plan from several streams or threads are safe.  C must not
 * overlap A or B.
 *
 * Errors: functions returning int give GEMM_OK (0) or a negative
 * gemm_status; functions returning a pointer give NULL.  The reason is kept
 * per thread and read with gemm_last_error().  Only errors detectable on the
 * host are reported (argument checks, launch failures via hipGetLastError);
 * a fault inside a kernel surfaces at the caller's next synchronisation.
 */
#ifndef TGEMM_H
#define TGEMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = -1,   /* NULL or misaligned pointer, bad enum, negative size */
    GEMM_ERR_UNSUPPORTED = -2,   /* shape outside the supported set, wrong GPU       */
    GEMM_ERR_HIP = -3            /* a HIP runtime call or kernel launch failed        */
} gemm_status;

typedef enum {
    GEMM_BF16_OUT_F32 = 0,       /* A, B bf16; C fp32 (no rounding of the fp32 sum)   */
    GEMM_BF16_OUT_BF16 = 1,      /* A, B bf16; C bf16                                 */
    GEMM_E4M3_OUT_BF16 = 2,      /* A, B OCP fp8 e4m3fn (max 448); C bf16             */
    GEMM_MXFP8_OUT_BF16 = 3,     /* A, B MX: e4m3fn elements + E8M0 scales; C bf16    */
    GEMM_MXFP4_OUT_BF16 = 4,     /* A, B MX: e2m1 elements (2 per byte) + E8M0; C bf16 */
    GEMM_I8_OUT_BF16 = 5,        /* A, B int8, exact int32 sums; C bf16               */
    GEMM_W4A8_OUT_BF16 = 6       /* A int8, B int4 (2 per byte), int32 sums; C bf16   */
} gemm_dtype;

typedef enum {
    GEMM_LAYOUT_BT = 0,               /* B is N x K row-major                        */
    GEMM_LAYOUT_BT_PRESHUFFLED = 1,   /* B is the image written by gemm_preshuffle_b */
    GEMM_LAYOUT_BN = 2,               /* B is K x N row-major: C = A * B (bf16, e4m3, int8) */
    GEMM_LAYOUT_AT = 3,               /* A is K x M row-major, B N x K (bf16, e4m3, int8)   */
    GEMM_LAYOUT_AT_BN = 4             /* A is K x M, B K x N row-major (bf16, e4m3, int8)   */
} gemm_layout;

typedef struct gemm_plan gemm_plan;   /* opaque, immutable after creation */

/*
 * gemm_plan_create -- validate a problem and pick its kernel and tiling.
 *   M, N, K  sizes in elements; M may be 0 (gemm_run then does nothing),
 *            K may be 0 (C is then all zeros).
 *   dtype    gemm_dtype; layout gemm_layout.
 * Requirements (else NULL with GEMM_ERR_UNSUPPORTED / GEMM_ERR_INVALID_ARG):
 *   0 <= M, N, K <= 2^30;  N % 16 == 0;
 *   K * elem_bytes % 64 == 0 -- the 64-byte K step of the pages' GEMM (Kernel
 *   Authoring skill, section 10 "Troubleshooting", tile_k rule);
 *   K * elem_bytes < 2^23 and N * out_bytes * 256 < 2^31 (a 256-row tile of
 *   any operand stays inside one 2^31-byte buffer range).
 * Host only: no device work, no allocation on the device.  Returns a plan the
 * caller frees with gemm_plan_destroy.
 */
gemm_plan *gemm_plan_create(int64_t M, int64_t N, int64_t K, int dtype, int layout);

/*
 * Kernel choice for gemm_plan_create_opt.  GEMM_KERNEL_AUTO is the planner's
 * own pick by shape, dtype and layout (what gemm_plan_create does); the others
 * force one kernel family for every shape, so that each family the planner
 * may pick can be checked and timed on any shape.  Every choice computes the
 * same C within the same bound; only speed differs.
 */
typedef enum {
    GEMM_KERNEL_AUTO = 0,         /* the planner's table                                      */
    GEMM_KERNEL_GENERIC_128 = 1,  /* generic tiled kernel, 128 x 128 tiles (bf16, e4m3)       */
    GEMM_KERNEL_GENERIC_256 = 2,  /* generic tiled kernel, 256 x 256 tiles (bf16, e4m3)       */
    GEMM_KERNEL_TILE256 = 3,      /* the planner's 256 x 256 kernel at any size (no skinny
                                     kernel, no 128 x 128 tiles)                              */
    GEMM_KERNEL_PIPE = 4,         /* 256 x 256, B straight to registers, 8 waves (bf16 and
                                     e4m3 with B N x K or pre-shuffled; integer operands)     */
    GEMM_KERNEL_PIPE4 = 5         /* the same with 4 waves and AGPR accumulators; for MX plans
                                     the 16x16x128 form of the scaled MFMA (block-scale image
                                     form 0)                                                   */
} gemm_kernel_choice;

typedef struct {
    int32_t kernel;               /* gemm_kernel_choice                                       */
    int32_t splits;               /* gemm_run_ws K slices: 0 the planner's choice, 1 never
                                     split, 2..64 that many (plans whose kernel can split)    */
} gemm_plan_options;

/*
 * gemm_plan_create_opt -- gemm_plan_create with an explicit kernel choice and
 * split count.  opt == NULL (or all fields 0) is exactly gemm_plan_create.
 * Errors as gemm_plan_create, plus GEMM_ERR_INVALID_ARG for an unknown choice
 * or a split count outside 0..64, and GEMM_ERR_UNSUPPORTED when the chosen
 * family has no kernel for the dtype and layout.  The library reads no
 * environment variables: a plan depends on these arguments only.
 */
gemm_plan *gemm_plan_create_opt(int64_t M, int64_t N, int64_t K, int dtype, int layout,
                                const gemm_plan_options *opt);

/* gemm_plan_destroy -- free a plan (NULL is ignored). */
void gemm_plan_destroy(gemm_plan *plan);

/*
 * gemm_preshuffled_b_bytes -- bytes of the pre-shuffled B image:
 * N * K * b_elem_bits / 8 (a pure permutation of B).  0 for a NULL plan.
 */
size_t gemm_preshuffled_b_bytes(const gemm_plan *plan);

/*
 * gemm_preshuffle_b -- write B (N x K row-major) in MFMA operand order.
 * The image is the 5-mode byte array (N/16, Kb/64, 4, 16, 16) taken in
 * row-major order, with Kb = K * b_elem_bits / 8 (B's row bytes): n-block, 64-byte k-block,
 * 16-byte k-quarter q, row r within the n-block, byte.  Each 1 KiB block is
 * therefore one wave's B operand for a 64-byte K step: lane 16*q + r loads
 * the 16 bytes of row 16*nb + r at k-bytes 64*kb + 16*q.  (Kernel Authoring
 * skill, section 6 "GEMM Pattern (Preshuffle)" step 1; K counted in bytes and
 * kpack = 16 bytes is this library's reading of that tuple.)
 *   B       device pointer, 16-byte aligned, N*K elements.
 *   B_shuf  device pointer, 16-byte aligned, gemm_preshuffled_b_bytes(plan)
 *           bytes, must not overlap B.
 *   stream  HIP stream (0 = default stream).
 * Any plan of the same (N, K, dtype) may be used; the image does not depend
 * on M or on the plan's layout.  Asynchronous; returns GEMM_OK or an error.
 */
int gemm_preshuffle_b(const gemm_plan *plan, const void *B, void *B_shuf, hipStream_t stream);

/*
 * gemm_run -- C = cvt((A * B^T) * s_a * s_b) on `stream`.
 *   A      device pointer, 16-byte aligned, M x K input elements (K x M
 *          for GEMM_LAYOUT_AT and GEMM_LAYOUT_AT_BN).
 *   B      device pointer, 16-byte aligned: N x K (GEMM_LAYOUT_BT,
 *          GEMM_LAYOUT_AT), the pre-shuffled image (GEMM_LAYOUT_BT_PRESHUFFLED)
 *          or K x N (GEMM_LAYOUT_BN, GEMM_LAYOUT_AT_BN).
 *   C      device pointer, 16-byte aligned, M x N output elements; overwritten.
 *   scale  device pointer to two floats {s_a, s_b}, or NULL for 1, 1.  Read
 *          on the device, so fp8 scales never force a host synchronisation.
 * Asynchronous; allocates nothing.  Returns GEMM_OK or an error code.
 */
int gemm_run(const gemm_plan *plan, const void *A, const void *B, void *C,
             const float *scale, hipStream_t stream);

/*
 * Fused epilogues.  The pages' GEMM takes scale_a, scale_b and bias tensors
 * and an epilogue choice of "none", "bias", "bias_relu", "bias_silu" or
 * "bias_gelu" (FlyDSL "Kernel authoring guide", section 11 "Complete
 * example: Preshuffle GEMM"), applying the scales as (acc * scale_a) *
 * scale_b in fp32 (FlyDSL "Kernel Authoring" skill, section 3).  This
 * library's reading of the shapes and formulas, all in fp32:
 *
 *   z[m][n] = (acc[m][n] * sa(m)) * sb(n)  (+ bias[n])
 *   C[m][n] = cvt( act(z[m][n]) )
 *
 *   sa(m) = scale_a[m] (per row of C) or scale_a[0], 1 when scale_a is NULL;
 *   sb(n) = scale_b[n] (per column of C) or scale_b[0], 1 when NULL;
 *   act:  none; ReLU z > 0 ? z : +0; SiLU z / (1 + e^-z);
 *         GELU by its definition z * Phi(z) = z / 2 * (1 + erf(z / sqrt 2)).
 */
typedef enum {
    GEMM_EPI_NONE = 0,           /* scales only; bias must be NULL            */
    GEMM_EPI_BIAS = 1,           /* + bias                                    */
    GEMM_EPI_BIAS_RELU = 2,      /* + bias, then ReLU                         */
    GEMM_EPI_BIAS_SILU = 3,      /* + bias, then SiLU                         */
    GEMM_EPI_BIAS_GELU = 4       /* + bias, then GELU (erf form)              */
} gemm_epilogue;

typedef struct {
    const float *scale_a;        /* device; NULL, 1 value, or M values; 4-byte aligned           */
    const float *scale_b;        /* device; NULL, 1 value, or N values; 4-byte aligned, 16-byte
                                    aligned when per column                                      */
    const float *bias;           /* device; N values, 16-byte aligned; required by the bias
                                    epilogues, NULL for GEMM_EPI_NONE                             */
    int32_t scale_a_per_row;     /* 0: scale_a[0] scales every row; 1: scale_a[m] scales row m    */
    int32_t scale_b_per_col;     /* 0: scale_b[0] scales every column; 1: scale_b[n] column n     */
    int32_t epilogue;            /* gemm_epilogue                                                 */
} gemm_epilogue_args;

/*
 * gemm_run_ex -- gemm_run with the fused epilogue above.
 *   A, B, C, stream  as for gemm_run.
 *   epi      host pointer to the description (read during the call only; the
 *            vectors it points to are read on the device, asynchronously, and
 *            must stay valid until the launch completes).  NULL = no scaling,
 *            no bias, no activation.
 * gemm_run(plan, A, B, C, scale, s) is gemm_run_ex with scale_a = scale,
 * scale_b = scale + 1 (per tensor) and GEMM_EPI_NONE.
 * Errors: GEMM_ERR_INVALID_ARG for an unknown epilogue, a per-row/column flag
 * other than 0 or 1, a missing bias (bias epilogues) or an unexpected one
 * (GEMM_EPI_NONE), or a misaligned vector; otherwise as gemm_run.
 */
int gemm_run_ex(const gemm_plan *plan, const void *A, const void *B, void *C,
                const gemm_epilogue_args *epi, hipStream_t stream);

/*
 * Split K with a caller-provided workspace.  When a problem has fewer
 * 256 x 256 output tiles than the chip has compute units (a few hundred rows
 * of A against a large B: batched decode, small prefill), each tile is
 * computed by s workgroups that take one K slice each and write fp32 partial
 * tiles to the workspace; a second kernel sums the s partials of every
 * element in slice order (deterministic) and applies the epilogue of
 * gemm_run_ex.  The plan decides s (gemm_plan_info.ws_splits); plans with
 * s == 1 need no workspace.  bf16, fp8 e4m3, int8 and W4A8 plans with
 * GEMM_LAYOUT_BT or GEMM_LAYOUT_BT_PRESHUFFLED split; MX plans and the other
 * layouts never do.  (The pages' GEMM
 * has no split K: this is this library's answer to shapes whose tile grid
 * leaves most of the chip idle.)
 *
 * gemm_workspace_bytes -- bytes gemm_run_ws needs to split K:
 *   ws_splits * M * N * 4, or 0 when the plan does not split (or NULL).
 */
size_t gemm_workspace_bytes(const gemm_plan *plan);

/*
 * gemm_run_ws -- gemm_run_ex, split over K when the workspace allows it.
 *   A, B, C, epi, stream  as for gemm_run_ex.
 *   workspace        device pointer, 16-byte aligned, not overlapping A, B
 *                    or C; owned by the caller, contents need not be
 *                    initialised and are undefined afterwards.
 *   workspace_bytes  its size.  With a NULL workspace or fewer than
 *                    gemm_workspace_bytes(plan) bytes the call is exactly
 *                    gemm_run_ex (no split).
 * Two launches on `stream` (tile kernel, then the reduction); asynchronous;
 * allocates nothing.  Calls that share one workspace must not overlap in time
 * (issue them on one stream).  Errors as gemm_run_ex, plus
 * GEMM_ERR_INVALID_ARG for a misaligned or overlapping workspace.
 */
int gemm_run_ws(const gemm_plan *plan, const void *A, const void *B, void *C,
                const gemm_epilogue_args *epi, void *workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * gemm_run_ws_noalloc -- gemm_run_ws on the library's own static workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * library holds one GEMM_STATIC_WORKSPACE_BYTES array per GPU it runs on,
 * from first use until the process ends; this call allocates nothing and
 * calls no allocating routine.
 *   A, B, C, epi, stream  as for gemm_run_ex.
 * A plan that does not split runs exactly as gemm_run_ex.  A plan whose
 * partials (gemm_workspace_bytes) exceed GEMM_STATIC_WORKSPACE_BYTES is
 * refused with GEMM_ERR_UNSUPPORTED (gemm_run_ws takes any workspace).
 * Every call on one GPU shares that GPU's array, whose contents are whatever
 * the last call left (every element a split reads is written first by the
 * same call, so nothing needs clearing): calls that overlap in time on one
 * GPU race -- issue them on one stream.  Errors as gemm_run_ws.
 */
#define GEMM_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int gemm_run_ws_noalloc(const gemm_plan *plan, const void *A, const void *B, void *C,
                        const gemm_epilogue_args *epi, hipStream_t stream);

/*
 * MX block-scaled operands (GEMM_MXFP8_OUT_BF16, GEMM_MXFP4_OUT_BF16).  The
 * pages' gfx950 scaled MFMA (FlyDSL "Kernel authoring guide", section 4.3
 * "ROCm intrinsics", MFMA instructions: mfma_scale_f32_16x16x128_f8f6f4)
 * takes E8M0 block scales per operand with block size 32 (FlyDSL "Kernel
 * Authoring" skill, section 6 "MFMA Integration", gfx1250 WMMA entry); the
 * element and scale formats are those of the OCP Microscaling formats:
 *
 *     C[m][n] = cvt( sum_k (a(m,k) * 2^(SA[m][k/32] - 127)) * (b(n,k) * 2^(SB[n][k/32] - 127)) )
 *
 *   A   M x K elements row-major (MXFP8: 1 byte each; MXFP4: 2 per byte,
 *       element 2t in the low nibble of byte t); B likewise N x K, or its
 *       pre-shuffled image (gemm_preshuffle_b on the bytes: for MXFP4 the
 *       64-byte k-blocks hold 128 elements);
 *   SA  M x K/32 E8M0 bytes row-major, SB N x K/32 (0xFF is NaN).
 * Requirements beyond gemm_plan_create's: K % 32 == 0; K * elem_bits / 8 % 64 == 0.
 * The scales go to the kernel as an image that lets each lane fetch the scales
 * of 4 row blocks for 4 MFMA K-slices (128 elements each) in one 16-byte load:
 * the bytes (ceil(R/64), G, 64, 4, 4), G = ceil(ceil(K/128)/4), row-major:
 * row quad, slice group g, lane l, 16-row block b, slice s holds
 * S[64 quad + 16 b + l % 16][4 (4 g + s) + l / 16] (127 past the rows or K).
 * That is form 0 (gemm_plan_info.scale_form), for the 16x16x128 MFMA.  MX
 * plans on 256 x 256 tiles run the 32x32x64 form of the instruction (twice
 * the e2m1 rate, 8 waves), whose lanes take the scale of row l % 32 and K
 * block 2 s' + l / 32 of 64-element slice s'; their image is form 1, with the
 * same size and record order: (quad, g, lane l, word w, byte b) holds
 * S[64 quad + 32 (w / 2) + l % 32][16 g + 2 (2 b + w % 2) + l / 32].
 * gemm_preshuffle_bscale writes the plan's form.
 */

/* gemm_bscale_image_bytes -- bytes of the image of A's (operand 0) or B's
 * (operand 1) block scales; 0 for a non-MX plan or another operand. */
size_t gemm_bscale_image_bytes(const gemm_plan *plan, int operand);

/*
 * gemm_preshuffle_bscale -- write the image above from R x K/32 E8M0 bytes
 * (R = M for operand 0, N for operand 1).
 *   scales  device pointer, R * K/32 bytes;  image  device pointer, 16-byte
 *   aligned, gemm_bscale_image_bytes(plan, operand) bytes, not overlapping.
 * Asynchronous on `stream`; GEMM_OK or an error (non-MX plan, bad operand,
 * NULL or misaligned pointers, overlap).
 */
int gemm_preshuffle_bscale(const gemm_plan *plan, int operand, const void *scales, void *image,
                           hipStream_t stream);

/*
 * gemm_run_mx -- C = cvt(epilogue(A * B^T)) for an MX plan.
 *   A, B, C    as for gemm_run (B plain or pre-shuffled per the plan's layout).
 *   A_bscale, B_bscale  device pointers to the images of SA and SB, 16-byte
 *              aligned (gemm_preshuffle_bscale).
 *   epi        the fused epilogue (see gemm_run_ex), or NULL.
 * gemm_run and gemm_run_ex reject MX plans.  Asynchronous; GEMM_OK or an error.
 */
int gemm_run_mx(const gemm_plan *plan, const void *A, const void *A_bscale, const void *B,
                const void *B_bscale, void *C, const gemm_epilogue_args *epi, hipStream_t stream);

/*
 * Integer operands (GEMM_I8_OUT_BF16, GEMM_W4A8_OUT_BF16).  The pages' int8
 * MFMA accumulates i8 x i8 products in int32 (FlyDSL "Kernel authoring
 * guide", section 4.3 "ROCm intrinsics", MFMA instructions; "Kernel
 * Authoring" skill, section 6 "MFMA Integration"), and their W4A8 GEMM takes
 * an int8 A with a B of packed int4 values unpacked to int8 inside the kernel
 * (the same skill, section 10 "Troubleshooting", INT4 item).  This library's
 * reading:
 *
 *     acc[m][n] = sum_k a(m,k) * b(n,k)            exact, in int32
 *     C[m][n]   = cvt( act( (float(acc) * sa(m)) * sb(n) (+ bias[n]) ) )
 *
 *   int8 two's complement (-128 .. 127); int4 two's complement (-8 .. 7), two
 *   per byte, element 2t in the low nibble of byte t.  float() rounds to
 *   nearest even (exact while |acc| < 2^24).  The scales and epilogue are
 *   those of gemm_run / gemm_run_ex, typically per-row and per-column
 *   dequantisation scales.
 *   A   M x K bytes row-major;  B  N x K bytes (int8) or N x K/2 bytes (int4)
 *       row-major, or the pre-shuffled image (gemm_preshuffle_b on B's bytes:
 *       for int4 a 64-byte k-block holds 128 values).
 * Requirements beyond gemm_plan_create's: K % 64 == 0 (int8) or K % 128 == 0
 * (W4A8), so every row of B is whole 64-byte K steps; K < 2^17, so no sum of
 * products (each at most 2^14 in magnitude) can leave the int32 range.
 * Run through gemm_run or gemm_run_ex.
 */

/* gemm_last_error -- message for the calling thread's last failure ("" if none). */
const char *gemm_last_error(void);

/* ------------------------------------------------------------------------
 * Planner introspection (host only).  A layout is (shape, stride) of up to
 * GEMM_MAX_RANK modes; a coordinate maps to sum(c_i * stride_i) (Kernel
 * Authoring skill, section 2 "Layout System", "Coordinate Mapping").
 * ------------------------------------------------------------------------ */
#define GEMM_MAX_RANK 8

typedef struct {
    int64_t M, N, K;
    int32_t dtype, layout;
    int32_t elem_bytes, out_bytes;
    int32_t kernel;          /* 0 tiled, 1 skinny (M <= 64, B N x K or pre-shuffled)  */
    int32_t tile_m, tile_n;  /* output tile of one workgroup                          */
    int32_t tile_k_bytes;    /* K bytes consumed per main-loop step (multiple of 64)  */
    int32_t threads;         /* threads per workgroup                                 */
    int32_t lds_stages;      /* LDS buffers in the software pipeline                  */
    int32_t lds_bytes;       /* static LDS per workgroup (<= 160 KiB on gfx950)       */
    int32_t grid;            /* workgroups per gemm_run launch                        */
    int32_t tiles_m, tiles_n;
    int32_t group_m;         /* tile rows per raster group within one XCD             */
    int32_t split_k;         /* K slices reduced inside a workgroup (skinny kernel)   */
    int32_t elem_bits;       /* bits per input element of A (16, 8 or 4); elem_bytes
                                is elem_bits / 8, so 0 for MXFP4                       */
    int32_t b_elem_bits;     /* bits per input element of B (4 for W4A8, else elem_bits) */
    int32_t ws_splits;       /* K slices gemm_run_ws uses with a large enough
                                workspace (1: it runs as gemm_run_ex)                 */
    int32_t ws_grid;         /* workgroups of gemm_run_ws's tile launch               */
    int32_t scale_form;      /* MX plans: form of the block-scale image (0 or 1, see
                                gemm_preshuffle_bscale); 0 for other plans            */
} gemm_plan_info;

/* gemm_plan_query -- copy the plan's decisions into *info. */
int gemm_plan_query(const gemm_plan *plan, gemm_plan_info *info);

typedef enum {
    GEMM_VIEW_A = 0,          /* A bytes:       (M, Ka):(Ka, 1), Ka = K * elem_bits / 8;
                                 A stored K x M: (K, 2M):(2M, 1)                            */
    GEMM_VIEW_B = 1,          /* B bytes:       (N, Kb):(Kb, 1), Kb = K * b_elem_bits / 8    */
    GEMM_VIEW_B_SHUF = 2,     /* pre-shuffled:  (N/16, Kb/64, 4, 16, 16):(16Kb, 1024, 256, 16, 1) */
    GEMM_VIEW_B_SRC = 3,      /* B bytes seen through the same 5 coordinates:
                                 (N/16, Kb/64, 4, 16, 16):(16Kb, 64, 16, Kb, 1)           */
    GEMM_VIEW_C = 4,          /* C bytes:       (M, N):(N*out_bytes, out_bytes)              */
    GEMM_VIEW_LDS_A = 5,      /* one LDS stage of A, before the XOR swizzle:
                                 (tile_m, tile_k_bytes/16, 16):(tile_k_bytes, 16, 1)     */
    GEMM_VIEW_TILE = 6        /* C tile grid:   (tiles_m, tiles_n):(tile_m*N*ob, tile_n*ob) */
} gemm_view;

/* gemm_plan_layout -- the byte layout of one view; rank and GEMM_MAX_RANK-long arrays out. */
int gemm_plan_layout(const gemm_plan *plan, int view, int32_t *rank, int64_t *shape, int64_t *stride);

/* gemm_layout_crd2idx -- sum(crd_i * stride_i); -1 and GEMM_ERR_INVALID_ARG
 * in gemm_last_error when a coordinate lies outside its mode. */
int64_t gemm_layout_crd2idx(int32_t rank, const int64_t *shape, const int64_t *stride, const int64_t *crd);

/* gemm_layout_idx2crd -- c_i = (idx / stride_i) % shape_i (the inverse of
 * crd2idx on an injective layout whose modes do not overlap). */
int gemm_layout_idx2crd(int32_t rank, const int64_t *shape, const int64_t *stride, int64_t idx, int64_t *crd);

/* gemm_lds_swizzle -- physical 16-byte chunk of logical chunk `chunk` of row
 * `row` in an LDS tile of `chunks_per_row` chunks (the XOR-16 swizzle the
 * pages name in section 6 of the Kernel Authoring skill; the function is this
 * library's choice).  -1 on bad arguments. */
int32_t gemm_lds_swizzle(int32_t row, int32_t chunk, int32_t chunks_per_row);

/* gemm_tile_of_workgroup -- the (tile_m index, tile_n index) the plan's
 * XCD-aware raster assigns to workgroup `wg` (0 <= wg < grid). */
int gemm_tile_of_workgroup(const gemm_plan *plan, int32_t wg, int32_t *tm, int32_t *tn);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H */
