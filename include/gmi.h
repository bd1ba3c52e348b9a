/*
 * gmi.h -- grouped, mixed-input and implicit-convolution GEMM on AMD MI355X
 * (gfx950).  Plain C ABI: device pointers, host sizes, no exceptions.
 *
 * One tiled GEMM mainloop computes D = alpha * A B + beta * C with fp32
 * accumulation.  A persistent tile scheduler runs it over a list of problems
 * (grouped: a shape and leading dimensions per problem; pointer-array: one
 * shape, one pointer per batch).  The same mainloop serves two variants: a
 * mixed-input product Y = X W^T whose 4-bit weights are prepacked once and
 * dequantised in registers with per-group scales and zero points, and an
 * implicit-GEMM convolution forward pass that addresses an NHWC activation
 * and a KRSC filter directly instead of building an im2col buffer.
 *
 * Conventions shared by every call
 *   - Memory.  Every tensor argument is a device pointer to caller-owned
 *     memory, except where a parameter says "host".  The library allocates
 *     nothing and keeps no pointer after a call returns.
 *   - Ordering.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) and the call returns without synchronising.
 *   - Layouts.  Leading dimensions and strides count elements.  A is
 *     row-major [M][lda] (K contiguous); B is column-major, column n at
 *     B + n * ldb (K contiguous); C and D are row-major [M][ldc / ldd]
 *     (N contiguous).
 *   - Rounding.  The fp32 result alpha * acc + beta * C is rounded to the
 *     output type to nearest, ties to even.  beta == 0 means C is never read.
 *   - Alignment.  Base pointers of A, B, C, D, X, Y, W, x, w, y must be
 *     16-byte aligned and every leading dimension a multiple of 8 elements
 *     (128-bit accesses), else GMI_ERR_MISALIGNED.
 *   - Errors.  Every argument is checked on the host before any HIP call; a
 *     failed check returns a status, records a message for gmi_last_error()
 *     and launches nothing.  A failed launch returns GMI_ERR_HIP.
 *   - Aliasing.  D may be C exactly (same pointer and leading dimension);
 *     any other overlap between an output and an input is undefined.
 */
#ifndef GMI_H
#define GMI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GMI_OK = 0,
  GMI_ERR_INVALID_ARG = 1, /* negative size, NULL pointer, ld too small, ... */
  GMI_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels cover  */
  GMI_ERR_MISALIGNED = 3,  /* pointer or leading dimension not 128-bit aligned */
  GMI_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required   */
  GMI_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed   */
} gmi_status;

/* Element types.  GMI_F8E4M3 (GEMM calls only): A and B are OCP fp8 E4M3
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, largest finite 448), C and D are bf16; the product of
 * two fp8 values and their sum are formed exactly in fp32 by the matrix
 * instruction, then accumulated in fp32.  This is the fp8 grouped GEMM the
 * element-type aliases of the grouped kernel page admit, on gfx950's
 * v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales. */
typedef enum { GMI_F16 = 0, GMI_BF16 = 1, GMI_F8E4M3 = 2 } gmi_dtype;

/* One problem of a grouped GEMM (host memory; the pointers are device
 * pointers).  Mirrors the per-group problem shape (M, N, K) and the per-group
 * strides of the grouped mode on the page
 * sm90_gemm_array_tma_warpspecialized_cooperative.hpp (Arguments; the
 * grouped-vs-array distinction of its stride types).  A problem with M == 0
 * or N == 0 is a valid no-op and its pointers may be NULL.  K == 0 gives
 * D = beta * C. */
typedef struct {
  int32_t M, N, K;
  int64_t lda, ldb, ldc, ldd; /* lda >= K, ldb >= K, ldc >= N (if C read), ldd >= N */
  const void* A;
  const void* B;
  const void* C; /* may be NULL iff beta == 0 */
  void* D;
} gmi_problem;

/* Device workspace needed by gmi_gemm_grouped for `problem_count` problems:
 * the per-problem descriptor table (80 bytes each) plus a 256-byte header.
 * Returns 0 for a negative count. */
size_t gmi_workspace_bytes(int32_t problem_count);

/* Grouped GEMM: D_g = alpha * A_g B_g + beta * C_g for g < count, all in one
 * persistent launch.  Follows the grouped problem mode of
 * sm90_gemm_array_tma_warpspecialized_cooperative.hpp (problem_shape per
 * group, per-group strides, persistent tile loop with a per-group shape
 * refresh; can_implement).
 *   problems   host array of `count` descriptors; it may be reused as soon as
 *              the call returns (the table is staged into `workspace`).
 *   dtype      element type of A, B, C and D (fp16 or bf16), or GMI_F8E4M3
 *              (A and B fp8, C and D bf16; K, lda and ldb multiples of 16,
 *              else GMI_ERR_UNSUPPORTED); fp32 accumulate.  Leading dimensions
 *              count elements of their own operand.
 *   workspace  device buffer of at least gmi_workspace_bytes(count) bytes,
 *              16-byte aligned; overwritten by the call and read by the kernel
 *              until it completes on `stream`.
 * count == 0, or all problems empty, launches nothing and returns GMI_OK. */
gmi_status gmi_gemm_grouped(const gmi_problem* problems, int32_t count, gmi_dtype dtype, float alpha,
                            float beta, void* workspace, size_t workspace_bytes, void* stream);

/* Grouped GEMM whose group sizes exist only on the device -- the
 * mixture-of-experts layout, where a routing kernel writes how many rows
 * each expert received and the host never reads them back.  The grouped
 * kernel page allows problem shapes that only the device holds (its grid may
 * then be larger than the tiles, and a workgroup that finds no work returns);
 * here the device-held shapes take the form of row offsets:
 *   group g < count owns rows [offsets[g], offsets[g + 1]) of A (row-major,
 *   [rows][lda], K contiguous) and of D (and C), and multiplies them by its
 *   own B_g = B + g * stride_b elements (column-major as for
 *   gmi_gemm_grouped: column n at B_g + n * ldb); N and K are shared.
 *   offsets    device array of count + 1 int32, non-decreasing, offsets[0] >= 0,
 *              offsets[count] <= rows.  Read on the device only, when the
 *              work runs on `stream`.  A group whose range is empty, reversed
 *              or outside [0, rows) is clipped to the part inside (or skipped),
 *              so no access leaves the buffers; its rows of D are then
 *              unspecified.
 *   rows       host: number of rows A, C and D hold (the capacity, e.g. tokens
 *              x experts per token); sizes the tile shape and bounds the grid.
 *   count      1 .. 1024 groups, else GMI_ERR_UNSUPPORTED (0 is a no-op).
 *   stride_b   elements between consecutive B_g; a multiple of 8 (16 for fp8).
 *   dtype      as for gmi_gemm_grouped.
 *   workspace  at least gmi_workspace_bytes(count) bytes, 16-byte aligned; a
 *              first launch writes the group table there (groups in decreasing
 *              order of work per tile, tile prefix sums, the tile total), the
 *              GEMM launch reads it.
 * Rows of D outside every group are not written. */
gmi_status gmi_gemm_grouped_offsets(int32_t count, const int32_t* offsets, int32_t rows, int32_t N, int32_t K,
                                    const void* A, int64_t lda, const void* B, int64_t ldb, int64_t stride_b,
                                    const void* C, int64_t ldc, void* D, int64_t ldd, gmi_dtype dtype,
                                    float alpha, float beta, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* For callers that cannot allocate device memory -- work captured into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc -- the same call
 * as gmi_gemm_grouped_offsets without a workspace argument: the group table
 * and tile total live in a static device array of the library, 82,176 bytes
 * (256 + 80 * 1024), one per device, which each device holds from the
 * library's load until the process ends.  The call allocates nothing; on a
 * device's first call it looks up that device's address of the array.
 *   count  1 .. 1024 (the table's capacity), else GMI_ERR_UNSUPPORTED.
 * Every call on one device shares that device's array and leaves the last
 * call's table in it (each call rewrites every entry it reads, so nothing
 * needs clearing): two calls that overlap on one device, on different
 * streams or from different threads, race on the array and give undefined
 * results; order them on one stream.  A failed address lookup returns
 * GMI_ERR_HIP.  Every other argument, layout and rule as for
 * gmi_gemm_grouped_offsets. */
gmi_status gmi_gemm_grouped_offsets_noalloc(int32_t count, const int32_t* offsets, int32_t rows, int32_t N,
                                            int32_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                                            int64_t stride_b, const void* C, int64_t ldc, void* D, int64_t ldd,
                                            gmi_dtype dtype, float alpha, float beta, void* stream);

/* Pointer-array batched GEMM: L problems of one shape (M, N, K) and shared
 * leading dimensions, each operand a separate device buffer.  The pointer
 * arrays themselves are device arrays of L device pointers.  Follows the
 * array problem mode (rank-4 problem shape (M, N, K, L), one stride per
 * operand shared by all batches) of
 * sm90_gemm_array_tma_warpspecialized_cooperative.hpp.
 *   C        may be NULL iff beta == 0; otherwise L valid pointers.
 *   dtype    as for gmi_gemm_grouped (fp8 A and B give bf16 C and D).
 * No workspace is needed. */
gmi_status gmi_gemm_ptr_array(int32_t L, int32_t M, int32_t N, int32_t K, const void* const* A, int64_t lda,
                              const void* const* B, int64_t ldb, const void* const* C, int64_t ldc,
                              void* const* D, int64_t ldd, gmi_dtype dtype, float alpha, float beta,
                              void* stream);

/* Size in bytes of a prepacked uint4 weight: N * K / 2. */
size_t gmi_prepack_w4_bytes(int32_t N, int32_t K);

/* Prepack a uint4 weight W, logically [N][K] (Y = X W^T), from its plain
 * packed form [N][K/2] bytes (element (n, k) in byte n*K/2 + k/2, even k in
 * the low nibble) into the order the W4A16 kernels consume.  The design note
 * of machete_mainloop.cuh motivates it: reorder the narrow operand once so
 * that each lane's values for several consecutive matrix instructions arrive
 * in one 128-bit load.  The permutation (requires N % 16 == 0, K % 128 == 0):
 *   block b = (n/16) * (K/128) + k/128, 1024 bytes at offset 1024 b;
 *   inside a block, lane L = 16 * ((k % 32) / 8) + n % 16 owns 16 bytes at
 *   16 L: four little-endian 32-bit words, word j = (k % 128) / 32, each
 *   holding the 8 consecutive k = 8 * ((k % 32) / 8) + e of its row, element
 *   e in nibble slot e/2 + 4 (e % 2) (even elements in bits 0-15, odd ones in
 *   bits 16-31).
 * A bijection on the N*K/2 bytes; `w_u4` and `w_prepacked` must not overlap. */
gmi_status gmi_prepack_w4(const uint8_t* w_u4, int32_t N, int32_t K, uint8_t* w_prepacked, void* stream);

/* Bytes of the optional workspace that lets gmi_gemm_w4a16 and
 * gmi_gemm_mixed split K across workgroups for this shape on the current
 * device: fp32 partial products of the k-ranges for every 128 x 128 output
 * tile (rows rounded up to 128 tokens, columns to 128 weight rows), summed in
 * k-range order by a second launch; 0 when no split is used.  bf16
 * activations may use more k-ranges than fp16; the size covers either type,
 * and a call whose workspace is smaller than its own type needs runs
 * unsplit.  The layout is private to the library. */
size_t gmi_w4a16_workspace_bytes(int32_t M, int32_t N, int32_t K);

/* Mixed-input GEMM Y = X W^T, 4-bit weights with per-group scales and zero
 * points: w[n][k] = (q[n][k] - z[k/g][n]) * s[k/g][n], the conversion mode
 * "convert, scale, add zero" of machete_mainloop.cuh (ConversionMode
 * ConvertAndScaleWithZero; scale_k = ceil(K / group_size) from
 * to_underlying_arguments; transform_A_kblock).  The zero point is read here
 * as an unsigned 4-bit offset subtracted before scaling.  For M <= 48 the
 * matrix instruction takes the exact integers q - z (fp16) and each group's
 * scale multiplies the fp32 partial sum over that group; otherwise each
 * weight is dequantised to fp16 as RN16((q - z) * s) and multiplied in fp16.
 * Accumulation is fp32 either way; Y is rounded to fp16.
 *   workspace    optional device memory of at least
 *                gmi_w4a16_workspace_bytes(M, N, K) bytes, 16-byte aligned,
 *                no initialisation needed: with it, shapes whose output tiles
 *                cannot fill the device split K (partials then a summing
 *                launch, both on `stream`); NULL or smaller runs unsplit.
 *                Contents are scratch; calls sharing one workspace must be
 *                ordered (same stream).
 *   X            fp16 [M][ldx], ldx >= K.
 *   w_prepacked  gmi_prepack_w4 output for the [N][K] weight.
 *   scales       fp16 [K/group_size][N] (n contiguous).
 *   zeros        uint4 [K/group_size][N/2] bytes, even n in the low nibble.
 *   group_size   > 0, K % group_size == 0, and group_size == K or
 *                group_size % 128 == 0 (the page's rule: the group size is K
 *                or a whole number of K tiles).
 *   Y            fp16 [M][ldy], ldy >= N.
 * Requires N % 16 == 0, K % 128 == 0, scales and zeros 16-byte aligned. */
gmi_status gmi_gemm_w4a16(int32_t M, int32_t N, int32_t K, const void* X, int64_t ldx, const uint8_t* w_prepacked,
                          const void* scales, const uint8_t* zeros, int32_t group_size, void* Y, int64_t ldy,
                          void* workspace, size_t workspace_bytes, void* stream);

/* 4-bit weight element types: GMI_W4_UINT4 holds 0..15, GMI_W4_INT4 holds
 * -8..7 in two's complement (nibble 8 is -8).  Both are stored and prepacked
 * alike (gmi_prepack_w4 moves nibbles and never reads their values). */
typedef enum { GMI_W4_UINT4 = 0, GMI_W4_INT4 = 1 } gmi_w4_type;

/* Mixed-input GEMM Y = X W^T in each conversion mode of machete_mainloop.cuh
 * (ConversionMode, chosen there by which of scale and zero types is void):
 *   DirectConvert            scales == NULL, zeros == NULL: w = v(q)
 *   ConvertAndScale          zeros == NULL:                 w = v(q) * s[k/g][n]
 *   ConvertAndScaleWithZero  both given:                    w = (v(q) - v(z[k/g][n])) * s[k/g][n]
 * where v() is the value of a 4-bit element of type `w_type`; the zero
 * points have the weight's type and are subtracted before the scale, as in
 * gmi_gemm_w4a16 (which is this call with fp16, uint4 and both arrays).
 * Zero points without scales are GMI_ERR_UNSUPPORTED (no such mode).
 *   x_dtype      GMI_F16 or GMI_BF16: the type of X, of the scales and of Y
 *                (the page's fp16 and bf16 activation / scale types).
 *   group_size   as for gmi_gemm_w4a16; ignored when scales == NULL.
 *   other arguments, layouts, workspace and errors as for gmi_gemm_w4a16.
 * Numerics: with bf16 activations, and with fp16 for M <= 48, the matrix
 * instruction takes exact integer weights and the scale multiplies each
 * group's fp32 partial sum: v(q) - v(z) (for the bf16 decode kernel the
 * offset-binary nibble plus 128, with (128 + zero point) times the group's
 * activation sum taken off that partial sum).  fp16 with M > 48 rounds every
 * weight first, RN16((v(q) - v(z)) * s), as the page does.  fp32
 * accumulation; Y is rounded to nearest even. */
gmi_status gmi_gemm_mixed(int32_t M, int32_t N, int32_t K, gmi_dtype x_dtype, const void* X, int64_t ldx,
                          const uint8_t* w_prepacked, gmi_w4_type w_type, const void* scales, const uint8_t* zeros,
                          int32_t group_size, void* Y, int64_t ldy, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Grouped mixed-input GEMM, the mixture-of-experts form that combines the
 * grouped problem list of sm90_gemm_array_tma_warpspecialized_cooperative.hpp
 * (group sizes held on the device, as for gmi_gemm_grouped_offsets) with the
 * conversion of machete_mainloop.cuh: group g < count owns rows
 * [offsets[g], offsets[g + 1]) of X and Y and computes
 * Y_g = X_g W_g^T with its own weight, scales and zero points:
 *   W_g = w_prepacked + g * w_stride      (bytes; a gmi_prepack_w4 output of [N][K])
 *   s_g = scales      + g * s_stride      (elements of x_dtype; [K/group][N])
 *   z_g = zeros       + g * z_stride      (bytes; [K/group][N/2])
 *   offsets  device int32 [count + 1], read on the device; ranges are
 *            clipped to [0, rows) and an empty or reversed one is skipped, so
 *            no access leaves the buffers; rows outside every group are not
 *            written.
 *   rows     host: rows X and Y hold.
 *   count    0 .. 65535 groups.
 *   strides  at least one group's data when count > 1 (N*K/2 bytes,
 *            (K/group)*N scales, (K/group)*N/2 zero bytes) and keeping every
 *            group's data 16-byte aligned; ignored for a NULL array.
 * Modes, types and layouts as for gmi_gemm_mixed.  By default a group runs
 * 16 rows at a time through the decode kernel body (exact integer weights
 * into the matrix instruction, each group's scale on the fp32 partial sums,
 * as gmi_gemm_mixed does for M <= 48).  When count <= 1024 and rows > 256, groups of at most 32
 * rows instead run the same body over both 16-row tiles at once (each weight
 * streamed once; the same bits), and larger groups a second launch over
 * their 128 x 128 output tiles through the tiled mainloop (each weight
 * dequantised once to the activation type, as gmi_gemm_mixed does for
 * M > 64).  Both launches are enqueued on `stream` and write disjoint rows.
 * No workspace. */
gmi_status gmi_gemm_mixed_grouped(int32_t count, const int32_t* offsets, int32_t rows, int32_t N, int32_t K,
                                  gmi_dtype x_dtype, const void* X, int64_t ldx, const uint8_t* w_prepacked,
                                  int64_t w_stride, gmi_w4_type w_type, const void* scales, int64_t s_stride,
                                  const uint8_t* zeros, int64_t z_stride, int32_t group_size, void* Y, int64_t ldy,
                                  void* stream);

/* Implicit-GEMM conv2d forward (cross-correlation, groups == 1):
 *   y[n][p][q][k] = alpha * sum_{r,s,c} x[n][p*sh - ph + r*dh][q*sw - pw + s*dw][c] * w[k][r][s][c]
 *                   + beta * c_in[n][p][q][k]
 * taps outside the image read as 0.  P = (H + 2 ph - dh (R-1) - 1) / sh + 1,
 * Q likewise.  The GEMM view is M = N*P*Q, N = K, K = R*S*C with (r, s, c),
 * c fastest, so the KRSC filter is the column-major B operand unchanged.
 * Follows sm100_implicit_gemm_umma_warpspecialized.hpp: the activation
 * addressed through im2col with padding, traversal stride and dilation
 * (get_tma_load_a_instance), the linearised problem shape
 * (get_problem_shape_MNKL), and can_implement (cross-correlation only,
 * channel-innermost tensors, traversal stride 1..8).
 *   x      NHWC, w KRSC, c_in and y NPQK (all packed), element type dtype.
 *   c_in   may be NULL iff beta == 0.
 * Requires C % 8 == 0 and K % 8 == 0 (128-bit channel runs, else
 * GMI_ERR_MISALIGNED), stride in [1, 8] (a larger stride gives
 * GMI_ERR_UNSUPPORTED), dilation >= 1, padding >= 0, P >= 1, Q >= 1, and
 * N*P*Q, N*H*W below 2^31. */
gmi_status gmi_conv2d_fprop_implicit(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S,
                                     int32_t pad_h, int32_t pad_w, int32_t stride_h, int32_t stride_w,
                                     int32_t dil_h, int32_t dil_w, const void* x, const void* w, const void* c_in,
                                     void* y, gmi_dtype dtype, float alpha, float beta, void* stream);

/* Activation of the fused conv epilogue. */
typedef enum { GMI_ACT_NONE = 0, GMI_ACT_RELU = 1 } gmi_activation;

/* gmi_conv2d_fprop_implicit with a fused epilogue:
 *   v = alpha * sum(...) + beta * c_in[n][p][q][k] + bias[k]
 *   y[n][p][q][k] = RN(act(v)),   act: identity (GMI_ACT_NONE) or max(v, 0) (GMI_ACT_RELU)
 * The conv page leaves its collective epilogue a template parameter (the
 * kernel only hands it the accumulator tile); this is the common bias +
 * activation instance of it, evaluated in fp32 on the accumulator before the
 * single rounding to the output type.
 *   bias   K elements of `dtype` (one per output channel), 16-byte aligned, or
 *          NULL for none.
 *   act    GMI_ACT_NONE or GMI_ACT_RELU; any other value gives
 *          GMI_ERR_INVALID_ARG.
 * All other arguments, layouts and errors as for gmi_conv2d_fprop_implicit. */
gmi_status gmi_conv2d_fprop_implicit_fused(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R,
                                           int32_t S, int32_t pad_h, int32_t pad_w, int32_t stride_h,
                                           int32_t stride_w, int32_t dil_h, int32_t dil_w, const void* x,
                                           const void* w, const void* c_in, const void* bias, void* y,
                                           gmi_dtype dtype, float alpha, float beta, gmi_activation act,
                                           void* stream);

/* Bytes of the workspace gmi_conv2d_dgrad_implicit needs: the filter
 * rearranged to [C][R][S][K] (C*K*R*S*2, rounded up to 256); 0 for a
 * non-positive size. */
size_t gmi_conv2d_dgrad_workspace_bytes(int32_t C, int32_t K, int32_t R, int32_t S);

/* Bytes of the workspace gmi_conv2d_wgrad_implicit needs for this problem
 * on the current device (the transposed operands and fp32 partial sums of
 * the split over taps); 0 if the problem is rejected. */
size_t gmi_conv2d_wgrad_workspace_bytes(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S,
                                        int32_t pad_h, int32_t pad_w, int32_t stride_h, int32_t stride_w,
                                        int32_t dil_h, int32_t dil_w, int32_t groups);

/* Implicit-GEMM conv2d weight gradient (the page's wgrad operator, and its
 * grouped wgrad), the adjoint of the forward convolution in its filter:
 *   dw[k][r][s][c] = alpha * sum over (n, p, q) of dy[n][p][q][k] *
 *                    x[n][p*sh - ph + r*dh][q*sw - pw + s*dw][g(k) * C/groups + c]
 *                    (taps inside the image) + beta * c_in[k][r][s][c],
 *   c < C/groups, g(k) = k / (K/groups): output channel k of group g sees
 *   only input channels g*C/groups .. (g+1)*C/groups - 1 (groups == 1 is the
 *   plain weight gradient of gmi_conv2d_fprop_implicit).
 * Arguments describe the forward problem: x NHWC (N x H x W x C), dy NPQK
 * with P, Q as for the forward pass, dw and c_in K x R x S x C/groups.  The page gathers the
 * activation as the im2col operand with dy tiled; here the sum is computed
 * as a forward convolution of the channel-major activation (each channel an
 * image whose channels are the batch) with dy as the filter, stride and
 * dilation exchanged, after two transposes into `workspace`; it is split over
 * taps into fp32 partials that a last launch sums in a fixed order, scales,
 * rounds to nearest even and writes as KRSC.
 *   workspace  at least gmi_conv2d_wgrad_workspace_bytes(...) bytes, 16-byte
 *              aligned, scratch for the call.
 * Requires N >= 1, C % 8 == 0 and K % 8 == 0 (else GMI_ERR_MISALIGNED),
 * groups dividing C and K with K/groups % 8 == 0, stride and dilation in
 * [1, 8], 16-byte aligned pointers, c_in NULL iff beta == 0. */
gmi_status gmi_conv2d_wgrad_implicit(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S,
                                     int32_t pad_h, int32_t pad_w, int32_t stride_h, int32_t stride_w,
                                     int32_t dil_h, int32_t dil_w, int32_t groups, const void* x, const void* dy,
                                     const void* c_in,
                                     void* dw, gmi_dtype dtype, float alpha, float beta, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Implicit-GEMM conv2d data gradient (the page's dgrad operator), the
 * adjoint of gmi_conv2d_fprop_implicit in its activation:
 *   dx[n][h][w][c] = alpha * sum over (p, q, k, r, s) with p*sh - ph + r*dh = h,
 *                    q*sw - pw + s*dw = w of dy[n][p][q][k] * w[k][r][s][c]
 *                    + beta * c_in[n][h][w][c]
 * Arguments describe the forward problem: x was N x H x W x C, the filter is
 * w KRSC, dy is N x P x Q x K with P, Q as for the forward pass; dx and c_in
 * are NHWC.  As on the page, dgrad gathers dy through the im2col addressing
 * with the filter-tap strides negated (padding -ph and dilation -dh over
 * dy); the GEMM view is M = N*H*W, N = C, K = R*S*K.  A forward stride above
 * 1 runs the page's strided dgrad: the dx pixels split into sh x sw phases
 * (rows h with h + ph in one residue class of sh, crossed with the columns'
 * classes), and each phase gathers dy over only the taps that reach it
 * (r*dh = h + ph mod sh), so no multiply touches a tap that misses; a phase
 * that no tap reaches gets alpha * 0 + beta * c_in.  Up to 16 phases run as
 * one launch (longest reduction first), more as a launch per phase.
 *   workspace  at least gmi_conv2d_dgrad_workspace_bytes(C, K, R, S) bytes,
 *              16-byte aligned: the filter rearranged per phase, [C][taps of
 *              the phase][K], one phase after another (the phases partition
 *              the taps), written and read by the call's launches.
 * Traversal strides in [1, 8] in each dimension, else GMI_ERR_UNSUPPORTED;
 * for a stride above 1, dx must stay below 2^31 bytes.  Other rules as for
 * the forward pass: C % 8 == 0 and K % 8 == 0, 16-byte aligned pointers, c_in
 * NULL iff beta == 0. */
gmi_status gmi_conv2d_dgrad_implicit(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S,
                                     int32_t pad_h, int32_t pad_w, int32_t stride_h, int32_t stride_w,
                                     int32_t dil_h, int32_t dil_w, const void* dy, const void* w, const void* c_in,
                                     void* dx, gmi_dtype dtype, float alpha, float beta, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Text of the last failed check or HIP error on the calling thread ("" if
 * none).  The pointer stays valid until the next gmi_* call on that thread. */
const char* gmi_last_error(void);

/* Measurement hook, for benchmarks and profilers of the GEMM path.  `start`
 * and `stop` are hipEvent_t handles that the caller created (with timing
 * enabled) and owns.  The next GEMM kernel that gmi_gemm_grouped,
 * gmi_gemm_grouped_offsets(_noalloc) or gmi_gemm_ptr_array launches on the
 * calling thread is launched through hipExtLaunchKernel with this pair, so
 * the runtime stamps them with that kernel's own start and end: their
 * elapsed time is the kernel's execution time, without the dispatch and
 * completion work that events recorded before and after the launch also
 * time.  The request is used by one kernel and then cleared; a call that
 * launches no GEMM kernel (a failed check, no work) leaves it pending.  The
 * table-building launches of the grouped calls are not timed.  Both NULL
 * cancels a pending request; exactly one NULL returns GMI_ERR_INVALID_ARG.
 * Makes no HIP call. */
gmi_status gmi_time_next_gemm(void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* GMI_H */
