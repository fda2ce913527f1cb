/*
 * fp4.h -- C ABI of the MI355X (gfx950) W4A4 block-scaled FP4 linear library.
 *
 * What it computes (the pages this project works from):
 *   - NVFP4: blocks of 16 consecutive values along K share one E4M3 scale
 *     s_b = cast_E4M3(max|x| / 6); each value is an E2M1 code q from
 *     {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}; x^ = s_b * q
 *     ("Hardware FP4 inference for speech on Blackwell", section "NVFP4, and
 *     the two ways it fails", both display equations). A second, per-tensor
 *     FP32 scale S_t keeps block scales under E4M3's 448 and block scales
 *     saturate (same section, paragraph on scale overflow; and "FP4 n'existe
 *     pas ...", section "Deux dialectes", two-level scaling). Here
 *     S_t = RN_fp32(max|x| / 2688) (dynamic) or a caller-given value (static),
 *     and x^ = q * s_b * S_t.
 *   - MXFP4: blocks of 32 values share one E8M0 power-of-two scale
 *     ("FP4 n'existe pas ...", section "Deux dialectes" and its table).
 *     Block exponent e_b = clamp(floor(log2 max|x|) - 2, -127, 127).
 *   - Weights are quantized once and cached; activations are quantized on
 *     every call; the product runs on the quantized operands with FP32
 *     accumulation (forum post on a standalone FP4 GEMM library with a
 *     pre-quantized weight cache, opening paragraphs).
 *   - The GEMM follows a linear layer: C[M,N] = A[M,K] * W[N,K]^T.
 *
 * Codes: E2M1 nibbles, sign in bit 3, magnitude index in bits 0-2 (S|EE|M,
 * exponent bias 1); two per byte, even k in the low nibble. Element rounding
 * is nearest with ties to even, against the rounded block scale.
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     allocates no memory and keeps no per-call state.
 *   - Work is enqueued on `stream` (0 = default stream) and the call returns
 *     without waiting. Faults inside kernels surface at the caller's next
 *     synchronization.
 *   - Arguments are validated on the host before anything is launched; a
 *     rejected call launches nothing and returns a non-zero fp4_status, with
 *     a description available from fp4_last_error() on the same thread.
 *   - Inputs are bf16, row-major, contiguous, 16-byte aligned, finite.
 *   - The library runs on gfx950 devices only (FP4_ERR_DEVICE otherwise).
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FP4_NVFP4 = 0, FP4_MXFP4 = 1 } fp4_format;

/*
 * Quantization recipe flags, OR-ed into a format value wherever an int32_t
 * fmt is taken (fp4_format | flags). They change how values are quantized,
 * not the stored format, its layout or its sizes. A tensor descriptor keeps
 * the flags it was quantized with; fp4_linear quantizes the activations with
 * the weight's flags.
 *
 * FP4_ROTATE: before quantization, each block of B values along K (B = the
 *   format's block: 16 or 32) is rotated, y = H_B x / sqrt(B), H_B the
 *   Sylvester Hadamard matrix: the online rotation the MXFP4 path applies to
 *   activations ("FP4 on a consumer RTX 5090: the Blackwell headline loses to
 *   plain int4", section "Finding 3 - the real-FP4 path"; the page gives no
 *   rotation size, the block is the one used here). Each rotated value is
 *   the exact real RN_fp32(1/sqrt(B)) * sum_j H[i][j] x[j] rounded once to
 *   bf16 (nearest, ties to even; an exact zero gives +0), so the result does
 *   not depend on the order of the additions; the block is quantized from
 *   those bf16 values. Weights and activations must both be rotated, or neither:
 *   then H_B H_B^T / B = I and the GEMM approximates the unrotated product.
 *   fp4_gemm rejects operands that differ in this flag. The NVFP4 dynamic
 *   tensor scale is taken over the rotated values. fp4_dequantize returns the
 *   rotated-domain values. Inputs must satisfy |x| < 2^120 (no overflow in
 *   the transform).
 * FP4_MX_OAS (MXFP4 only): overflow-aware block exponent, the smallest e with
 *   max|x| <= 6 * 2^e (clamped to [-127, 127]), so no element saturates
 *   ("FP4 n'existe pas ...", section "L'ecart de qualite - et comment il se
 *   reduit"); the default exponent floor(log2 max|x|) - 2 lets block maxima
 *   in (6, 8) * 2^e saturate. Operands may differ in this flag.
 * FP4_MX_MBS (MXFP4 only): macro-block scaling, a second-level scale over a
 *   macro-block of several 32-value blocks that brings MXFP4 closer to
 *   two-level scaling without changing its base format ("FP4 n'existe
 *   pas ...", same section; the page gives neither the macro-block size nor
 *   the scale's format). Here a macro-block is the four blocks of one
 *   128-value segment of a row along K, and its scale is the FP32 number
 *   S_mb = RN_fp32(g / (6 * 2^j)) in [1, 2), g the segment's largest
 *   magnitude and j = floor(log2(g / 6)) (1 when g = 0), which puts the
 *   segment's largest value on the top code. Each block's E8M0 exponent is
 *   the rule above applied to its values divided by S_mb, and elements round
 *   against 2^e_b * S_mb: x^ = q * 2^e_b * S_mb. The S_mb are stored after the
 *   E8M0 bytes in the scales buffer (fp4_scales_bytes includes them): TILED,
 *   16 floats per fragment (one per fragment row) after all fragments' E8M0
 *   bytes; CANONICAL, [rows][K_pad / 128] floats starting at the first
 *   16-byte boundary past rows * scales_pitch bytes. Both operands of a
 *   product must carry this flag, or neither (fp4_gemm: FP4_ERR_FORMAT_MISMATCH);
 *   the weight-only linear rejects it. Combines with FP4_ROTATE and FP4_MX_OAS
 *   (with OAS: the smallest e with a_b <= 6 * 2^e * S_mb).
 */
enum { FP4_ROTATE = 0x100, FP4_MX_OAS = 0x200, FP4_MX_MBS = 0x400 };

typedef enum {
    FP4_OK = 0,
    FP4_ERR_INVALID_ARG = 1,     /* null pointer, bad enum, non-positive size */
    FP4_ERR_SHAPE = 2,           /* K not a multiple of the block, mismatched K */
    FP4_ERR_ALIGNMENT = 3,       /* pointer or pitch not 16-byte aligned */
    FP4_ERR_WORKSPACE = 4,       /* workspace missing or smaller than required */
    FP4_ERR_FORMAT_MISMATCH = 5, /* operands of different formats or layouts */
    FP4_ERR_DEVICE = 6,          /* current device is not gfx950 */
    FP4_ERR_HIP = 7              /* a HIP runtime call or launch failed */
} fp4_status;

/*
 * CANONICAL: codes row-major [rows][codes_pitch] bytes (pitch >= K_pad/2),
 *   scales row-major [rows][scales_pitch] bytes (pitch >= K_pad/B); bytes
 *   past K within a row are zero. This is the activation layout and the
 *   layout used to compare with a reference byte for byte.
 * TILED: the weight cache layout, also accepted for activations (the linear
 *   path uses it internally). Rows are padded to round_up(rows, 16) and K to
 *   K_pad = round_up(K, 128); the matrix is cut into
 *   fragments of 16 rows x 128 values, stored fragment-major
 *   ((row / 16) * (K_pad / 128) + k / 128). A fragment's codes are 1024 bytes:
 *   16 bytes per lane l = 16 * c + r holding row r, values 32c .. 32c+31 of
 *   the fragment. Its scales follow the same lane order: 128 bytes (NVFP4,
 *   two E4M3 bytes per lane) or 64 bytes (MXFP4, one E8M0 byte per lane).
 *   Padding codes and scales are zero.
 * K_pad = round_up(K, 128) in both layouts.
 */
typedef enum { FP4_LAYOUT_CANONICAL = 0, FP4_LAYOUT_TILED = 1 } fp4_layout;

typedef struct {
    int32_t fmt;            /* fp4_format */
    int32_t layout;         /* fp4_layout */
    int64_t rows;           /* logical rows (M for activations, N for weights) */
    int64_t cols;           /* logical K */
    int64_t codes_pitch;    /* CANONICAL: bytes per row of codes; TILED: 0 */
    int64_t scales_pitch;   /* CANONICAL: bytes per row of scales; TILED: 0 */
    void *codes;            /* device, caller-owned */
    void *scales;           /* device, caller-owned */
    float *tensor_scale;    /* device FP32 S_t (NVFP4); ignored for MXFP4 */
} fp4_tensor;

/* Block size along K: 16 (NVFP4) or 32 (MXFP4); 0 for a bad format. */
int32_t fp4_block_size(int32_t fmt);

/* Bytes needed for the codes / scales of a [rows, k] tensor in `layout`
 * (padding included). 0 for invalid arguments. */
size_t fp4_codes_bytes(int32_t fmt, int32_t layout, int64_t rows, int64_t k);
size_t fp4_scales_bytes(int32_t fmt, int32_t layout, int64_t rows, int64_t k);

/* Fill `t` for caller-allocated buffers sized by the two calls above
 * (canonical pitches are the minimum: K_pad/2 and K_pad/B bytes). */
fp4_status fp4_tensor_init(fp4_tensor *t, int32_t fmt, int32_t layout, int64_t rows,
                           int64_t k, void *codes, void *scales, float *tensor_scale);

/* Workspace for fp4_quantize_act / fp4_quantize_weight (NVFP4: the per-tensor
 * maximum reduction; MXFP4: 0). It must be zero-filled before its first use;
 * every call leaves it reusable. Calls sharing a workspace must not overlap
 * in time. */
size_t fp4_quantize_workspace_bytes(int32_t fmt, int64_t rows, int64_t k);

/*
 * Quantize a weight W bf16 [n, k] once, into `out` (TILED, filled by
 * fp4_tensor_init with rows = n, cols = k). NVFP4 uses the dynamic per-tensor
 * scale, written to *out->tensor_scale. k must be a multiple of the block.
 */
fp4_status fp4_quantize_weight(int32_t fmt, const void *w_bf16, int64_t n, int64_t k,
                               fp4_tensor *out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * Quantize activations A bf16 [m, k] into `out` (CANONICAL or TILED). NVFP4:
 * static_scale == NULL selects the dynamic per-tensor scale; otherwise
 * *static_scale (device FP32, > 0, finite) is used as S_t and block scales
 * saturate at 448. MXFP4 requires static_scale == NULL.
 */
fp4_status fp4_quantize_act(int32_t fmt, const void *a_bf16, int64_t m, int64_t k,
                            const float *static_scale, fp4_tensor *out, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Workspace for fp4_gemm: for CANONICAL activations with M > 128, room for a
 * tiled copy of them (then the product runs on the LDS-staged tile kernel);
 * for TILED activations with 33 <= M <= 128 on a weight large enough for the
 * mid-size GEMM (fp4_set_mid_gemm), room for its FP32 partial sums (K split
 * over workgroups; 0 when the shape takes one slice); otherwise 0. No zero-filling or persistence is needed. */
size_t fp4_gemm_workspace_bytes(int32_t fmt, int64_t m, int64_t n, int64_t k);

/*
 * C[m, n] (bf16, row stride ldc elements) = bf16_RNE(alpha * sum_k a^'[m,k] w^'[n,k]),
 * with a^' = q * s_b (per-tensor factors pulled into alpha = S_tA * S_tW for
 * NVFP4, alpha = 1 for MXFP4). `a` is CANONICAL or TILED, `w` is TILED,
 * same format and K. Accumulation is FP32. CANONICAL `a` with M > 128 is
 * first copied into the tiled layout in `workspace` when it holds
 * fp4_gemm_workspace_bytes (16-byte aligned); with a smaller or NULL
 * workspace such a product runs on a slower kernel that reads the canonical
 * layout directly. TILED `a` with 33 <= M <= 128 on a large weight runs on
 * the mid-size kernel (fp4_set_mid_gemm) when the workspace holds
 * fp4_gemm_workspace_bytes, else on the skinny kernel; the two agree within
 * the GEMM tolerance. Calls sharing a workspace must not overlap in time.
 * FP4_ERR_SHAPE when M <= 128 with CANONICAL `a` whose M * max(codes pitch,
 * scales pitch) reaches 2^31 bytes (the skinny kernels use 32-bit offsets).
 */
fp4_status fp4_gemm(const fp4_tensor *a, const fp4_tensor *w, void *c_bf16, int64_t ldc,
                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace for fp4_linear: the quantized activations and the quantizer's
 * scratch (and, for 33-128 rows, the mid-size GEMM's partial sums, at most
 * 12 MiB, within the allocation-free array where the rest fits). Same contract as the quantize workspace: zero-filled before its
 * first use, left reusable by every call, not shared by overlapping calls.
 * One workspace may serve calls of different shapes (and formats) in
 * sequence when it is at least as large as each call requires: the words that
 * persist between calls sit at a fixed offset. */
size_t fp4_linear_workspace_bytes(int32_t fmt, int64_t m, int64_t n, int64_t k);

/*
 * y[m, N] (bf16, contiguous) = x[m, K] (bf16) through the cached weight `w`:
 * quantize x as fp4_quantize_act would (same static_scale rule), then
 * fp4_gemm. All intermediate data lives in `workspace`.
 * Small activations (M * K small enough for every workgroup to quantize them
 * itself) take one launch of the skinny GEMM with that quantization inside.
 * Otherwise, for M <= 32 without macro-block scales or rotation, and with
 * fp4_set_decode_linear_fusion(1), this is one launch of the skinny GEMM: its
 * first workgroups quantize the activations into the workspace while the
 * GEMM workgroups issue their first weight loads and then wait for them. That
 * wait is bounded like the quantizer's maximum exchange (FP4_WS_EXCHANGE_TIMEOUT,
 * NaN outputs, the workspace to be zero-filled again before reuse, as below).
 * With fp4_set_large_linear_fusion(1), M > 128 with a static NVFP4 scale, or
 * MXFP4 without macro-block scales, is one launch: its first workgroups
 * quantize the activations (each row panel of output tiles once, split along
 * K among several workgroups) and the tile workgroups wait for their panel
 * before reading it. That wait is bounded like the quantizer's maximum
 * exchange: a tile that gives up makes its outputs NaN and sets
 * FP4_WS_EXCHANGE_TIMEOUT (fp4_workspace_flags); the workspace must then be
 * zero-filled again before it is reused.
 */
fp4_status fp4_linear(const void *x_bf16, int64_t m, const fp4_tensor *w,
                      const float *static_scale, void *y_bf16, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * fp4_linear for callers that cannot allocate device memory: code under
 * stream capture, tight serving loops, harnesses that forbid allocation. The
 * same computation and kernels as fp4_linear, without a workspace argument:
 * the workspace is a device array inside the library, FP4_NOALLOC_SCRATCH_BYTES
 * on every GPU the library runs on, held until the process ends. The call
 * allocates nothing. A call that would need more workspace than that
 * (fp4_linear_workspace_bytes) returns FP4_ERR_WORKSPACE before launching
 * anything. All calls on one GPU share that GPU's array, which keeps what the
 * last call left there: calls that overlap in time on one GPU (other streams
 * or threads) race and must be serialized by the caller. The first call on a
 * GPU clears the array's persistent words with a kernel on its stream.
 */
#define FP4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
fp4_status fp4_linear_noalloc(const void *x_bf16, int64_t m, const fp4_tensor *w,
                              const float *static_scale, void *y_bf16, hipStream_t stream);

/*
 * Weight-only linear (W4A16): y[m, N] (bf16, row stride ldy elements) =
 * bf16_RNE(S_tW * sum_k x[m, k] * (q * s_b)[n, k]) with the activations x
 * [m, K] kept in bf16 (contiguous, 16-byte aligned) and only the cached weight
 * `w` (TILED) in FP4; FP32 accumulation ("Hardware FP4 inference for speech
 * on Blackwell", section "Weights are safe" for the W4A16 regime, and section
 * "Two Triton kernels for the SM120 gaps" for a W4A16 GEMM on pre-packed FP4
 * weights). S_tW = 1 for MXFP4. One launch, no workspace. A rotated weight
 * (FP4_ROTATE) is rejected (FP4_ERR_FORMAT_MISMATCH): its activations would
 * need the same rotation, which fp4_linear applies. MXFP4 weights must stay
 * below 2^127 in magnitude (their dequantized values are formed in bf16).
 */
fp4_status fp4_linear_w4a16(const void *x_bf16, int64_t m, const fp4_tensor *w, void *y_bf16,
                            int64_t ldy, hipStream_t stream);

/* Number of kernel launches fp4_linear makes for this shape under the
 * current switches: 1 when the activation quantization is fused into the
 * GEMM (small M * K on the skinny path without rotation or macro-block
 * scales; with fp4_set_decode_linear_fusion(1), M <= 32 without either; with
 * fp4_set_large_linear_fusion(1), M > 128 with a static NVFP4 scale or MXFP4
 * without macro-block scales), 2 for quantize + GEMM, one more when the
 * quantizer needs a separate reduction launch (NVFP4 activations with a
 * dynamic scale past 16384 fragments of 16 x 128 values, or rotated and past
 * the single-launch quantizer's size), and one more when the mid-size GEMM
 * (33-128 rows) splits K (its partial sums are added by a launch of their
 * own). 0 for invalid arguments. */
int32_t fp4_linear_launches(int32_t fmt, int64_t m, int64_t n, int64_t k, int32_t static_scale);

/*
 * Sticky error flags that kernels record in a quantize or linear workspace
 * (the flags sit at the same offset in both). FP4_WS_EXCHANGE_TIMEOUT: a
 * workgroup of the single-launch NVFP4 quantizer (dynamic scale, activations
 * of up to 2^17 blocks) gave up waiting for the other workgroups' maxima. That
 * exchange assumes every workgroup of its grid (at most 128 workgroups of at
 * most 512 threads) is resident at once; a workgroup that is not, for as long
 * as the bounded wait lasts (about 2^22 polls), makes the call fail visibly:
 * its tensor scale is NaN (so is every product computed from it) and the flag
 * is set. The flags stay set until cleared here.
 * Waits for `stream`, writes the flags to *flags and, when clear != 0, clears
 * them. Not for use inside a stream capture.
 */
enum { FP4_WS_EXCHANGE_TIMEOUT = 1 };
fp4_status fp4_workspace_flags(const void *workspace, size_t workspace_bytes, uint32_t *flags,
                               int32_t clear, hipStream_t stream);

/* Test aid: the number of polls after which a workgroup of that exchange gives
 * up (default 2^22; 0 gives up at once, which makes every such call fail as
 * described above). Process-wide; returns the previous value. */
uint32_t fp4_set_exchange_spin_limit(uint32_t polls);

/* Whether fp4_linear quantizes large-M activations inside the GEMM launch
 * where it can (1) or in a launch of its own (0, the default: the separate
 * quantizer keeps many waves on every CU, the producers inside the GEMM only
 * as many as the tile kernel does, and the two-launch form measured as fast
 * or faster). Same results either way. Process-wide; returns the previous
 * setting. */
int32_t fp4_set_large_linear_fusion(int32_t on);

/* Whether fp4_linear with at most 32 activation rows quantizes them inside the
 * skinny GEMM's launch (1) or in a launch of its own (0, the default: the
 * GEMM workgroups can prefetch only their first weight fragments while they
 * wait, and the producers' chain of loads, stores and counts took longer
 * than a launch of its own). Same results either way. Process-wide; returns
 * the previous setting. */
int32_t fp4_set_decode_linear_fusion(int32_t on);

/* Whether the GEMM of 33-128 activation rows (tiled activations, no
 * macro-block scales; fp4_linear, and fp4_gemm with a workspace of
 * fp4_gemm_workspace_bytes) on large weights runs on the mid-size kernel (1,
 * the default: four weight tiles per workgroup, so each activation fragment is
 * loaded and converted once per 64 output columns; K split over at most one
 * workgroup per CU, whose FP32 partial sums a second launch adds in a fixed
 * order) or on the skinny kernel (0: one 16-row weight tile per workgroup
 * over the whole K). The mid-size kernel takes a shape only when every wave
 * streams at least 8 of K's 128-value fragments (about K * N >= 2^26 at
 * 256 CUs); smaller shapes keep the skinny kernel either way. Results agree
 * within the GEMM tolerance, not bit for bit (another summation order).
 * Process-wide; returns the previous setting. */
int32_t fp4_set_mid_gemm(int32_t on);

/* Test aid: the number of K slices the mid-size GEMM of fp4_linear uses for
 * this shape under the current switches (1: one launch that writes the
 * output; more: a combining launch adds the slices), or 0 when fp4_linear
 * runs another GEMM kernel (or the arguments are invalid). */
int32_t fp4_linear_mid_splits(int32_t fmt, int64_t m, int64_t n, int64_t k);

/* Where the NVFP4 product on 256 x 256 output tiles (large M) converts codes
 * to exact f16 values: 0 = in the registers of each wave that uses a fragment
 * (two waves per fragment), 1 = once per workgroup into LDS, the waves then
 * reading f16 operands. Same results either way. Process-wide; returns the
 * previous mode, or -1 for an invalid mode (nothing changed). */
int32_t fp4_set_nvfp4_tile_mode(int32_t mode);

/* Test aids (not on the hot path). */
/* Copy a TILED tensor into a CANONICAL one of the same format/shape
 * (including the tensor scale when both pointers are set). */
fp4_status fp4_export_canonical(const fp4_tensor *tiled, fp4_tensor *canonical,
                                hipStream_t stream);
/* x^ as FP32 [rows, cols] with row stride ldo (RN_fp32 of q * s_b * S_t). */
fp4_status fp4_dequantize(const fp4_tensor *t, float *out_f32, int64_t ldo,
                          hipStream_t stream);

const char *fp4_status_string(int32_t status);
/* Detail of the last non-OK status returned on this thread ("" if none). */
const char *fp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H */
