/*
 * fp4_oracle.c -- plain, slow CPU oracle for block-scaled FP4 (NVFP4 and MXFP4)
 * quantization, dequantization and the GEMM over dequantized operands.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library. The GPU library shares no code,
 * header, table or helper with it, and neither side includes or calls the other.
 *
 * Sources (the web pages this project works from):
 *   [SPEECH]  "Hardware FP4 inference for speech on Blackwell",
 *             section "NVFP4, and the two ways it fails": the E2M1 code set
 *             (first display equation), the block scale s = cast_E4M3(max|x|/6)
 *             with dequantization x^ = s*q (second display equation), the
 *             max/12 and max/24 facts, the 1000-outlier example, the E4M3
 *             ceiling of 448 and the 6*448 = 2688 overflow threshold, and the
 *             per-tensor FP32 scale with saturation used by hardware paths.
 *   [DIALECT] "FP4 n'existe pas : il existe des FP4, et chaque runtime choisit
 *             son dialecte", section "Deux dialectes, deux strategies de
 *             scaling" and its comparison table: E2M1 elements (1 sign,
 *             2 exponent, 1 mantissa bit), MXFP4 = 32-value blocks sharing an
 *             E8M0 (power-of-two) scale, NVFP4 = 16-value blocks with an E4M3
 *             block scale plus an FP32 per-tensor scale; ~4.5 / ~4.25 bits per
 *             value.
 *   [GEMMLIB] Forum post on a standalone FP4 GEMM library with a pre-quantized
 *             weight cache (opening paragraphs): weights are quantized once,
 *             activations per call, and the product runs on the quantized
 *             operands.
 *   [REALFP4] "FP4 on a consumer RTX 5090: the Blackwell headline loses to
 *             plain int4", section "Finding 3 - the real-FP4 path (QuTLASS
 *             MXFP4)": the MXFP4 path rotates activations with an online
 *             Hadamard transform before quantizing them.
 *   [DIALECT], section "L'ecart de qualite - et comment il se reduit": the
 *             overflow-aware scaling variant (OAS) picks the per-block scale
 *             so that the block's extreme values do not saturate.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - E2M1 bit layout S|EE|M with exponent bias 1 (the only IEEE-style layout
 *     that yields the printed code set).
 *   - "cast" is round-to-nearest, ties to even.
 *   - E4M3 is the variant whose largest finite value is 448 (no infinities,
 *     0x7F/0xFF are NaN).
 *   - Per-tensor scale (NVFP4, dynamic): S_t = RN_fp32(g / 2688), g = max|x|
 *     over the tensor; S_t = 1 when g = 0. It is the decode multiplier:
 *     x^ = q * s_b * S_t. Block scales then saturate at 448 (the hardware
 *     recipe); the naive single-level variant (S_t = 1, no saturation, NaN on
 *     overflow) is provided only to reproduce the pages' failure example.
 *   - Element rounding uses the rounded block scale: the code is the nearest
 *     point of {0, .5, 1, 1.5, 2, 3, 4, 6} * d_b to |x| (d_b = s_b * S_t),
 *     ties to the even index, saturating at 6 * d_b.
 *   - Blocks run along the contraction dimension K of both operands; even k
 *     goes to the low nibble of each byte; negative values that round to zero
 *     keep their sign bit.
 *   - MXFP4 block exponent: e_b = clamp(floor(log2 a_b) - 2, -127, 127),
 *     a_b = 0 -> -127; the scale byte is e_b + 127. The pages name the open MX
 *     specification without printing its rule, so this rule is pinned only by
 *     invariants (block max lands on 4 or 6, nothing saturates), not by a value
 *     the pages print.
 *   - Rotation (optional, either format): within each quantization block of
 *     B values along k, y = H_B x / sqrt(B) with H_B the Sylvester Hadamard
 *     matrix (H[i][j] = (-1)^popcount(i & j)); the pages give no rotation
 *     size, and B keeps each rotation inside the block it feeds. The pages
 *     give no precision either; the rotation's output decides codes, so it is
 *     defined without any order-dependent rounding: the exact real
 *     c * sum_j H[i][j] x[j], c = RN_fp32(1/sqrt(B)) (exactly 1/4 for B = 16),
 *     rounded once to bf16 (nearest even), the activation type the quantizer
 *     takes; an exact zero gives +0. The weights are rotated the same way, so
 *     the GEMM of the two rotated operands approximates the unrotated product
 *     (H H^T / B = I).
 *   - OAS (MXFP4 only): e_b = the smallest exponent with a_b <= 6 * 2^e_b
 *     (clamped to [-127, 127]), so no element saturates; the default rule
 *     lets block maxima in (6, 8) * 2^e_b saturate to 6 * 2^e_b.
 *   - MBS (MXFP4 only; [DIALECT], same section: a second-level scale over a
 *     macro-block grouping several 32-value blocks, bringing MXFP4 closer to
 *     two-level scaling without changing the base format). The pages give
 *     neither the macro-block size nor the scale's format or rule. Reading:
 *     a macro-block is the 32-value blocks of one 128-value segment of a row
 *     along k (the last segment shorter when k % 128 != 0); its scale is an
 *     FP32 number in [1, 2), S_mb = RN_fp32(g / (6 * 2^j)) with g the
 *     segment's largest magnitude and j = floor(log2(g / 6)) (S_mb = 1 when
 *     g = 0), the non-power-of-two factor that puts the segment's largest
 *     value on the top code 6 * 2^j, as a two-level scale puts a block's on
 *     6 * s_b. Each block then takes the MX exponent of its values divided by
 *     S_mb: e_b = clamp(floor(log2(a_b / S_mb)) - 2, -127, 127) (with OAS the
 *     smallest e with a_b <= 6 * 2^e * S_mb); its decode step is
 *     d_b = 2^e_b * S_mb and x^ = q * 2^e_b * S_mb. The E2M1 codes and E8M0
 *     bytes keep their format; the S_mb are stored beside them.
 *
 * Precision: every decision is taken on exact values. bf16 inputs, E4M3 scales,
 * FP32 tensor scales and the thresholds t * s_b * S_t (<= 31 significant bits)
 * are exact in binary64, so all comparisons below are exact. The two divisions
 * (a_b / (6 S_t) and g / 2688) are argued exact-in-effect where they occur.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_DYNAMIC = 0, ORC_STATIC = 1, ORC_NAIVE = 2 };
enum { ORC_NVFP4 = 0, ORC_MXFP4 = 1 };

/* ------------------------------------------------------------------ codecs */

/* bf16 bit pattern -> exact binary64 value. */
double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E2M1 nibble -> value. [DIALECT]: 1 sign, 2 exponent, 1 mantissa bit;
 * reading: exponent bias 1, exponent field 0 is subnormal (M * 0.5). */
double orc_e2m1_value(int code)
{
    int s = (code >> 3) & 1, ee = (code >> 1) & 3, m = code & 1;
    double mag = (ee == 0) ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, ee - 1);
    return s ? -mag : mag;
}

/* E4M3 byte -> value: S|EEEE|MMM, bias 7, largest finite 448 [SPEECH],
 * 0x7F and 0xFF are NaN, no infinities. */
double orc_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = m * ldexp(1.0, -9);            /* subnormal: M/8 * 2^-6 */
    else
        mag = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -mag : mag;
}

/* E8M0 byte -> value 2^(byte - 127); 0xFF is NaN [DIALECT: exponent only]. */
double orc_e8m0_value(int byte)
{
    if (byte == 0xFF)
        return NAN;
    return ldexp(1.0, byte - 127);
}

/* Round a non-negative real v to E4M3, nearest, ties to even mantissa.
 * The grid is extended past 448 with the same spacing; a result above 448
 * becomes 448 when saturating and NaN (0x7F) otherwise. Returns the byte. */
int orc_e4m3_from_real(double v, int saturate)
{
    if (isnan(v))
        return 0x7F;
    if (v <= 0.0)
        return 0x00;
    int e2;
    frexp(v, &e2);                 /* v = f * 2^e2, f in [0.5, 1) */
    int fl = e2 - 1;               /* floor(log2 v) */
    if (fl < -6)
        fl = -6;                   /* subnormals share the 2^-6 binade spacing */
    double quantum = ldexp(1.0, fl - 3);  /* 3 mantissa bits per binade */
    double n = v / quantum;        /* exact: power-of-two division */
    double whole = floor(n), frac = n - whole;
    if (frac > 0.5 || (frac == 0.5 && fmod(whole, 2.0) != 0.0))
        whole += 1.0;              /* nearest, ties to even multiple */
    double r = whole * quantum;
    if (r > 448.0)
        return saturate ? 0x7E : 0x7F;
    if (r == 0.0)
        return 0x00;
    if (r < ldexp(1.0, -6))
        return (int)(r / ldexp(1.0, -9));            /* subnormal mantissa */
    frexp(r, &e2);
    fl = e2 - 1;
    int mant = (int)((r / ldexp(1.0, fl) - 1.0) * 8.0);
    return ((fl + 7) << 3) | mant;
}

/* Nearest E2M1 magnitude index (0..7) of ax against the grid
 * {0, .5, 1, 1.5, 2, 3, 4, 6} * d, ties to the even index, saturating at 6d.
 * Written as the count of midpoints that ax passes: a midpoint between an
 * odd and an even index goes to the even one, so it is passed with ">" when
 * the upper neighbour is odd and with ">=" when it is even. t * d is exact
 * in binary64 (<= 3 + 28 significant bits). A zero or NaN scale gives 0. */
static int e2m1_magnitude_index(double ax, double d)
{
    if (!(d > 0.0))
        return 0;
    int m = 0;
    m += ax > 0.25 * d;   /* 0   | 0.5 -> tie to 0   */
    m += ax >= 0.75 * d;  /* 0.5 | 1   -> tie to 1   */
    m += ax > 1.25 * d;   /* 1   | 1.5 -> tie to 1   */
    m += ax >= 1.75 * d;  /* 1.5 | 2   -> tie to 2   */
    m += ax > 2.5 * d;    /* 2   | 3   -> tie to 2   */
    m += ax >= 3.5 * d;   /* 3   | 4   -> tie to 4   */
    m += ax > 5.0 * d;    /* 4   | 6   -> tie to 4   */
    return m;
}

/* ----------------------------------------------------------- quantization */

/* Largest |x| over n bf16 values (exact). */
double orc_amax(const uint16_t *x, int64_t n)
{
    double g = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double a = fabs(orc_bf16_value(x[i]));
        if (a > g)
            g = a;
    }
    return g;
}

/* Dynamic per-tensor scale S_t = RN_fp32(g / 2688), or 1 when g = 0.
 * 2688 = 6 * 448 [SPEECH]. The binary64 quotient is rounded once more to
 * binary32; that equals the correctly rounded binary32 quotient because
 * g / 2688 = g / (21 * 2^7) either terminates within 8 bits (21 | g) or has
 * a period-6 binary expansion that never runs near a binary32 midpoint
 * closer than the binary64 rounding error. */
float orc_tensor_scale(const uint16_t *x, int64_t n)
{
    double g = orc_amax(x, n);
    if (g == 0.0)
        return 1.0f;
    return (float)(g / 2688.0);
}

/* Encode one block of `bs` values with decode step d (exact), writing codes. */
static void encode_block(const uint16_t *x, int bs, double d, uint8_t *codes_nibbles)
{
    for (int i = 0; i < bs; ++i) {
        double v = orc_bf16_value(x[i]);
        int sign = signbit(v) ? 1 : 0;
        int mag = e2m1_magnitude_index(fabs(v), d);
        codes_nibbles[i] = (uint8_t)((sign << 3) | mag);
    }
}

/* Pack nibbles: byte j = code(2j) | code(2j+1) << 4. */
static void pack_row(const uint8_t *nib, int64_t k, uint8_t *out)
{
    for (int64_t j = 0; j < k / 2; ++j)
        out[j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));
}

/*
 * NVFP4 quantization of a row-major bf16 matrix x[rows][k], k % 16 == 0.
 *   mode DYNAMIC: S_t from the tensor's own maximum, block scales saturate.
 *   mode STATIC:  S_t = static_scale (> 0), block scales saturate.
 *   mode NAIVE:   S_t = 1, no saturation (block scale NaN above 464).
 * Per block of 16 along k [SPEECH, second display equation]:
 *   a_b = max|x|, s_b = RNE_E4M3(a_b / (6 S_t)), d_b = s_b * S_t,
 *   each element -> nearest code of |x| / d_b, sign kept.
 * Outputs: codes[rows][k/2], scales[rows][k/16] (E4M3 bytes), *tensor_scale.
 * Returns 0, or -1 on a bad argument.
 *
 * The quotient a_b / (6 S_t) is formed in binary64. 6 S_t is exact; if the
 * real quotient were an E4M3 rounding midpoint (<= 5 significant bits) it
 * would be exactly representable and computed exactly; otherwise its distance
 * to any midpoint is at least ~2^-32 relative (a_b has 8 significant bits,
 * midpoint * 6 S_t at most 31), far above binary64's 2^-53, so rounding the
 * binary64 quotient gives the byte of the real quotient.
 */
int orc_quantize_nvfp4(const uint16_t *x, int64_t rows, int64_t k, int mode,
                       float static_scale, uint8_t *codes, uint8_t *scales,
                       float *tensor_scale)
{
    if (k <= 0 || rows < 0 || k % 16 != 0)
        return -1;
    float st;
    if (mode == ORC_DYNAMIC)
        st = orc_tensor_scale(x, rows * k);
    else if (mode == ORC_STATIC) {
        if (!(static_scale > 0.0f) || isinf(static_scale))
            return -1;
        st = static_scale;
    } else if (mode == ORC_NAIVE)
        st = 1.0f;
    else
        return -1;
    *tensor_scale = st;
    int saturate = (mode != ORC_NAIVE);

    uint8_t *nib = (uint8_t *)malloc((size_t)k);
    if (!nib)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * k;
        for (int64_t b = 0; b < k / 16; ++b) {
            double ab = orc_amax(xr + b * 16, 16);
            double quotient = ab / (6.0 * (double)st);
            int sbyte = orc_e4m3_from_real(quotient, saturate);
            scales[r * (k / 16) + b] = (uint8_t)sbyte;
            double d = orc_e4m3_value(sbyte) * (double)st;   /* exact */
            encode_block(xr + b * 16, 16, d, nib + b * 16);
        }
        pack_row(nib, k, codes + r * (k / 2));
    }
    free(nib);
    return 0;
}

/* MXFP4 block exponent for block maximum ab (reading stated in the header). */
int orc_mx_exponent(double ab)
{
    if (ab == 0.0)
        return -127;
    int e2;
    frexp(ab, &e2);                /* floor(log2 ab) = e2 - 1 */
    int e = (e2 - 1) - 2;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

/* OAS block exponent [DIALECT, quality-gap section]: the smallest e with
 * ab <= 6 * 2^e, clamped to [-127, 127]. The default exponent leaves
 * ab / 2^e in [4, 8); when that quotient exceeds 6 one more step brings it
 * into (3, 4). 6 * 2^e is exact, so the comparison is exact. */
int orc_mx_exponent_oas(double ab)
{
    int e = orc_mx_exponent(ab);
    if (ab > 6.0 * ldexp(1.0, e) && e < 127)
        e += 1;
    return e;
}

/*
 * MXFP4 quantization [DIALECT]: blocks of 32 along k share one E8M0 scale
 * 2^e_b; elements are the nearest E2M1 codes of |x| / 2^e_b (same rounding
 * as NVFP4). Outputs codes[rows][k/2], scales[rows][k/32] (byte e_b + 127).
 * oas != 0 takes the overflow-aware exponent instead of the default one.
 */
int orc_quantize_mxfp4_rule(const uint16_t *x, int64_t rows, int64_t k, int oas,
                            uint8_t *codes, uint8_t *scales)
{
    if (k <= 0 || rows < 0 || k % 32 != 0)
        return -1;
    uint8_t *nib = (uint8_t *)malloc((size_t)k);
    if (!nib)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * k;
        for (int64_t b = 0; b < k / 32; ++b) {
            double ab = orc_amax(xr + b * 32, 32);
            int e = oas ? orc_mx_exponent_oas(ab) : orc_mx_exponent(ab);
            scales[r * (k / 32) + b] = (uint8_t)(e + 127);
            encode_block(xr + b * 32, 32, ldexp(1.0, e), nib + b * 32);
        }
        pack_row(nib, k, codes + r * (k / 2));
    }
    free(nib);
    return 0;
}

int orc_quantize_mxfp4(const uint16_t *x, int64_t rows, int64_t k,
                       uint8_t *codes, uint8_t *scales)
{
    return orc_quantize_mxfp4_rule(x, rows, k, 0, codes, scales);
}

/* Macro-block scale of a segment whose largest magnitude is g (reading in the
 * header). g / 6 in binary64 never rounds across a power of two (g has 8
 * significant bits, so g < 6 * 2^j implies g <= 6 * 2^j (1 - 2^-8)), and
 * g / 6 = g / (3 * 2) has a period-2 binary expansion (or terminates), so
 * its binary64 value never lies on a binary32 rounding midpoint it was not
 * already on: rounding it to binary32 equals rounding the real quotient. */
float orc_mbs_scale(double g)
{
    if (g == 0.0)
        return 1.0f;
    double q = g / 6.0;
    int e2;
    frexp(q, &e2);                     /* floor(log2 q) = e2 - 1 */
    return (float)ldexp(q, -(e2 - 1));
}

/* MX block exponent of a_b / s for s in [1, 2), exactly: floor(log2(a_b / s))
 * is floor(log2 a_b) or one less, decided by a_b >= s * 2^floor(log2 a_b)
 * (an exact binary64 product). OAS: one more step while a_b > 6 * 2^e * s. */
int orc_mbs_exponent(double ab, float s, int oas)
{
    if (ab == 0.0)
        return -127;
    int e2;
    frexp(ab, &e2);
    int fl = e2 - 1;
    if (ab < (double)s * ldexp(1.0, fl))
        fl -= 1;
    int e = fl - 2;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    if (oas && ab > 6.0 * ldexp(1.0, e) * (double)s && e < 127)
        e += 1;
    return e;
}

/*
 * MXFP4 with macro-block scaling (reading in the header): codes [rows][k/2],
 * E8M0 bytes [rows][k/32] as for MXFP4, and the FP32 macro-block scales
 * mscales [rows][ceil(k/128)]. Elements are the nearest E2M1 codes of
 * |x| / d_b with d_b = 2^e_b * S_mb (exact in binary64), ties to even.
 */
int orc_quantize_mxfp4_mbs(const uint16_t *x, int64_t rows, int64_t k, int oas,
                           uint8_t *codes, uint8_t *scales, float *mscales)
{
    if (k <= 0 || rows < 0 || k % 32 != 0)
        return -1;
    int64_t nseg = (k + 127) / 128;
    uint8_t *nib = (uint8_t *)malloc((size_t)k);
    if (!nib)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * k;
        for (int64_t sgi = 0; sgi < nseg; ++sgi) {
            int64_t k0 = sgi * 128, k1 = k0 + 128 < k ? k0 + 128 : k;
            float smb = orc_mbs_scale(orc_amax(xr + k0, k1 - k0));
            mscales[r * nseg + sgi] = smb;
            for (int64_t b = k0 / 32; b < k1 / 32; ++b) {
                int e = orc_mbs_exponent(orc_amax(xr + b * 32, 32), smb, oas);
                scales[r * (k / 32) + b] = (uint8_t)(e + 127);
                encode_block(xr + b * 32, 32, ldexp(1.0, e) * (double)smb, nib + b * 32);
            }
        }
        pack_row(nib, k, codes + r * (k / 2));
    }
    free(nib);
    return 0;
}

/* --------------------------------------------------------------- rotation */

/* RN_fp32(1/sqrt(bs)): exactly 0.25 for 16; for 32 the binary64 value of
 * 1/sqrt(32) is rounded to binary32 (a test checks it is the binary32 value
 * nearest to the real 1/sqrt(32)). */
float orc_hadamard_norm(int bs)
{
    return bs == 16 ? 0.25f : (float)(1.0 / sqrt((double)bs));
}

/*
 * Exact rotation sums. A finite bf16 value is an integer multiple of 2^-133
 * (its smallest subnormal): |x| = N * 2^-133 with N < 2^261. A row of H_bs
 * applied to a block is a signed sum of at most 32 such integers (< 2^266),
 * and multiplying by the 24-bit significand of RN_fp32(1/sqrt(bs)) stays
 * below 2^290. Those integers are held here as little-endian arrays of
 * 32-bit words, wide enough for 320 bits.
 */
#define ROT_WORDS 10

typedef struct { uint32_t w[ROT_WORDS]; } rot_int;

/* a += m * 2^shift (m < 2^9, shift <= 253). */
static void rot_add(rot_int *a, uint32_t m, int shift)
{
    int i = shift / 32;
    uint64_t carry = (uint64_t)m << (shift % 32);
    while (carry != 0 && i < ROT_WORDS) {
        uint64_t t = (uint64_t)a->w[i] + (carry & 0xFFFFFFFFu);
        a->w[i] = (uint32_t)t;
        carry = (carry >> 32) + (t >> 32);
        ++i;
    }
}

/* -1, 0, +1 as a <, =, > b. */
static int rot_cmp(const rot_int *a, const rot_int *b)
{
    for (int i = ROT_WORDS - 1; i >= 0; --i)
        if (a->w[i] != b->w[i])
            return a->w[i] < b->w[i] ? -1 : 1;
    return 0;
}

/* a -= b, given a >= b. */
static void rot_sub(rot_int *a, const rot_int *b)
{
    uint64_t borrow = 0;
    for (int i = 0; i < ROT_WORDS; ++i) {
        uint64_t t = (uint64_t)a->w[i] - b->w[i] - borrow;
        a->w[i] = (uint32_t)t;
        borrow = (t >> 63) & 1u;
    }
}

/* a *= c (c < 2^24). */
static void rot_mul(rot_int *a, uint32_t c)
{
    uint64_t carry = 0;
    for (int i = 0; i < ROT_WORDS; ++i) {
        uint64_t t = (uint64_t)a->w[i] * c + carry;
        a->w[i] = (uint32_t)t;
        carry = t >> 32;
    }
}

static int rot_bit(const rot_int *a, int i)
{
    return i < 0 ? 0 : (int)((a->w[i / 32] >> (i % 32)) & 1u);
}

/* Number of significant bits (0 for zero). */
static int rot_bitlen(const rot_int *a)
{
    for (int i = ROT_WORDS - 1; i >= 0; --i)
        if (a->w[i])
            for (int b = 31; b >= 0; --b)
                if ((a->w[i] >> b) & 1u)
                    return 32 * i + b + 1;
    return 0;
}

/* bf16 bits of (-1)^neg * a * 2^scale_exp rounded to nearest, ties to even
 * (a > 0; the result is finite for the inputs accepted below). bf16 keeps 8
 * significant bits down to 2^-126 and a fixed quantum of 2^-133 below. */
static uint16_t rot_round_bf16(const rot_int *a, int scale_exp, int neg)
{
    int len = rot_bitlen(a);
    int top = len - 1 + scale_exp;                 /* floor(log2 |value|) */
    int q = top - 7 > -133 ? top - 7 : -133;       /* exponent of the bf16 quantum */
    int drop = q - scale_exp;                      /* bits of a below the quantum */
    uint32_t r = 0;
    for (int i = 8; i >= 0; --i)                   /* a >> drop has at most 9 bits */
        r = (r << 1) | (uint32_t)rot_bit(a, drop + i);
    int half = rot_bit(a, drop - 1), sticky = 0;
    for (int i = drop - 2; i >= 0 && !sticky; --i)
        sticky = rot_bit(a, i);
    if (half && (sticky || (r & 1u)))
        r += 1;                                    /* may carry into the next binade */
    float f = ldexpf((float)r, q);                 /* exact: r <= 256 */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)((u >> 16) | (neg ? 0x8000u : 0u));
}

static int popcount_parity(int v)
{
    int p = 0;
    for (; v; v >>= 1)
        p ^= v & 1;
    return p;
}

/*
 * Rotation reading in the header [REALFP4]: within each block of bs values
 * along k, out[i] = RN_bf16( c * sum_j H[i][j] x[j] ) with
 * H[i][j] = (-1)^popcount(i & j) (Sylvester order) and c = RN_fp32(1/sqrt(bs)):
 * the sum and the product are exact and the bf16 rounding (nearest, ties to
 * even) is the only one, so the result does not depend on the order in which
 * a transform adds. An exact zero sum gives +0. bs is 16 or 32, k a multiple
 * of bs, inputs finite with |x| < 2^120. Returns 0, or -1 on a bad argument.
 */
int orc_hadamard_bf16(const uint16_t *x, int64_t rows, int64_t k, int bs, uint16_t *out)
{
    if ((bs != 16 && bs != 32) || k <= 0 || rows < 0 || k % bs != 0)
        return -1;
    /* c = C * 2^(ce - 24) with C the 24-bit integer significand */
    int ce;
    double cf = frexp((double)orc_hadamard_norm(bs), &ce);
    uint32_t cint = (uint32_t)ldexp(cf, 24);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < k / bs; ++b) {
            const uint16_t *xb = x + r * k + b * bs;
            for (int i = 0; i < bs; ++i) {
                rot_int pos, neg;
                memset(&pos, 0, sizeof pos);
                memset(&neg, 0, sizeof neg);
                for (int j = 0; j < bs; ++j) {
                    uint32_t bits = xb[j], e = (bits >> 7) & 0xFFu, m = bits & 0x7Fu;
                    if (e == 0 && m == 0)
                        continue;                  /* +-0 */
                    /* |x| = N * 2^-133: N = m (subnormal) or (128 + m) << (e - 1) */
                    uint32_t sig = e ? (128u | m) : m;
                    int shift = e ? (int)e - 1 : 0;
                    int negative = (int)(bits >> 15) ^ popcount_parity(i & j);
                    rot_add(negative ? &neg : &pos, sig, shift);
                }
                int c = rot_cmp(&pos, &neg);
                uint16_t y = 0;
                if (c > 0) {
                    rot_sub(&pos, &neg);
                    rot_mul(&pos, cint);
                    y = rot_round_bf16(&pos, -133 + ce - 24, 0);
                } else if (c < 0) {
                    rot_sub(&neg, &pos);
                    rot_mul(&neg, cint);
                    y = rot_round_bf16(&neg, -133 + ce - 24, 1);
                }
                out[r * k + b * bs + i] = y;
            }
        }
    return 0;
}

/* --------------------------------------------------------- dequantization */

/* One dequantized element without the per-tensor factor: v(code) * s_b, times
 * the macro-block scale S_mb when the row has them (macro_row != NULL;
 * MXFP4 with MBS). Exact in binary64 (2 + 1 + 24 significant bits at most). */
static double element_value(int fmt, const uint8_t *codes_row, const uint8_t *scales_row,
                            const float *macro_row, int64_t kk)
{
    int byte = codes_row[kk / 2];
    int code = (kk % 2 == 0) ? (byte & 15) : (byte >> 4);
    double q = orc_e2m1_value(code);
    double s = (fmt == ORC_NVFP4) ? orc_e4m3_value(scales_row[kk / 16])
                                  : orc_e8m0_value(scales_row[kk / 32]);
    if (macro_row)
        s *= (double)macro_row[kk / 128];
    return q * s;
}

/* x^ = q * s_b * S_t (NVFP4), q * 2^e_b (MXFP4) or q * 2^e_b * S_mb (MXFP4
 * with MBS: mscales [rows][ceil(k/128)], else NULL), exact in binary64.
 * out[rows][k]. tensor_scale is ignored for MXFP4. */
void orc_dequantize_ms(int fmt, const uint8_t *codes, const uint8_t *scales,
                       const float *mscales, float tensor_scale, int64_t rows, int64_t k,
                       double *out)
{
    int64_t bs = (fmt == ORC_NVFP4) ? 16 : 32, nseg = (k + 127) / 128;
    double st = (fmt == ORC_NVFP4) ? (double)tensor_scale : 1.0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t kk = 0; kk < k; ++kk)
            out[r * k + kk] = element_value(fmt, codes + r * (k / 2), scales + r * (k / bs),
                                            mscales ? mscales + r * nseg : NULL, kk) * st;
}

void orc_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales,
                    float tensor_scale, int64_t rows, int64_t k, double *out)
{
    orc_dequantize_ms(fmt, codes, scales, NULL, tensor_scale, rows, k, out);
}

/* ------------------------------------------------------------------- GEMM */

/*
 * C[m][n] = alpha * sum_k a'[m][k] * w'[n][k], with a' = q * s_b (per-tensor
 * factors pulled out into alpha = S_tA * S_tW for NVFP4, alpha = 1 for MXFP4),
 * i.e. C = A^ W^T in the orientation of a linear layer. Binary64, summed in
 * increasing k. L[m][n] = alpha * sum_k |a' w'| is the magnitude bound the
 * tolerance is stated against. Either output pointer may be NULL.
 */
static void gemm_entry(int fmt, const uint8_t *a_codes, const uint8_t *a_scales,
                       const float *a_ms, const uint8_t *w_codes, const uint8_t *w_scales,
                       const float *w_ms, int64_t k, int64_t m, int64_t n, double alpha,
                       double *c_out, double *l_out)
{
    int64_t bs = (fmt == ORC_NVFP4) ? 16 : 32, nseg = (k + 127) / 128;
    const uint8_t *ac = a_codes + m * (k / 2), *as = a_scales + m * (k / bs);
    const uint8_t *wc = w_codes + n * (k / 2), *ws = w_scales + n * (k / bs);
    const float *am = a_ms ? a_ms + m * nseg : NULL, *wm = w_ms ? w_ms + n * nseg : NULL;
    double acc = 0.0, mag = 0.0;
    for (int64_t kk = 0; kk < k; ++kk) {
        double p = element_value(fmt, ac, as, am, kk) * element_value(fmt, wc, ws, wm, kk);
        acc += p;
        mag += fabs(p);
    }
    if (c_out)
        *c_out = alpha * acc;
    if (l_out)
        *l_out = alpha * mag;
}

static double gemm_alpha(int fmt, float a_ts, float w_ts)
{
    return (fmt == ORC_NVFP4) ? (double)a_ts * (double)w_ts : 1.0;
}

/* Full GEMM: c[M][N], l[M][N]; a_ms / w_ms are the operands' macro-block
 * scales (MXFP4 with MBS) or NULL. */
void orc_gemm_ms(int fmt, const uint8_t *a_codes, const uint8_t *a_scales, const float *a_ms,
                 float a_ts, const uint8_t *w_codes, const uint8_t *w_scales, const float *w_ms,
                 float w_ts, int64_t M, int64_t N, int64_t K, double *c, double *l)
{
    double alpha = gemm_alpha(fmt, a_ts, w_ts);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            gemm_entry(fmt, a_codes, a_scales, a_ms, w_codes, w_scales, w_ms, K, m, n, alpha,
                       c ? c + m * N + n : NULL, l ? l + m * N + n : NULL);
}

void orc_gemm(int fmt, const uint8_t *a_codes, const uint8_t *a_scales, float a_ts,
              const uint8_t *w_codes, const uint8_t *w_scales, float w_ts,
              int64_t M, int64_t N, int64_t K, double *c, double *l)
{
    orc_gemm_ms(fmt, a_codes, a_scales, NULL, a_ts, w_codes, w_scales, NULL, w_ts, M, N, K, c, l);
}

/* Sampled GEMM: entries (rows[i], cols[i]) for i < count. */
void orc_gemm_sampled_ms(int fmt, const uint8_t *a_codes, const uint8_t *a_scales,
                         const float *a_ms, float a_ts, const uint8_t *w_codes,
                         const uint8_t *w_scales, const float *w_ms, float w_ts, int64_t K,
                         const int64_t *rows, const int64_t *cols, int64_t count,
                         double *c, double *l)
{
    double alpha = gemm_alpha(fmt, a_ts, w_ts);
    for (int64_t i = 0; i < count; ++i)
        gemm_entry(fmt, a_codes, a_scales, a_ms, w_codes, w_scales, w_ms, K, rows[i], cols[i],
                   alpha, c ? c + i : NULL, l ? l + i : NULL);
}

void orc_gemm_sampled(int fmt, const uint8_t *a_codes, const uint8_t *a_scales, float a_ts,
                      const uint8_t *w_codes, const uint8_t *w_scales, float w_ts,
                      int64_t K, const int64_t *rows, const int64_t *cols, int64_t count,
                      double *c, double *l)
{
    orc_gemm_sampled_ms(fmt, a_codes, a_scales, NULL, a_ts, w_codes, w_scales, NULL, w_ts, K,
                        rows, cols, count, c, l);
}

/*
 * Weight-only variant (W4A16): the activations stay bf16 and only the cached
 * weight is quantized [SPEECH, section "Weights are safe" (the W4A16
 * checkpoint) and section "Two Triton kernels for the SM120 gaps" (a W4A16
 * GEMM of bf16 activations with pre-packed FP4 weights)].
 * C[m][n] = S_tW * sum_k x[m][k] * (q * s_b)[n][k] (S_tW = 1 for MXFP4),
 * binary64, increasing k; L the same sum of magnitudes. x is bf16 [M][K],
 * the weight canonical (codes [N][K/2], scales [N][K/B]).
 */
static void gemm_w4a16_entry(int fmt, const uint16_t *x, const uint8_t *w_codes,
                             const uint8_t *w_scales, int64_t k, int64_t m, int64_t n,
                             double alpha, double *c_out, double *l_out)
{
    int64_t bs = (fmt == ORC_NVFP4) ? 16 : 32;
    const uint16_t *xr = x + m * k;
    const uint8_t *wc = w_codes + n * (k / 2), *ws = w_scales + n * (k / bs);
    double acc = 0.0, mag = 0.0;
    for (int64_t kk = 0; kk < k; ++kk) {
        double p = orc_bf16_value(xr[kk]) * element_value(fmt, wc, ws, NULL, kk);
        acc += p;
        mag += fabs(p);
    }
    if (c_out)
        *c_out = alpha * acc;
    if (l_out)
        *l_out = alpha * mag;
}

void orc_gemm_w4a16(int fmt, const uint16_t *x, const uint8_t *w_codes,
                    const uint8_t *w_scales, float w_ts, int64_t M, int64_t N, int64_t K,
                    double *c, double *l)
{
    double alpha = (fmt == ORC_NVFP4) ? (double)w_ts : 1.0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            gemm_w4a16_entry(fmt, x, w_codes, w_scales, K, m, n, alpha,
                             c ? c + m * N + n : NULL, l ? l + m * N + n : NULL);
}

void orc_gemm_w4a16_sampled(int fmt, const uint16_t *x, const uint8_t *w_codes,
                            const uint8_t *w_scales, float w_ts, int64_t K,
                            const int64_t *rows, const int64_t *cols, int64_t count,
                            double *c, double *l)
{
    double alpha = (fmt == ORC_NVFP4) ? (double)w_ts : 1.0;
    for (int64_t i = 0; i < count; ++i)
        gemm_w4a16_entry(fmt, x, w_codes, w_scales, K, rows[i], cols[i], alpha,
                         c ? c + i : NULL, l ? l + i : NULL);
}

/* Vector helper for the pins: RNE to E4M3 of n reals. */
void orc_e4m3_from_real_array(const double *v, int64_t n, int saturate, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)orc_e4m3_from_real(v[i], saturate);
}
