// fp4_internal.h -- declarations shared by the library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace fp4i {

constexpr int kFragK = 128;          // K values per fragment (one scaled-MFMA K step)
constexpr int kFragRows = 16;        // rows per fragment
constexpr int kFragCodeBytes = 1024; // 16 rows x 128 values x 4 bits
constexpr int kMaxAmaxParts = 1024;  // partial maxima of the per-tensor reduction
constexpr int kDecodeMaxM = 128;     // M up to which the skinny (decode) GEMM is used
constexpr int kW16DecodeMaxM = 32;   // the same for the weight-only (W4A16) linear

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t k_pad(int64_t k) { return round_up(k, kFragK); }
inline int block_of(int fmt) { return fmt == 0 ? 16 : 32; }
inline int frag_scale_bytes(int fmt) { return fmt == 0 ? 128 : 64; }

constexpr int kActGrid = 128;         // workgroups of the single-launch quantizer
constexpr int kActBpt = 4;            // single-launch quantizer capacity: kActGrid * 256 * kActBpt blocks
constexpr int64_t kActRedundantMaxValues = 49152;  // M * K up to which each workgroup finds the maximum alone
// Quantize scratch (32-bit words, zero-filled once): kMaxAmaxParts partial
// maxima; the single-launch quantizer's kActGrid tagged maximum words, one per
// 128-byte line; a line holding the sticky error flags; a line holding the
// exchange's arrival count (reset by the last workgroup of every call).
constexpr int kSlotStride = 32;
constexpr int kErrWord = kMaxAmaxParts + kActGrid * kSlotStride;
constexpr int kArriveWord = kErrWord + kSlotStride;
// The fused large-M linear's per-panel words: (ready count, finished count)
// for each row panel of output tiles, reset by the panel's last consumer.
constexpr int kPanelWords = kArriveWord + kSlotStride;
constexpr int kMaxPanels = 1024;
// The one-pass quantizer of mid-size NVFP4 tensors (dynamic scale, tiled
// layout): at most kMidGrid workgroups of kMidThreads threads, each wave
// holding up to kMidFragsPerWave fragments, exchange their maxima through
// kMidGrid tagged words of their own (one 128-byte line each).
constexpr int kMidGrid = 256;
constexpr int kMidThreads = 1024;
constexpr int kMidFragsPerWave = 4;
constexpr int kMidSlotWord = kPanelWords + 2 * kMaxPanels;
constexpr size_t kQuantScratchBytes = (size_t)(kMidSlotWord + kMidGrid * kSlotStride) * sizeof(uint32_t);
// Error flag: a workgroup of the maximum exchange gave up waiting.
constexpr uint32_t kErrExchangeTimeout = 1u;
constexpr uint32_t kDefaultSpinLimit = 1u << 22;
// Polls of the maximum exchange before a workgroup gives up (test hook).
uint32_t exchange_spin_limit();
uint32_t set_exchange_spin_limit(uint32_t polls);

// Number of partial maxima the large-tensor path produces for n elements.
int amax_parts(int64_t n);
// Whether a [rows, k] tensor takes the single-launch path.
bool quant_fits_small(int fmt, int64_t rows, int64_t k, int tiled);
// Whether NVFP4 with the dynamic scale (recipe bits in `recipe`) takes the
// one-pass mid-size path (one launch instead of maxima + encode).
bool quant_fits_mid(int fmt, uint32_t recipe, int64_t rows, int64_t k, int tiled);

// ---- launchers (all asynchronous on `stream`) ----

// Quantization recipe bits: rotate every block (block Hadamard) before it is
// quantized; MXFP4 overflow-aware block exponent.
constexpr uint32_t kRecipeRotate = 1u;
constexpr uint32_t kRecipeOas = 2u;
constexpr uint32_t kRecipeMbs = 4u;   // MXFP4 macro-block scales (one FP32 per 128-value segment)

// Quantize x [rows, k] (bf16, row-major) into the canonical (tiled = 0) or
// fragment-tiled (tiled = 1) layout; fmt 0 = NVFP4, 1 = MXFP4. NVFP4 takes S_t
// from *static_scale when non-null, else from the tensor's maximum (of the
// rotated values when rotating); writes *ts_out when non-null. `scratch` holds
// kQuantScratchBytes. MXFP4 with kRecipeMbs writes the macro-block scales to
// `macro`: canonical [rows][mpitch] floats, tiled [fragment][16 rows] floats.
hipError_t launch_quantize(int fmt, uint32_t recipe, int tiled, const uint16_t *x, int64_t rows,
                           int64_t k, const float *static_scale, uint8_t *codes, int64_t cpitch,
                           uint8_t *scales, int64_t spitch, float *macro, int64_t mpitch,
                           float *ts_out, uint32_t *scratch, hipStream_t stream);

// Macro-block scale arrays (MBS) travel with the codes in the export, import
// and dequantization: tiled [fragment][16] floats, canonical [rows][mpitch]
// floats; nullptr without MBS.
hipError_t launch_export_canonical(int fmt, const uint8_t *tcodes, const uint8_t *tscales,
                                   const float *tmacro, int64_t rows, int64_t k, uint8_t *codes,
                                   int64_t cpitch, uint8_t *scales, int64_t spitch, float *macro,
                                   int64_t mpitch, const float *ts_in, float *ts_out,
                                   hipStream_t stream);

// Canonical [rows, k] codes/scales -> the fragment-tiled layout (rows padded
// to 16, zero padding).
hipError_t launch_import_tiled(int fmt, const uint8_t *codes, int64_t cpitch, const uint8_t *scales,
                              int64_t spitch, const float *macro, int64_t mpitch, int64_t rows,
                              int64_t k, uint8_t *tcodes, uint8_t *tscales, float *tmacro,
                              hipStream_t stream);

hipError_t launch_dequant(int fmt, int tiled, const uint8_t *codes, int64_t cpitch,
                          const uint8_t *scales, int64_t spitch, const float *macro,
                          int64_t mpitch, const float *ts, int64_t rows, int64_t k, float *out,
                          int64_t ldo, hipStream_t stream);

struct GemmArgs {
  int fmt;
  int a_tiled;
  const uint8_t *a_codes; int64_t a_cpitch;
  const uint8_t *a_scales; int64_t a_spitch;
  const float *a_ts;
  const uint8_t *w_codes; const uint8_t *w_scales;
  const float *w_ts;
  int64_t m, n, k;
  uint16_t *c; int64_t ldc;
  // MXFP4 macro-block scales (both operands, or neither): A tiled
  // [fragment][16] or canonical [m][a_mpitch] floats, W tiled [fragment][16]
  const float *a_ms = nullptr; int64_t a_mpitch = 0;
  const float *w_ms = nullptr;
};

hipError_t launch_gemm_prefill(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_decode(const GemmArgs &g, hipStream_t stream);

// GEMM for 33-128 activation rows with tiled activations and no macro-block
// scales: four weight tiles per workgroup, K split into `splits` slices whose
// FP32 partial sums go to `part` (splits * m * n floats, unused when splits
// is 1) and are added in slice order by a second launch.
// gemm_mid_splits: the slice count for a shape (0: the kernel does not apply),
// with at most `cap` bytes of partial sums. mid_gemm: whether the GEMM
// launches use it (1, the default) or the skinny kernel (0).
int gemm_mid_splits(int64_t m, int64_t n, int64_t k, int64_t cap);
hipError_t launch_gemm_mid(const GemmArgs &g, int splits, float *part, hipStream_t stream);
int mid_gemm();
int set_mid_gemm(int on);

// LDS-staged GEMM for large M; both operands fragment-tiled. cfg selects the
// workgroup tile (88: 256 x 256, 44: 128 x 128; 0: by shape).
int gemm_tile_config(int fmt, int64_t m, int64_t n);
// NVFP4 256 x 256 tiles: 0 = conversion in registers by each wave that uses a
// fragment, 1 = conversion once per workgroup into LDS (k_gemm_tile_nvlds).
int nvfp4_tile_mode();
int set_nvfp4_tile_mode(int mode);
hipError_t launch_gemm_tile(const GemmArgs &g, int cfg, hipStream_t stream);

// Single-launch linear for large M (NVFP4 with a static tensor scale, or
// MXFP4 without macro-block scales): the first workgroups quantize the bf16
// activations x [m, k] into the tiled layout at g.a_codes / g.a_scales (each
// row panel of output tiles split along K among several of them), the others
// compute the output tiles, each waiting (bounded) for its panel. `scratch` is
// the quantize scratch (kQuantScratchBytes, zero-filled once): its panel words
// and error flags. Whether it applies: linear_fused_large_ok.
bool linear_fused_large_ok(int fmt, uint32_t recipe, int64_t m, int64_t n, int64_t k,
                           bool static_scale);
// Whether fp4_linear uses it when it applies (1) or quantizes in a separate
// launch (0, the default).
int large_linear_fusion();
int set_large_linear_fusion(int on);
hipError_t launch_linear_fused_large(const GemmArgs &g, const uint16_t *x,
                                     const float *static_scale, uint32_t recipe,
                                     uint32_t *scratch, hipStream_t stream);

// Single-launch linear for 1-32 activation rows (no macro-block scales): the
// skinny GEMM's launch, whose first workgroups quantize x [m, k] into the
// tiled layout at g.a_codes / g.a_scales while the GEMM workgroups issue their
// first weight loads and wait (bounded) for them. g.a_ts: the static NVFP4
// scale, or the word the dynamic S_t is written to. `scratch`: the quantize
// scratch (kQuantScratchBytes, zero-filled once). Whether fp4_linear uses it
// (where k_linear_decode does not apply): decode_linear_fusion() (0, the
// default: quantize + GEMM measured faster).
bool linear_fused_decode_ok(int fmt, uint32_t recipe, int64_t m, int64_t n, int64_t k);
int decode_linear_fusion();
int set_decode_linear_fusion(int on);
hipError_t launch_linear_fused_decode(const GemmArgs &g, const uint16_t *x,
                                      const float *static_scale, uint32_t recipe,
                                      uint32_t *scratch, hipStream_t stream);

// Single-launch linear (activation quantization fused) for small activations.
constexpr int kFusedMaxM = 16;
constexpr int64_t kFusedMaxMK = 65536;        // M * K_pad bound (LDS staging, MXFP4)
constexpr int64_t kFusedMaxWork = 16 << 20;   // M * K_pad * N tiles bound
constexpr int64_t kFusedMaxWorkNv = 4 << 20;  // NVFP4: M * K_pad * N tiles bound
constexpr int64_t kFusedMaxTilesNv = 512;      // NVFP4: at most this many weight tiles
bool linear_fused_ok(int fmt, int64_t m, int64_t n, int64_t k);
hipError_t launch_linear_fused(int fmt, uint32_t recipe, const uint16_t *x, int64_t m, int64_t k,
                               const float *static_scale, const uint8_t *w_codes,
                               const uint8_t *w_scales, const float *w_ts, int64_t n,
                               uint16_t *y, int64_t ldy, hipStream_t stream);

// Weight-only linear (W4A16): y[m, n] = S_tW * x[m, :] . (q s_b)[n, :], x bf16
// with row pitch ldx elements (a multiple of 8), the weight in the tiled cache.
hipError_t launch_linear_w4a16(int fmt, const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_ts,
                               int64_t n, uint16_t *y, int64_t ldy, hipStream_t stream);

}  // namespace fp4i
