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
// Quantize scratch: kMaxAmaxParts partial maxima, then the single-launch
// quantizer's kActGrid tagged maximum words, one per 128-byte line
// (zero-filled once).
constexpr int kSlotStride = 32;
constexpr size_t kQuantScratchBytes = (kMaxAmaxParts + kActGrid * kSlotStride) * sizeof(uint32_t);

// Number of partial maxima the large-tensor path produces for n elements.
int amax_parts(int64_t n);
// Whether a [rows, k] tensor takes the single-launch path.
bool quant_fits_small(int fmt, int64_t rows, int64_t k, int tiled);

// ---- launchers (all asynchronous on `stream`) ----

// Quantization recipe bits: rotate every block (block Hadamard) before it is
// quantized; MXFP4 overflow-aware block exponent.
constexpr uint32_t kRecipeRotate = 1u;
constexpr uint32_t kRecipeOas = 2u;

// Quantize x [rows, k] (bf16, row-major) into the canonical (tiled = 0) or
// fragment-tiled (tiled = 1) layout; fmt 0 = NVFP4, 1 = MXFP4. NVFP4 takes S_t
// from *static_scale when non-null, else from the tensor's maximum (of the
// rotated values when rotating); writes *ts_out when non-null. `scratch` holds
// kQuantScratchBytes.
hipError_t launch_quantize(int fmt, uint32_t recipe, int tiled, const uint16_t *x, int64_t rows,
                           int64_t k, const float *static_scale, uint8_t *codes, int64_t cpitch,
                           uint8_t *scales, int64_t spitch, float *ts_out, uint32_t *scratch,
                           hipStream_t stream);

hipError_t launch_export_canonical(int fmt, const uint8_t *tcodes, const uint8_t *tscales,
                                   int64_t rows, int64_t k, uint8_t *codes, int64_t cpitch,
                                   uint8_t *scales, int64_t spitch, const float *ts_in,
                                   float *ts_out, hipStream_t stream);

hipError_t launch_dequant(int fmt, int tiled, const uint8_t *codes, int64_t cpitch,
                          const uint8_t *scales, int64_t spitch, const float *ts, int64_t rows,
                          int64_t k, float *out, int64_t ldo, hipStream_t stream);

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
};

hipError_t launch_gemm_prefill(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_decode(const GemmArgs &g, hipStream_t stream);

// LDS-staged GEMM for large M; both operands fragment-tiled. cfg selects the
// workgroup tile (88: 256 x 256, 44: 128 x 128; 0: by shape).
int gemm_tile_config(int fmt, int64_t m, int64_t n);
hipError_t launch_gemm_tile(const GemmArgs &g, int cfg, hipStream_t stream);

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
