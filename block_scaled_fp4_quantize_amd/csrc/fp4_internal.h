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
constexpr int kDecodeMaxM = 32;      // M up to which the skinny (decode) GEMM is used

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t k_pad(int64_t k) { return round_up(k, kFragK); }
inline int block_of(int fmt) { return fmt == 0 ? 16 : 32; }
inline int frag_scale_bytes(int fmt) { return fmt == 0 ? 128 : 64; }

// Number of partial maxima the amax kernel produces for n elements.
int amax_parts(int64_t n);

// Split-K plan of the skinny GEMM (identical in workspace sizing and launch).
struct DecodePlan {
  int mg;        // 16-row groups of A (1 or 2)
  int splits;    // K splits across workgroups
  int frags;     // fragments per wave
  int kt_per_wg; // fragments per workgroup (4 waves)
};
DecodePlan decode_plan(int fmt, int64_t m, int64_t n, int64_t k);
size_t decode_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k);

// ---- launchers (all asynchronous on `stream`) ----
hipError_t launch_amax_parts(const uint16_t *x, int64_t n, uint32_t *parts, int nparts,
                             hipStream_t stream);

// Quantize rows of x [rows, k] (bf16) into the canonical layout (fmt 0 = NVFP4,
// 1 = MXFP4). NVFP4 takes S_t from `static_scale` when non-null, else from the
// `nparts` partial maxima. Writes *ts_out (NVFP4) and zeroes `zero_n` ints at
// `zero_ptr` (split-K counters of a following GEMM) when zero_n > 0.
hipError_t launch_quant_canonical(int fmt, const uint16_t *x, int64_t rows, int64_t k,
                                  const uint32_t *parts, int nparts, const float *static_scale,
                                  uint8_t *codes, int64_t cpitch, uint8_t *scales,
                                  int64_t spitch, float *ts_out, int *zero_ptr, int zero_n,
                                  hipStream_t stream);

// Quantize a weight [n, k] into the fragment-tiled layout (dynamic S_t for NVFP4).
hipError_t launch_quant_tiled(int fmt, const uint16_t *w, int64_t n, int64_t k,
                              const uint32_t *parts, int nparts, uint8_t *codes,
                              uint8_t *scales, float *ts_out, hipStream_t stream);

hipError_t launch_export_canonical(int fmt, const uint8_t *tcodes, const uint8_t *tscales,
                                   int64_t rows, int64_t k, uint8_t *codes, int64_t cpitch,
                                   uint8_t *scales, int64_t spitch, const float *ts_in,
                                   float *ts_out, hipStream_t stream);

hipError_t launch_dequant(int fmt, int tiled, const uint8_t *codes, int64_t cpitch,
                          const uint8_t *scales, int64_t spitch, const float *ts, int64_t rows,
                          int64_t k, float *out, int64_t ldo, hipStream_t stream);

hipError_t launch_zero_ints(int *p, int n, hipStream_t stream);

struct GemmArgs {
  int fmt;
  const uint8_t *a_codes; int64_t a_cpitch;
  const uint8_t *a_scales; int64_t a_spitch;
  const float *a_ts;
  const uint8_t *w_codes; const uint8_t *w_scales;
  const float *w_ts;
  int64_t m, n, k;
  uint16_t *c; int64_t ldc;
};

hipError_t launch_gemm_prefill(const GemmArgs &g, hipStream_t stream);
// Skinny GEMM; `partials`/`counters` may be null when the plan has splits == 1.
hipError_t launch_gemm_decode(const GemmArgs &g, const DecodePlan &plan, float *partials,
                              int *counters, hipStream_t stream);

}  // namespace fp4i
