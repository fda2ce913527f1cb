// quant.hip -- activation and weight quantization kernels for gfx950.
//
// NVFP4 (16-value blocks, E4M3 block scale, FP32 per-tensor scale) and MXFP4
// (32-value blocks, E8M0 block scale), per "Hardware FP4 inference for speech
// on Blackwell" (section "NVFP4, and the two ways it fails") and "FP4 n'existe
// pas ..." (section "Deux dialectes, deux strategies de scaling"). The dynamic
// per-tensor scale needs the tensor's largest magnitude before any block can be
// encoded, so it is a two-launch reduction: partial maxima per workgroup, then
// every quantize workgroup folds the (at most 1024) partials itself. No atomics
// and no memory clearing are involved, so the result is deterministic and the
// scratch needs no initialization.
#include "fp4_device.h"
#include "fp4_internal.h"

namespace fp4i {
using namespace fp4d;

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Workgroup-wide max of v (all threads receive it).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *lds4) {
  v = wave_max_u32(v);
  int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) lds4[wave] = v;
  __syncthreads();
  uint32_t r = lds4[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = max(r, lds4[i]);
  return r;
}

// |x| max as bf16 bit patterns (magnitudes order like their bit patterns).
__device__ __forceinline__ uint32_t absmax_bits8(uint4 v) {
  uint32_t m = 0;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, w[i] & 0x7FFFu);
    m = max(m, (w[i] >> 16) & 0x7FFFu);
  }
  return m;
}

__global__ __launch_bounds__(kThreads) void k_amax_parts(const uint4 *__restrict__ x, int64_t n8,
                                                         uint32_t *__restrict__ parts) {
  __shared__ uint32_t lds[4];
  uint32_t m = 0;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride)
    m = max(m, absmax_bits8(x[i]));
  m = block_max_u32(m, lds);
  if (threadIdx.x == 0) parts[blockIdx.x] = m;
}

// Per-tensor scale for this launch: static value or the fold of the partials.
__device__ __forceinline__ float resolve_tensor_scale(const uint32_t *parts, int nparts,
                                                      const float *static_scale, uint32_t *lds4) {
  if (static_scale) return *static_scale;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = max(m, parts[i]);
  m = block_max_u32(m, lds4);
  return tensor_scale_from_amax(bf16_bits_to_f32(m));
}

// One thread per 16-value block (NVFP4) of the padded row, canonical layout.
__global__ __launch_bounds__(kThreads) void k_quant_nv_canon(
    const uint16_t *__restrict__ x, int64_t rows, int64_t k, int64_t nb_pad,
    const uint32_t *__restrict__ parts, int nparts, const float *__restrict__ static_scale,
    uint8_t *__restrict__ codes, int64_t cpitch, uint8_t *__restrict__ scales, int64_t spitch,
    float *__restrict__ ts_out, int *__restrict__ zero_ptr, int zero_n) {
  __shared__ uint32_t lds[4];
  float st = resolve_tensor_scale(parts, nparts, static_scale, lds);
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0 && ts_out) *ts_out = st;
    for (int i = threadIdx.x; i < zero_n; i += blockDim.x) zero_ptr[i] = 0;
  }
  const int64_t nb = k / 16, total = rows * nb_pad;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    int64_t r = t / nb_pad, b = t - r * nb_pad;
    uint8_t *crow = codes + r * cpitch;
    if (b >= nb) {  // zero padding up to K_pad
      *(uint2 *)(crow + b * 8) = make_uint2(0u, 0u);
      scales[r * spitch + b] = 0;
      continue;
    }
    const uint4 *src = (const uint4 *)(x + r * k + b * 16);
    uint4 v0 = src[0], v1 = src[1];
    uint32_t abits = max(absmax_bits8(v0), absmax_bits8(v1));
    double q = (double)bf16_bits_to_f32(abits) / (6.0 * (double)st);
    uint32_t sbyte = e4m3_rne_sat(q);
    NvBlockEnc enc = nv_block_encoder(sbyte, st);
    uint2 out = make_uint2(nv_encode8(enc, v0), nv_encode8(enc, v1));
    *(uint2 *)(crow + b * 8) = out;
    scales[r * spitch + b] = (uint8_t)sbyte;
  }
}

// One thread per 32-value block (MXFP4) of the padded row, canonical layout.
__global__ __launch_bounds__(kThreads) void k_quant_mx_canon(
    const uint16_t *__restrict__ x, int64_t rows, int64_t k, int64_t nb_pad,
    uint8_t *__restrict__ codes, int64_t cpitch, uint8_t *__restrict__ scales, int64_t spitch,
    int *__restrict__ zero_ptr, int zero_n) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < zero_n; i += blockDim.x) zero_ptr[i] = 0;
  const int64_t nb = k / 32, total = rows * nb_pad;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    int64_t r = t / nb_pad, b = t - r * nb_pad;
    uint8_t *crow = codes + r * cpitch;
    if (b >= nb) {
      *(uint4 *)(crow + b * 16) = make_uint4(0u, 0u, 0u, 0u);
      scales[r * spitch + b] = 0;
      continue;
    }
    const uint4 *src = (const uint4 *)(x + r * k + b * 32);
    uint4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
    uint32_t abits = max(max(absmax_bits8(v0), absmax_bits8(v1)),
                         max(absmax_bits8(v2), absmax_bits8(v3)));
    int e = mx_exponent_from_bits(abits);
    uint4 out = make_uint4(mx_encode8(e, v0), mx_encode8(e, v1), mx_encode8(e, v2),
                           mx_encode8(e, v3));
    *(uint4 *)(crow + b * 16) = out;
    scales[r * spitch + b] = (uint8_t)(e + 127);
  }
}

// Weight quantization into the fragment-tiled layout. One thread per block of
// the padded [N_pad, K_pad] matrix; padding blocks get zero codes and scales.
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_quant_tiled(
    const uint16_t *__restrict__ w, int64_t n, int64_t k, int64_t n_pad, int64_t kt_n,
    const uint32_t *__restrict__ parts, int nparts, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ scales, float *__restrict__ ts_out) {
  constexpr int B = FMT == 0 ? 16 : 32;
  constexpr int BPF = 128 / B;                   // blocks per fragment row
  constexpr int SFB = FMT == 0 ? 128 : 64;       // scale bytes per fragment
  __shared__ uint32_t lds[4];
  float st = 1.0f;
  if (FMT == 0) {
    st = resolve_tensor_scale(parts, nparts, nullptr, lds);
    if (blockIdx.x == 0 && threadIdx.x == 0) *ts_out = st;
  }
  const int64_t nb = k / B, nb_pad = kt_n * BPF, total = n_pad * nb_pad;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    int64_t row = t / nb_pad, b = t - row * nb_pad;
    int64_t frag = (row >> 4) * kt_n + b / BPF;
    int r = (int)(row & 15), bi = (int)(b % BPF);
    uint8_t *cdst, *sdst;
    if (FMT == 0) {  // lane 16*(bi/2) + r holds blocks bi (low 8 bytes) and bi^1
      int lane = 16 * (bi >> 1) + r;
      cdst = codes + frag * kFragCodeBytes + lane * 16 + (bi & 1) * 8;
      sdst = scales + frag * SFB + lane * 2 + (bi & 1);
    } else {
      int lane = 16 * bi + r;
      cdst = codes + frag * kFragCodeBytes + lane * 16;
      sdst = scales + frag * SFB + lane;
    }
    if (row >= n || b >= nb) {
      if (FMT == 0) *(uint2 *)cdst = make_uint2(0u, 0u);
      else *(uint4 *)cdst = make_uint4(0u, 0u, 0u, 0u);
      *sdst = 0;
      continue;
    }
    const uint4 *src = (const uint4 *)(w + row * k + b * B);
    if (FMT == 0) {
      uint4 v0 = src[0], v1 = src[1];
      uint32_t abits = max(absmax_bits8(v0), absmax_bits8(v1));
      double q = (double)bf16_bits_to_f32(abits) / (6.0 * (double)st);
      uint32_t sbyte = e4m3_rne_sat(q);
      NvBlockEnc enc = nv_block_encoder(sbyte, st);
      *(uint2 *)cdst = make_uint2(nv_encode8(enc, v0), nv_encode8(enc, v1));
      *sdst = (uint8_t)sbyte;
    } else {
      uint4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
      uint32_t abits = max(max(absmax_bits8(v0), absmax_bits8(v1)),
                           max(absmax_bits8(v2), absmax_bits8(v3)));
      int e = mx_exponent_from_bits(abits);
      *(uint4 *)cdst = make_uint4(mx_encode8(e, v0), mx_encode8(e, v1), mx_encode8(e, v2),
                                  mx_encode8(e, v3));
      *sdst = (uint8_t)(e + 127);
    }
  }
}

// Tiled -> canonical copy (one thread per block of the padded canonical row).
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_export(
    const uint8_t *__restrict__ tc, const uint8_t *__restrict__ ts, int64_t rows, int64_t kt_n,
    uint8_t *__restrict__ codes, int64_t cpitch, uint8_t *__restrict__ scales, int64_t spitch,
    const float *__restrict__ tsc_in, float *__restrict__ tsc_out) {
  constexpr int B = FMT == 0 ? 16 : 32;
  constexpr int BPF = 128 / B;
  constexpr int SFB = FMT == 0 ? 128 : 64;
  if (blockIdx.x == 0 && threadIdx.x == 0 && tsc_in && tsc_out) *tsc_out = *tsc_in;
  const int64_t nb_pad = kt_n * BPF, total = rows * nb_pad;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    int64_t row = t / nb_pad, b = t - row * nb_pad;
    int64_t frag = (row >> 4) * kt_n + b / BPF;
    int r = (int)(row & 15), bi = (int)(b % BPF);
    if (FMT == 0) {
      int lane = 16 * (bi >> 1) + r;
      *(uint2 *)(codes + row * cpitch + b * 8) =
          *(const uint2 *)(tc + frag * kFragCodeBytes + lane * 16 + (bi & 1) * 8);
      scales[row * spitch + b] = ts[frag * SFB + lane * 2 + (bi & 1)];
    } else {
      int lane = 16 * bi + r;
      *(uint4 *)(codes + row * cpitch + b * 16) =
          *(const uint4 *)(tc + frag * kFragCodeBytes + lane * 16);
      scales[row * spitch + b] = ts[frag * SFB + lane];
    }
  }
}

// x^ = q * s_b * S_t rounded once to FP32. One thread per element.
template <int FMT, int TILED>
__global__ __launch_bounds__(kThreads) void k_dequant(
    const uint8_t *__restrict__ codes, int64_t cpitch, const uint8_t *__restrict__ scales,
    int64_t spitch, const float *__restrict__ tsc, int64_t rows, int64_t k, int64_t kt_n,
    float *__restrict__ out, int64_t ldo) {
  constexpr int B = FMT == 0 ? 16 : 32;
  constexpr int SFB = FMT == 0 ? 128 : 64;
  const double st = (FMT == 0 && tsc) ? (double)*tsc : 1.0;
  const int64_t total = rows * k;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    int64_t row = t / k, kk = t - row * k;
    uint32_t byte, sbyte;
    if (!TILED) {
      byte = codes[row * cpitch + kk / 2];
      sbyte = scales[row * spitch + kk / B];
    } else {
      int64_t frag = (row >> 4) * kt_n + kk / 128;
      int r = (int)(row & 15), kin = (int)(kk % 128);
      int lane = 16 * (kin / 32) + r;
      byte = codes[frag * kFragCodeBytes + lane * 16 + (kin % 32) / 2];
      sbyte = FMT == 0 ? scales[frag * SFB + lane * 2 + (kin % 32) / 16]
                       : scales[frag * SFB + lane];
    }
    uint32_t code = (kk & 1) ? (byte >> 4) : (byte & 15u);
    uint32_t ee = (code >> 1) & 3u, mm = code & 1u;
    float qmag = ee == 0 ? 0.5f * (float)mm : ldexpf(1.0f + 0.5f * (float)mm, (int)ee - 1);
    double s = FMT == 0 ? (double)e4m3_to_f32(sbyte) : ldexp(1.0, (int)sbyte - 127);
    double v = (double)qmag * s * st;
    out[row * ldo + kk] = (code & 8u) ? -(float)v : (float)v;
  }
}

__global__ void k_zero_ints(int *p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

int grid_for(int64_t work, int cap) {
  int64_t g = (work + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

}  // namespace

int amax_parts(int64_t n) {
  int64_t per = (int64_t)kThreads * 8 * 4;   // >= 4 uint4 loads per thread
  int64_t p = (n + per - 1) / per;
  if (p < 1) p = 1;
  if (p > kMaxAmaxParts) p = kMaxAmaxParts;
  return (int)p;
}

hipError_t launch_amax_parts(const uint16_t *x, int64_t n, uint32_t *parts, int nparts,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_amax_parts, dim3(nparts), dim3(kThreads), 0, stream,
                     (const uint4 *)x, n / 8, parts);
  return hipGetLastError();
}

hipError_t launch_quant_canonical(int fmt, const uint16_t *x, int64_t rows, int64_t k,
                                  const uint32_t *parts, int nparts, const float *static_scale,
                                  uint8_t *codes, int64_t cpitch, uint8_t *scales,
                                  int64_t spitch, float *ts_out, int *zero_ptr, int zero_n,
                                  hipStream_t stream) {
  int64_t nb_pad = k_pad(k) / block_of(fmt);
  int grid = grid_for(rows * nb_pad, 4096);
  if (fmt == 0)
    hipLaunchKernelGGL(k_quant_nv_canon, dim3(grid), dim3(kThreads), 0, stream, x, rows, k,
                       nb_pad, parts, nparts, static_scale, codes, cpitch, scales, spitch, ts_out,
                       zero_ptr, zero_n);
  else
    hipLaunchKernelGGL(k_quant_mx_canon, dim3(grid), dim3(kThreads), 0, stream, x, rows, k,
                       nb_pad, codes, cpitch, scales, spitch, zero_ptr, zero_n);
  return hipGetLastError();
}

hipError_t launch_quant_tiled(int fmt, const uint16_t *w, int64_t n, int64_t k,
                              const uint32_t *parts, int nparts, uint8_t *codes, uint8_t *scales,
                              float *ts_out, hipStream_t stream) {
  int64_t n_pad = round_up(n, 16), kt_n = k_pad(k) / 128;
  int64_t work = n_pad * kt_n * (128 / block_of(fmt));
  int grid = grid_for(work, 8192);
  if (fmt == 0)
    hipLaunchKernelGGL(k_quant_tiled<0>, dim3(grid), dim3(kThreads), 0, stream, w, n, k, n_pad,
                       kt_n, parts, nparts, codes, scales, ts_out);
  else
    hipLaunchKernelGGL(k_quant_tiled<1>, dim3(grid), dim3(kThreads), 0, stream, w, n, k, n_pad,
                       kt_n, parts, nparts, codes, scales, ts_out);
  return hipGetLastError();
}

hipError_t launch_export_canonical(int fmt, const uint8_t *tcodes, const uint8_t *tscales,
                                   int64_t rows, int64_t k, uint8_t *codes, int64_t cpitch,
                                   uint8_t *scales, int64_t spitch, const float *ts_in,
                                   float *ts_out, hipStream_t stream) {
  int64_t kt_n = k_pad(k) / 128;
  int grid = grid_for(rows * kt_n * (128 / block_of(fmt)), 8192);
  if (fmt == 0)
    hipLaunchKernelGGL(k_export<0>, dim3(grid), dim3(kThreads), 0, stream, tcodes, tscales, rows,
                       kt_n, codes, cpitch, scales, spitch, ts_in, ts_out);
  else
    hipLaunchKernelGGL(k_export<1>, dim3(grid), dim3(kThreads), 0, stream, tcodes, tscales, rows,
                       kt_n, codes, cpitch, scales, spitch, ts_in, ts_out);
  return hipGetLastError();
}

hipError_t launch_dequant(int fmt, int tiled, const uint8_t *codes, int64_t cpitch,
                          const uint8_t *scales, int64_t spitch, const float *ts, int64_t rows,
                          int64_t k, float *out, int64_t ldo, hipStream_t stream) {
  int64_t kt_n = k_pad(k) / 128;
  int grid = grid_for(rows * k, 8192);
#define FP4_DQ(F, T)                                                                       \
  hipLaunchKernelGGL((k_dequant<F, T>), dim3(grid), dim3(kThreads), 0, stream, codes, cpitch, \
                     scales, spitch, ts, rows, k, kt_n, out, ldo)
  if (fmt == 0 && !tiled) FP4_DQ(0, 0);
  else if (fmt == 0) FP4_DQ(0, 1);
  else if (!tiled) FP4_DQ(1, 0);
  else FP4_DQ(1, 1);
#undef FP4_DQ
  return hipGetLastError();
}

hipError_t launch_zero_ints(int *p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_ints, dim3((n + 255) / 256), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace fp4i
