// gemm_w4a16.hip -- weight-only FP4 linear (W4A16) for gfx950.
//
// y[m, n] = bf16_RNE(S_tW * sum_k x[m, k] (q s_b)[n, k]): the activations stay
// bf16 and only the cached weight is FP4, the weight-only regime the pages
// measure next to W4A4 ("Hardware FP4 inference for speech on Blackwell",
// section "Weights are safe" for the W4A16 checkpoint, and section "Two Triton
// kernels for the SM120 gaps" for a W4A16 GEMM of bf16 activations with
// pre-packed FP4 weights). FP32 accumulation.
//
// The weight cache is the same fragment-tiled cache the W4A4 GEMM reads. Each
// lane's 32 FP4 values are dequantized to exact bf16 values q * s_b (at most
// 6 significant bits; NVFP4 range [2^-10, 2688], MXFP4 q * 2^e within the bf16
// range for weights below 2^127) and fed to the bf16 matrix instruction
// (V_MFMA_F32_16X16X32_BF16) as values 8g..8g+7 (g = 0..3) of the lane's 32;
// the activation operand takes the same K permutation, so lane l (column
// l % 16) reads x[m][128 kt + 32 (l / 16) + 8g .. + 7]: 64 contiguous bytes
// per fragment.
//   NVFP4: codes -> FP32 by the hardware FP4 convert (scale 1), times the
//          E4M3 block scale in FP32 (exact), packed to bf16 (exact).
//   MXFP4: the convert applies the power-of-two block scale itself (the
//          convert's scale carries an exponent only, which is all an E8M0
//          scale is); a block scale of 2^-127, not a normal FP32 number, takes
//          the FP32 route.
#include "fp4_device.h"
#include "fp4_internal.h"

namespace fp4i {
using namespace fp4d;

namespace {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf2_bits(bf2v v) { return __builtin_bit_cast(uint32_t, v); }

// Two FP4 codes (byte b of q) -> FP32 values (exact).
__device__ __forceinline__ f2v fp4x2_to_f2(uint32_t q, int b) {
  switch (b) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
  }
}

// Two FP4 codes (byte b of q) -> bf16 values q * 2^e, e the exponent of s.
__device__ __forceinline__ uint32_t fp4x2_to_bf2_scaled(uint32_t q, float s, int b) {
  switch (b) {
    case 0: return bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 0));
    case 1: return bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 1));
    case 2: return bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 2));
    default: return bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 3));
  }
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return bf2_bits(__builtin_convertvector((f2v){lo, hi}, bf2v));
}

// One dword of codes (values 8g .. 8g+7 of the lane) with block scale sv
// (FP32) -> 8 exact bf16 values, FP32 route.
__device__ __forceinline__ bf8v deq8_f32(uint32_t d, float sv) {
  uint32_t r[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f2v v = fp4x2_to_f2(d, b);
    r[b] = pack_bf2(v[0] * sv, v[1] * sv);
  }
  return __builtin_bit_cast(bf8v, make_uint4(r[0], r[1], r[2], r[3]));
}

// The lane's 32 weight values as four groups of 8 bf16 (group g = values
// 8g .. 8g+7). sc: NVFP4 two E4M3 bytes (values 0-15, 16-31); MXFP4 one E8M0.
template <int FMT>
__device__ __forceinline__ void deq_w32(uint4 q, uint32_t sc, bf8v out[4]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  if constexpr (FMT == 0) {
    const float s0 = e4m3_to_f32(sc & 0x7Fu), s1 = e4m3_to_f32((sc >> 8) & 0x7Fu);
#pragma unroll
    for (int g = 0; g < 4; ++g) out[g] = deq8_f32(w[g], g < 2 ? s0 : s1);
  } else {
    const uint32_t e = sc & 0xFFu;
    if (e != 0u) {
      const float s = __uint_as_float(e << 23);  // 2^(e - 127), a normal FP32 number
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t r[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) r[b] = fp4x2_to_bf2_scaled(w[g], s, b);
        out[g] = __builtin_bit_cast(bf8v, make_uint4(r[0], r[1], r[2], r[3]));
      }
    } else {
      const float s = 0x1p-127f;  // subnormal: exact FP32 multiply instead
#pragma unroll
      for (int g = 0; g < 4; ++g) out[g] = deq8_f32(w[g], s);
    }
  }
}

// The lane's part of weight fragment f: 16 code bytes and its scale bytes.
template <int FMT>
__device__ __forceinline__ void load_wfrag(const uint8_t *__restrict__ w_codes,
                                           const uint8_t *__restrict__ w_sc, int64_t f, int lane,
                                           uint4 &q, uint32_t &sc) {
  q = *(const uint4 *)(w_codes + f * kFragCodeBytes + lane * 16);
  sc = FMT == 0 ? (uint32_t)*(const uint16_t *)(w_sc + f * 128 + lane * 2)
                : (uint32_t)w_sc[f * 64 + lane];
}

// The lane's activation operand for K step kt: row `row` (zero past m or for
// a K tail beyond k), values 128 kt + 32 (lane / 16) + 0 .. 31 as four groups.
__device__ __forceinline__ void load_x(const uint16_t *__restrict__ x, int64_t ldx, int row,
                                       int m, int k, int kt, int lane, uint4 out[4]) {
  const int k0 = kt * kFragK + 32 * (lane >> 4);
  if (row >= m || k0 >= k) {
#pragma unroll
    for (int g = 0; g < 4; ++g) out[g] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  // k is a multiple of the block (16 or 32), so a lane's 32 values are either
  // all inside k or (NVFP4 only) split at k0 + 16
  const uint4 *src = (const uint4 *)(x + (int64_t)row * ldx + k0);
  out[0] = src[0];
  out[1] = src[1];
  if (k0 + 16 < k) {
    out[2] = src[2];
    out[3] = src[3];
  } else {
    out[2] = make_uint4(0u, 0u, 0u, 0u);
    out[3] = make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ v4f mma_bf16(bf8v a, uint4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf8v, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ decode
//
// M <= 32: one workgroup per NT 16-row weight tiles covering all of K, eight
// waves taking interleaved K steps (kt = wave + 8 j), the next step's loads
// issued before the current step's arithmetic; partial sums added in LDS in a
// fixed order. The weight tile is the matrix instruction's A operand, so the
// accumulator holds y^T (rows n, columns m). Every workgroup reads the bf16
// activation rows of the whole K from L2, which bounds the kernel once there
// are many rows: NT > 1 tiles per workgroup read them once for NT tiles.
constexpr int kW16Waves = 8;

template <int FMT, int MG, int NT>
__global__ __launch_bounds__(64 * kW16Waves) void k_w4a16_decode(
    const uint16_t *__restrict__ x, int64_t ldx, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_sc, const float *__restrict__ w_ts, int m, int n, int k,
    int kt_n, int nt_n, uint16_t *__restrict__ y, int64_t ldy) {
  constexpr int NW = kW16Waves;
  __shared__ float red[NW][NT * MG][4][64];
  const int nt0 = blockIdx.x * NT;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  v4f acc[NT][MG];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < MG; ++g) acc[t][g] = v4f{0.f, 0.f, 0.f, 0.f};
  uint4 wq[2][NT], xa[2][MG][4];
  uint32_t ws[2][NT];
  auto load = [&](int buf, int kt) __attribute__((always_inline)) {
    if (kt < kt_n) {
#pragma unroll
      for (int t = 0; t < NT; ++t)  // a tile past the last reads the last again (never stored)
        load_wfrag<FMT>(w_codes, w_sc, (int64_t)min(nt0 + t, nt_n - 1) * kt_n + kt, lane,
                        wq[buf][t], ws[buf][t]);
#pragma unroll
      for (int g = 0; g < MG; ++g) load_x(x, ldx, 16 * g + (lane & 15), m, k, kt, lane, xa[buf][g]);
    }
  };
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bf8v wh[4];
      deq_w32<FMT>(wq[buf][t], ws[buf][t], wh);
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[t][g] = mma_bf16(wh[s], xa[buf][g][s], acc[t][g]);
    }
  };
  load(0, wave);
  for (int kt = wave; kt < kt_n; kt += 2 * NW) {
    load(1, kt + NW);
    compute(0);
    if (kt + NW >= kt_n) break;
    load(0, kt + 2 * NW);
    compute(1);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < MG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][t * MG + g][r][lane] = acc[t][g][r];
  __syncthreads();
  const int tg = threadIdx.x >> 6;
  if (tg >= NT * MG) return;
  const int t = tg / MG, g = tg % MG;
  const Alpha alpha = FMT == 0 ? make_alpha(1.0f, w_ts[0]) : Alpha{1.0f, 0};
  const int col = 16 * g + (lane & 15);  // activation row m
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = red[0][tg][r][lane];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) v += red[w2][tg][r][lane];
    const int row = (nt0 + t) * 16 + 4 * (lane >> 4) + r;  // output column n
    if (col < m && row < n) y[(int64_t)col * ldy + row] = f32_to_bf16_rne(apply_alpha(v, alpha));
  }
}

// ------------------------------------------------------------------- tiles
//
// M > 32: 128 x 128 output tiles, four waves in a 2 x 2 grid of 64 x 64 (4 x 4
// matrix tiles of 16 x 16). Per K step a wave reads its four weight fragments
// and the activation operands of its 64 rows straight into registers
// (coalesced: a weight fragment is 1 KB contiguous, an activation row's
// 256 bytes are read by four lanes), dequantizes the weights once and runs
// 64 matrix instructions. The weight is the A operand, so a lane ends with
// four consecutive output columns of one row.
template <int FMT>
__global__ __launch_bounds__(256) void k_w4a16_tile(
    const uint16_t *__restrict__ x, int64_t ldx, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_sc, const float *__restrict__ w_ts, int m, int n, int k,
    int kt_n, int nt_n, uint16_t *__restrict__ y, int64_t ldy) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int m0 = blockIdx.y * 128 + (wave >> 1) * 64;
  const int nt0 = (blockIdx.x * 128 + (wave & 1) * 64) >> 4;
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int kt = 0; kt < kt_n; ++kt) {
    uint4 wq[4], xa[4][4];
    uint32_t ws[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nt = min(nt0 + j, nt_n - 1);  // past N: a valid tile, never stored
      load_wfrag<FMT>(w_codes, w_sc, (int64_t)nt * kt_n + kt, lane, wq[j], ws[j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) load_x(x, ldx, m0 + 16 * i + (lane & 15), m, k, kt, lane, xa[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf8v wh[4];
      deq_w32<FMT>(wq[j], ws[j], wh);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[i][j] = mma_bf16(wh[s], xa[i][s], acc[i][j]);
    }
  }
  const Alpha alpha = FMT == 0 ? make_alpha(1.0f, w_ts[0]) : Alpha{1.0f, 0};
  const int rl = lane & 15, cl = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + 16 * i + rl;
    if (row >= m) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col0 = (nt0 + j) * 16 + cl;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (col0 + r < n) y[(int64_t)row * ldy + col0 + r] = f32_to_bf16_rne(apply_alpha(acc[i][j][r], alpha));
    }
  }
}

}  // namespace

hipError_t launch_linear_w4a16(int fmt, const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_ts,
                               int64_t n, uint16_t *y, int64_t ldy, hipStream_t stream) {
  const int kt_n = (int)(k_pad(k) / kFragK);
  const int nt_n = (int)(round_up(n, 16) / 16);
  if (m <= kW16DecodeMaxM) {
    const int mg = m <= 16 ? 1 : 2;
    // weight tiles per workgroup (measured on the decode shapes): with 17-32
    // rows the activation reads from L2 dominate, so 4 tiles (>= 1024 tiles)
    // or 2 (>= 256, leaving 128+ workgroups); MXFP4 from 8 rows also gains
    // with 4; otherwise one (fewer, longer workgroups lost at M = 1, and for
    // NVFP4, whose weight dequantization is the heavier part, at M = 8).
    const int per = mg == 2 ? (nt_n >= 1024 ? 4 : nt_n >= 256 ? 2 : 1)
                            : (fmt == 1 && m >= 8 && nt_n >= 1024 ? 4 : 1);
#define FP4_W16D(F, G, T)                                                                      \
  hipLaunchKernelGGL((k_w4a16_decode<F, G, T>), dim3((unsigned)((nt_n + T - 1) / T)),         \
                     dim3(64 * kW16Waves), 0, stream, x, ldx, w_codes, w_scales, w_ts, (int)m, \
                     (int)n, (int)k, kt_n, nt_n, y, ldy)
#define FP4_W16P(F, G) do { if (per == 4) FP4_W16D(F, G, 4); else if (per == 2) FP4_W16D(F, G, 2); \
                            else FP4_W16D(F, G, 1); } while (0)
    if (fmt == 0 && mg == 1) FP4_W16P(0, 1);
    else if (fmt == 0) FP4_W16P(0, 2);
    else if (mg == 1) FP4_W16P(1, 1);
    else FP4_W16P(1, 2);
#undef FP4_W16P
#undef FP4_W16D
    return hipGetLastError();
  }
  dim3 grid((unsigned)((n + 127) / 128), (unsigned)((m + 127) / 128));
  if (fmt == 0)
    hipLaunchKernelGGL(k_w4a16_tile<0>, grid, dim3(256), 0, stream, x, ldx, w_codes, w_scales,
                       w_ts, (int)m, (int)n, (int)k, kt_n, nt_n, y, ldy);
  else
    hipLaunchKernelGGL(k_w4a16_tile<1>, grid, dim3(256), 0, stream, x, ldx, w_codes, w_scales,
                       w_ts, (int)m, (int)n, (int)k, kt_n, nt_n, y, ldy);
  return hipGetLastError();
}

}  // namespace fp4i
