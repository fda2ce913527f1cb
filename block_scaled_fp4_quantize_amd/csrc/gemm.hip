// gemm.hip -- W4A4 block-scaled FP4 GEMM kernels for gfx950.
//
// C[m, n] = alpha * sum_k (q_a s_a)[m, k] (q_w s_w)[n, k], FP32 accumulation,
// bf16 output, as a linear layer (weights [N, K]). The product of the
// dequantized operands is what the pages' GEMM library computes on the
// quantized weight cache (forum post on a standalone FP4 GEMM library, opening
// paragraphs).
//
// MXFP4 runs natively on the block-scaled FP4 matrix instruction
// (V_MFMA_SCALE_F32_16X16X128_F8F6F4): per lane 32 E2M1 values along K and
// one E8M0 scale for its 32-value block, which is exactly MXFP4's block.
//
// NVFP4 cannot: its 16-value blocks carry E4M3 scales with a mantissa, while
// the matrix unit applies one power-of-two scale per 32 values. q * s_b needs
// up to 6 significant bits, more than any FP4/FP6/FP8 element holds, so the
// exact path dequantizes each lane's codes to f16 (q * s_b is exact in f16:
// <= 6 significant bits, range [2^-10, 2688]) and runs the f16 matrix
// instruction (V_MFMA_F32_16X16X32_F16), whose f16 x f16 products are exact
// in its FP32 accumulator. Each lane's 32 values feed four K=32 instructions
// as values 8g..8g+7 (g = 0..3) of both operands; any K permutation applied to
// both operands leaves the contraction unchanged.
#include "fp4_device.h"
#include "fp4_internal.h"

namespace fp4i {
using namespace fp4d;

namespace {

__device__ __forceinline__ v4f mfma_mx(uint4 a, uint4 b, v4f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(frag_v8i(a), frag_v8i(b), c, 4, 4, 0,
                                                           (int)sa, 0, (int)sb);
}

__device__ __forceinline__ v4f mfma_nv(const h8v a[4], const h8v b[4], v4f c) {
#pragma unroll
  for (int g = 0; g < 4; ++g) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[g], b[g], c, 0, 0, 0);
  return c;
}

// ------------------------------------------------------------------ prefill
//
// Workgroup tile 128 x 128 (4 waves in a 2 x 2 grid, 64 x 64 per wave as
// 4 x 4 tiles of 16 x 16). Operands are read per lane straight into the MFMA
// operand registers: an A fragment lane l reads 16 bytes of row (l % 16) at
// K offset 32 (l / 16) of the canonical layout; a W fragment is one 1 KB
// contiguous tile of the weight cache.
template <int FMT>
__global__ __launch_bounds__(256) void k_gemm_prefill(
    const uint8_t *__restrict__ a_codes, int64_t a_cp, const uint8_t *__restrict__ a_sc,
    int64_t a_sp, const float *__restrict__ a_ts, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_sc, const float *__restrict__ w_ts, int m, int n, int kt_n,
    int nt_n, uint16_t *__restrict__ c, int64_t ldc) {
  constexpr int SFB = FMT == 0 ? 128 : 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m0 = blockIdx.y * 128 + (wave >> 1) * 64;
  const int nt0 = (blockIdx.x * 128 + (wave & 1) * 64) >> 4;
  const int lr = lane & 15, lc = lane >> 4;
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kt = 0; kt < kt_n; ++kt) {
    uint4 aq[4], wq[4];
    uint32_t as[4], ws[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = m0 + 16 * i + lr;
      if (row < m) {
        aq[i] = *(const uint4 *)(a_codes + (int64_t)row * a_cp + kt * 64 + lc * 16);
        as[i] = FMT == 0 ? *(const uint16_t *)(a_sc + (int64_t)row * a_sp + kt * 8 + lc * 2)
                         : a_sc[(int64_t)row * a_sp + kt * 4 + lc];
      } else {
        aq[i] = make_uint4(0u, 0u, 0u, 0u);
        as[i] = 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int nt = nt0 + j;
      if (nt < nt_n) {
        int64_t f = (int64_t)nt * kt_n + kt;
        wq[j] = *(const uint4 *)(w_codes + f * kFragCodeBytes + lane * 16);
        ws[j] = FMT == 0 ? *(const uint16_t *)(w_sc + f * SFB + lane * 2) : w_sc[f * SFB + lane];
      } else {
        wq[j] = make_uint4(0u, 0u, 0u, 0u);
        ws[j] = 0u;
      }
    }
    if (FMT == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_mx(aq[i], wq[j], acc[i][j], as[i], ws[j]);
    } else {
      h8v ah[4][4], wh[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) nv_dequant32(aq[i], as[i], ah[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) nv_dequant32(wq[j], ws[j], wh[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_nv(ah[i], wh[j], acc[i][j]);
    }
  }
  const float alpha = FMT == 0 ? a_ts[0] * w_ts[0] : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int col = (nt0 + j) * 16 + lr;
      if (col >= n) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int row = m0 + 16 * i + 4 * lc + r;
        if (row < m) c[(int64_t)row * ldc + col] = f32_to_bf16_rne(acc[i][j][r] * alpha);
      }
    }
}

// ------------------------------------------------------------------- decode
//
// Skinny GEMM for M <= 32: the weight is streamed once at HBM rate. Workgroup
// (nt, s) owns one 16-row weight tile and a K range of kt_per_wg fragments;
// its 4 waves take interleaved fragments so the workgroup reads a contiguous
// run of the weight cache. The weight tile is the MFMA's A operand (rows n)
// and the activations its B operand (columns m, MG groups of 16), so the
// accumulator holds C^T. Waves are summed in LDS in a fixed order; with
// several K splits each workgroup stores its partial tile and the last one to
// arrive (counted with an atomic) sums the partials in split order, so the
// result does not depend on scheduling.
template <int FMT, int MG>
__global__ __launch_bounds__(256) void k_gemm_decode(
    const uint8_t *__restrict__ a_codes, int64_t a_cp, const uint8_t *__restrict__ a_sc,
    int64_t a_sp, const float *__restrict__ a_ts, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_sc, const float *__restrict__ w_ts, int m, int n, int kt_n,
    uint16_t *__restrict__ c, int64_t ldc, int splits, int kt_per_wg,
    float *__restrict__ partials, int *__restrict__ counters) {
  constexpr int SFB = FMT == 0 ? 128 : 64;
  constexpr int U = 2;
  __shared__ float red[4][MG][4][64];
  __shared__ int last_flag;
  const int nt = blockIdx.x, s = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lc = lane >> 4;
  const int kt_begin = s * kt_per_wg;
  const int kt_end = min(kt_n, kt_begin + kt_per_wg);
  v4f acc[MG];
#pragma unroll
  for (int g = 0; g < MG; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kt0 = kt_begin + wave; kt0 < kt_end; kt0 += 4 * U) {
    uint4 wq[U], aq[U][MG];
    uint32_t ws[U], as[U][MG];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int kt = kt0 + 4 * u;
      bool ok = kt < kt_end;
      int64_t f = (int64_t)nt * kt_n + kt;
      wq[u] = ok ? *(const uint4 *)(w_codes + f * kFragCodeBytes + lane * 16)
                 : make_uint4(0u, 0u, 0u, 0u);
      ws[u] = ok ? (FMT == 0 ? (uint32_t)*(const uint16_t *)(w_sc + f * SFB + lane * 2)
                             : (uint32_t)w_sc[f * SFB + lane])
                 : 0u;
#pragma unroll
      for (int g = 0; g < MG; ++g) {
        int row = 16 * g + lr;
        bool aok = ok && row < m;
        aq[u][g] = aok ? *(const uint4 *)(a_codes + (int64_t)row * a_cp + kt * 64 + lc * 16)
                       : make_uint4(0u, 0u, 0u, 0u);
        as[u][g] = aok ? (FMT == 0
                              ? (uint32_t)*(const uint16_t *)(a_sc + (int64_t)row * a_sp + kt * 8 +
                                                              lc * 2)
                              : (uint32_t)a_sc[(int64_t)row * a_sp + kt * 4 + lc])
                       : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (FMT == 1) {
#pragma unroll
        for (int g = 0; g < MG; ++g) acc[g] = mfma_mx(wq[u], aq[u][g], acc[g], ws[u], as[u][g]);
      } else {
        h8v wh[4];
        nv_dequant32(wq[u], ws[u], wh);
#pragma unroll
        for (int g = 0; g < MG; ++g) {
          h8v ah[4];
          nv_dequant32(aq[u][g], as[u][g], ah);
          acc[g] = mfma_nv(wh, ah, acc[g]);
        }
      }
    }
  }
  // Sum the 4 waves in a fixed order.
#pragma unroll
  for (int g = 0; g < MG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][g][r][lane] = acc[g][r];
  __syncthreads();
  // Threads 0..64*MG-1 each own one (g, lane) column of 4 values.
  const float alpha = FMT == 0 ? a_ts[0] * w_ts[0] : 1.0f;
  const int tg = threadIdx.x >> 6;  // group handled by this thread (if < MG)
  float tot[4] = {0.f, 0.f, 0.f, 0.f};
  if (tg < MG) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      tot[r] = ((red[0][tg][r][lane] + red[1][tg][r][lane]) + red[2][tg][r][lane]) +
               red[3][tg][r][lane];
  }
  if (splits > 1) {
    float *mine = partials + ((int64_t)nt * splits + s) * (MG * 256);
    if (tg < MG) {
#pragma unroll
      for (int r = 0; r < 4; ++r) mine[tg * 256 + r * 64 + lane] = tot[r];
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) last_flag = (atomicAdd(&counters[nt], 1) == splits - 1);
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    if (tg < MG) {
      const float *base = partials + (int64_t)nt * splits * (MG * 256);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = 0.f;
        for (int ss = 0; ss < splits; ++ss)
          v += __builtin_nontemporal_load(base + (int64_t)ss * (MG * 256) + tg * 256 + r * 64 + lane);
        tot[r] = v;
      }
    }
  }
  if (tg < MG) {
    int col = 16 * tg + lr;  // activation row m
    if (col < m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int row = nt * 16 + 4 * lc + r;  // output column n
        if (row < n) c[(int64_t)col * ldc + row] = f32_to_bf16_rne(tot[r] * alpha);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs &g, hipStream_t stream) {
  int kt_n = (int)(k_pad(g.k) / 128);
  int nt_n = (int)(round_up(g.n, 16) / 16);
  dim3 grid((unsigned)((g.n + 127) / 128), (unsigned)((g.m + 127) / 128));
  if (g.fmt == 0)
    hipLaunchKernelGGL(k_gemm_prefill<0>, grid, dim3(256), 0, stream, g.a_codes, g.a_cpitch,
                       g.a_scales, g.a_spitch, g.a_ts, g.w_codes, g.w_scales, g.w_ts, (int)g.m,
                       (int)g.n, kt_n, nt_n, g.c, g.ldc);
  else
    hipLaunchKernelGGL(k_gemm_prefill<1>, grid, dim3(256), 0, stream, g.a_codes, g.a_cpitch,
                       g.a_scales, g.a_spitch, g.a_ts, g.w_codes, g.w_scales, g.w_ts, (int)g.m,
                       (int)g.n, kt_n, nt_n, g.c, g.ldc);
  return hipGetLastError();
}

DecodePlan decode_plan(int fmt, int64_t m, int64_t n, int64_t k) {
  (void)fmt;
  DecodePlan p;
  p.mg = m <= 16 ? 1 : 2;
  int64_t kt_n = k_pad(k) / 128, nt_n = round_up(n, 16) / 16;
  // Aim for ~16 waves per CU over 256 CUs (4 waves per workgroup) while each
  // wave streams at least 2 fragments.
  int64_t target_wg = 1024;
  int64_t splits = (target_wg + nt_n - 1) / nt_n;
  int64_t max_splits = (kt_n + 7) / 8;   // >= 8 fragments per workgroup
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t kpw = (kt_n + splits - 1) / splits;
  p.kt_per_wg = (int)kpw;
  p.splits = (int)((kt_n + kpw - 1) / kpw);
  p.frags = (int)((kpw + 3) / 4);
  return p;
}

size_t decode_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
  DecodePlan p = decode_plan(fmt, m, n, k);
  if (p.splits <= 1) return 0;
  int64_t nt_n = round_up(n, 16) / 16;
  size_t counters = (size_t)round_up(nt_n * 4, 256);
  size_t parts = (size_t)nt_n * p.splits * p.mg * 256 * 4;
  return counters + parts;
}

hipError_t launch_gemm_decode(const GemmArgs &g, const DecodePlan &p, float *partials,
                              int *counters, hipStream_t stream) {
  int kt_n = (int)(k_pad(g.k) / 128);
  int nt_n = (int)(round_up(g.n, 16) / 16);
  dim3 grid((unsigned)nt_n, (unsigned)p.splits);
#define FP4_DEC(F, G)                                                                           \
  hipLaunchKernelGGL((k_gemm_decode<F, G>), grid, dim3(256), 0, stream, g.a_codes, g.a_cpitch, \
                     g.a_scales, g.a_spitch, g.a_ts, g.w_codes, g.w_scales, g.w_ts, (int)g.m,  \
                     (int)g.n, kt_n, g.c, g.ldc, p.splits, p.kt_per_wg, partials, counters)
  if (g.fmt == 0 && p.mg == 1) FP4_DEC(0, 1);
  else if (g.fmt == 0) FP4_DEC(0, 2);
  else if (p.mg == 1) FP4_DEC(1, 1);
  else FP4_DEC(1, 2);
#undef FP4_DEC
  return hipGetLastError();
}

}  // namespace fp4i
