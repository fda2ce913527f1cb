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

#include <algorithm>

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

// One lane's part of the A fragment (16 rows from 16*g, K values 128*kt ..
// 128*kt+127): 16 bytes of codes and its scale bytes, from the canonical
// layout (row-major, 64 bytes of a row per fragment) or the tiled layout (the
// fragment is 1 KB contiguous, in lane order). Rows at or past m read as zero.
template <int FMT, int ATILED>
__device__ __forceinline__ void load_a(const uint8_t *__restrict__ a_codes, int64_t a_cp,
                                       const uint8_t *__restrict__ a_sc, int64_t a_sp, int kt_n,
                                       int g, int kt, int lane, int m, uint4 &q, uint32_t &sc) {
  const int row = 16 * g + (lane & 15);
  if (row >= m) {
    q = make_uint4(0u, 0u, 0u, 0u);
    sc = 0u;
    return;
  }
  if (ATILED) {
    const int64_t f = (int64_t)g * kt_n + kt;
    q = *(const uint4 *)(a_codes + f * kFragCodeBytes + lane * 16);
    sc = FMT == 0 ? (uint32_t)*(const uint16_t *)(a_sc + f * 128 + lane * 2)
                  : (uint32_t)a_sc[f * 64 + lane];
  } else {
    const int lc = lane >> 4;
    q = *(const uint4 *)(a_codes + (int64_t)row * a_cp + kt * 64 + lc * 16);
    sc = FMT == 0 ? (uint32_t)*(const uint16_t *)(a_sc + (int64_t)row * a_sp + kt * 8 + lc * 2)
                  : (uint32_t)a_sc[(int64_t)row * a_sp + kt * 4 + lc];
  }
}

// One lane's part of weight fragment (nt, kt) of the tiled weight cache.
template <int FMT>
__device__ __forceinline__ void load_w(const uint8_t *__restrict__ w_codes,
                                       const uint8_t *__restrict__ w_sc, int64_t f, int lane,
                                       uint4 &q, uint32_t &sc) {
  q = *(const uint4 *)(w_codes + f * kFragCodeBytes + lane * 16);
  sc = FMT == 0 ? (uint32_t)*(const uint16_t *)(w_sc + f * 128 + lane * 2)
                : (uint32_t)w_sc[f * 64 + lane];
}

// ------------------------------------------------------------------ prefill
//
// Workgroup tile 128 x 128 (4 waves in a 2 x 2 grid, 64 x 64 per wave as
// 4 x 4 tiles of 16 x 16). Operands are read per lane straight into the MFMA
// operand registers: an A fragment lane l reads 16 bytes of row (l % 16) at
// K offset 32 (l / 16) of the canonical layout; a W fragment is one 1 KB
// contiguous tile of the weight cache.
template <int FMT, int ATILED>
__global__ __launch_bounds__(256) void k_gemm_prefill(
    const uint8_t *__restrict__ a_codes, int64_t a_cp, const uint8_t *__restrict__ a_sc,
    int64_t a_sp, const float *__restrict__ a_ts, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_sc, const float *__restrict__ w_ts, int m, int n, int kt_n,
    int nt_n, uint16_t *__restrict__ c, int64_t ldc) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
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
    for (int i = 0; i < 4; ++i)
      load_a<FMT, ATILED>(a_codes, a_cp, a_sc, a_sp, kt_n, (m0 >> 4) + i, kt, lane, m, aq[i], as[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nt = nt0 + j;
      if (nt < nt_n) {
        load_w<FMT>(w_codes, w_sc, (int64_t)nt * kt_n + kt, lane, wq[j], ws[j]);
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
  const Alpha alpha = FMT == 0 ? make_alpha(a_ts[0], w_ts[0]) : Alpha{1.0f, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int col = (nt0 + j) * 16 + lr;
      if (col >= n) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int row = m0 + 16 * i + 4 * lc + r;
        if (row < m) c[(int64_t)row * ldc + col] = f32_to_bf16_rne(apply_alpha(acc[i][j][r], alpha));
      }
    }
}

// ------------------------------------------------------------------- decode
//
// Skinny GEMM for M <= 128: the weight is streamed once at HBM rate. One
// workgroup per NT 16-row weight tiles covers the whole K range, so there is
// no cross-workgroup reduction: every workgroup is resident at once and HBM
// bandwidth is shared among them. The kDecWaves waves take interleaved
// fragments (kt = wave + kDecWaves * j) in groups of FM; the next group's
// loads are issued before the current group's arithmetic, whose wait then
// covers both groups (the fragment guards put loads under branches, and the
// compiler merges their wait counts), so a wave drains its loads every group.
// MXFP4 uses this kernel: for its one-instruction fragments it measured faster
// than every deeper pipeline tried (the ring kernel below). The weight tile is
// the MFMA's A operand (rows n) and the activations its B operand (columns m,
// MG groups of 16: 1, 2, 4 or 8), so the accumulator holds C^T. The waves'
// partial sums are added in LDS in a fixed order. Up to M = 128 this beats the
// tiled kernels, whose few output tiles (M / 128 rows of them) leave most CUs
// idle; every workgroup reads the (small, L2-resident) activations once.
constexpr int kDecWaves = 8;
constexpr int kDecFrags = 2;

template <int FMT, int MG, int ATILED, int NT>
__global__ __launch_bounds__(64 * kDecWaves) void k_gemm_decode(
    const uint8_t *__restrict__ a_codes, int64_t a_cp, const uint8_t *__restrict__ a_sc,
    int64_t a_sp, const float *__restrict__ a_ts, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_sc, const float *__restrict__ w_ts, int m, int n, int kt_n,
    int nt_n, uint16_t *__restrict__ c, int64_t ldc) {
  // fragments per group: two, or one for eight activation groups (registers)
  constexpr int NW = kDecWaves, FM = MG >= 8 ? 1 : kDecFrags;
  __shared__ float red[NW][NT * MG][4][64];
  const int nt0 = blockIdx.x * NT;  // first of this workgroup's NT weight tiles
  // readfirstlane makes the wave index (and every fragment guard derived from
  // it) a scalar, so the guards compile to branches around the matrix
  // instructions rather than to EXEC masks they would not honour.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  v4f acc[NT][MG];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < MG; ++g) acc[t][g] = v4f{0.f, 0.f, 0.f, 0.f};
  uint4 wq[2][FM][NT], aq[2][FM][MG];
  uint32_t ws[2][FM][NT], as[2][FM][MG];

  auto load = [&](int buf, int base) {
#pragma unroll
    for (int u = 0; u < FM; ++u) {
      const int kt = base + NW * u;
      if (kt < kt_n) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          // a tile past the last one reads the last again (its sums are never stored)
          const int nt = min(nt0 + t, nt_n - 1);
          load_w<FMT>(w_codes, w_sc, (int64_t)nt * kt_n + kt, lane, wq[buf][u][t], ws[buf][u][t]);
        }
#pragma unroll
        for (int g = 0; g < MG; ++g)
          load_a<FMT, ATILED>(a_codes, a_cp, a_sc, a_sp, kt_n, g, kt, lane, m, aq[buf][u][g],
                              as[buf][u][g]);
      }
    }
  };
  auto compute = [&](int buf, int base) {
#pragma unroll
    for (int u = 0; u < FM; ++u) {
      if (base + NW * u >= kt_n) break;  // wave-uniform
      if (FMT == 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int g = 0; g < MG; ++g)
            acc[t][g] = mfma_mx(wq[buf][u][t], aq[buf][u][g], acc[t][g], ws[buf][u][t], as[buf][u][g]);
      } else {
        // each activation group is dequantized once for the NT weight tiles
        h8v wh[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t) nv_dequant32(wq[buf][u][t], ws[buf][u][t], wh[t]);
#pragma unroll
        for (int g = 0; g < MG; ++g) {
          h8v ah[4];
          nv_dequant32(aq[buf][u][g], as[buf][u][g], ah);
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t][g] = mfma_nv(wh[t], ah, acc[t][g]);
        }
      }
    }
  };
  constexpr int STEP = NW * FM;
  load(0, wave);
  for (int base = wave; base < kt_n; base += 2 * STEP) {
    load(1, base + STEP);
    compute(0, base);
    if (base + STEP >= kt_n) break;
    load(0, base + 2 * STEP);
    compute(1, base + STEP);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < MG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][t * MG + g][r][lane] = acc[t][g][r];
  __syncthreads();
  const int tg = threadIdx.x >> 6;  // accumulator group reduced by this wave
  if (tg >= NT * MG) return;
  const int t = tg / MG, g = tg % MG;
  const Alpha alpha = FMT == 0 ? make_alpha(a_ts[0], w_ts[0]) : Alpha{1.0f, 0};
  const int col = 16 * g + (lane & 15);  // activation row m
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = red[0][tg][r][lane];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) v += red[w2][tg][r][lane];
    const int row = (nt0 + t) * 16 + 4 * (lane >> 4) + r;  // output column n
    if (col < m && row < n) c[(int64_t)col * ldc + row] = f32_to_bf16_rne(apply_alpha(v, alpha));
  }
}

// ------------------------------------------------------------ decode, ring
//
// The same skinny GEMM (one workgroup per one or two 16-row weight tiles, its
// waves split over K, partial sums added in LDS in a fixed order) with its operands read
// through a ring of kRingDepth register slots per wave: slot d is consumed and
// at once refilled with the fragment kRingDepth steps ahead. Every operand is
// read with a buffer load whose resource ends at the operand's last valid
// byte; reads past it (fragments past K, activation rows past M, tiles past N)
// return zero. The loop body has no memory access under a branch, which keeps
// the compiler's wait counts exact: a slot waits only for its own loads. NVFP4
// uses it: its per-fragment dequantization then overlaps the next fragments'
// loads (decode benchmark, GEMM kernels only: 142 -> 131 us per step). MXFP4,
// whose fragments cost one matrix instruction, measured slower with any ring
// depth than with the group-of-two loads of k_gemm_decode (97 us: 104, 109,
// 113 and 125 us at depths 1 to 4).
constexpr int kRingWaves = 8;
constexpr int kRingDepth = 2;

typedef unsigned int u4v __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at p (raw, stride 0; gfx9 word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u4v v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int FMT>
__device__ __forceinline__ uint32_t buf_load_scale(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if (FMT == 0) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// The operand pointers are not declared __restrict__: the compiler would then
// take the buffer loads as invariant and move them across the ordering
// statements below.
template <int FMT, int MG, int ATILED, int NT, int NWT>
__global__ __launch_bounds__(64 * NWT) void k_gemm_decode_ring(
    const uint8_t *a_codes, int64_t a_cp, const uint8_t *a_sc, int64_t a_sp,
    const float *__restrict__ a_ts, const uint8_t *w_codes, const uint8_t *w_sc,
    const float *__restrict__ w_ts, int m, int n, int kt_n, int nt_n, uint16_t *c, int64_t ldc) {
  constexpr int NW = NWT, D = kRingDepth;
  constexpr int SFB = FMT == 0 ? 128 : 64;  // scale bytes per fragment
  __shared__ float red[NW][NT * MG][4][64];
  const int nt0 = blockIdx.x * NT;  // first of this workgroup's NT weight tiles
  // readfirstlane makes the wave index (and every guard derived from it) a
  // scalar, so guards compile to branches rather than to EXEC masks that a
  // matrix instruction would not honour.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tiles = min(NT, nt_n - nt0);
  const __amdgpu_buffer_rsrc_t wr = buf_rsrc(w_codes + (int64_t)nt0 * kt_n * kFragCodeBytes,
                                             (uint32_t)(tiles * kt_n * kFragCodeBytes));
  const __amdgpu_buffer_rsrc_t wsr = buf_rsrc(w_sc + (int64_t)nt0 * kt_n * SFB,
                                              (uint32_t)(tiles * kt_n * SFB));
  // Activations: tiled = ceil(m / 16) groups of kt_n fragments; canonical =
  // m rows of pitch a_cp (codes) and a_sp (scales).
  const int ag = (m + 15) >> 4;
  const __amdgpu_buffer_rsrc_t ar =
      buf_rsrc(a_codes, (uint32_t)(ATILED ? (int64_t)ag * kt_n * kFragCodeBytes : (int64_t)m * a_cp));
  const __amdgpu_buffer_rsrc_t asr =
      buf_rsrc(a_sc, (uint32_t)(ATILED ? (int64_t)ag * kt_n * SFB : (int64_t)m * a_sp));
  const int lr = lane & 15, lc = lane >> 4;

  v4f acc[NT][MG];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < MG; ++g) acc[t][g] = v4f{0.f, 0.f, 0.f, 0.f};
  uint4 wq[D][NT], aq[D][MG];
  uint32_t ws[D][NT], as[D][MG];

  // Byte offsets of fragment kt. Loads that must not happen (kt >= kt_n,
  // activation rows >= m) take an offset past every resource's end (each is
  // below 2^31 bytes), so they return zero without reading memory.
  constexpr uint32_t kOut = 0x80000000u;
  auto issue = [&](int d, int kt) {
    const bool kin = kt < kt_n;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t f = (uint32_t)(t * kt_n + kt);
      wq[d][t] = buf_load16(wr, kin ? f * kFragCodeBytes + lane * 16 : kOut);
      ws[d][t] = buf_load_scale<FMT>(wsr, kin ? f * SFB + lane * (FMT == 0 ? 2 : 1) : kOut);
    }
#pragma unroll
    for (int g = 0; g < MG; ++g) {
      const int row = 16 * g + lr;
      uint32_t co = kOut, so = kOut;
      if (kin && row < m) {
        if (ATILED) {
          const uint32_t f = (uint32_t)(g * kt_n + kt);
          co = f * kFragCodeBytes + lane * 16;
          so = f * SFB + lane * (FMT == 0 ? 2 : 1);
        } else {
          co = (uint32_t)((int64_t)row * a_cp + kt * 64 + lc * 16);
          so = (uint32_t)((int64_t)row * a_sp + kt * (FMT == 0 ? 8 : 4) + lc * (FMT == 0 ? 2 : 1));
        }
      }
      aq[d][g] = buf_load16(ar, co);
      as[d][g] = buf_load_scale<FMT>(asr, so);
    }
  };
  auto compute = [&](int d) {
    if (FMT == 1) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int g = 0; g < MG; ++g) acc[t][g] = mfma_mx(wq[d][t], aq[d][g], acc[t][g], ws[d][t], as[d][g]);
    } else {
      // each activation group is dequantized once for the NT weight tiles
      h8v wh[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t) nv_dequant32(wq[d][t], ws[d][t], wh[t]);
#pragma unroll
      for (int g = 0; g < MG; ++g) {
        h8v ah[4];
        nv_dequant32(aq[d][g], as[d][g], ah);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t][g] = mfma_nv(wh[t], ah, acc[t][g]);
      }
    }
  };

  const int J = wave < kt_n ? (kt_n - 1 - wave) / NW + 1 : 0;  // this wave's fragments
  // An empty asm statement with a memory clobber between slots keeps the
  // slots' loads in slot order (the order in which they are consumed), so
  // that each slot waits only for its own and older loads.
#pragma unroll
  for (int d = 0; d < D; ++d) {
    issue(d, wave + NW * d);
    asm volatile("" ::: "memory");
  }
  for (int j0 = 0; j0 < J; j0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (j0 + d < J) compute(d);  // wave-uniform; no memory access inside
      issue(d, wave + NW * (j0 + d + D));
      asm volatile("" ::: "memory");
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < MG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][t * MG + g][r][lane] = acc[t][g][r];
  __syncthreads();
  const Alpha alpha = FMT == 0 ? make_alpha(a_ts[0], w_ts[0]) : Alpha{1.0f, 0};
  for (int tg = wave; tg < NT * MG; tg += NW) {  // accumulator groups reduced by this wave
    const int t = tg / MG, g = tg % MG;
    const int col = 16 * g + lr;  // activation row m
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = red[0][tg][r][lane];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) v += red[w2][tg][r][lane];
      const int row = (nt0 + t) * 16 + 4 * lc + r;  // output column n
      if (col < m && row < n) c[(int64_t)col * ldc + row] = f32_to_bf16_rne(apply_alpha(v, alpha));
    }
  }
}

// --------------------------------------------------------- fused linear
//
// Skinny linear with the activation quantization fused in, for activations
// small enough that every workgroup can quantize all of them itself (the
// bf16 tensor is L2-resident): each workgroup issues the loads of its first
// weight fragments, takes the activations' maximum (NVFP4), encodes every
// block exactly as the standalone quantizer does and stages the result in LDS,
// then runs the decode main loop with the activation operand read from LDS.
// No value crosses workgroups and there is no separate quantize launch.
//   NVFP4: LDS holds the activations already dequantized to f16 (q * s_b is
//          exact in f16), so the main loop converts only the weight operand.
//   MXFP4: LDS holds codes and E8M0 bytes for the scaled matrix instruction.
// LDS rows are padded by 16 bytes so the rows of a fragment use other banks.
template <int FMT>
__global__ __launch_bounds__(64 * kDecWaves) void k_linear_decode(
    const uint16_t *__restrict__ x, int m, int k, const float *__restrict__ static_scale,
    const uint8_t *__restrict__ w_codes, const uint8_t *__restrict__ w_sc,
    const float *__restrict__ w_ts, int n, int kt_n, uint16_t *__restrict__ y, int64_t ldy,
    uint32_t recipe) {
  constexpr int NW = kDecWaves, FM = kDecFrags;
  constexpr int B = FMT == 0 ? 16 : 32, V = B / 8;
  const bool rot = recipe & kRecipeRotate;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float red[NW][4][64];
  __shared__ uint32_t lmax[NW];
  // NVFP4: f16 rows of K_pad values; MXFP4: code rows then scale rows
  const int ap = FMT == 0 ? kt_n * 256 + 16 : kt_n * 64 + 16;
  const int sp = kt_n * 4;
  uint8_t *lscales = smem + (size_t)m * ap;
  const int nt = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;

  uint4 wq[2][FM];
  uint32_t ws[2][FM];
  auto load = [&](int buf, int base) {
#pragma unroll
    for (int u = 0; u < FM; ++u) {
      const int kt = base + NW * u;
      if (kt < kt_n) load_w<FMT>(w_codes, w_sc, (int64_t)nt * kt_n + kt, lane, wq[buf][u], ws[buf][u]);
    }
  };
  load(0, wave);

  const int nb = k / B, nb_pad = kt_n * (128 / B), total = m * nb_pad;
  float st = 1.0f;
  if (FMT == 0) {
    if (static_scale) {
      st = *static_scale;
    } else {
      uint32_t amax = 0;
      for (int t = threadIdx.x; t < m * nb; t += 64 * NW) {
        const int r = t / nb, c = t - r * nb;
        const uint4 *src = (const uint4 *)(x + (int64_t)r * k + c * B);
        uint4 v[2] = {src[0], src[1]};
        if (rot) hadamard_block<16>(v);
        amax = max(amax, max(absmax_bits8(v[0]), absmax_bits8(v[1])));
      }
      st = tensor_scale_from_amax(bf16_bits_to_f32(block_max_u32(amax, lmax)));
    }
  }
#pragma unroll 1
  for (int t = threadIdx.x; t < total; t += 64 * NW) {
    const int r = t / nb_pad, c = t - r * nb_pad;
    uint4 v[V];
    if (c < nb) {
      const uint4 *src = (const uint4 *)(x + (int64_t)r * k + c * B);
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = src[i];
      if (rot) hadamard_block<B>(v);
    }
    if constexpr (FMT == 0) {
      uint4 *dst = (uint4 *)(smem + r * ap + c * 32);
      if (c < nb) {
        uint2 q;
        uint32_t sbyte;
        nv_encode_block(v[0], v[1], st, q, sbyte);
        dst[0] = nv_dequant8_u4(q.x, sbyte);
        dst[1] = nv_dequant8_u4(q.y, sbyte);
      } else {
        dst[0] = make_uint4(0u, 0u, 0u, 0u);
        dst[1] = make_uint4(0u, 0u, 0u, 0u);
      }
    } else {
      uint4 q = make_uint4(0u, 0u, 0u, 0u);
      uint32_t sbyte = 0;
      if (c < nb) mx_encode_block(v, q, sbyte, recipe & kRecipeOas);
      *(uint4 *)(smem + r * ap + c * 16) = q;
      lscales[r * sp + c] = (uint8_t)sbyte;
    }
  }
  __syncthreads();

  const int row = lane & 15, lc = lane >> 4;
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, int base) {
#pragma unroll
    for (int u = 0; u < FM; ++u) {
      const int kt = base + NW * u;
      if (kt >= kt_n) break;  // wave-uniform
      if constexpr (FMT == 1) {
        uint4 aq = make_uint4(0u, 0u, 0u, 0u);
        uint32_t as = 0u;
        if (row < m) {
          aq = *(const uint4 *)(smem + row * ap + kt * 64 + lc * 16);
          as = lscales[row * sp + kt * 4 + lc];
        }
        acc = mfma_mx(wq[buf][u], aq, acc, ws[buf][u], as);
      } else {
        h8v wh[4], ah[4];
        nv_dequant32(wq[buf][u], ws[buf][u], wh);
        const uint4 *arow = (const uint4 *)(smem + row * ap + kt * 256 + lc * 64);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          ah[g] = __builtin_bit_cast(h8v, row < m ? arow[g] : make_uint4(0u, 0u, 0u, 0u));
        acc = mfma_nv(wh, ah, acc);
      }
    }
  };
  constexpr int STEP = NW * FM;
  for (int base = wave; base < kt_n; base += 2 * STEP) {
    load(1, base + STEP);
    compute(0, base);
    if (base + STEP >= kt_n) break;
    load(0, base + 2 * STEP);
    compute(1, base + STEP);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  if (wave != 0) return;
  const Alpha alpha = FMT == 0 ? make_alpha(st, w_ts[0]) : Alpha{1.0f, 0};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float sum = red[0][r][lane];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) sum += red[w2][r][lane];
    const int ncol = nt * 16 + 4 * lc + r;
    if (row < m && ncol < n) y[(int64_t)row * ldy + ncol] = f32_to_bf16_rne(apply_alpha(sum, alpha));
  }
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs &g, hipStream_t stream) {
  const int kt_n = (int)(k_pad(g.k) / kFragK);
  const int nt_n = (int)(round_up(g.n, 16) / 16);
  dim3 grid((unsigned)((g.n + 127) / 128), (unsigned)((g.m + 127) / 128));
#define FP4_PRE(F, T)                                                                          \
  hipLaunchKernelGGL((k_gemm_prefill<F, T>), grid, dim3(256), 0, stream, g.a_codes,           \
                     g.a_cpitch, g.a_scales, g.a_spitch, g.a_ts, g.w_codes, g.w_scales, g.w_ts, \
                     (int)g.m, (int)g.n, kt_n, nt_n, g.c, g.ldc)
  if (g.fmt == 0 && !g.a_tiled) FP4_PRE(0, 0);
  else if (g.fmt == 0) FP4_PRE(0, 1);
  else if (!g.a_tiled) FP4_PRE(1, 0);
  else FP4_PRE(1, 1);
#undef FP4_PRE
  return hipGetLastError();
}

hipError_t launch_gemm_decode(const GemmArgs &g, hipStream_t stream) {
  const int kt_n = (int)(k_pad(g.k) / kFragK);
  const int nt_n = (int)(round_up(g.n, 16) / 16);
  const int mg = g.m <= 16 ? 1 : g.m <= 32 ? 2 : g.m <= 64 ? 4 : 8;
  if (g.fmt == 0) {
    // the ring kernel's buffer resources (and offsets) stay below 2^31 bytes
    const int64_t a_bytes = g.a_tiled ? round_up(g.m, 16) / 16 * kt_n * kFragCodeBytes
                                      : g.m * std::max(g.a_cpitch, g.a_spitch) + (int64_t)kt_n * 64;
    if (a_bytes >= (int64_t(1) << 31) || (int64_t)kt_n * kFragCodeBytes >= (int64_t(1) << 30))
      return hipErrorInvalidValue;
    // Two weight tiles per workgroup, so that the activations are loaded and
    // dequantized once per two tiles:
    //  - 1-16 activation rows, 256-511 tiles: 16 waves per workgroup keep the
    //    waves per CU of one tile per 8-wave workgroup (decode shapes with
    //    N = 5120: 7.0 -> 6.5 us at K = 5120, 17.7 -> 14.9 us at K = 17408);
    //    with >= 512 tiles the second tile measured slower at 8 and 16 waves;
    //  - 17-32 activation rows, >= 256 tiles (N = 5120, M = 32: 9.0 -> 7.5 us
    //    at K = 5120, 23.9 -> 18.3 us at K = 17408; N = 17408: 20.4 -> 18.4 us).
    const bool two1 = mg == 1 && nt_n >= 256 && nt_n < 512;
    const bool two2 = mg == 2 && nt_n >= 256;
    const bool two = two1 || two2;
    dim3 grid((unsigned)(two ? (nt_n + 1) / 2 : nt_n));
#define FP4_RING1(G, T, P, W)                                                                   \
  hipLaunchKernelGGL((k_gemm_decode_ring<0, G, T, P, W>), grid, dim3(64 * W), 0, stream,    \
                     g.a_codes, g.a_cpitch, g.a_scales, g.a_spitch, g.a_ts, g.w_codes,      \
                     g.w_scales, g.w_ts, (int)g.m, (int)g.n, kt_n, nt_n, g.c, g.ldc)
#define FP4_RING_T(G, P, W) do { if (g.a_tiled) FP4_RING1(G, 1, P, W); else FP4_RING1(G, 0, P, W); } while (0)
    if (two1) FP4_RING_T(1, 2, 2 * kRingWaves);
    else if (mg == 1) FP4_RING_T(1, 1, kRingWaves);
    else if (two2) FP4_RING_T(2, 2, kRingWaves);
    else if (mg == 2) FP4_RING_T(2, 1, kRingWaves);
    else if (mg == 4) FP4_RING_T(4, 1, kRingWaves);
    else FP4_RING_T(8, 1, kRingWaves);
#undef FP4_RING_T
#undef FP4_RING1
    return hipGetLastError();
  }
  // MXFP4 with 17-32 activation rows: two weight tiles per workgroup when
  // that still leaves >= 256 workgroups, so the activations are read once per
  // two tiles (measured: 17.7 -> 15.8 us at M = 32, N = 17408).
  // (at 256-511 tiles it measured mixed: M = 32, N = 5120: 5.7 -> 5.9 us at
  // K = 5120, 18.3 -> 17.4 us at K = 17408)
  const int nt_per = (mg == 2 && nt_n >= 512) ? 2 : 1;
  dim3 grid((unsigned)((nt_n + nt_per - 1) / nt_per));
#define FP4_DEC(F, G, T, P)                                                                     \
  hipLaunchKernelGGL((k_gemm_decode<F, G, T, P>), grid, dim3(64 * kDecWaves), 0, stream,       \
                     g.a_codes, g.a_cpitch, g.a_scales, g.a_spitch, g.a_ts, g.w_codes,         \
                     g.w_scales, g.w_ts, (int)g.m, (int)g.n, kt_n, nt_n, g.c, g.ldc)
#define FP4_DEC_T(F, G, P) do { if (g.a_tiled) FP4_DEC(F, G, 1, P); else FP4_DEC(F, G, 0, P); } while (0)
  if (mg == 1) FP4_DEC_T(1, 1, 1);
  else if (mg == 2 && nt_per == 2) FP4_DEC_T(1, 2, 2);
  else if (mg == 2) FP4_DEC_T(1, 2, 1);
  else if (mg == 4) FP4_DEC_T(1, 4, 1);
  else FP4_DEC_T(1, 8, 1);
#undef FP4_DEC_T
#undef FP4_DEC
  return hipGetLastError();
}

bool linear_fused_ok(int fmt, int64_t m, int64_t n, int64_t k) {
  const int64_t mk = m * k_pad(k);
  // LDS staging bound, and a bound on the redundant quantization work that
  // every weight tile's workgroup repeats.
  // NVFP4's encoding prologue (maximum pass + exact encode) is long enough
  // that only about two workgroups per CU (512 weight tiles) should repeat it,
  // and the separate quantizer plus the skinny GEMM wins once M * K_pad * tiles
  // passes about 4M (320 tiles, measured: K = 5120 fused at M = 2, 11.9 us
  // against 13.5; separate at M = 4, 13.4 us against 15.5, and at M = 1 with
  // K = 17408, 22.4 us against 23.0).
  const int64_t nt = round_up(n, 16) / 16;
  if (fmt == 0)
    return m <= kFusedMaxM && mk <= kFusedMaxMK / 2 && mk * nt <= kFusedMaxWorkNv &&
           nt <= kFusedMaxTilesNv;
  return m <= kFusedMaxM && mk <= kFusedMaxMK && mk * nt <= kFusedMaxWork;
}

hipError_t launch_linear_fused(int fmt, uint32_t recipe, const uint16_t *x, int64_t m, int64_t k,
                               const float *static_scale, const uint8_t *w_codes,
                               const uint8_t *w_scales, const float *w_ts, int64_t n,
                               uint16_t *y, int64_t ldy, hipStream_t stream) {
  const int kt_n = (int)(k_pad(k) / kFragK);
  const int nt_n = (int)(round_up(n, 16) / 16);
  const size_t lds = fmt == 0 ? (size_t)m * (kt_n * 256 + 16)
                              : (size_t)m * (kt_n * 64 + 16) + (size_t)m * kt_n * 4;
  if (fmt == 0)
    hipLaunchKernelGGL(k_linear_decode<0>, dim3(nt_n), dim3(64 * kDecWaves), lds, stream, x,
                       (int)m, (int)k, static_scale, w_codes, w_scales, w_ts, (int)n, kt_n, y, ldy,
                       recipe);
  else
    hipLaunchKernelGGL(k_linear_decode<1>, dim3(nt_n), dim3(64 * kDecWaves), lds, stream, x,
                       (int)m, (int)k, static_scale, w_codes, w_scales, w_ts, (int)n, kt_n, y, ldy,
                       recipe);
  return hipGetLastError();
}

}  // namespace fp4i
