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
#include <atomic>

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

// MXFP4 with macro-block scales: one fragment (K = 128, one 128-value segment
// of both operands) as its own product, added with the segment scales of its
// output rows and columns: acc += p * (s4 * s1), s4 the scales of the lane's
// four accumulator rows, s1 that of its column.
__device__ __forceinline__ v4f mfma_mx_mbs(uint4 a, uint4 b, v4f c, uint32_t sa, uint32_t sb,
                                           float4 s4, float s1) {
  const v4f p = mfma_mx(a, b, v4f{0.f, 0.f, 0.f, 0.f}, sa, sb);
  c[0] = __builtin_fmaf(p[0], s4.x * s1, c[0]);
  c[1] = __builtin_fmaf(p[1], s4.y * s1, c[1]);
  c[2] = __builtin_fmaf(p[2], s4.z * s1, c[2]);
  c[3] = __builtin_fmaf(p[3], s4.w * s1, c[3]);
  return c;
}

// Macro-block scale of activation row `row` at fragment kt (0 past m).
template <int ATILED>
__device__ __forceinline__ float a_macro(const float *a_ms, int64_t a_mp, int kt_n, int row, int kt,
                                         int m) {
  if (row >= m) return 0.f;
  return ATILED ? a_ms[((int64_t)(row >> 4) * kt_n + kt) * 16 + (row & 15)]
                : a_ms[(int64_t)row * a_mp + kt];
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

// ------------------------------------------------- decode, single launch
//
// fp4_linear for 1-32 activation rows as one launch of the skinny GEMM: its
// first nprod workgroups quantize the activations into the workspace's tiled
// layout, one wave per 16-row fragment, with device-coherent stores, and
// count themselves in a ready word once their stores are complete; the GEMM
// workgroups (numbered after them) issue their first weight loads, wait,
// bounded, for the count, and only then load the activations. The count is
// kept in kReadyCopies words on lines of their own (producers add to all, GEMM
// workgroup b polls copy b % kReadyCopies with one wave): with every wave of
// a thousand resident workgroups polling one word, the polls swamped that
// word's memory channel and the decode calls ran 1.3-3x slower. Dispatch
// follows the workgroup index, so the producers are running before any
// GEMM workgroup waits for them. NVFP4 with a dynamic tensor scale: the
// producers first exchange their maxima (group_max_u32), as the single-launch
// quantizer's workgroups do, and the last to arrive publishes S_t. A wait
// that gives up sets the sticky error flag and makes the output NaN; the last
// GEMM workgroup to pass its wait resets the ready word for the next call.
struct DecFused {
  const uint16_t *x;   // bf16 activations [m, k]
  const float *st;     // NVFP4 static tensor scale (device), or null
  uint32_t *ts_out;    // NVFP4 dynamic: the tensor scale's bits go here
  uint32_t *slots;     // tagged maximum slots (kActGrid, kSlotStride words apart)
  uint32_t *err;       // sticky error flags
  uint32_t *arrive;    // producers past the exchange (low half), gave up (high half)
  uint32_t *ready;     // [r * kSlotStride] (r < kReadyCopies) producers done;
                       // [kReadyCopies * kSlotStride] GEMM workgroups past their wait
  int nprod, k;
  uint32_t recipe, spin;
};

// Fragments per producer wave at most: one, so that the producers' registers
// stay below the GEMM workgroups' (the kernel's count is the larger of the two).
constexpr int kDecProdFrags = 1;
constexpr int kReadyCopies = 16;
static_assert((kReadyCopies + 1) * kSlotStride <= 2 * kMaxPanels,
              "the ready words fit the quantize scratch's panel words");

// Producer p of the single-launch decode linear: fragments p * NW + wave +
// u * nprod * NW (u < kDecProdFrags) of the activations' tiled layout.
template <int FMT, int NW>
__device__ void decode_produce(const DecFused &fz, int m, int kt_n, uint8_t *a_codes,
                               uint8_t *a_sc, uint32_t *lds) {
  constexpr int SCB = FMT == 0 ? 128 : 64, U = kDecProdFrags;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, r = lane & 15, c = lane >> 4;
  const int nfr = ((m + 15) >> 4) * kt_n, P = fz.nprod, p = blockIdx.x;
  uint4 v[U][4];
  uint32_t amax = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int f = p * NW + wave + u * P * NW;
    const int row = (f / kt_n) * 16 + r, k0 = (f % kt_n) * kFragK + 32 * c;
    const bool live = f < nfr && row < m;
    const uint4 *src = (const uint4 *)(fz.x + (int64_t)row * fz.k + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[u][j] = (live && k0 + 8 * j < fz.k) ? src[j] : make_uint4(0u, 0u, 0u, 0u);
  }
  // (no rotation here: its code would raise the kernel's register count for
  // every call; rotated activations take the two-launch path)
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = max(amax, absmax_bits8(v[u][j]));
  float st = 1.0f;
  if (FMT == 0) {
    if (fz.st) {
      st = *fz.st;
    } else {
      // this call's tag: one more than the previous call's (slot p is written
      // only by producer p)
      const uint32_t tag = ((__hip_atomic_load(&fz.slots[p * kSlotStride], __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) >> 16) + 1u) & 0xFFFFu;
      const uint32_t g = group_max_u32<kActGrid, kSlotStride>(block_max_u32(amax, lds), tag,
                                                              fz.slots, p, P, fz.spin, lds);
      const bool gave_up = g >= 0x8000u;
      st = gave_up ? __builtin_nanf("") : tensor_scale_from_amax(bf16_bits_to_f32(g));
      if (threadIdx.x == 0) {
        if (gave_up)
          __hip_atomic_fetch_or(fz.err, kErrExchangeTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t before = __hip_atomic_fetch_add(fz.arrive, gave_up ? 0x10001u : 1u,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((before & 0xFFFFu) == (uint32_t)P - 1) {
          // the last producer past the exchange: every other one has decided
          const bool any = gave_up || (before >> 16) != 0u;
          __hip_atomic_store(fz.ts_out, __float_as_uint(any ? __builtin_nanf("") : st),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(fz.arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int f = p * NW + wave + u * P * NW;
    if (f >= nfr) break;  // wave-uniform
    const int row = (f / kt_n) * 16 + r, k0 = (f % kt_n) * kFragK + 32 * c;
    uint4 q = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (FMT == 0) {
      uint2 c0 = make_uint2(0u, 0u), c1 = make_uint2(0u, 0u);
      uint32_t s0 = 0, s1 = 0;
      if (row < m && k0 < fz.k) nv_encode_block(v[u][0], v[u][1], st, c0, s0);
      if (row < m && k0 + 16 < fz.k) nv_encode_block(v[u][2], v[u][3], st, c1, s1);
      q = make_uint4(c0.x, c0.y, c1.x, c1.y);
      store2_dev(dev_rsrc(a_sc + (int64_t)f * SCB, SCB), lane * 2, s0 | (s1 << 8));
    } else {
      uint32_t sc = 0;
      if (row < m && k0 < fz.k) mx_encode_block(v[u], q, sc, fz.recipe & kRecipeOas);
      store1_dev(dev_rsrc(a_sc + (int64_t)f * SCB, SCB), lane, sc);
    }
    store16_dev(dev_rsrc(a_codes + (int64_t)f * kFragCodeBytes, kFragCodeBytes), lane * 16, q);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are complete
  __syncthreads();
  if (threadIdx.x < kReadyCopies)
    __hip_atomic_fetch_add(&fz.ready[threadIdx.x * kSlotStride], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// A GEMM workgroup's wait for the producers: wave 0 polls its copy of the
// count (bounded), the workgroup's barrier releases the other waves. Returns
// whether the wait gave up (every thread gets the answer), having set the
// sticky flag. `flag`: one LDS word.
__device__ __forceinline__ bool decode_wait(const DecFused &fz, uint32_t *flag) {
  if (threadIdx.x < 64) {
    const uint32_t b = blockIdx.x - (uint32_t)fz.nprod;
    const uint32_t *word = &fz.ready[(b % kReadyCopies) * kSlotStride];
    bool ok = false;
    for (uint32_t it = 0; it < fz.spin; ++it) {
      if (__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)fz.nprod) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (threadIdx.x == 0) {
      if (!ok)
        __hip_atomic_fetch_or(fz.err, kErrExchangeTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = ok ? 0u : 1u;
    }
  }
  __syncthreads();
  return *flag != 0u;
}

// After every wave of the workgroup has passed its wait (thread 0): the last
// GEMM workgroup resets the ready words.
__device__ __forceinline__ void decode_finish(const DecFused &fz) {
  const uint32_t ngemm = gridDim.x - (uint32_t)fz.nprod;
  uint32_t *fin = &fz.ready[kReadyCopies * kSlotStride];
  const uint32_t done = __hip_atomic_fetch_add(fin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (done == ngemm - 1) {
    for (int r = 0; r < kReadyCopies; ++r)
      __hip_atomic_store(&fz.ready[r * kSlotStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(fin, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The activation pointers, as the loads after a wait must see them: an empty
// asm statement that "changes" them, so that no load through them can be
// moved above the wait.
template <typename T>
__device__ __forceinline__ T *after_wait(T *p) {
  asm volatile("" : "+s"(p)::"memory");
  return p;
}

// ------------------------------------------------------------------ prefill
//
// Workgroup tile 128 x 128 (4 waves in a 2 x 2 grid, 64 x 64 per wave as
// 4 x 4 tiles of 16 x 16). Operands are read per lane straight into the MFMA
// operand registers: an A fragment lane l reads 16 bytes of row (l % 16) at
// K offset 32 (l / 16) of the canonical layout; a W fragment is one 1 KB
// contiguous tile of the weight cache.
// MB: MXFP4 with macro-block scales (a_ms, w_ms).
template <int FMT, int ATILED, int MB = 0>
__global__ __launch_bounds__(256) void k_gemm_prefill(
    const uint8_t *__restrict__ a_codes, int64_t a_cp, const uint8_t *__restrict__ a_sc,
    int64_t a_sp, const float *__restrict__ a_ts, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_sc, const float *__restrict__ w_ts, int m, int n, int kt_n,
    int nt_n, uint16_t *__restrict__ c, int64_t ldc, const float *__restrict__ a_ms,
    int64_t a_mp, const float *__restrict__ w_ms) {
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
    if (FMT == 1 && MB) {
      // accumulator rows are activation rows 16 i + 4 lc + r, its column the
      // weight row 16 j + lr
      float4 sa[4];
      float sw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = m0 + 16 * i + 4 * lc;
        sa[i] = make_float4(a_macro<ATILED>(a_ms, a_mp, kt_n, r0, kt, m),
                            a_macro<ATILED>(a_ms, a_mp, kt_n, r0 + 1, kt, m),
                            a_macro<ATILED>(a_ms, a_mp, kt_n, r0 + 2, kt, m),
                            a_macro<ATILED>(a_ms, a_mp, kt_n, r0 + 3, kt, m));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sw[j] = nt0 + j < nt_n ? w_ms[((int64_t)(nt0 + j) * kt_n + kt) * 16 + lr] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mfma_mx_mbs(aq[i], wq[j], acc[i][j], as[i], ws[j], sa[i], sw[j]);
    } else if (FMT == 1) {
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

// MB: MXFP4 with macro-block scales (a_ms, w_ms): each fragment's product is
// added with its rows' and columns' segment scales.
// FUSED: the single-launch linear (DecFused): the first fz.nprod workgroups
// quantize the activations, the rest wait for them after their first weight
// loads.
template <int FMT, int MG, int ATILED, int NT, int MB = 0, int FUSED = 0>
__global__ __launch_bounds__(64 * kDecWaves) void k_gemm_decode(
    const uint8_t *__restrict__ a_codes, int64_t a_cp, const uint8_t *__restrict__ a_sc,
    int64_t a_sp, const float *__restrict__ a_ts, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_sc, const float *__restrict__ w_ts, int m, int n, int kt_n,
    int nt_n, uint16_t *__restrict__ c, int64_t ldc, const float *__restrict__ a_ms,
    int64_t a_mp, const float *__restrict__ w_ms, DecFused fz) {
  // fragments per group: two, or one for eight activation groups (registers)
  constexpr int NW = kDecWaves, FM = MG >= 8 ? 1 : kDecFrags;
  __shared__ float red[NW][NT * MG][4][64];
  if (FUSED && (int)blockIdx.x < fz.nprod) {
    decode_produce<FMT, NW>(fz, m, kt_n, (uint8_t *)a_codes, (uint8_t *)a_sc, (uint32_t *)red);
    return;
  }
  // first of this workgroup's NT weight tiles
  const int nt0 = (FUSED ? (int)blockIdx.x - fz.nprod : (int)blockIdx.x) * NT;
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
  float4 wm[2][FM][NT];   // MB: the lane's four weight rows' segment scales
  float am[2][FM][MG];    // MB: its activation row's

  auto load = [&](int buf, int base, bool lw = true, bool la = true) {
#pragma unroll
    for (int u = 0; u < FM; ++u) {
      const int kt = base + NW * u;
      if (kt < kt_n) {
        if (lw) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            // a tile past the last one reads the last again (its sums are never stored)
            const int nt = min(nt0 + t, nt_n - 1);
            load_w<FMT>(w_codes, w_sc, (int64_t)nt * kt_n + kt, lane, wq[buf][u][t], ws[buf][u][t]);
            if (MB)
              wm[buf][u][t] = *(const float4 *)(w_ms + ((int64_t)nt * kt_n + kt) * 16 + 4 * (lane >> 4));
          }
        }
        if (la) {
#pragma unroll
          for (int g = 0; g < MG; ++g) {
            load_a<FMT, ATILED>(a_codes, a_cp, a_sc, a_sp, kt_n, g, kt, lane, m, aq[buf][u][g],
                                as[buf][u][g]);
            if (MB) am[buf][u][g] = a_macro<ATILED>(a_ms, a_mp, kt_n, 16 * g + (lane & 15), kt, m);
          }
        }
      }
    }
  };
  auto compute = [&](int buf, int base) {
#pragma unroll
    for (int u = 0; u < FM; ++u) {
      if (base + NW * u >= kt_n) break;  // wave-uniform
      if (FMT == 1 && MB) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int g = 0; g < MG; ++g)
            acc[t][g] = mfma_mx_mbs(wq[buf][u][t], aq[buf][u][g], acc[t][g], ws[buf][u][t],
                                    as[buf][u][g], wm[buf][u][t], am[buf][u][g]);
      } else if (FMT == 1) {
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
  bool gave_up = false;
  if (FUSED) {
    load(0, wave, true, false);
    __shared__ uint32_t wait_flag;
    gave_up = decode_wait(fz, &wait_flag);
    a_codes = after_wait(a_codes);
    a_sc = after_wait(a_sc);
    load(0, wave, false, true);
  } else {
    load(0, wave);
  }
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
      for (int r = 0; r < 4; ++r)
        red[wave][t * MG + g][r][lane] = gave_up ? __builtin_nanf("") : acc[t][g][r];
  __syncthreads();
  if (FUSED && threadIdx.x == 0) decode_finish(fz);
  const int tg = threadIdx.x >> 6;  // accumulator group reduced by this wave
  if (tg >= NT * MG) return;
  const int t = tg / MG, g = tg % MG;
  // (the single-launch linear's dynamic S_t is written during this launch)
  const float sa = FMT != 0 ? 1.0f
                   : FUSED ? __uint_as_float(__hip_atomic_load((const uint32_t *)a_ts, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT))
                           : a_ts[0];
  const Alpha alpha = FMT == 0 ? make_alpha(sa, w_ts[0]) : Alpha{1.0f, 0};
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
// FUSED: the single-launch linear, as in k_gemm_decode.
template <int FMT, int MG, int ATILED, int NT, int NWT, int FUSED = 0>
__global__ __launch_bounds__(64 * NWT) void k_gemm_decode_ring(
    const uint8_t *a_codes, int64_t a_cp, const uint8_t *a_sc, int64_t a_sp,
    const float *__restrict__ a_ts, const uint8_t *w_codes, const uint8_t *w_sc,
    const float *__restrict__ w_ts, int m, int n, int kt_n, int nt_n, uint16_t *c, int64_t ldc,
    DecFused fz) {
  constexpr int NW = NWT, D = kRingDepth;
  constexpr int SFB = FMT == 0 ? 128 : 64;  // scale bytes per fragment
  __shared__ float red[NW][NT * MG][4][64];
  if (FUSED && (int)blockIdx.x < fz.nprod) {
    decode_produce<FMT, NW>(fz, m, kt_n, (uint8_t *)a_codes, (uint8_t *)a_sc, (uint32_t *)red);
    return;
  }
  // first of this workgroup's NT weight tiles
  const int nt0 = (FUSED ? (int)blockIdx.x - fz.nprod : (int)blockIdx.x) * NT;
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
  const uint32_t a_bytes = (uint32_t)(ATILED ? (int64_t)ag * kt_n * kFragCodeBytes : (int64_t)m * a_cp);
  const uint32_t as_bytes = (uint32_t)(ATILED ? (int64_t)ag * kt_n * SFB : (int64_t)m * a_sp);
  // (rebuilt after the wait in the single-launch linear)
  __amdgpu_buffer_rsrc_t ar = buf_rsrc(a_codes, a_bytes), asr = buf_rsrc(a_sc, as_bytes);
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
  auto issue = [&](int d, int kt, bool lw = true, bool la = true) {
    const bool kin = kt < kt_n;
    if (lw) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t f = (uint32_t)(t * kt_n + kt);
        wq[d][t] = buf_load16(wr, kin ? f * kFragCodeBytes + lane * 16 : kOut);
        ws[d][t] = buf_load_scale<FMT>(wsr, kin ? f * SFB + lane * (FMT == 0 ? 2 : 1) : kOut);
      }
    }
    if (!la) return;
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
  bool gave_up = false;
  if (FUSED) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      issue(d, wave + NW * d, true, false);
      asm volatile("" ::: "memory");
    }
    __shared__ uint32_t wait_flag;
    gave_up = decode_wait(fz, &wait_flag);
    ar = buf_rsrc(after_wait(a_codes), a_bytes);
    asr = buf_rsrc(after_wait(a_sc), as_bytes);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      issue(d, wave + NW * d, false, true);
      asm volatile("" ::: "memory");
    }
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      issue(d, wave + NW * d);
      asm volatile("" ::: "memory");
    }
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
      for (int r = 0; r < 4; ++r)
        red[wave][t * MG + g][r][lane] = gave_up ? __builtin_nanf("") : acc[t][g][r];
  __syncthreads();
  if (FUSED && threadIdx.x == 0) decode_finish(fz);
  // (the single-launch linear's dynamic S_t is written during this launch)
  const float sa = FMT != 0 ? 1.0f
                   : FUSED ? __uint_as_float(__hip_atomic_load((const uint32_t *)a_ts, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT))
                           : a_ts[0];
  const Alpha alpha = FMT == 0 ? make_alpha(sa, w_ts[0]) : Alpha{1.0f, 0};
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

// ------------------------------------------------------------ mid-size M
//
// 33-128 activation rows (tiled activations, no macro-block scales). The
// skinny kernels give each 16-row weight tile its own workgroup, so at these
// sizes every workgroup loads all M activation rows (and, NVFP4, dequantizes
// them) for 16 output columns: the activation side, not the weight stream,
// bounds them. Here a workgroup takes kMidTiles consecutive weight tiles (64
// output columns) for all the rows, over one of S slices of K, and its four
// waves split the slice's fragments (wave w: fragments kb + w, kb + w + 4,
// ...), so each activation fragment a wave loads and converts serves four
// weight tiles. The waves' sums meet in LDS in a fixed order; with S > 1 each
// workgroup writes its slice's FP32 sums to `part` [S][m][n] and k_mid_sum
// adds the slices in order, so the result does not depend on timing.
constexpr int kMidTiles = 4;
constexpr int kMidWaves = 4;

template <int FMT, int MG>
__global__ __launch_bounds__(64 * kMidWaves) void k_gemm_mid(
    const uint8_t *a_codes, const uint8_t *a_sc, const float *__restrict__ a_ts,
    const uint8_t *w_codes, const uint8_t *w_sc, const float *__restrict__ w_ts, int m, int n,
    int kt_n, int nt_n, int kps, uint16_t *c, int64_t ldc, float *part) {
  constexpr int NT = kMidTiles, NW = kMidWaves, D = kRingDepth;
  constexpr int SFB = FMT == 0 ? 128 : 64;  // scale bytes per fragment
  constexpr int SLOTS = NT * MG * 4;         // accumulator values per lane
  __shared__ float red[2][SLOTS][64];
  const int nt0 = (int)blockIdx.x * NT;
  const int split = (int)blockIdx.y;
  const int kb = split * kps, ke = min(kt_n, kb + kps);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tiles = min(NT, nt_n - nt0);
  const __amdgpu_buffer_rsrc_t wr = buf_rsrc(w_codes + (int64_t)nt0 * kt_n * kFragCodeBytes,
                                             (uint32_t)(tiles * kt_n * kFragCodeBytes));
  const __amdgpu_buffer_rsrc_t wsr = buf_rsrc(w_sc + (int64_t)nt0 * kt_n * SFB,
                                              (uint32_t)(tiles * kt_n * SFB));
  const int ag = (m + 15) >> 4;
  const __amdgpu_buffer_rsrc_t ar = buf_rsrc(a_codes, (uint32_t)(ag * kt_n * kFragCodeBytes));
  const __amdgpu_buffer_rsrc_t asr = buf_rsrc(a_sc, (uint32_t)(ag * kt_n * SFB));
  const int lr = lane & 15, lc = lane >> 4;

  v4f acc[NT][MG];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < MG; ++g) acc[t][g] = v4f{0.f, 0.f, 0.f, 0.f};
  uint4 wq[D][NT], aq[D][MG];
  uint32_t ws[D][NT], as[D][MG];

  // Loads that must not happen (fragments past the slice, tiles past n,
  // activation rows past m) take an offset past every resource's end (each
  // below 2^31 bytes): they return zero without reading memory.
  constexpr uint32_t kOut = 0x80000000u;
  auto issue = [&](int d, int kt) {
    const bool kin = kt < ke;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t f = (uint32_t)(t * kt_n + kt);
      const bool in = kin && t < tiles;
      wq[d][t] = buf_load16(wr, in ? f * kFragCodeBytes + lane * 16 : kOut);
      ws[d][t] = buf_load_scale<FMT>(wsr, in ? f * SFB + lane * (FMT == 0 ? 2 : 1) : kOut);
    }
#pragma unroll
    for (int g = 0; g < MG; ++g) {
      const uint32_t f = (uint32_t)(g * kt_n + kt);
      const bool in = kin && 16 * g + lr < m;
      aq[d][g] = buf_load16(ar, in ? f * kFragCodeBytes + lane * 16 : kOut);
      as[d][g] = buf_load_scale<FMT>(asr, in ? f * SFB + lane * (FMT == 0 ? 2 : 1) : kOut);
    }
  };
  auto compute = [&](int d) {
    if (FMT == 1) {
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t][g] = mfma_mx(wq[d][t], aq[d][g], acc[t][g], ws[d][t], as[d][g]);
    } else {
      // each activation fragment is dequantized once for the NT weight tiles
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

  const int first = kb + wave;
  const int J = first < ke ? (ke - 1 - first) / NW + 1 : 0;  // this wave's fragments
  // (an empty asm statement with a memory clobber between slots keeps the
  // slots' loads in the order they are consumed, as in the ring kernel)
#pragma unroll
  for (int d = 0; d < D; ++d) {
    issue(d, first + NW * d);
    asm volatile("" ::: "memory");
  }
  for (int j0 = 0; j0 < J; j0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (j0 + d < J) compute(d);  // wave-uniform; no memory access inside
      issue(d, first + NW * (j0 + d + D));
      asm volatile("" ::: "memory");
    }
  }

  // waves 2, 3 hand their sums to waves 0, 1; those then to everyone:
  // value = (sum of waves 0 and 2) + (sum of waves 1 and 3)
  if (wave >= 2) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave - 2][(t * MG + g) * 4 + r][lane] = acc[t][g][r];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][g][r] += red[wave][(t * MG + g) * 4 + r][lane];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][(t * MG + g) * 4 + r][lane] = acc[t][g][r];
  }
  __syncthreads();
  // wave w writes weight tile nt0 + w
  const int t = wave;
  const int col0 = (nt0 + t) * 16 + 4 * lc;  // output columns col0 .. col0 + 3
  const Alpha alpha = FMT == 0 ? make_alpha(a_ts[0], w_ts[0]) : Alpha{1.0f, 0};
#pragma unroll
  for (int g = 0; g < MG; ++g) {
    const int row = 16 * g + lr;  // activation row
    if (row >= m) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = (t * MG + g) * 4 + r;
      const float v = red[0][i][lane] + red[1][i][lane];
      const int col = col0 + r;
      if (col >= n) continue;
      if (part) part[((int64_t)split * m + row) * n + col] = v;
      else c[(int64_t)row * ldc + col] = f32_to_bf16_rne(apply_alpha(v, alpha));
    }
  }
}

// The slices' partial sums of k_gemm_mid added in slice order, scaled and
// rounded: c[row, col] = bf16_RNE(alpha * (((p_0 + p_1) + p_2) + ...)).
__global__ __launch_bounds__(256) void k_mid_sum(const float *__restrict__ part, int splits, int m,
                                                 int n, int fmt, const float *__restrict__ a_ts,
                                                 const float *__restrict__ w_ts, uint16_t *c,
                                                 int64_t ldc) {
  const int64_t mn = (int64_t)m * n;
  const Alpha alpha = fmt == 0 ? make_alpha(a_ts[0], w_ts[0]) : Alpha{1.0f, 0};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v = part[i];
    for (int s = 1; s < splits; ++s) v += part[s * mn + i];
    const int64_t row = i / n, col = i - row * n;
    c[row * ldc + col] = f32_to_bf16_rne(apply_alpha(v, alpha));
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
  // (rotated and macro-block-scaled activations never come here: the host
  // sends them to the separate quantizer, and leaving their code out keeps
  // this kernel's registers low)
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
#define FP4_PRE(F, T, MB)                                                                      \
  hipLaunchKernelGGL((k_gemm_prefill<F, T, MB>), grid, dim3(256), 0, stream, g.a_codes,       \
                     g.a_cpitch, g.a_scales, g.a_spitch, g.a_ts, g.w_codes, g.w_scales, g.w_ts, \
                     (int)g.m, (int)g.n, kt_n, nt_n, g.c, g.ldc, g.a_ms, g.a_mpitch, g.w_ms)
  const bool mb = g.fmt == 1 && g.w_ms;
  if (g.fmt == 0 && !g.a_tiled) FP4_PRE(0, 0, 0);
  else if (g.fmt == 0) FP4_PRE(0, 1, 0);
  else if (mb && !g.a_tiled) FP4_PRE(1, 0, 1);
  else if (mb) FP4_PRE(1, 1, 1);
  else if (!g.a_tiled) FP4_PRE(1, 0, 0);
  else FP4_PRE(1, 1, 0);
#undef FP4_PRE
  return hipGetLastError();
}

namespace {

// The skinny GEMM's launch; with fz, the single-launch linear (tiled
// activations, at most 32 rows, no macro-block scales: checked by the caller),
// whose grid is fz->nprod producers followed by the GEMM workgroups. The
// producer count is set here from the chosen kernel's waves.
hipError_t decode_launch(const GemmArgs &g, DecFused *fz, hipStream_t stream) {
  const int kt_n = (int)(k_pad(g.k) / kFragK);
  const int nt_n = (int)(round_up(g.n, 16) / 16);
  const int mg = g.m <= 16 ? 1 : g.m <= 32 ? 2 : g.m <= 64 ? 4 : 8;
  const int nfr = (int)(round_up(g.m, 16) / 16) * kt_n;
  auto producers = [&](int waves) {
    if (!fz) return 0;
    fz->nprod = std::min(kActGrid, (nfr + waves * kDecProdFrags - 1) / (waves * kDecProdFrags));
    return fz->nprod;
  };
  const DecFused none{};
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
    const int ngemm = two ? (nt_n + 1) / 2 : nt_n;
#define FP4_RING1(G, T, P, W, FU)                                                                   \
  hipLaunchKernelGGL((k_gemm_decode_ring<0, G, T, P, W, FU>), dim3((unsigned)(ngemm + producers(W))), \
                     dim3(64 * W), 0, stream, g.a_codes, g.a_cpitch, g.a_scales, g.a_spitch, g.a_ts,  \
                     g.w_codes, g.w_scales, g.w_ts, (int)g.m, (int)g.n, kt_n, nt_n, g.c, g.ldc,       \
                     fz ? *fz : none)
#define FP4_RING_T(G, P, W)                         \
  do {                                              \
    if (fz) FP4_RING1(G, 1, P, W, 1);               \
    else if (g.a_tiled) FP4_RING1(G, 1, P, W, 0);   \
    else FP4_RING1(G, 0, P, W, 0);                  \
  } while (0)
#define FP4_RING_N(G, P, W)                         \
  do {                                              \
    if (g.a_tiled) FP4_RING1(G, 1, P, W, 0);        \
    else FP4_RING1(G, 0, P, W, 0);                  \
  } while (0)
    if (two1) FP4_RING_T(1, 2, 2 * kRingWaves);
    else if (mg == 1) FP4_RING_T(1, 1, kRingWaves);
    else if (two2) FP4_RING_T(2, 2, kRingWaves);
    else if (mg == 2) FP4_RING_T(2, 1, kRingWaves);
    else if (mg == 4) FP4_RING_N(4, 1, kRingWaves);
    else FP4_RING_N(8, 1, kRingWaves);
#undef FP4_RING_N
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
  const int ngemm = (nt_n + nt_per - 1) / nt_per;
#define FP4_DEC(F, G, T, P, MB, FU)                                                                  \
  hipLaunchKernelGGL((k_gemm_decode<F, G, T, P, MB, FU>), dim3((unsigned)(ngemm + producers(kDecWaves))), \
                     dim3(64 * kDecWaves), 0, stream, g.a_codes, g.a_cpitch, g.a_scales, g.a_spitch,    \
                     g.a_ts, g.w_codes, g.w_scales, g.w_ts, (int)g.m, (int)g.n, kt_n, nt_n, g.c, g.ldc, \
                     g.a_ms, g.a_mpitch, g.w_ms, fz ? *fz : none)
#define FP4_DEC_N(F, G, P)                                                       \
  do {                                                                           \
    if (g.w_ms) {                                                                \
      if (g.a_tiled) FP4_DEC(F, G, 1, P, 1, 0); else FP4_DEC(F, G, 0, P, 1, 0); \
    } else {                                                                     \
      if (g.a_tiled) FP4_DEC(F, G, 1, P, 0, 0); else FP4_DEC(F, G, 0, P, 0, 0); \
    }                                                                            \
  } while (0)
#define FP4_DEC_T(F, G, P)                        \
  do {                                            \
    if (fz) FP4_DEC(F, G, 1, P, 0, 1);            \
    else FP4_DEC_N(F, G, P);                      \
  } while (0)
  if (mg == 1) FP4_DEC_T(1, 1, 1);
  else if (mg == 2 && nt_per == 2) FP4_DEC_T(1, 2, 2);
  else if (mg == 2) FP4_DEC_T(1, 2, 1);
  else if (mg == 4) FP4_DEC_N(1, 4, 1);
  else FP4_DEC_N(1, 8, 1);
#undef FP4_DEC_T
#undef FP4_DEC_N
#undef FP4_DEC
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_decode(const GemmArgs &g, hipStream_t stream) {
  return decode_launch(g, nullptr, stream);
}

namespace {
std::atomic<int> g_mid{1};
}  // namespace

int mid_gemm() { return g_mid.load(std::memory_order_relaxed); }
int set_mid_gemm(int on) { return g_mid.exchange(on ? 1 : 0, std::memory_order_relaxed); }

// The slice count: at most one workgroup per CU (a workgroup holds all four
// SIMDs' registers, so a second round of workgroups costs a whole slice:
// measured, 270 workgroups for 256 CUs took 1.4x as long as 180), each wave
// keeping at least one fragment, the partial sums within `cap`. The kernel is
// used only where every wave then streams at least kMidMinWaveFrags
// fragments: its fixed costs (the combining launch, the LDS sums, one wave
// per SIMD waiting on its loads) are paid back only over a long stream. Measured
// against the skinny kernel (graph replay, 64 and 128 rows): K x N = 17408 x
// 5120 (46 fragments a slice) 1.4-1.7x faster, 5120 x 17408 (40, one slice)
// 1.1-1.2x; 5120 x 5120 (14) and every shape of 2880-5760 (at most 12) slower.
constexpr int kMidMinWaveFrags = 8;
// Below 33 rows the skinny kernel already takes two weight tiles per
// workgroup for 17-32 rows; a two-group instance of this kernel measured
// 0.91-0.93x there on K x N = 5120 x 17408 and 1.0-1.13x on 17408 x 5120
// (the decode benchmark within 1.5% either way), so it is not used.
constexpr int kMidMinM = 33;

int gemm_mid_splits(int64_t m, int64_t n, int64_t k, int64_t cap) {
  if (m < kMidMinM || m > kDecodeMaxM) return 0;
  const int64_t kt_n = k_pad(k) / kFragK, nt_n = round_up(n, 16) / 16;
  // 32-bit buffer offsets: the workgroup's weight tiles and all activation groups
  if (kt_n * kFragCodeBytes * std::max(kMidTiles, 8) >= (int64_t(1) << 31)) return 0;
  const int64_t ncol = (nt_n + kMidTiles - 1) / kMidTiles;
  int64_t s = std::max<int64_t>(1, 256 / ncol);
  s = std::min(s, std::max<int64_t>(1, kt_n / kMidWaves));
  while (s > 1 && s * m * n * (int64_t)sizeof(float) > cap) --s;
  if ((kt_n + s - 1) / s < (int64_t)kMidWaves * kMidMinWaveFrags) return 0;
  return (int)s;
}

hipError_t launch_gemm_mid(const GemmArgs &g, int splits, float *part, hipStream_t stream) {
  if (!g.a_tiled || g.w_ms || g.m < kMidMinM || g.m > kDecodeMaxM || splits < 1 || (splits > 1 && !part))
    return hipErrorInvalidValue;
  const int kt_n = (int)(k_pad(g.k) / kFragK);
  const int nt_n = (int)(round_up(g.n, 16) / 16);
  const int ncol = (nt_n + kMidTiles - 1) / kMidTiles;
  const int kps = (kt_n + splits - 1) / splits;
  float *p = splits > 1 ? part : nullptr;
  const dim3 grid((unsigned)ncol, (unsigned)splits);
#define FP4_MID(F, G)                                                                         \
  hipLaunchKernelGGL((k_gemm_mid<F, G>), grid, dim3(64 * kMidWaves), 0, stream, g.a_codes,   \
                     g.a_scales, g.a_ts, g.w_codes, g.w_scales, g.w_ts, (int)g.m, (int)g.n, kt_n, \
                     nt_n, kps, g.c, g.ldc, p)
  if (g.fmt == 0 && g.m <= 64) FP4_MID(0, 4);
  else if (g.fmt == 0) FP4_MID(0, 8);
  else if (g.m <= 64) FP4_MID(1, 4);
  else FP4_MID(1, 8);
#undef FP4_MID
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t mn = g.m * g.n;
  const unsigned blocks = (unsigned)std::min<int64_t>(2048, (mn + 255) / 256);
  hipLaunchKernelGGL(k_mid_sum, dim3(blocks), dim3(256), 0, stream, part, splits, (int)g.m,
                     (int)g.n, g.fmt, g.a_ts, g.w_ts, g.c, g.ldc);
  return hipGetLastError();
}

namespace {
std::atomic<int> g_fuse_decode{0};
}  // namespace

int decode_linear_fusion() { return g_fuse_decode.load(std::memory_order_relaxed); }
int set_decode_linear_fusion(int on) {
  return g_fuse_decode.exchange(on ? 1 : 0, std::memory_order_relaxed);
}

static_assert(kRingWaves == kDecWaves, "the producer bound assumes eight-wave workgroups at least");

bool linear_fused_decode_ok(int fmt, uint32_t recipe, int64_t m, int64_t n, int64_t k) {
  (void)fmt;
  (void)n;
  // every fragment has a producer wave: at most kActGrid producers (the
  // exchange's slots) of at least kRingWaves = kDecWaves waves
  const int64_t nfr = round_up(m, 16) / 16 * (k_pad(k) / kFragK);
  return decode_linear_fusion() && m <= 32 && !(recipe & (kRecipeMbs | kRecipeRotate)) &&
         nfr <= (int64_t)kActGrid * kDecWaves * kDecProdFrags;
}

hipError_t launch_linear_fused_decode(const GemmArgs &g, const uint16_t *x,
                                      const float *static_scale, uint32_t recipe,
                                      uint32_t *scratch, hipStream_t stream) {
  // g: tiled activations at g.a_codes / g.a_scales (written by this launch),
  // g.a_ts = static_scale or the word the dynamic S_t goes to
  DecFused fz;
  fz.x = x;
  fz.st = static_scale;
  fz.ts_out = (uint32_t *)g.a_ts;
  fz.slots = scratch + kMaxAmaxParts;
  fz.err = scratch + kErrWord;
  fz.arrive = scratch + kArriveWord;
  fz.ready = scratch + kPanelWords;
  fz.nprod = 0;
  fz.k = (int)g.k;
  fz.recipe = recipe;
  fz.spin = exchange_spin_limit();
  return decode_launch(g, &fz, stream);
}

bool linear_fused_ok(int fmt, int64_t m, int64_t n, int64_t k) {
  const int64_t mk = m * k_pad(k);
  // LDS staging bound, and a bound on the redundant quantization work that
  // every weight tile's workgroup repeats.
  // NVFP4's encoding prologue (maximum pass + exact encode) is long enough
  // that with two or more rows only about two workgroups per CU (512 weight
  // tiles) should repeat it, and the separate quantizer plus the skinny GEMM
  // wins once M * K_pad * tiles passes about 4M (320 tiles, K = 5120,
  // measured: fused at M = 2, 11.9 us against 13.5; separate at M = 4, 12.3
  // us against 14.7). A single row's prologue is short enough for twice that
  // work and any tile count (K = 5120, N = 17408: fused 19.0 us against 20.0;
  // K = 17408, N = 5120: 20.8 against 21.1; at M = 2, N = 17408 the separate
  // quantizer wins, 20.4 against 22.9).
  const int64_t nt = round_up(n, 16) / 16;
  if (fmt == 0 && m == 1) return mk <= kFusedMaxMK / 2 && mk * nt <= 2 * kFusedMaxWorkNv;
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
