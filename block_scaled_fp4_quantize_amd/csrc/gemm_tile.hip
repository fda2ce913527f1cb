// gemm_tile.hip -- LDS-staged W4A4 GEMM for large M (prefill and square
// shapes), gfx950.
//
// Same product as the other GEMM kernels: C[m, n] = alpha * sum_k
// (q_a s_a)[m, k] (q_w s_w)[n, k], FP32 accumulation, bf16 output (forum post
// on a standalone FP4 GEMM library, opening paragraphs: weights quantized once
// into a cache, activations per call).
//
// Both operands are in the fragment-tiled layout (16 rows x 128 values per
// fragment, 1 KB of codes in the matrix instruction's lane order, then the
// fragment's scale bytes in a separate array), so a stage of the K loop is a
// set of whole 1 KB fragments. They are copied global -> LDS with the direct
// LDS load (global_load_lds_dwordx4: lane i of the wave writes bytes
// 16i..16i+15 of a 1 KB LDS run), which needs no registers and no LDS store
// instructions. The scale bytes are copied a dword at a time (one dword holds
// the scales of 4 lanes (MXFP4) or 2 lanes (NVFP4) of one fragment) and
// regrouped on the way: each lane's copy reads whichever global dword the LDS
// order wants, and the stage stores them as [operand][lane group][fragment],
// so that a lane finds its scales for all of its fragments in consecutive
// dwords (a few 16-byte LDS reads instead of one byte read per fragment). A four-stage ring: while stage s is consumed, the copies of
// stages s+1 and s+2 are in flight and those of s+3 are issued; the copies
// and the LDS reads of the next stage are spread between the matrix
// instructions so the matrix unit is not left idle while they issue.
//
// Workgroup: four waves in a 2 x 2 grid; wave tile TM x TN fragments
// (16 TM rows of A by 16 TN rows of W). The weight fragment is the matrix
// instruction's A operand and the activation fragment its B operand, so each
// lane ends with four consecutive output columns of one row (one 8-byte
// store).
//   MXFP4: V_MFMA_SCALE_F32_16X16X128_F8F6F4, E8M0 byte per lane.
//   NVFP4: exact f16 dequantization of each lane's codes (q * s_b has at most
//          6 significant bits) and V_MFMA_F32_16X16X32_F16, as in the other
//          kernels.
// Workgroups are numbered so that consecutive tiles land on the same XCD
// (the hardware deals workgroups to the eight XCDs round-robin), and tiles are
// walked in groups of tile rows, so the tiles an XCD runs at one time share
// A and W K-slices in that XCD's L2.
#include "fp4_device.h"
#include "fp4_internal.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

// clang notes that M0 is a reserved register when it appears in an inline
// assembly clobber list (the direct-LDS copies below set it); no
// compiler-generated code in these kernels uses M0.
#pragma clang diagnostic ignored "-Winline-asm"

namespace fp4i {
using namespace fp4d;

namespace {

constexpr int kStages = 4;
constexpr int kXcds = 8;
constexpr int kGroupRows = 8;

template <int FMT, int TM, int TN>
struct TileCfg {
  static constexpr int FA = 2 * TM, FW = 2 * TN, NF = FA + FW;  // fragments per stage
  static constexpr int SCB = FMT == 0 ? 128 : 64;                // scale bytes per fragment
  static constexpr int SC_DW = NF * SCB / 4;                     // scale dwords per stage
  // scale copies (64 dwords each), rounded up so every wave issues as many
  static constexpr int SC_INSTR = ((SC_DW + 63) / 64 + 3) / 4 * 4;
  static constexpr int CODE_BYTES = NF * kFragCodeBytes;
  static constexpr int STAGE = CODE_BYTES + SC_INSTR * 256;
  // copies per wave per stage: NF / 4 code fragments + SC_INSTR / 4 scale runs
  static constexpr int PS = NF / 4 + SC_INSTR / 4;
  static_assert(NF % 4 == 0, "fragments per stage must split over four waves");
  static_assert(2 * PS < 64, "vmcnt range");
};

// s_waitcnt vmcnt(N), other counters left alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS only: this wave's LDS reads are complete, then
// s_barrier. (The LDS copies are waited for explicitly with vmcnt; a fence
// here would also wait for every copy still in flight.) The wait is the
// builtin so that the compiler's own counter bookkeeping sees it; the empty
// asm statements keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt at their maxima
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global -> LDS copies: lane i writes bytes [size*i, size*i + size) of
// the wave's LDS run starting at the wave-uniform LDS address dst (M0). They
// are written as assembly so that the compiler does not treat every later LDS
// read as dependent on every copy still in flight (it cannot tell the ring's
// stages apart and would wait for all of them); the K loop waits for exactly
// the copies it needs with vmcnt. The copies have no register results.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}
// The source address is a wave-uniform base (SGPR pair) plus a per-lane
// 32-bit byte offset, which keeps the copy addresses out of vector registers.
// The base is uniform by construction; it passes through readfirstlane so
// that the compiler never hands the scalar operand a vector register (free
// where the base already is scalar).
__device__ __forceinline__ const uint8_t *sgpr_ptr(const uint8_t *p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const uint8_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void lds_copy16(const uint8_t *base, uint32_t off, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(sgpr_ptr(base)), "s"(dst) : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const uint8_t *base, uint32_t off, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(sgpr_ptr(base)), "s"(dst) : "memory", "m0");
}

__device__ __forceinline__ v4f mma_mx(uint4 w, uint4 a, v4f c, uint32_t sw, uint32_t sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(frag_v8i(w), frag_v8i(a), c, 4, 4, 0,
                                                           (int)sw, 0, (int)sa);
}

template <int S>
using Stage = std::integral_constant<int, S>;

// Two floats -> two bf16 (round to nearest even; v_cvt_pk_bf16_f32), packed.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
}

// The fused linear's extra arguments (k_gemm_tile with FUSED = 1).
struct Fused {
  const uint16_t *x;        // bf16 activations [m, k]
  const float *st;          // NVFP4 static tensor scale (device)
  uint32_t *panel;          // per panel: ready count, finished count
  uint32_t *err;            // sticky error flags
  int nprod, parts;         // producer workgroups; producers per panel
  int k;
  uint32_t recipe, spin;
};

// Producer of the fused linear: quantizes part `part` (of `parts`) of row
// panel `panel` of the activations into the tiled layout, one wave per
// fragment (lane 16c + r: row r, values 32c .. 32c + 31), with the same
// encoders as the quantize kernels; then counts itself in the panel's ready
// word once its stores are complete.
template <int FMT, int FA>
__device__ void fused_produce(const Fused &fz, int panel, int part, int m, int kt_n, int ga_n,
                             uint8_t *a_codes, uint8_t *a_sc) {
  constexpr int SCB = FMT == 0 ? 128 : 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, r = lane & 15, c = lane >> 4;
  const int g_lo = panel * FA, g_hi = min(g_lo + FA, ga_n);
  const int nfr = (g_hi - g_lo) * kt_n, per = (nfr + fz.parts - 1) / fz.parts;
  const int f_lo = part * per, f_hi = min(f_lo + per, nfr);
  const float st = FMT == 0 ? *fz.st : 1.0f;
  // U fragments per wave in flight: all their loads are issued before the
  // first is encoded (a producer workgroup holds the tile kernel's LDS, so
  // few of them share a CU and each must keep many loads outstanding); two
  // for the 128-row tiles, whose kernels keep two waves per SIMD
  constexpr int U = FA >= 16 ? 4 : 2;
  for (int i0 = f_lo + wave; i0 < f_hi; i0 += 4 * U) {
    uint4 v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + 4 * u;
      const int g = g_lo + i / kt_n, kt = i % kt_n;
      const int row = g * 16 + r, k0 = kt * kFragK + 32 * c;
      const bool live = i < f_hi && row < m;
      const uint4 *src = (const uint4 *)(fz.x + (int64_t)row * fz.k + k0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[u][j] = (live && k0 + 8 * j < fz.k) ? src[j] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + 4 * u;
      if (i >= f_hi) break;
      const int g = g_lo + i / kt_n, kt = i % kt_n;
      const int64_t f = (int64_t)g * kt_n + kt;
      const int row = g * 16 + r, k0 = kt * kFragK + 32 * c;
      if (fz.recipe & kRecipeRotate) {
        if constexpr (FMT == 0) {
          uint4 b0[2] = {v[u][0], v[u][1]}, b1[2] = {v[u][2], v[u][3]};
          hadamard_block<16>(b0);
          hadamard_block<16>(b1);
          v[u][0] = b0[0]; v[u][1] = b0[1]; v[u][2] = b1[0]; v[u][3] = b1[1];
        } else {
          hadamard_block<32>(v[u]);
        }
      }
      uint4 q = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (FMT == 0) {
        uint2 c0 = make_uint2(0u, 0u), c1 = make_uint2(0u, 0u);
        uint32_t s0 = 0, s1 = 0;
        if (row < m && k0 < fz.k) nv_encode_block(v[u][0], v[u][1], st, c0, s0);
        if (row < m && k0 + 16 < fz.k) nv_encode_block(v[u][2], v[u][3], st, c1, s1);
        q = make_uint4(c0.x, c0.y, c1.x, c1.y);
        store2_dev(dev_rsrc(a_sc + f * SCB, SCB), lane * 2, s0 | (s1 << 8));
      } else {
        uint32_t sc = 0;
        if (row < m && k0 < fz.k) mx_encode_block(v[u], q, sc, fz.recipe & kRecipeOas);
        store1_dev(dev_rsrc(a_sc + f * SCB, SCB), lane, sc);
      }
      store16_dev(dev_rsrc(a_codes + f * kFragCodeBytes, kFragCodeBytes), lane * 16, q);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(&fz.panel[2 * panel], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int TM, int TN, int FUSED = 0>
__global__ __launch_bounds__(256) void k_gemm_tile(
    const uint8_t *__restrict__ a_codes, const uint8_t *__restrict__ a_sc,
    const float *__restrict__ a_ts, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_sc, const float *__restrict__ w_ts, int m, int n, int kt_n,
    int ga_n, int nt_n, int tiles_m, int tiles_n, uint16_t *__restrict__ c, int64_t ldc,
    int vec_store, Fused fz) {
  using C = TileCfg<FMT, TM, TN>;
  // One LDS array per ring stage and a K loop unrolled four times, so every
  // stage buffer is a compile-time constant in its body (with a run-time
  // stage index the accumulators were shuffled between register files).
  __shared__ __align__(1024) uint8_t lds0[C::STAGE];
  __shared__ __align__(1024) uint8_t lds1[C::STAGE];
  __shared__ __align__(1024) uint8_t lds2[C::STAGE];
  __shared__ __align__(1024) uint8_t lds3[C::STAGE];
  auto stage_ptr = [&](auto sc) __attribute__((always_inline)) -> uint8_t * {
    constexpr int S = decltype(sc)::value % kStages;
    if constexpr (S == 0) return lds0;
    else if constexpr (S == 1) return lds1;
    else if constexpr (S == 2) return lds2;
    else return lds3;
  };
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;

  // ---- fused linear: the first nprod workgroups quantize the activations
  // (they run before any tile workgroup of their XCD: dispatch follows the
  // workgroup index) and end; the rest are the tiles, numbered from 0
  // (nprod is a multiple of the XCD count, so the XCD of tile b is still b % 8)
  if (FUSED && (int)blockIdx.x < fz.nprod) {
    fused_produce<FMT, C::FA>(fz, blockIdx.x / fz.parts, blockIdx.x % fz.parts, m, kt_n, ga_n,
                              (uint8_t *)a_codes, (uint8_t *)a_sc);
    return;
  }

  // ---- tile of this workgroup (XCD-contiguous, grouped by tile rows)
  int tm, tn;
  {
    const int nwg = tiles_m * tiles_n, b = blockIdx.x - (FUSED ? fz.nprod : 0);
    const int xcd = b % kXcds, slot = b / kXcds, q = nwg / kXcds, r = nwg % kXcds;
    const int L = xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
    const int per_group = kGroupRows * tiles_n, grp = L / per_group, first = grp * kGroupRows;
    const int gsz = min(tiles_m - first, kGroupRows), in = L - grp * per_group;
    tm = first + in % gsz;
    tn = in / gsz;
  }
  const int g0 = tm * C::FA, n0 = tn * C::FW;

  // ---- fused linear: wait (bounded) until every producer of this tile row's
  // activation panel has finished; the panel's fragments are then read with
  // ordinary loads, this kernel having read none of them before. A wait that
  // gives up sets the sticky error flag and makes the tile's output NaN.
  __shared__ uint32_t gave_up_s;
  if (FUSED) {
    if (threadIdx.x == 0) {
      uint32_t ok = 0;
      for (uint32_t it = 0; it < fz.spin; ++it) {
        if (__hip_atomic_load(&fz.panel[2 * tm], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
            (uint32_t)fz.parts) {
          ok = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (!ok)
        __hip_atomic_fetch_or(fz.err, kErrExchangeTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      gave_up_s = !ok;
    }
    __syncthreads();
  }

  // ---- this wave's share of every stage's copies: code fragments
  // wave + 4u (one 16-byte copy per lane, 1 KB per wave), then scale runs
  // wave + 4v (one dword per lane). Fragment rows past the operand (A rows
  // >= m, W rows >= n, rounded to 16) copy the last valid fragment instead:
  // they only feed output rows/columns that are never stored, and every wave
  // issues the same number of copies at every stage.
  constexpr int NCP = C::NF / 4, NSP = C::SC_INSTR / 4;
  // Copy sources: a wave-uniform fragment-row base and a per-lane offset
  // (lane * 16 for the code fragments; for the scale runs the lane's dword,
  // relative to the run's first row: a run never crosses from A's scales into
  // W's, A's scale dwords per stage being a multiple of 64).
  auto row_of = [&](int f) __attribute__((always_inline)) {
    return f < C::FA ? min(g0 + f, ga_n - 1) : min(n0 + f - C::FA, nt_n - 1);
  };
  const uint8_t *code_base[NCP];
  const uint32_t code_off = lane * 16;
#pragma unroll
  for (int u = 0; u < NCP; ++u) {
    const int f = wave + 4 * u;
    code_base[u] = (f < C::FA ? a_codes : w_codes) + (int64_t)row_of(f) * kt_n * kFragCodeBytes;
  }
  // Stage scale region. Grouped (GS, the MXFP4 256 x 256 tile): dword d <
  // A_DW is A's chunk d / FA (lane group) of fragment d % FA; the W section
  // follows with FW fragments per chunk. A_DW is a multiple of 64, so a copy
  // run (64 dwords) never mixes A and W. Otherwise the global order is kept
  // (fragment-major, one byte (MXFP4) or byte pair (NVFP4) per lane): the
  // 128 x 128 tiles and NVFP4 measured no faster with the grouped order.
  constexpr bool GS = FMT == 1 && TM == 8 && TN == 8;
  constexpr int DPF = C::SCB / 4;            // scale dwords per fragment
  constexpr int A_DW = DPF * C::FA;
  static_assert(!GS || A_DW % 64 == 0, "a scale copy run stays within one operand");
  auto frag_chunk = [&](int d, int &f, int &pc) __attribute__((always_inline)) {
    if (!GS) {
      f = d / DPF;
      pc = d % DPF;
    } else if (d < A_DW) {
      pc = d / C::FA;
      f = d % C::FA;
    } else {
      pc = (d - A_DW) / C::FW;
      f = C::FA + (d - A_DW) % C::FW;
    }
  };
  const uint8_t *sc_base[NSP];
  uint32_t sc_off[NSP];
#pragma unroll
  for (int v = 0; v < NSP; ++v) {
    const int j = wave + 4 * v;
    int f0, pc0, f, pc;
    frag_chunk(min(64 * j, C::SC_DW - 1), f0, pc0);
    frag_chunk(min(64 * j + lane, C::SC_DW - 1), f, pc);
    const int r0 = row_of(f0);
    sc_base[v] = (f0 < C::FA ? a_sc : w_sc) + (int64_t)r0 * kt_n * C::SCB;
    sc_off[v] = (uint32_t)((row_of(f) - r0) * kt_n * C::SCB + pc * 4);
  }

  // copy unit u of this wave's share of stage kt: units 0..NCP-1 are code
  // fragments, NCP..NCP+NSP-1 scale runs
  constexpr int NU = NCP + NSP;
  auto issue_unit = [&](uint8_t *st, int kt, int u) __attribute__((always_inline)) {
    if (u < NCP)
      lds_copy16(code_base[u] + (int64_t)kt * kFragCodeBytes, code_off,
                 lds_addr(st + (wave + 4 * u) * kFragCodeBytes));
    else
      lds_copy4(sc_base[u - NCP] + (int64_t)kt * C::SCB, sc_off[u - NCP],
                lds_addr(st + C::CODE_BYTES + (wave + 4 * (u - NCP)) * 256));
  };
  auto issue = [&](auto sc, int kt) __attribute__((always_inline)) {
    uint8_t *st = stage_ptr(sc);
#pragma unroll
    for (int u = 0; u < NU; ++u) issue_unit(st, kt, u);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int fa0 = wm * TM, fw0 = C::FA + wn * TN;  // this wave's first fragments in a stage

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  struct Ops {
    uint4 aq[TM], wq[TN];
    uint32_t as[TM], ws[TN];
  };
  // read unit r of a stage into registers: A fragment r (r < TM) or W
  // fragment r - TM, each with its scale, or in the grouped order codes only
  // and (r = TM + TN) the lane's scales of all of them: TM and TN consecutive dwords, each holding the lane's scale
  // byte (MXFP4) or byte pair (NVFP4) at bit 32 * (lane % LPD) / LPD. The
  // shifted dword is kept whole: the scaled matrix instruction reads byte 0
  // of its scale operand and the NVFP4 dequantization masks each byte.
  static_assert(TM % 4 == 0 && TN % 4 == 0, "scale reads take 4 fragments per 16 bytes");
  constexpr int LPD = 256 / C::SCB;          // lanes per scale dword
  const int s_chunk = lane / LPD, s_shift = (lane % LPD) * (32 / LPD);
  auto read_unit = [&](const uint8_t *st, Ops &o, int r) __attribute__((always_inline)) {
    if (!GS) {  // code bytes and scale of one fragment
      const int f = r < TM ? fa0 + r : fw0 + r - TM;
      const uint4 q = *(const uint4 *)(st + f * kFragCodeBytes + lane * 16);
      const uint32_t sv = FMT == 0 ? (uint32_t) * (const uint16_t *)(st + C::CODE_BYTES + f * 128 + lane * 2)
                                   : (uint32_t)st[C::CODE_BYTES + f * 64 + lane];
      if (r < TM) {
        o.aq[r] = q;
        o.as[r] = sv;
      } else {
        o.wq[r - TM] = q;
        o.ws[r - TM] = sv;
      }
      return;
    }
    if (r < TM + TN) {
      const int f = r < TM ? fa0 + r : fw0 + r - TM;
      const uint4 q = *(const uint4 *)(st + f * kFragCodeBytes + lane * 16);
      if (r < TM) o.aq[r] = q;
      else o.wq[r - TM] = q;
      return;
    }
    const uint32_t *sr = (const uint32_t *)(st + C::CODE_BYTES);
    const uint4 *sa = (const uint4 *)(sr + s_chunk * C::FA + fa0);
    const uint4 *sw = (const uint4 *)(sr + A_DW + s_chunk * C::FW + (fw0 - C::FA));
#pragma unroll
    for (int i = 0; i < TM / 4; ++i) {
      const uint4 d = sa[i];
      o.as[4 * i] = d.x >> s_shift;
      o.as[4 * i + 1] = d.y >> s_shift;
      o.as[4 * i + 2] = d.z >> s_shift;
      o.as[4 * i + 3] = d.w >> s_shift;
    }
#pragma unroll
    for (int j = 0; j < TN / 4; ++j) {
      const uint4 d = sw[j];
      o.ws[4 * j] = d.x >> s_shift;
      o.ws[4 * j + 1] = d.y >> s_shift;
      o.ws[4 * j + 2] = d.z >> s_shift;
      o.ws[4 * j + 3] = d.w >> s_shift;
    }
  };
  constexpr int NR = TM + TN + (GS ? 1 : 0);  // read units per stage
  auto read = [&](auto sc, Ops &o) __attribute__((always_inline)) {
    const uint8_t *st = stage_ptr(sc);
#pragma unroll
    for (int r = 0; r < NR; ++r) read_unit(st, o, r);
  };

  auto mma = [&](const Ops &o) __attribute__((always_inline)) {
    if constexpr (FMT == 1) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mma_mx(o.wq[j], o.aq[i], acc[i][j], o.ws[j], o.as[i]);
    } else {
      // K sub-block g: dword g of every lane's 16 code bytes (values
      // 8g..8g+7 of its 32), the same permutation of K for both operands.
      // Software-pipelined: sub-block g+1 is dequantized while sub-block g's
      // matrix instructions run (no scheduling barrier between sub-blocks, so
      // the scheduler interleaves the two), and the two units work side by
      // side. The weight operands of g+1 are double-buffered; each activation
      // row's operand for g+1 replaces its g value right after that row's
      // instructions. (Explicit MFMA/VALU scheduling groups made the
      // scheduler spill.)
      auto deq_a = [&](int g, int i) __attribute__((always_inline)) {
        const uint32_t d = g == 0 ? o.aq[i].x : g == 1 ? o.aq[i].y : g == 2 ? o.aq[i].z : o.aq[i].w;
        return __builtin_bit_cast(h8v, nv_dequant8_u4(d, g < 2 ? (o.as[i] & 0xFFu) : (o.as[i] >> 8)));
      };
      auto deq_w = [&](int g, int j) __attribute__((always_inline)) {
        const uint32_t d = g == 0 ? o.wq[j].x : g == 1 ? o.wq[j].y : g == 2 ? o.wq[j].z : o.wq[j].w;
        return __builtin_bit_cast(h8v, nv_dequant8_u4(d, g < 2 ? (o.ws[j] & 0xFFu) : (o.ws[j] >> 8)));
      };
      h8v ah[TM], wh[2][TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) wh[0][j] = deq_w(0, j);
#pragma unroll
      for (int i = 0; i < TM; ++i) ah[i] = deq_a(0, i);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g < 3) {
#pragma unroll
          for (int j = 0; j < TN; ++j) wh[(g + 1) & 1][j] = deq_w(g + 1, j);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh[g & 1][j], ah[i], acc[i][j], 0, 0, 0);
          if (g < 3) ah[i] = deq_a(g + 1, i);
        }
      }
    }
  };

  // ---- K loop over a four-stage ring. Stages kt+1 and kt+2 are in flight
  // while stage kt is waited for; stage kt+3 is issued after the barrier into
  // the buffer stage kt-1 used. Past the last stage the copies repeat the
  // last stage into buffers nobody reads any more, so every iteration issues
  // the same copies and waits for the same count (no branches in the loop
  // body). MXFP4 reads stage kt+1 into registers while stage kt's matrix
  // instructions run.
  auto src_kt = [&](int kt) __attribute__((always_inline)) { return min(kt, kt_n - 1); };
  issue(Stage<0>{}, 0);
  issue(Stage<1>{}, src_kt(1));
  issue(Stage<2>{}, src_kt(2));

  Ops ops[2];
  constexpr bool kDouble = FMT == 1;
  if constexpr (kDouble) {
    wait_vm<2 * C::PS>();
    lds_barrier();
    read(Stage<0>{}, ops[0]);
  }
  auto body = [&](auto sc, int kt) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    if constexpr (kDouble) {
      wait_vm<C::PS>();  // stage kt+1 has landed (kt+2 may be in flight)
      lds_barrier();
      // Stage kt's matrix instructions, with the copies of stage kt+3 and the
      // register reads of stage kt+1 spread between them: each copy or LDS
      // read issues while a matrix instruction runs instead of holding the
      // matrix unit idle. The scheduling barriers keep that order. (After the
      // last stage the reads fetch values that are never used.)
      constexpr int NQ = TM * TN;
      constexpr int DMA_EVERY = NQ / NU > 0 ? NQ / NU : 1;

      const int kcopy = src_kt(kt + 3);
      uint8_t *st_copy = stage_ptr(Stage<S + 3>{});
      const uint8_t *st_read = stage_ptr(Stage<S + 1>{});
      const Ops &cur = ops[S & 1];
      Ops &nxt = ops[(S + 1) & 1];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q % DMA_EVERY == 0 && q / DMA_EVERY < NU) issue_unit(st_copy, kcopy, q / DMA_EVERY);
        // read units spread evenly: unit u at the first q with (q+1) NR / NQ > u
        if ((q + 1) * NR / NQ > q * NR / NQ) read_unit(st_read, nxt, q * NR / NQ);
        const int i = q / TN, j = q % TN;
        acc[i][j] = mma_mx(cur.wq[j], cur.aq[i], acc[i][j], cur.ws[j], cur.as[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      wait_vm<2 * C::PS>();  // stage kt has landed (kt+1, kt+2 may be in flight)
      lds_barrier();
      issue(Stage<S + 3>{}, src_kt(kt + 3));
      read(sc, ops[0]);
      mma(ops[0]);
    }
  };
  for (int kt = 0; kt < kt_n; kt += kStages) {
    body(Stage<0>{}, kt);
    if (kt + 1 < kt_n) body(Stage<1>{}, kt + 1);
    if (kt + 2 < kt_n) body(Stage<2>{}, kt + 2);
    if (kt + 3 < kt_n) body(Stage<3>{}, kt + 3);
  }
  // every copy has landed before the workgroup can end (its LDS is then
  // handed to the next workgroup)
  wait_vm<0>();

  Alpha alpha = FMT == 0 ? make_alpha(a_ts[0], w_ts[0]) : Alpha{1.0f, 0};
  if (FUSED) {
    // this tile reads no more activations: count it finished; the panel's
    // last tile resets the panel's words for the next call
    if (gave_up_s) alpha.m = __builtin_nanf("");
    if (threadIdx.x == 0) {
      const uint32_t done = __hip_atomic_fetch_add(&fz.panel[2 * tm + 1], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      if (done == (uint32_t)tiles_n - 1) {
        __hip_atomic_store(&fz.panel[2 * tm], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&fz.panel[2 * tm + 1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // ---- epilogue: lane holds C[row][col0 .. col0+3] of each 16 x 16 tile
  const int rl = lane & 15, cl = 4 * (lane >> 4);
  if (vec_store == 2) {
    // Staged through LDS: each wave writes its 16TM x 16TN quadrant as bf16
    // rows into one ring buffer (the ring is free once every wave has left the
    // K loop), then stores whole rows, 16 bytes per lane, so that every store
    // instruction covers whole 128-byte lines (the accumulator layout alone
    // gives 32-byte pieces of 16 different rows per instruction).
    lds_barrier();
    constexpr int QR = 16 * TM, QC = 16 * TN;
    constexpr int QP = 2 * QC + 16;  // padded LDS row pitch in bytes
    static_assert(QR * QP <= C::STAGE, "a wave's output quadrant fits one ring buffer");
    uint8_t *q = wave == 0 ? lds0 : wave == 1 ? lds1 : wave == 2 ? lds2 : lds3;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f &a = acc[i][j];
        const uint32_t lo = pack_bf16x2(apply_alpha(a[0], alpha), apply_alpha(a[1], alpha));
        const uint32_t hi = pack_bf16x2(apply_alpha(a[2], alpha), apply_alpha(a[3], alpha));
        *(uint2 *)(q + (16 * i + rl) * QP + 2 * (16 * j + cl)) = make_uint2(lo, hi);
      }
    constexpr int LPR = QC / 8, RPI = 64 / LPR;  // lanes per row, rows per instruction
    const int lr = lane / LPR, lc = 8 * (lane % LPR);
    const int row0 = (g0 + fa0) * 16, col = (n0 + wn * TN) * 16 + lc;
#pragma unroll 4
    for (int it = 0; it < QR / RPI; ++it) {
      const int r = it * RPI + lr, row = row0 + r;
      const uint4 v = *(const uint4 *)(q + r * QP + 2 * lc);
      if (row >= m) continue;
      uint16_t *dst = c + (int64_t)row * ldc + col;
      if (col + 7 < n) {
        *(uint4 *)dst = v;
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < n) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = (g0 + fa0 + i) * 16 + rl;
    if (row >= m) continue;
    uint16_t *crow = c + (int64_t)row * ldc;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col0 = (n0 + wn * TN + j) * 16 + cl;
      const v4f &a = acc[i][j];
      const uint32_t lo = pack_bf16x2(apply_alpha(a[0], alpha), apply_alpha(a[1], alpha));
      const uint32_t hi = pack_bf16x2(apply_alpha(a[2], alpha), apply_alpha(a[3], alpha));
      if (vec_store && col0 + 3 < n) {
        *(uint2 *)(crow + col0) = make_uint2(lo, hi);
      } else {
        if (col0 < n) crow[col0] = (uint16_t)lo;
        if (col0 + 1 < n) crow[col0 + 1] = (uint16_t)(lo >> 16);
        if (col0 + 2 < n) crow[col0 + 2] = (uint16_t)hi;
        if (col0 + 3 < n) crow[col0 + 3] = (uint16_t)(hi >> 16);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// NVFP4 with the conversion in LDS: every fragment of a stage is dequantized
// once per workgroup (in the kernel above, each A and W fragment is converted
// by both waves that use it). Per K = 32 sub-block (dword g of every lane's
// 16 code bytes, the same K permutation for both operands), each wave converts
// eight of the stage's fragments to exact f16 q * s_b and writes them to a
// double-buffered f16 area (1 KB per fragment, in operand lane order); after a
// barrier every wave reads its TM + TN f16 operands back and runs its TM x TN
// matrix instructions while the next sub-block is converted into the other
// buffer. The FP4 ring has two stages (LDS: 2 x 36 KB ring + 2 x 32 KB f16);
// stage s is copied while stages s - 2 and s - 1 are consumed, its codes read
// into registers at the last sub-block of stage s - 1.
template <int TM, int TN>
__global__ __launch_bounds__(256) void k_gemm_tile_nvlds(
    const uint8_t *__restrict__ a_codes, const uint8_t *__restrict__ a_sc,
    const float *__restrict__ a_ts, const uint8_t *__restrict__ w_codes,
    const uint8_t *__restrict__ w_sc, const float *__restrict__ w_ts, int m, int n, int kt_n,
    int ga_n, int nt_n, int tiles_m, int tiles_n, uint16_t *__restrict__ c, int64_t ldc,
    int vec_store) {
  using C = TileCfg<0, TM, TN>;
  constexpr int F16B = C::NF * kFragCodeBytes;            // one sub-block's f16 operands
  constexpr int QR = 16 * TM, QC = 16 * TN, QP = 2 * QC + 16;
  constexpr int RING = C::STAGE;
  constexpr int USE = 2 * RING + 2 * F16B;
  constexpr int TOTAL = USE > 4 * QR * QP ? USE : 4 * QR * QP;
  static_assert(C::NF == 32 && TOTAL <= 160 * 1024, "256 x 256 tile: 32 fragments per stage");
  __shared__ __align__(1024) uint8_t smem[TOTAL];
  auto ring = [&](auto r) __attribute__((always_inline)) -> uint8_t * {
    return smem + (decltype(r)::value & 1) * RING;
  };
  auto f16buf = [&](auto b) __attribute__((always_inline)) -> uint8_t * {
    return smem + 2 * RING + (decltype(b)::value & 1) * F16B;
  };
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;

  // ---- tile of this workgroup (XCD-contiguous, grouped by tile rows)
  int tm, tn;
  {
    const int nwg = tiles_m * tiles_n, b = blockIdx.x;
    const int xcd = b % kXcds, slot = b / kXcds, q = nwg / kXcds, r = nwg % kXcds;
    const int L = xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
    const int per_group = kGroupRows * tiles_n, grp = L / per_group, first = grp * kGroupRows;
    const int gsz = min(tiles_m - first, kGroupRows), in = L - grp * per_group;
    tm = first + in % gsz;
    tn = in / gsz;
  }
  const int g0 = tm * C::FA, n0 = tn * C::FW;

  // ---- copies: code fragments wave + 4u, scale runs wave + 4v (as above)
  constexpr int NCP = C::NF / 4, NSP = C::SC_INSTR / 4;
  auto row_of = [&](int f) __attribute__((always_inline)) {
    return f < C::FA ? min(g0 + f, ga_n - 1) : min(n0 + f - C::FA, nt_n - 1);
  };
  const uint8_t *code_base[NCP];
  const uint32_t code_off = lane * 16;
#pragma unroll
  for (int u = 0; u < NCP; ++u) {
    const int f = wave + 4 * u;
    code_base[u] = (f < C::FA ? a_codes : w_codes) + (int64_t)row_of(f) * kt_n * kFragCodeBytes;
  }
  constexpr int DPF = C::SCB / 4;
  const uint8_t *sc_base[NSP];
  uint32_t sc_off[NSP];
#pragma unroll
  for (int v = 0; v < NSP; ++v) {
    const int j = wave + 4 * v;
    const int d0 = min(64 * j, C::SC_DW - 1), d = min(64 * j + lane, C::SC_DW - 1);
    const int f0 = d0 / DPF, f = d / DPF;
    const int r0 = row_of(f0);
    sc_base[v] = (f0 < C::FA ? a_sc : w_sc) + (int64_t)r0 * kt_n * C::SCB;
    sc_off[v] = (uint32_t)((row_of(f) - r0) * kt_n * C::SCB + (d % DPF) * 4);
  }
  auto issue = [&](uint8_t *st, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NCP; ++u)
      lds_copy16(code_base[u] + (int64_t)kt * kFragCodeBytes, code_off,
                 lds_addr(st + (wave + 4 * u) * kFragCodeBytes));
#pragma unroll
    for (int v = 0; v < NSP; ++v)
      lds_copy4(sc_base[v] + (int64_t)kt * C::SCB, sc_off[v],
                lds_addr(st + C::CODE_BYTES + (wave + 4 * v) * 256));
  };
  auto src_kt = [&](int kt) __attribute__((always_inline)) { return min(kt, kt_n - 1); };

  // ---- this wave's conversions: fragments wave + 4d, d = 0..7
  constexpr int ND = C::NF / 4;
  uint4 cq[ND];
  uint32_t cs[ND / 2];   // scale byte pairs of fragments 2e (low half) and 2e + 1
  auto read_codes = [&](const uint8_t *st) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const int f = wave + 4 * d;
      cq[d] = *(const uint4 *)(st + f * kFragCodeBytes + lane * 16);
      const uint32_t sp = *(const uint16_t *)(st + C::CODE_BYTES + f * 128 + lane * 2);
      if (d & 1) cs[d / 2] |= sp << 16;
      else cs[d / 2] = sp;
    }
  };
  auto convert = [&](auto gc, uint8_t *dst) __attribute__((always_inline)) {
    constexpr int G = decltype(gc)::value;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const uint32_t q = G == 0 ? cq[d].x : G == 1 ? cq[d].y : G == 2 ? cq[d].z : cq[d].w;
      const uint32_t sp = cs[d / 2] >> (16 * (d & 1));
      const uint32_t sb = G < 2 ? (sp & 0xFFu) : ((sp >> 8) & 0xFFu);
      *(uint4 *)(dst + (wave + 4 * d) * kFragCodeBytes + lane * 16) = nv_dequant8_u4(q, sb);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int fa0 = wm * TM, fw0 = C::FA + wn * TN;
  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // the activation operands are held, the weight operands streamed one at a
  // time (registers: the accumulators fill the AGPRs)
  auto mma_sub = [&](const uint8_t *src) __attribute__((always_inline)) {
    h8v ah[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) ah[i] = *(const h8v *)(src + (fa0 + i) * kFragCodeBytes + lane * 16);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const h8v wh = *(const h8v *)(src + (fw0 + j) * kFragCodeBytes + lane * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh, ah[i], acc[i][j], 0, 0, 0);
    }
  };

  // ---- prologue: stages 0 and 1 copied, stage 0's first sub-block converted
  issue(ring(Stage<0>{}), 0);
  issue(ring(Stage<1>{}), src_kt(1));
  wait_vm<C::PS>();
  lds_barrier();
  read_codes(ring(Stage<0>{}));
  convert(Stage<0>{}, f16buf(Stage<0>{}));
  lds_barrier();
  issue(ring(Stage<0>{}), src_kt(2));

  // stage kt (ring R = kt % 2): sub-blocks 0..3 from the f16 buffers 0, 1, 0, 1
  // while sub-blocks 1..3 and the next stage's sub-block 0 are converted
  auto stage = [&](auto rc, int kt) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value;
    mma_sub(f16buf(Stage<0>{}));
    convert(Stage<1>{}, f16buf(Stage<1>{}));
    lds_barrier();
    mma_sub(f16buf(Stage<1>{}));
    convert(Stage<2>{}, f16buf(Stage<0>{}));
    lds_barrier();
    mma_sub(f16buf(Stage<0>{}));
    convert(Stage<3>{}, f16buf(Stage<1>{}));
    lds_barrier();
    // the next stage's copies have landed (the one after may be in flight)
    wait_vm<C::PS>();
    lds_barrier();
    const bool more = kt + 1 < kt_n;
    if (more) read_codes(ring(Stage<R + 1>{}));
    mma_sub(f16buf(Stage<1>{}));
    if (more) convert(Stage<0>{}, f16buf(Stage<0>{}));
    lds_barrier();
    // stage kt + 1's codes are in registers: its ring takes stage kt + 3
    issue(ring(Stage<R + 1>{}), src_kt(kt + 3));
  };
  for (int kt = 0; kt < kt_n; kt += 2) {
    stage(Stage<0>{}, kt);
    if (kt + 1 < kt_n) stage(Stage<1>{}, kt + 1);
  }
  wait_vm<0>();

  // ---- epilogue: as in the kernel above (quadrants staged through LDS)
  const Alpha alpha = make_alpha(a_ts[0], w_ts[0]);
  const int rl = lane & 15, cl = 4 * (lane >> 4);
  if (vec_store == 2) {
    lds_barrier();
    uint8_t *q = smem + wave * (QR * QP);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f &a = acc[i][j];
        const uint32_t lo = pack_bf16x2(apply_alpha(a[0], alpha), apply_alpha(a[1], alpha));
        const uint32_t hi = pack_bf16x2(apply_alpha(a[2], alpha), apply_alpha(a[3], alpha));
        *(uint2 *)(q + (16 * i + rl) * QP + 2 * (16 * j + cl)) = make_uint2(lo, hi);
      }
    constexpr int LPR = QC / 8, RPI = 64 / LPR;
    const int lr = lane / LPR, lc = 8 * (lane % LPR);
    const int row0 = (g0 + fa0) * 16, col = (n0 + wn * TN) * 16 + lc;
#pragma unroll 4
    for (int it = 0; it < QR / RPI; ++it) {
      const int r = it * RPI + lr, row = row0 + r;
      const uint4 v = *(const uint4 *)(q + r * QP + 2 * lc);
      if (row >= m) continue;
      uint16_t *dst = c + (int64_t)row * ldc + col;
      if (col + 7 < n) {
        *(uint4 *)dst = v;
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < n) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = (g0 + fa0 + i) * 16 + rl;
    if (row >= m) continue;
    uint16_t *crow = c + (int64_t)row * ldc;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col0 = (n0 + wn * TN + j) * 16 + cl;
      const v4f &a = acc[i][j];
      const uint32_t lo = pack_bf16x2(apply_alpha(a[0], alpha), apply_alpha(a[1], alpha));
      const uint32_t hi = pack_bf16x2(apply_alpha(a[2], alpha), apply_alpha(a[3], alpha));
      if (vec_store && col0 + 3 < n) {
        *(uint2 *)(crow + col0) = make_uint2(lo, hi);
      } else {
        if (col0 < n) crow[col0] = (uint16_t)lo;
        if (col0 + 1 < n) crow[col0 + 1] = (uint16_t)(lo >> 16);
        if (col0 + 2 < n) crow[col0 + 2] = (uint16_t)hi;
        if (col0 + 3 < n) crow[col0 + 3] = (uint16_t)(hi >> 16);
      }
    }
  }
}

}  // namespace

namespace {
std::atomic<int> g_nv_tile_mode{0};
std::atomic<int> g_fuse_large{0};
}  // namespace

int large_linear_fusion() { return g_fuse_large.load(std::memory_order_relaxed); }
int set_large_linear_fusion(int on) { return g_fuse_large.exchange(on ? 1 : 0, std::memory_order_relaxed); }

int nvfp4_tile_mode() { return g_nv_tile_mode.load(std::memory_order_relaxed); }
int set_nvfp4_tile_mode(int mode) { return g_nv_tile_mode.exchange(mode, std::memory_order_relaxed); }

int gemm_tile_config(int fmt, int64_t m, int64_t n) {
  // 256 x 256 tiles when they give every CU (256) at least one tile; 128 x
  // 128 otherwise (measured on the prefill and square shapes: the smaller
  // tile wins whenever the larger one leaves CUs idle).
  (void)fmt;
  const int64_t t88 = ((m + 255) / 256) * ((n + 255) / 256);
  return t88 >= 256 ? 88 : 44;
}

hipError_t launch_gemm_tile(const GemmArgs &g, int cfg, hipStream_t stream) {
  const int kt_n = (int)(k_pad(g.k) / kFragK);
  const int ga_n = (int)(round_up(g.m, 16) / 16);
  const int nt_n = (int)(round_up(g.n, 16) / 16);
  if (cfg == 0) cfg = gemm_tile_config(g.fmt, g.m, g.n);
  const int bm = cfg == 88 ? 256 : 128, bn = bm;
  const int tiles_m = (int)((g.m + bm - 1) / bm), tiles_n = (int)((g.n + bn - 1) / bn);
  // 2: 16-byte row stores through LDS; 1: 8-byte stores; 0: element stores
  const int vec = (g.ldc % 8 == 0 && (uintptr_t)g.c % 16 == 0)  ? 2
                  : (g.ldc % 4 == 0 && (uintptr_t)g.c % 8 == 0) ? 1
                                                                : 0;
  dim3 grid((unsigned)(tiles_m * tiles_n));
#define FP4_TILE(F, A, B)                                                                       \
  hipLaunchKernelGGL((k_gemm_tile<F, A, B>), grid, dim3(256), 0, stream, g.a_codes, g.a_scales, \
                     g.a_ts, g.w_codes, g.w_scales, g.w_ts, (int)g.m, (int)g.n, kt_n, ga_n,      \
                     nt_n, tiles_m, tiles_n, g.c, g.ldc, vec, Fused{})
  if (g.fmt == 1) {
    if (cfg == 88) FP4_TILE(1, 8, 8);
    else FP4_TILE(1, 4, 4);
  } else {
    if (cfg == 88 && nvfp4_tile_mode() == 1)
      hipLaunchKernelGGL((k_gemm_tile_nvlds<8, 8>), grid, dim3(256), 0, stream, g.a_codes,
                         g.a_scales, g.a_ts, g.w_codes, g.w_scales, g.w_ts, (int)g.m, (int)g.n,
                         kt_n, ga_n, nt_n, tiles_m, tiles_n, g.c, g.ldc, vec);
    else if (cfg == 88) FP4_TILE(0, 8, 8);
    else FP4_TILE(0, 4, 4);
  }
#undef FP4_TILE
  return hipGetLastError();
}

bool linear_fused_large_ok(int fmt, uint32_t recipe, int64_t m, int64_t n, int64_t k,
                           bool static_scale) {
  (void)k;
  if (!large_linear_fusion() || m <= kDecodeMaxM || (recipe & kRecipeMbs)) return false;
  if (fmt == 0 && !static_scale) return false;   // a dynamic scale needs the whole tensor first
  const int bm = gemm_tile_config(fmt, m, n) == 88 ? 256 : 128;
  return (m + bm - 1) / bm <= kMaxPanels;
}

hipError_t launch_linear_fused_large(const GemmArgs &g, const uint16_t *x,
                                     const float *static_scale, uint32_t recipe,
                                     uint32_t *scratch, hipStream_t stream) {
  const int kt_n = (int)(k_pad(g.k) / kFragK);
  const int ga_n = (int)(round_up(g.m, 16) / 16);
  const int nt_n = (int)(round_up(g.n, 16) / 16);
  const int cfg = gemm_tile_config(g.fmt, g.m, g.n);
  const int bm = cfg == 88 ? 256 : 128;
  const int tiles_m = (int)((g.m + bm - 1) / bm), tiles_n = (int)((g.n + bm - 1) / bm);
  // about one producer per CU, each panel split along K among `parts` of them;
  // a multiple of the XCD count in all, so the tiles' XCD numbering holds
  int parts = std::max(1, std::min(16, 256 / tiles_m));
  while ((tiles_m * parts) % kXcds) ++parts;
  const int nprod = tiles_m * parts;
  const int vec = (g.ldc % 8 == 0 && (uintptr_t)g.c % 16 == 0)  ? 2
                  : (g.ldc % 4 == 0 && (uintptr_t)g.c % 8 == 0) ? 1
                                                                : 0;
  Fused fz;
  fz.x = x;
  fz.st = static_scale;
  fz.panel = scratch + kPanelWords;
  fz.err = scratch + kErrWord;
  fz.nprod = nprod;
  fz.parts = parts;
  fz.k = (int)g.k;
  fz.recipe = recipe;
  fz.spin = exchange_spin_limit();
  dim3 grid((unsigned)(nprod + tiles_m * tiles_n));
#define FP4_FTILE(F, A, B)                                                                        \
  hipLaunchKernelGGL((k_gemm_tile<F, A, B, 1>), grid, dim3(256), 0, stream, g.a_codes, g.a_scales, \
                     g.a_ts, g.w_codes, g.w_scales, g.w_ts, (int)g.m, (int)g.n, kt_n, ga_n,         \
                     nt_n, tiles_m, tiles_n, g.c, g.ldc, vec, fz)
  if (g.fmt == 1) {
    if (cfg == 88) FP4_FTILE(1, 8, 8);
    else FP4_FTILE(1, 4, 4);
  } else {
    if (cfg == 88) FP4_FTILE(0, 8, 8);
    else FP4_FTILE(0, 4, 4);
  }
#undef FP4_FTILE
  return hipGetLastError();
}

}  // namespace fp4i
