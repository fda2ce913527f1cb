// quant.hip -- activation and weight quantization kernels for gfx950.
//
// NVFP4 (16-value blocks, E4M3 block scale, FP32 per-tensor scale) and MXFP4
// (32-value blocks, E8M0 block scale), per "Hardware FP4 inference for speech
// on Blackwell" (section "NVFP4, and the two ways it fails") and "FP4 n'existe
// pas ..." (section "Deux dialectes, deux strategies de scaling").
//
// One thread encodes one block. Output goes to the canonical row-major layout
// or to the fragment-tiled layout (16 rows x 128 values per 1 KB fragment, the
// operand order of the scaled matrix instruction), padding included.
//
// The dynamic NVFP4 per-tensor scale needs the tensor's largest magnitude
// before any block can be encoded. Two ways are used:
//   * small tensors (activations of skinny GEMMs): one launch of a fixed grid
//     of kActGrid workgroups. Each workgroup keeps its blocks in registers,
//     publishes its maximum in its own tagged word and waits (bounded) until
//     every workgroup's word carries this call's tag (grid_max_u32). Only
//     these 32-bit words cross workgroups, through device-coherent accesses,
//     so no cache writeback is needed. Zero-filled words are the initial state.
//   * large tensors: partial maxima per workgroup, then a second launch in
//     which every workgroup folds the (at most 1024) partials itself.
// Both are deterministic: a maximum does not depend on evaluation order.
#include "fp4_device.h"
#include "fp4_internal.h"

#include <algorithm>
#include <atomic>

namespace fp4i {
using namespace fp4d;

namespace {

constexpr int kThreads = 256;
constexpr unsigned kLdsPerCu = 160 * 1024;  // LDS per CU (gfx950)

template <int FMT>
struct Blk {
  static constexpr int B = FMT == 0 ? 16 : 32;  // values per block
  static constexpr int V = B / 8;               // uint4 loads per block
  static constexpr int BPF = 128 / B;           // blocks per fragment row
  static constexpr int SFB = FMT == 0 ? 128 : 64;
};

// Where block b (of 16/32 values) of row r goes.
template <int FMT, int TILED>
__device__ __forceinline__ void block_dst(int64_t r, int64_t b, int64_t kt_n, uint8_t *codes,
                                          int64_t cpitch, uint8_t *scales, int64_t spitch,
                                          uint8_t *&cdst, uint8_t *&sdst) {
  using K = Blk<FMT>;
  if (!TILED) {
    cdst = codes + r * cpitch + b * (K::B / 2);
    sdst = scales + r * spitch + b;
    return;
  }
  const int64_t frag = (r >> 4) * kt_n + b / K::BPF;
  const int rr = (int)(r & 15), bi = (int)(b % K::BPF);
  if (FMT == 0) {  // lane 16*(bi/2) + rr holds blocks bi (low 8 bytes) and bi^1
    const int lane = 16 * (bi >> 1) + rr;
    cdst = codes + frag * kFragCodeBytes + lane * 16 + (bi & 1) * 8;
    sdst = scales + frag * K::SFB + lane * 2 + (bi & 1);
  } else {
    const int lane = 16 * bi + rr;
    cdst = codes + frag * kFragCodeBytes + lane * 16;
    sdst = scales + frag * K::SFB + lane;
  }
}

template <int FMT>
__device__ __forceinline__ uint32_t block_absmax(const uint4 (&v)[Blk<FMT>::V]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < Blk<FMT>::V; ++i) m = max(m, absmax_bits8(v[i]));
  return m;
}

// Recipe bits (a kernel argument, uniform over the grid): rotate each block
// before anything else looks at its values; MXFP4 overflow-aware exponent;
// MXFP4 macro-block scales.
__device__ __forceinline__ bool rotates(uint32_t recipe) { return recipe & kRecipeRotate; }
__device__ __forceinline__ bool oas_rule(uint32_t recipe) { return recipe & kRecipeOas; }
__device__ __forceinline__ bool mbs(uint32_t recipe) { return recipe & kRecipeMbs; }

// Macro-block scale of a 128-value segment whose four blocks sit on lanes
// lane ^ {0, D, 2D, 3D} (D = 1: one block per thread, consecutive threads;
// D = 16: the tiled kernel's lane groups), from each lane's block maximum.
template <int D>
__device__ __forceinline__ float segment_mbs_scale(uint32_t bmax) {
  uint32_t g = max(bmax, (uint32_t)__shfl_xor((int)bmax, D, 64));
  g = max(g, (uint32_t)__shfl_xor((int)g, 2 * D, 64));
  return mbs_scale_from_bits(g);
}

// Where the macro-block scale of segment seg of row r goes.
template <int TILED>
__device__ __forceinline__ float *macro_dst(int64_t r, int64_t seg, int64_t kt_n, float *macro,
                                            int64_t mpitch) {
  if (!TILED) return macro + r * mpitch + seg;
  return macro + ((r >> 4) * kt_n + seg) * 16 + (r & 15);
}

template <int FMT>
__device__ __forceinline__ void maybe_rotate(uint4 (&v)[Blk<FMT>::V], uint32_t recipe) {
  if (rotates(recipe)) hadamard_block<Blk<FMT>::B>(v);
}

// Encode one block (values in v) and store codes + scale byte.
// smb: the block's macro-block scale (MXFP4 with MBS).
template <int FMT>
__device__ __forceinline__ void encode_store(const uint4 (&v)[Blk<FMT>::V], float st, float smb,
                                             uint8_t *cdst, uint8_t *sdst, uint32_t recipe) {
  uint32_t sbyte;
  if constexpr (FMT == 0) {
    uint2 c;
    nv_encode_block(v[0], v[1], st, c, sbyte);
    *(uint2 *)cdst = c;
  } else {
    uint4 c;
    if (mbs(recipe)) mbs_encode_block(v, smb, c, sbyte, oas_rule(recipe));
    else mx_encode_block(v, c, sbyte, oas_rule(recipe));
    *(uint4 *)cdst = c;
  }
  *sdst = (uint8_t)sbyte;
}

template <int FMT>
__device__ __forceinline__ void zero_store(uint8_t *cdst, uint8_t *sdst) {
  if (FMT == 0) *(uint2 *)cdst = make_uint2(0u, 0u);
  else *(uint4 *)cdst = make_uint4(0u, 0u, 0u, 0u);
  *sdst = 0;
}

// ------------------------------------------------------------------ large

// Partial maxima: grid-stride over 16-byte groups, four loads in flight per
// thread (one per stride) before their maxima are taken.
__global__ __launch_bounds__(kThreads) void k_amax_parts(const uint4 *__restrict__ x, int64_t n8,
                                                         uint32_t *__restrict__ parts) {
  __shared__ uint32_t lds[4];
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    const uint4 a = x[i], b = x[i + stride], c = x[i + 2 * stride], d = x[i + 3 * stride];
    m = max(m, max(max(absmax_bits8(a), absmax_bits8(b)), max(absmax_bits8(c), absmax_bits8(d))));
  }
  for (; i < n8; i += stride) m = max(m, absmax_bits8(x[i]));
  m = block_max_u32(m, lds);
  if (threadIdx.x == 0) parts[blockIdx.x] = m;
}

// Partial maxima of the rotated tensor (NVFP4 with rotation): block by block,
// each block rotated first. nblocks = rows * k / 16 (blocks never straddle
// rows, k being a multiple of 16).
__global__ __launch_bounds__(kThreads) void k_amax_parts_rot(const uint4 *__restrict__ x,
                                                             int64_t nblocks,
                                                             uint32_t *__restrict__ parts) {
  __shared__ uint32_t lds[4];
  uint32_t m = 0;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nblocks; i += stride) {
    uint4 v[2] = {x[2 * i], x[2 * i + 1]};
    hadamard_block<16>(v);
    m = max(m, max(absmax_bits8(v[0]), absmax_bits8(v[1])));
  }
  m = block_max_u32(m, lds);
  if (threadIdx.x == 0) parts[blockIdx.x] = m;
}

// Grid-stride over every block of the padded output; S_t (NVFP4) from the
// static value or the fold of the partial maxima.
template <int FMT, int TILED, int FULL>
__global__ __launch_bounds__(kThreads) void k_quant(
    const uint16_t *__restrict__ x, int64_t rows, int64_t k, int64_t rows_pad, int64_t kt_n,
    const uint32_t *__restrict__ parts, int nparts, const float *__restrict__ static_scale,
    uint8_t *__restrict__ codes, int64_t cpitch, uint8_t *__restrict__ scales, int64_t spitch,
    float *__restrict__ ts_out, uint32_t recipe, float *__restrict__ macro, int64_t mpitch) {
  using K = Blk<FMT>;
  if (!FULL) recipe &= kRecipeOas;  // the plain recipe: no rotation or MBS code
  __shared__ uint32_t lds[4];
  float st = 1.0f;
  if (FMT == 0) {
    if (static_scale) {
      st = *static_scale;
    } else {
      uint32_t m = 0;
      for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = max(m, parts[i]);
      st = tensor_scale_from_amax(bf16_bits_to_f32(block_max_u32(m, lds)));
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && ts_out) *ts_out = st;
  }
  const int64_t nb = k / K::B, nb_pad = kt_n * K::BPF, total = rows_pad * nb_pad;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // (with MBS the four blocks of a segment are four consecutive threads of
  // one iteration: nb_pad and the stride are multiples of 4)
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t r = t / nb_pad, b = t - r * nb_pad;
    uint8_t *cdst, *sdst;
    block_dst<FMT, TILED>(r, b, kt_n, codes, cpitch, scales, spitch, cdst, sdst);
    const bool pad = r >= rows || b >= nb;
    uint4 v[K::V];
    if (!pad) {
      const uint4 *src = (const uint4 *)(x + r * k + b * K::B);
#pragma unroll
      for (int i = 0; i < K::V; ++i) v[i] = src[i];
      maybe_rotate<FMT>(v, recipe);
    } else {
#pragma unroll
      for (int i = 0; i < K::V; ++i) v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    float smb = 1.0f;
    if (FMT == 1 && mbs(recipe)) {
      smb = segment_mbs_scale<1>(block_absmax<FMT>(v));
      if ((b & 3) == 0) *macro_dst<TILED>(r, b >> 2, kt_n, macro, mpitch) = smb;
    }
    if (pad) zero_store<FMT>(cdst, sdst);
    else encode_store<FMT>(v, st, smb, cdst, sdst, recipe);
  }
}

// Large tensors into the fragment-tiled layout: one wave per fragment of 16
// rows x 128 values, lane l = 16c + r taking row r's values 32c .. 32c + 31 —
// exactly the 16 code bytes and 2 (NVFP4) or 1 (MXFP4) scale bytes the lane
// owns in the fragment. Each lane reads 64 contiguous bytes of its row (a
// wave covers 16 rows x 256 bytes, whole cache lines) and the wave writes its
// fragment's 1 KB of codes and its scale bytes contiguously.
template <int FMT, int FULL>
__global__ __launch_bounds__(kThreads) void k_quant_tiled(
    const uint16_t *__restrict__ x, int64_t rows, int64_t k, int64_t rows_pad, int64_t kt_n,
    const uint32_t *__restrict__ parts, int nparts, const float *__restrict__ static_scale,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ ts_out,
    uint32_t recipe, float *__restrict__ macro) {
  using K = Blk<FMT>;
  if (!FULL) recipe &= kRecipeOas;  // the plain recipe: no rotation or MBS code
  __shared__ uint32_t lds[4];
  float st = 1.0f;
  if (FMT == 0) {
    if (static_scale) {
      st = *static_scale;
    } else {
      uint32_t m = 0;
      for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = max(m, parts[i]);
      st = tensor_scale_from_amax(bf16_bits_to_f32(block_max_u32(m, lds)));
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && ts_out) *ts_out = st;
  }
  const int lane = threadIdx.x & 63, r = lane & 15, c = lane >> 4;
  const int64_t frags = (rows_pad >> 4) * kt_n;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t f = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); f < frags;
       f += waves) {
    const int64_t row = (f / kt_n) * 16 + r, k0 = (f % kt_n) * kFragK + 32 * c;
    uint4 v[4];
    const uint4 *src = (const uint4 *)(x + row * k + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j)  // values k0 + 8j .. k0 + 8j + 7 (blocks never straddle k)
      v[j] = (row < rows && k0 + 8 * j < k) ? src[j] : make_uint4(0u, 0u, 0u, 0u);
    if (rotates(recipe)) {  // whole blocks only: a padding block stays zero
      if constexpr (FMT == 0) {
        uint4 b0[2] = {v[0], v[1]}, b1[2] = {v[2], v[3]};
        hadamard_block<16>(b0);
        hadamard_block<16>(b1);
        v[0] = b0[0]; v[1] = b0[1]; v[2] = b1[0]; v[3] = b1[1];
      } else {
        hadamard_block<32>(v);
      }
    }
    uint4 q;
    uint32_t sc;
    if constexpr (FMT == 0) {
      uint2 c0 = make_uint2(0u, 0u), c1 = make_uint2(0u, 0u);
      uint32_t s0 = 0, s1 = 0;
      if (row < rows && k0 < k) nv_encode_block(v[0], v[1], st, c0, s0);
      if (row < rows && k0 + 16 < k) nv_encode_block(v[2], v[3], st, c1, s1);
      q = make_uint4(c0.x, c0.y, c1.x, c1.y);
      sc = s0 | (s1 << 8);
      *(uint16_t *)(scales + f * K::SFB + lane * 2) = (uint16_t)sc;
    } else {
      q = make_uint4(0u, 0u, 0u, 0u);
      sc = 0;
      if (mbs(recipe)) {
        // lanes r, r + 16, r + 32, r + 48 hold the segment's four blocks
        const float smb = segment_mbs_scale<16>(max(max(absmax_bits8(v[0]), absmax_bits8(v[1])),
                                                    max(absmax_bits8(v[2]), absmax_bits8(v[3]))));
        if (row < rows && k0 < k) mbs_encode_block(v, smb, q, sc, oas_rule(recipe));
        if (c == 0) macro[f * 16 + r] = smb;
      } else if (row < rows && k0 < k) {
        mx_encode_block(v, q, sc, oas_rule(recipe));
      }
      scales[f * K::SFB + lane] = (uint8_t)sc;
    }
    *(uint4 *)(codes + f * kFragCodeBytes + lane * 16) = q;
  }
}

// ------------------------------------------------------------------ small

// Maximum over every workgroup of the grid (group_max_u32 with the grid as
// the group). The wait assumes every workgroup of the grid (at most kActGrid
// of at most 512 threads) runs at the same time.
__device__ __forceinline__ uint32_t grid_max_u32(uint32_t wg_max, uint32_t tag, uint32_t *slots,
                                                 uint32_t spin_limit, uint32_t *lds) {
  return group_max_u32<kActGrid, kSlotStride>(wg_max, tag, slots, blockIdx.x, gridDim.x,
                                              spin_limit, lds);
}

// Largest magnitude (bf16 bits) of the whole tensor, taken by one workgroup
// alone: its threads read every block (rotated first when the recipe says
// so) and the workgroup takes the maximum. Four blocks per thread are loaded
// before any is used; past the end the last block is read again, which the
// maximum does not mind.
template <int FMT>
__device__ __forceinline__ uint32_t tensor_absmax_wg(const uint16_t *x, int64_t nblk,
                                                     uint32_t recipe, uint32_t *lds) {
  using K = Blk<FMT>;
  uint32_t m = 0;
  for (int64_t t = threadIdx.x; t < nblk; t += 4 * (int64_t)blockDim.x) {
    uint4 u[4][K::V];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t b = min(t + j * (int64_t)blockDim.x, nblk - 1);
      const uint4 *src = (const uint4 *)(x + b * K::B);
#pragma unroll
      for (int i = 0; i < K::V; ++i) u[j][i] = src[i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      maybe_rotate<FMT>(u[j], recipe);
      m = max(m, block_absmax<FMT>(u[j]));
    }
  }
  return block_max_u32(m, lds);
}

// Single-launch quantization of a tensor of at most kActGrid * 256 * kActBpt
// (= kActGrid * 512 * 2) blocks. Every thread loads its (at most BPT) blocks first, so the values are
// in registers while the maximum is found. The dynamic-scale form runs as few
// workgroups as hold the tensor; with DYN = 1 they exchange their maxima,
// with DYN = 2 (small tensors) each workgroup reads the whole tensor and
// takes the maximum itself, with no exchange.
//
// When a workgroup of the exchange gives up (grid_max_u32), it encodes with a
// NaN tensor scale (zero codes and scales), sets kErrExchangeTimeout in the
// workspace's sticky error word, and the tensor scale written for the call is
// NaN: the last workgroup to finish writes S_t, and it knows from the arrival
// count (which also counts the workgroups that gave up) whether any did.
template <int FMT, int TILED, int DYN, int BPT, int NTH, int FULL>
__global__ __launch_bounds__(NTH) void k_quant_small(
    const uint16_t *__restrict__ x, int64_t rows, int64_t k, int64_t rows_pad, int64_t kt_n,
    const float *__restrict__ static_scale, uint8_t *__restrict__ codes, int64_t cpitch,
    uint8_t *__restrict__ scales, int64_t spitch, float *__restrict__ ts_out,
    uint32_t *__restrict__ sync, uint32_t recipe, uint32_t spin_limit, float *__restrict__ macro,
    int64_t mpitch) {
  using K = Blk<FMT>;
  if (!FULL) recipe &= kRecipeOas;  // the plain recipe: no rotation or MBS code
  __shared__ uint32_t lds[NTH / 64];
  const int64_t nb = k / K::B, nb_pad = kt_n * K::BPF, total = rows_pad * nb_pad;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t tag = 0;
  if (DYN == 1)  // this call's tag: one more than the previous call's (any slot)
    tag = ((__hip_atomic_load(&sync[blockIdx.x * kSlotStride], __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT) >> 16) + 1u) & 0xFFFFu;
  uint4 v[BPT][K::V];
  float smb[BPT];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int64_t t = t0 + i * stride;
    const int64_t r = t / nb_pad, b = t - r * nb_pad;
    if (t < total && r < rows && b < nb) {
      const uint4 *src = (const uint4 *)(x + r * k + b * K::B);
#pragma unroll
      for (int j = 0; j < K::V; ++j) v[i][j] = src[j];
    } else {
#pragma unroll
      for (int j = 0; j < K::V; ++j) v[i][j] = make_uint4(0u, 0u, 0u, 0u);
    }
    maybe_rotate<FMT>(v[i], recipe);
    const uint32_t bm = block_absmax<FMT>(v[i]);
    m = max(m, bm);
    // a segment's four blocks are four consecutive threads (nb_pad and the
    // grid stride are multiples of 4)
    smb[i] = (FMT == 1 && mbs(recipe)) ? segment_mbs_scale<1>(bm) : 1.0f;
  }
  float st = 1.0f;
  bool gave_up = false;
  uint32_t arrived_before = 0;
  if (FMT == 0) {
    if (DYN == 1) {
      const uint32_t g = grid_max_u32(block_max_u32(m, lds), tag, sync, spin_limit, lds);
      gave_up = g >= 0x8000u;
      st = gave_up ? __builtin_nanf("") : tensor_scale_from_amax(bf16_bits_to_f32(g));
      if (threadIdx.x == 0) {
        if (gave_up)
          __hip_atomic_fetch_or(&sync[kErrWord - kMaxAmaxParts], kErrExchangeTimeout,
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // arrivals in the low half, workgroups that gave up in the high half;
        // the result is first needed after the encoding below
        arrived_before = __hip_atomic_fetch_add(&sync[kArriveWord - kMaxAmaxParts],
                                                gave_up ? 0x10001u : 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      }
    } else if (DYN == 2) {
      st = tensor_scale_from_amax(bf16_bits_to_f32(tensor_absmax_wg<FMT>(x, rows * nb, recipe, lds)));
    } else {
      st = *static_scale;
    }
    if (DYN != 1 && blockIdx.x == 0 && threadIdx.x == 0 && ts_out) *ts_out = st;
  }
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int64_t t = t0 + i * stride;
    if (t >= total) break;
    const int64_t r = t / nb_pad, b = t - r * nb_pad;
    uint8_t *cdst, *sdst;
    block_dst<FMT, TILED>(r, b, kt_n, codes, cpitch, scales, spitch, cdst, sdst);
    if (r >= rows || b >= nb) zero_store<FMT>(cdst, sdst);
    else encode_store<FMT>(v[i], st, smb[i], cdst, sdst, recipe);
    if (FMT == 1 && mbs(recipe) && (b & 3) == 0)
      *macro_dst<TILED>(r, b >> 2, kt_n, macro, mpitch) = smb[i];
  }
  if (FMT == 0 && DYN == 1 && threadIdx.x == 0 && (arrived_before & 0xFFFFu) == gridDim.x - 1) {
    // the last workgroup: every other one has taken its decision
    const bool any_gave_up = gave_up || (arrived_before >> 16) != 0u;
    if (ts_out) *ts_out = any_gave_up ? __builtin_nanf("") : st;
    __hip_atomic_store(&sync[kArriveWord - kMaxAmaxParts], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One-pass NVFP4 quantization with the dynamic tensor scale of a mid-size
// tensor into the tiled layout: past the single-launch quantizer's capacity
// but small enough for the registers of kMidGrid resident workgroups. Wave w
// takes fragments w, w + W, ... (W waves in the grid; at most FPW of them),
// one fragment per wave step as in k_quant_tiled, and loads all of them
// before anything else; the workgroups then exchange their maxima through
// their own tagged words and encode from the registers, so the tensor is read
// from memory once instead of twice. A workgroup that gives up waiting
// behaves as in k_quant_small (NaN tensor scale, sticky error flag).
template <int FPW>
__global__ __launch_bounds__(kMidThreads) void k_quant_tiled_x(
    const uint16_t *__restrict__ x, int64_t rows, int64_t k, int64_t rows_pad, int64_t kt_n,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ ts_out,
    uint32_t *__restrict__ sync, uint32_t spin_limit) {
  __shared__ uint32_t lds[kMidThreads / 64];
  uint32_t *slots = sync + (kMidSlotWord - kMaxAmaxParts);
  // this call's tag: one more than the previous call's (any slot)
  const uint32_t tag = ((__hip_atomic_load(&slots[blockIdx.x * kSlotStride], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) >> 16) + 1u) & 0xFFFFu;
  const int lane = threadIdx.x & 63, r = lane & 15, c = lane >> 4;
  const int64_t frags = (rows_pad >> 4) * kt_n;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t w0 = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  uint4 v[FPW][4];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int64_t f = w0 + i * waves;
    const int64_t row = (f / kt_n) * 16 + r, k0 = (f % kt_n) * kFragK + 32 * c;
    const bool live = f < frags && row < rows;
    const uint4 *src = (const uint4 *)(x + row * k + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j)  // values k0 + 8j .. k0 + 8j + 7 (blocks never straddle k)
      v[i][j] = (live && k0 + 8 * j < k) ? src[j] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, absmax_bits8(v[i][j]));
  }
  const uint32_t g = group_max_u32<kMidGrid, kSlotStride>(block_max_u32(m, lds), tag, slots,
                                                          blockIdx.x, gridDim.x, spin_limit, lds);
  const bool gave_up = g >= 0x8000u;
  const float st = gave_up ? __builtin_nanf("") : tensor_scale_from_amax(bf16_bits_to_f32(g));
  uint32_t arrived_before = 0;
  if (threadIdx.x == 0) {
    if (gave_up)
      __hip_atomic_fetch_or(&sync[kErrWord - kMaxAmaxParts], kErrExchangeTimeout,
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    arrived_before = __hip_atomic_fetch_add(&sync[kArriveWord - kMaxAmaxParts],
                                            gave_up ? 0x10001u : 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int64_t f = w0 + i * waves;
    if (f >= frags) break;
    const int64_t row = (f / kt_n) * 16 + r, k0 = (f % kt_n) * kFragK + 32 * c;
    uint2 c0 = make_uint2(0u, 0u), c1 = make_uint2(0u, 0u);
    uint32_t s0 = 0, s1 = 0;
    if (row < rows && k0 < k) nv_encode_block(v[i][0], v[i][1], st, c0, s0);
    if (row < rows && k0 + 16 < k) nv_encode_block(v[i][2], v[i][3], st, c1, s1);
    *(uint16_t *)(scales + f * 128 + lane * 2) = (uint16_t)(s0 | (s1 << 8));
    *(uint4 *)(codes + f * kFragCodeBytes + lane * 16) = make_uint4(c0.x, c0.y, c1.x, c1.y);
  }
  if (threadIdx.x == 0 && (arrived_before & 0xFFFFu) == gridDim.x - 1) {
    // the last workgroup: every other one has taken its decision
    const bool any_gave_up = gave_up || (arrived_before >> 16) != 0u;
    if (ts_out) *ts_out = any_gave_up ? __builtin_nanf("") : st;
    __hip_atomic_store(&sync[kArriveWord - kMaxAmaxParts], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// --------------------------------------------------------------- test aids

// Tiled -> canonical copy (one thread per block of the padded canonical row).
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_export(
    const uint8_t *__restrict__ tc, const uint8_t *__restrict__ ts, int64_t rows, int64_t kt_n,
    uint8_t *__restrict__ codes, int64_t cpitch, uint8_t *__restrict__ scales, int64_t spitch,
    const float *__restrict__ tsc_in, float *__restrict__ tsc_out,
    const float *__restrict__ tmacro, float *__restrict__ macro, int64_t mpitch) {
  using K = Blk<FMT>;
  if (blockIdx.x == 0 && threadIdx.x == 0 && tsc_in && tsc_out) *tsc_out = *tsc_in;
  const int64_t nb_pad = kt_n * K::BPF, total = rows * nb_pad;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t r = t / nb_pad, b = t - r * nb_pad;
    uint8_t *tcd, *tsd, *ccd, *csd;
    block_dst<FMT, 1>(r, b, kt_n, (uint8_t *)tc, 0, (uint8_t *)ts, 0, tcd, tsd);
    block_dst<FMT, 0>(r, b, kt_n, codes, cpitch, scales, spitch, ccd, csd);
    if (FMT == 0) *(uint2 *)ccd = *(const uint2 *)tcd;
    else *(uint4 *)ccd = *(const uint4 *)tcd;
    *csd = *tsd;
    if (tmacro && (b & 3) == 0) *macro_dst<0>(r, b >> 2, kt_n, macro, mpitch) =
        *macro_dst<1>(r, b >> 2, kt_n, (float *)tmacro, 0);
  }
}

// Canonical -> tiled copy (one thread per block of the padded tiled layout;
// rows past the tensor and K padding come out zero).
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_import(
    const uint8_t *__restrict__ codes, int64_t cpitch, const uint8_t *__restrict__ scales,
    int64_t spitch, int64_t rows, int64_t rows_pad, int64_t kt_n, uint8_t *__restrict__ tc,
    uint8_t *__restrict__ ts, const float *__restrict__ macro, int64_t mpitch,
    float *__restrict__ tmacro) {
  using K = Blk<FMT>;
  const int64_t nb_pad = kt_n * K::BPF, total = rows_pad * nb_pad;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t r = t / nb_pad, b = t - r * nb_pad;
    uint8_t *tcd, *tsd;
    block_dst<FMT, 1>(r, b, kt_n, tc, 0, ts, 0, tcd, tsd);
    if (macro && (b & 3) == 0)   // padding rows: the scale of an all-zero segment
      *macro_dst<1>(r, b >> 2, kt_n, tmacro, 0) =
          r < rows ? *macro_dst<0>(r, b >> 2, kt_n, (float *)macro, mpitch) : 1.0f;
    if (r >= rows) {
      zero_store<FMT>(tcd, tsd);
      continue;
    }
    const uint8_t *ccd = codes + r * cpitch + b * (K::B / 2);
    if (FMT == 0) *(uint2 *)tcd = *(const uint2 *)ccd;
    else *(uint4 *)tcd = *(const uint4 *)ccd;
    *tsd = scales[r * spitch + b];
  }
}

// x^ = q * s_b * S_t (NVFP4) or q * 2^e_b (* S_mb with macro-block scales)
// rounded once to FP32. One thread per element.
template <int FMT, int TILED>
__global__ __launch_bounds__(kThreads) void k_dequant(
    const uint8_t *__restrict__ codes, int64_t cpitch, const uint8_t *__restrict__ scales,
    int64_t spitch, const float *__restrict__ tsc, int64_t rows, int64_t k, int64_t kt_n,
    float *__restrict__ out, int64_t ldo, const float *__restrict__ macro, int64_t mpitch) {
  using K = Blk<FMT>;
  const double st = (FMT == 0 && tsc) ? (double)*tsc : 1.0;
  const int64_t total = rows * k;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t r = t / k, kk = t - r * k;
    uint8_t *cd, *sd;
    block_dst<FMT, TILED>(r, kk / K::B, kt_n, (uint8_t *)codes, cpitch, (uint8_t *)scales,
                          spitch, cd, sd);
    const uint32_t byte = cd[(kk % K::B) / 2];
    const uint32_t code = (kk & 1) ? (byte >> 4) : (byte & 15u);
    const uint32_t ee = (code >> 1) & 3u, mm = code & 1u;
    const float qmag = ee == 0 ? 0.5f * (float)mm : ldexpf(1.0f + 0.5f * (float)mm, (int)ee - 1);
    double s = FMT == 0 ? (double)e4m3_to_f32(*sd) : ldexp(1.0, (int)*sd - 127);
    if (macro) s *= (double)*macro_dst<TILED>(r, kk / 128, kt_n, (float *)macro, mpitch);
    const double val = (double)qmag * s * st;
    out[r * ldo + kk] = (code & 8u) ? -(float)val : (float)val;
  }
}

int grid_for(int64_t work, int cap) {
  int64_t g = (work + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

std::atomic<uint32_t> g_spin_limit{kDefaultSpinLimit};

template <int FMT, int TILED>
void launch_small(const uint16_t *x, int64_t rows, int64_t k, int64_t rows_pad, int64_t kt_n,
                  const float *static_scale, uint8_t *codes, int64_t cpitch, uint8_t *scales,
                  int64_t spitch, float *ts_out, uint32_t *sync, uint32_t recipe, float *macro,
                  int64_t mpitch, hipStream_t stream) {
  const uint32_t spin = g_spin_limit.load(std::memory_order_relaxed);
  // the rotation and MBS code only in the kernels that need it: it holds
  // registers whether or not it runs
  const bool full = (recipe & (kRecipeRotate | kRecipeMbs)) != 0u;
  // One block per thread where the grid allows: encoding is the costly part
  // and spreads over as many CUs as there are blocks. The dynamic-scale form
  // also exchanges its maximum among the workgroups, so it stops at kActGrid
  // workgroups (of up to 512 threads with two blocks each); fewer workgroups
  // also means fewer polls of the exchange words.
  const int64_t total = rows_pad * kt_n * Blk<FMT>::BPF;
  const int64_t per_wg = (total + kThreads - 1) / kThreads;
  if (FMT == 0 && !static_scale) {
    // as few blocks per thread as the grid allows: the unrolled load and
    // encode steps of unused ones still cost time (1 instead of 4 blocks per
    // thread: 0.4-0.6 us per call on the decode shapes)
    int grid = (int)(per_wg < kActGrid ? per_wg : kActGrid);
#define FP4_QS1(D, BPT, NTH, FU)                                                                    \
  hipLaunchKernelGGL((k_quant_small<FMT, TILED, D, BPT, NTH, FU>), dim3(grid), dim3(NTH), 0, stream, \
                     x, rows, k, rows_pad, kt_n, static_scale, codes, cpitch, scales, spitch,        \
                     ts_out, sync, recipe, spin, macro, mpitch)
#define FP4_QS(D, BPT, NTH) do { if (full) FP4_QS1(D, BPT, NTH, 1); else FP4_QS1(D, BPT, NTH, 0); } while (0)
    // Small tensors: every workgroup reads the whole tensor for its maximum
    // rather than exchanging it (measured per call: M = 1, K = 5120: 4.9 ->
    // 3.9 us; M = 8, K = 5120: 5.15 -> 4.8 us; at M * K = 139264 it lost,
    // 5.2 -> 6.9 us, as each workgroup's reads grow). Not with the rotation:
    // every workgroup would rotate the whole tensor.
    if (rows * k <= kActRedundantMaxValues && per_wg <= kActGrid && !(recipe & kRecipeRotate))
      FP4_QS(2, 1, kThreads);
    else if (per_wg <= kActGrid) FP4_QS(1, 1, kThreads);
    else {
      // past 256 blocks per workgroup, 512-thread workgroups before two
      // blocks per thread (M = 32, K = 17408: 6.3 -> 5.85 us; with fewer
      // blocks the larger workgroups measured 0.5 us slower)
      const int64_t per_wg2 = (total + 2 * kThreads - 1) / (2 * kThreads);
      grid = (int)(per_wg2 < kActGrid ? per_wg2 : kActGrid);
      if (per_wg2 <= kActGrid) FP4_QS(1, 1, 2 * kThreads);
      else FP4_QS(1, 2, 2 * kThreads);
    }
#undef FP4_QS
#undef FP4_QS1
  } else if (full) {
    hipLaunchKernelGGL((k_quant_small<FMT, TILED, 0, 1, kThreads, 1>), dim3((unsigned)per_wg),
                       dim3(kThreads), 0, stream, x, rows, k, rows_pad, kt_n, static_scale, codes,
                       cpitch, scales, spitch, ts_out, sync, recipe, spin, macro, mpitch);
  } else {
    hipLaunchKernelGGL((k_quant_small<FMT, TILED, 0, 1, kThreads, 0>), dim3((unsigned)per_wg),
                       dim3(kThreads), 0, stream, x, rows, k, rows_pad, kt_n, static_scale, codes,
                       cpitch, scales, spitch, ts_out, sync, recipe, spin, macro, mpitch);
  }
}

template <int FMT, int TILED>
void launch_large(const uint16_t *x, int64_t rows, int64_t k, int64_t rows_pad, int64_t kt_n,
                  const uint32_t *parts, int nparts, const float *static_scale, uint8_t *codes,
                  int64_t cpitch, uint8_t *scales, int64_t spitch, float *ts_out, uint32_t recipe,
                  float *macro, int64_t mpitch, hipStream_t stream) {
  // the rotation and MBS code only in the kernels that need it: it holds
  // registers (the MXFP4 tiled quantizer: 183 of them with it) whether or
  // not it runs
  const bool full = (recipe & (kRecipeRotate | kRecipeMbs)) != 0u;
  if (TILED) {  // one wave per fragment, four waves per workgroup, grid-stride
    const int64_t frags = (rows_pad >> 4) * kt_n;
    const int grid = (int)std::min<int64_t>((frags + 3) / 4, 8192);
    // Plain MXFP4 on large tensors streams faster with fewer workgroups per
    // CU (its encode is short, so eight waves per SIMD only add concurrent
    // streams): dynamic LDS that is never touched caps residency at four
    // workgroups per CU from 64 MiB of bf16 input and at two from 384 MiB
    // (measured: 8192 x 8192 36.0 -> 32.2 us, 16384 x 16384 141.6 -> 123.6
    // us). NVFP4 (longer encode) and the recipe instances keep every wave.
    const int64_t in_bytes = rows * k * 2;
    const unsigned lds = FMT == 1 && !full && in_bytes >= (int64_t)384 << 20 ? kLdsPerCu / 2 - 1024
                         : FMT == 1 && !full && in_bytes >= (int64_t)64 << 20 ? kLdsPerCu / 4 - 1024
                                                                              : 0u;
#define FP4_QT(FU)                                                                               \
  hipLaunchKernelGGL((k_quant_tiled<FMT, FU>), dim3(grid), dim3(kThreads), lds, stream, x, rows, k, \
                     rows_pad, kt_n, parts, nparts, static_scale, codes, scales, ts_out, recipe,     \
                     macro)
    if (full) FP4_QT(1);
    else FP4_QT(0);
#undef FP4_QT
    return;
  }
  const int grid = grid_for(rows_pad * kt_n * Blk<FMT>::BPF, 8192);
#define FP4_QC(FU)                                                                                \
  hipLaunchKernelGGL((k_quant<FMT, TILED, FU>), dim3(grid), dim3(kThreads), 0, stream, x, rows, k, \
                     rows_pad, kt_n, parts, nparts, static_scale, codes, cpitch, scales, spitch,   \
                     ts_out, recipe, macro, mpitch)
  if (full) FP4_QC(1);
  else FP4_QC(0);
#undef FP4_QC
}

}  // namespace

uint32_t exchange_spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

uint32_t set_exchange_spin_limit(uint32_t polls) {
  return g_spin_limit.exchange(polls, std::memory_order_relaxed);
}

int amax_parts(int64_t n) {
  int64_t per = (int64_t)kThreads * 8 * 4;  // >= 4 uint4 loads per thread
  int64_t p = (n + per - 1) / per;
  if (p < 1) p = 1;
  if (p > kMaxAmaxParts) p = kMaxAmaxParts;
  return (int)p;
}

static_assert(kMidFragsPerWave == 4, "the mid-size quantizer has instances for 1, 2 and 4 fragments per wave");

bool quant_fits_mid(int fmt, uint32_t recipe, int64_t rows, int64_t k, int tiled) {
  if (fmt != 0 || !tiled || (recipe & kRecipeRotate) || quant_fits_small(fmt, rows, k, tiled))
    return false;
  const int64_t frags = round_up(rows, 16) / 16 * (k_pad(k) / kFragK);
  return frags <= (int64_t)kMidGrid * (kMidThreads / 64) * kMidFragsPerWave;
}

bool quant_fits_small(int fmt, int64_t rows, int64_t k, int tiled) {
  const int64_t rows_pad = tiled ? round_up(rows, 16) : rows;
  const int64_t blocks = rows_pad * (k_pad(k) / block_of(fmt));
  return blocks <= (int64_t)kActGrid * kThreads * kActBpt;
}

hipError_t launch_quantize(int fmt, uint32_t recipe, int tiled, const uint16_t *x, int64_t rows,
                           int64_t k, const float *static_scale, uint8_t *codes, int64_t cpitch,
                           uint8_t *scales, int64_t spitch, float *macro, int64_t mpitch,
                           float *ts_out, uint32_t *scratch, hipStream_t stream) {
  const int64_t rows_pad = tiled ? round_up(rows, 16) : rows;
  const int64_t kt_n = k_pad(k) / kFragK;
  if (quant_fits_small(fmt, rows, k, tiled)) {
    uint32_t *sync = scratch + kMaxAmaxParts;
#define FP4_QS(F, T) launch_small<F, T>(x, rows, k, rows_pad, kt_n, static_scale, codes, cpitch, \
                                        scales, spitch, ts_out, sync, recipe, macro, mpitch, stream)
    if (fmt == 0 && !tiled) FP4_QS(0, 0);
    else if (fmt == 0) FP4_QS(0, 1);
    else if (!tiled) FP4_QS(1, 0);
    else FP4_QS(1, 1);
#undef FP4_QS
    return hipGetLastError();
  }
  if (!static_scale && quant_fits_mid(fmt, recipe, rows, k, tiled)) {
    // as few fragments per wave and workgroups as hold the tensor
    const int64_t frags = (rows_pad >> 4) * kt_n, per_fpw = (int64_t)kMidGrid * (kMidThreads / 64);
    const int fpw = frags <= per_fpw ? 1 : frags <= 2 * per_fpw ? 2 : 4;
    const int grid = (int)((frags + fpw * (kMidThreads / 64) - 1) / (fpw * (kMidThreads / 64)));
    uint32_t *sync = scratch + kMaxAmaxParts;
    const uint32_t spin = exchange_spin_limit();
#define FP4_QX(F)                                                                                  \
  hipLaunchKernelGGL(k_quant_tiled_x<F>, dim3(grid), dim3(kMidThreads), 0, stream, x, rows, k,      \
                     rows_pad, kt_n, codes, scales, ts_out, sync, spin)
    if (fpw == 1) FP4_QX(1);
    else if (fpw == 2) FP4_QX(2);
    else FP4_QX(4);
#undef FP4_QX
    return hipGetLastError();
  }
  int nparts = 0;
  if (fmt == 0 && !static_scale) {
    // at most 512 partial maxima without rotation: fewer, longer-running
    // workgroups stream a large tensor faster (16384 x 16384: 111 -> ~100 us)
    nparts = amax_parts(rows * k);
    if (!(recipe & kRecipeRotate)) nparts = std::min(nparts, kMaxAmaxParts / 2);
    if (recipe & kRecipeRotate)
      hipLaunchKernelGGL(k_amax_parts_rot, dim3(nparts), dim3(kThreads), 0, stream,
                         (const uint4 *)x, rows * k / 16, scratch);
    else
      hipLaunchKernelGGL(k_amax_parts, dim3(nparts), dim3(kThreads), 0, stream, (const uint4 *)x,
                         rows * k / 8, scratch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#define FP4_QL(F, T) launch_large<F, T>(x, rows, k, rows_pad, kt_n, scratch, nparts, static_scale, \
                                        codes, cpitch, scales, spitch, ts_out, recipe, macro,       \
                                        mpitch, stream)
  if (fmt == 0 && !tiled) FP4_QL(0, 0);
  else if (fmt == 0) FP4_QL(0, 1);
  else if (!tiled) FP4_QL(1, 0);
  else FP4_QL(1, 1);
#undef FP4_QL
  return hipGetLastError();
}

hipError_t launch_export_canonical(int fmt, const uint8_t *tcodes, const uint8_t *tscales,
                                   const float *tmacro, int64_t rows, int64_t k, uint8_t *codes,
                                   int64_t cpitch, uint8_t *scales, int64_t spitch, float *macro,
                                   int64_t mpitch, const float *ts_in, float *ts_out,
                                   hipStream_t stream) {
  const int64_t kt_n = k_pad(k) / kFragK;
  const int grid = grid_for(rows * kt_n * (128 / block_of(fmt)), 8192);
  if (fmt == 0)
    hipLaunchKernelGGL(k_export<0>, dim3(grid), dim3(kThreads), 0, stream, tcodes, tscales, rows,
                       kt_n, codes, cpitch, scales, spitch, ts_in, ts_out, nullptr, nullptr,
                       (int64_t)0);
  else
    hipLaunchKernelGGL(k_export<1>, dim3(grid), dim3(kThreads), 0, stream, tcodes, tscales, rows,
                       kt_n, codes, cpitch, scales, spitch, ts_in, ts_out, tmacro, macro, mpitch);
  return hipGetLastError();
}

hipError_t launch_import_tiled(int fmt, const uint8_t *codes, int64_t cpitch, const uint8_t *scales,
                              int64_t spitch, const float *macro, int64_t mpitch, int64_t rows,
                              int64_t k, uint8_t *tcodes, uint8_t *tscales, float *tmacro,
                              hipStream_t stream) {
  const int64_t kt_n = k_pad(k) / kFragK, rows_pad = round_up(rows, 16);
  const int grid = grid_for(rows_pad * kt_n * (128 / block_of(fmt)), 8192);
  if (fmt == 0)
    hipLaunchKernelGGL(k_import<0>, dim3(grid), dim3(kThreads), 0, stream, codes, cpitch, scales,
                       spitch, rows, rows_pad, kt_n, tcodes, tscales, nullptr, (int64_t)0, nullptr);
  else
    hipLaunchKernelGGL(k_import<1>, dim3(grid), dim3(kThreads), 0, stream, codes, cpitch, scales,
                       spitch, rows, rows_pad, kt_n, tcodes, tscales, macro, mpitch, tmacro);
  return hipGetLastError();
}

hipError_t launch_dequant(int fmt, int tiled, const uint8_t *codes, int64_t cpitch,
                          const uint8_t *scales, int64_t spitch, const float *macro,
                          int64_t mpitch, const float *ts, int64_t rows, int64_t k, float *out,
                          int64_t ldo, hipStream_t stream) {
  const int64_t kt_n = k_pad(k) / kFragK;
  const int grid = grid_for(rows * k, 8192);
#define FP4_DQ(F, T)                                                                       \
  hipLaunchKernelGGL((k_dequant<F, T>), dim3(grid), dim3(kThreads), 0, stream, codes, cpitch, \
                     scales, spitch, ts, rows, k, kt_n, out, ldo, macro, mpitch)
  if (fmt == 0 && !tiled) FP4_DQ(0, 0);
  else if (fmt == 0) FP4_DQ(0, 1);
  else if (!tiled) FP4_DQ(1, 0);
  else FP4_DQ(1, 1);
#undef FP4_DQ
  return hipGetLastError();
}

}  // namespace fp4i
