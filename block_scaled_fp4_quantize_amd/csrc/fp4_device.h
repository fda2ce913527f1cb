// fp4_device.h -- device-side number formats for the gfx950 kernels.
//
// E2M1 element codes (S|EE|M, exponent bias 1) with magnitudes
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}, E4M3 block scales (largest finite 448) and
// E8M0 block exponents, as described on "Hardware FP4 inference for speech on
// Blackwell" (section "NVFP4, and the two ways it fails") and "FP4 n'existe
// pas ..." (section "Deux dialectes, deux strategies de scaling").
//
// Every rounding decision here is taken on exact values so that the result
// does not depend on evaluation order:
//   * block scales: the quotient a_b / (6 S_t) is a correctly rounded binary64
//     division, rounded to E4M3 from its binary64 bits (a real quotient that is
//     not an E4M3 midpoint stays >= ~2^-32 away from one, far above the
//     binary64 error, and an exact midpoint is computed exactly);
//   * element codes (NVFP4): each midpoint test |x| vs t * s_b * S_t is the sign
//     of one fused multiply-add, fma(t * s_b, S_t, -|x|), which is exact in
//     sign because t * s_b is exact in binary32 and the operands are pre-scaled
//     by 2^64 when S_t is tiny so that no nonzero difference underflows;
//   * element codes (MXFP4): x * 2^-e is exact, and the hardware FP4 convert
//     rounds it to nearest, ties to even, saturating at 6.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fp4d {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// bf16 round-to-nearest-even of a finite FP32 value (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// The GEMM output scale alpha = S_tA * S_tW (NVFP4; 1 for MXFP4), held as
// m * 2^e with m = fl(mA * mW) from the two scales' frexp mantissas, so that
// scaling an accumulator neither underflows nor overflows in an intermediate
// step: out = ldexp(acc * m, e), the power of two applied exactly (rounded
// once if the result is subnormal).
struct Alpha {
  float m;
  int e;
};
__device__ __forceinline__ Alpha make_alpha(float sa, float sw) {
  int ea, ew;
  const float ma = frexpf(sa, &ea), mw = frexpf(sw, &ew);
  return Alpha{ma * mw, ea + ew};
}
__device__ __forceinline__ float apply_alpha(float v, Alpha a) { return ldexpf(v * a.m, a.e); }

// E4M3 byte (sign clear, not NaN) -> exact FP32 value.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
  if (e == 0) return ldexpf((float)m, -9);
  return ldexpf((float)(8u + m), (int)e - 10);
}

// Nearest E4M3 byte to a non-negative binary64 value, ties to even mantissa,
// saturating at 448 (0x7E). Values >= 448 map to 0x7E (464 is the tie that
// still rounds to 448; anything above saturates).
__device__ __forceinline__ uint32_t e4m3_rne_sat(double q) {
  if (!(q > 0.0)) return 0u;
  if (q >= 448.0) return 0x7Eu;
  int e2;
  (void)frexp(q, &e2);          // q = f * 2^e2, f in [0.5, 1)
  int fl = e2 - 1;              // floor(log2 q)
  if (fl < -6) fl = -6;         // subnormals use the 2^-6 binade spacing
  double n = ldexp(q, 3 - fl);  // exact: q / 2^(fl-3)
  int r = (int)rint(n);         // round to nearest, ties to even
  if (r == 0) return 0u;
  if (fl == -6 && r < 8) return (uint32_t)r;         // subnormal
  if (r == 16) { fl += 1; r = 8; }
  return ((uint32_t)(fl + 7) << 3) | (uint32_t)(r - 8);
}

// Per-tensor NVFP4 decode scale from the tensor's largest magnitude g:
// S_t = RN_fp32(g / 2688) (2688 = 6 * 448), or 1 when g = 0.
__device__ __forceinline__ float tensor_scale_from_amax(float g) {
  if (!(g > 0.0f)) return 1.0f;
  return (float)((double)g / 2688.0);
}

// NVFP4 per-block encoder state: thresholds t * s_b for the seven midpoints of
// the E2M1 grid, the pre-scaled tensor scale and the pre-scale factor.
struct NvBlockEnc {
  float t[7];
  float st;      // S_t * sigma
  float sigma;   // 1 or 2^64
  bool zero;     // block scale rounded to zero: every code is +-0
};

__device__ __forceinline__ NvBlockEnc nv_block_encoder(uint32_t sbyte, float st) {
  NvBlockEnc e;
  float sv = e4m3_to_f32(sbyte);
  e.t[0] = 0.25f * sv; e.t[1] = 0.75f * sv; e.t[2] = 1.25f * sv; e.t[3] = 1.75f * sv;
  e.t[4] = 2.5f * sv;  e.t[5] = 3.5f * sv;  e.t[6] = 5.0f * sv;
  e.sigma = (st < 0x1p-64f) ? 0x1p64f : 1.0f;
  e.st = st * e.sigma;
  e.zero = (sbyte == 0u);
  return e;
}

// E2M1 magnitude index (0..7) of |x| (exact FP32) against the block's grid:
// midpoints between an odd and an even index are passed with '>', the others
// with '>=', so ties go to the even index; 6 * d_b saturates.
__device__ __forceinline__ uint32_t nv_encode_mag(const NvBlockEnc &e, float ax) {
  if (e.zero) return 0u;
  float axs = ax * e.sigma;
  uint32_t m = 0;
  m += (__builtin_fmaf(e.t[0], e.st, -axs) < 0.0f);
  m += (__builtin_fmaf(e.t[1], e.st, -axs) <= 0.0f);
  m += (__builtin_fmaf(e.t[2], e.st, -axs) < 0.0f);
  m += (__builtin_fmaf(e.t[3], e.st, -axs) <= 0.0f);
  m += (__builtin_fmaf(e.t[4], e.st, -axs) < 0.0f);
  m += (__builtin_fmaf(e.t[5], e.st, -axs) <= 0.0f);
  m += (__builtin_fmaf(e.t[6], e.st, -axs) < 0.0f);
  return m;
}

// Encode 8 bf16 values (one uint4) of an NVFP4 block into 8 nibbles (uint32).
__device__ __forceinline__ uint32_t nv_encode8(const NvBlockEnc &e, uint4 v) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t b = (w[i] >> (16 * h)) & 0xFFFFu;
      float ax = bf16_bits_to_f32(b & 0x7FFFu);
      uint32_t code = nv_encode_mag(e, ax) | ((b >> 12) & 8u);
      out |= code << (4 * (2 * i + h));
    }
  }
  return out;
}

// MXFP4 block exponent from the block maximum's bf16 bits (sign clear):
// e = clamp(floor(log2 a) - 2, -127, 127); the scale byte is e + 127.
// bf16 subnormals and zero have floor(log2 a) <= -127, so they clamp to -127.
// The overflow-aware rule (oas) takes the smallest e with a <= 6 * 2^e: with
// a = m * 2^E (m in [1, 2)) the default quotient a / 2^e is 4m, so one more
// step is needed exactly when m > 1.5, i.e. when the 7 stored mantissa bits
// exceed 0x40 (for the blocks that clamp to -127, a < 4 * 2^-127 already).
__device__ __forceinline__ int mx_exponent_from_bits(uint32_t abits, bool oas = false) {
  int ef = (int)(abits >> 7);      // biased exponent field
  int e = ef - 129;                // floor(log2 a) - 2 for normal a
  if (oas && (abits & 0x7Fu) > 0x40u) e += 1;
  return e < -127 ? -127 : e;
}

// Encode 8 bf16 values into 8 nibbles with the hardware FP4 convert applied to
// the exact quotient x * 2^-e (nearest, ties to even, saturating at 6).
__device__ __forceinline__ uint32_t mx_encode8(int e, uint4 v) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = ldexpf(bf16_bits_to_f32(w[i] & 0xFFFFu), -e);
    const float hi = ldexpf(bf16_bits_to_f32(w[i] >> 16), -e);
    // the byte-select operand writes byte i of `out` and keeps the others
    switch (i) {
      case 0: out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, lo, hi, 1.0f, 0); break;
      case 1: out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, lo, hi, 1.0f, 1); break;
      case 2: out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, lo, hi, 1.0f, 2); break;
      default: out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, lo, hi, 1.0f, 3); break;
    }
  }
  return out;
}

// ---- block helpers shared by the quantizers and the fused linear ----

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Workgroup-wide max of v (every thread receives it); lds holds one word per wave.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *lds) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  uint32_t r = lds[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = max(r, lds[i]);
  return r;
}

// Maximum over a group of G workgroups (this one is member g) through NS
// tagged 32-bit slots, ST words apart (one 128-byte line each, so that polls
// of different slots go to different lines): (call tag << 16) | a member's
// maximum as bf16 bits (< 2^15). Member g writes slots g, g + G, g + 2G, ...,
// so every call rewrites every slot whatever its group size, and after any
// call all slots carry that call's tag; a call's tag is therefore one more
// than any slot's tag at its start (a zero-filled array is tag 0). Thread
// t < G polls slot t until it carries this call's tag, and the workgroup takes
// the maximum. The values travel in the polled words themselves, so no cache
// writeback or fence is involved. The wait assumes every member runs at the
// same time; it is bounded by spin_limit polls per slot. A slot that does not
// arrive in time counts as 0xFFFF, so a result at or above 0x8000 (no bf16
// magnitude is) tells the caller this workgroup gave up.
template <int NS, int ST>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t wg_max, uint32_t tag, uint32_t *slots,
                                                  uint32_t g, uint32_t G, uint32_t spin_limit,
                                                  uint32_t *lds) {
  for (uint32_t s = g + threadIdx.x * G; s < (uint32_t)NS; s += blockDim.x * G)
    __hip_atomic_store(&slots[s * ST], (tag << 16) | wg_max, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  uint32_t v = 0;
  if (threadIdx.x < G) {
    bool arrived = false;
    for (uint32_t it = 0; it < spin_limit; ++it) {
      v = __hip_atomic_load(&slots[threadIdx.x * ST], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((v >> 16) == tag) {
        arrived = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    v = arrived ? (v & 0xFFFFu) : 0xFFFFu;
  }
  return block_max_u32(v, lds);
}

// Device-coherent stores (write through to memory, the cache policy of
// device-scope atomics), so that a reader in another workgroup of the same
// launch, on any XCD, sees them once the writer's stores are complete and it
// has said so through a device-scope atomic. The buffer resource is built
// from a wave-uniform base (a fragment's first byte) and each lane passes its
// byte offset: a resource is a scalar operand, and one built from a per-lane
// address makes the compiler issue the store once per distinct lane value.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}
__device__ __forceinline__ void store16_dev(__amdgpu_buffer_rsrc_t r, int off, uint4 v) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u4{v.x, v.y, v.z, v.w}, r, off, 0, 16);
}
__device__ __forceinline__ void store2_dev(__amdgpu_buffer_rsrc_t r, int off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, 16);
}
__device__ __forceinline__ void store1_dev(__amdgpu_buffer_rsrc_t r, int off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b8((unsigned char)v, r, off, 0, 16);
}

// |x| max of 8 bf16 values as a bit pattern (magnitudes order like their bits).
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

// Exact codes of the two values of bf16 pair word wv (byte I of the codes)
// from their bracket codes (below). The bracket is far narrower than any gap
// of the E2M1 grid, so where a value's two codes differ they are neighbours
// and its quotient x / d_b lies next to their midpoint mu. Then the sign of
// RN(mu * s_b * S_t - |x|) decides: mu * s_b is exact (at most 3 + 4
// significant bits), and with S_t >= 2^-100 every term is a multiple of
// 2^-134, so a nonzero difference keeps its sign through the one rounding.
// Ties go to the even code. Where the two codes agree every branch gives that
// code. hsv = s_b / 2; returns a mask of the nibbles that take hi's code.
template <int I>
__device__ __forceinline__ uint32_t nv_resolve_pair(uint32_t lo, uint32_t hi, uint32_t wv,
                                                    float hsv, float st) {
  const v2f gl = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(lo, 1.0f, I);
  const v2f gh = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(hi, 1.0f, I);
  const float a0 = __uint_as_float((wv << 16) & 0x7FFFFFFFu);
  const float a1 = __uint_as_float(wv & 0x7FFF0000u);
  // (|g_lo| + |g_hi|) / 2 is the midpoint (or the common grid value)
  const float t0 = __builtin_fmaf((__builtin_fabsf(gl.x) + __builtin_fabsf(gh.x)) * hsv, st, -a0);
  const float t1 = __builtin_fmaf((__builtin_fabsf(gl.y) + __builtin_fabsf(gh.y)) * hsv, st, -a1);
  const uint32_t odd0 = (lo >> (8 * I)) & 1u, odd1 = (lo >> (8 * I + 4)) & 1u;
  const bool up0 = t0 < 0.0f || (t0 == 0.0f && odd0);
  const bool up1 = t1 < 0.0f || (t1 == 0.0f && odd1);
  return ((up0 ? 0x0Fu : 0u) | (up1 ? 0xF0u : 0u)) << (8 * I);
}

// Fast NVFP4 element codes for 8 values with a bracket test. r ~ 1/d_b has a
// relative error below 2^-22, so r_lo = RN(r (1 - 2^-20)) and
// r_hi = RN(r (1 + 2^-20)) are strictly below and above 1/d_b, and the once-
// rounded products x r_lo and x r_hi strictly bracket the exact quotient
// x / d_b (their own rounding adds at most 2^-24). The hardware convert rounds
// two values at a time (nearest, ties to even, saturating) into one code byte,
// so each dword of bf16 pairs costs two converts, one per bracket end. When
// both ends give the same 8 codes, rounding is monotonic, so those are the
// exact quotient's codes; otherwise a quotient lies within 2^-19 of a rounding
// midpoint (or on it) and one exact comparison per value decides. Such
// quotients are common, not rare: with S_t = RN(amax / 2688), a bf16 value
// that is a small multiple of amax / 2688 gives a quotient that misses a
// midpoint only by S_t's rounding error (about 1% of 8-value groups of
// normal data). Returns the 8 nibbles.
__device__ __forceinline__ uint32_t nv_encode8_fast(uint32_t sbyte, float st, float r_lo,
                                                    float r_hi, uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = __uint_as_float(w[i] << 16), x1 = __uint_as_float(w[i] & 0xFFFF0000u);
    // the byte-select operand writes byte i and keeps the others
    switch (i) {
      case 0:
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x0 * r_lo, x1 * r_lo, 1.0f, 0);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x0 * r_hi, x1 * r_hi, 1.0f, 0);
        break;
      case 1:
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x0 * r_lo, x1 * r_lo, 1.0f, 1);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x0 * r_hi, x1 * r_hi, 1.0f, 1);
        break;
      case 2:
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x0 * r_lo, x1 * r_lo, 1.0f, 2);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x0 * r_hi, x1 * r_hi, 1.0f, 2);
        break;
      default:
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x0 * r_lo, x1 * r_lo, 1.0f, 3);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x0 * r_hi, x1 * r_hi, 1.0f, 3);
        break;
    }
  }
  if (lo != hi) {  // near a midpoint: exact comparisons
    // The empty statement hides v's value from the optimizer, so that the
    // exact path's per-value work is not hoisted into the common path.
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
    const float hsv = 0.5f * e4m3_to_f32(sbyte);
    // only the code bytes whose ends differ: a wave runs a pair's comparisons
    // when any of its lanes needs them, which for one pair of values is far
    // rarer than for the whole group of eight
    const uint32_t diff = lo ^ hi;
    uint32_t up = 0;
    if (diff & 0x000000FFu) up |= nv_resolve_pair<0>(lo, hi, v.x, hsv, st);
    if (diff & 0x0000FF00u) up |= nv_resolve_pair<1>(lo, hi, v.y, hsv, st);
    if (diff & 0x00FF0000u) up |= nv_resolve_pair<2>(lo, hi, v.z, hsv, st);
    if (diff & 0xFF000000u) up |= nv_resolve_pair<3>(lo, hi, v.w, hsv, st);
    lo = (lo & ~up) | (hi & up);
  }
  return lo;
}

// One NVFP4 block (16 values in v0, v1) under tensor scale st: 8 code bytes
// and the E4M3 scale byte.
__device__ __forceinline__ void nv_encode_block(uint4 v0, uint4 v1, float st, uint2 &codes,
                                                uint32_t &sbyte) {
  const uint32_t abits = max(absmax_bits8(v0), absmax_bits8(v1));
  const double q = (double)bf16_bits_to_f32(abits) / (6.0 * (double)st);
  sbyte = e4m3_rne_sat(q);
  if (sbyte != 0u && st >= 0x1p-100f) {
    // d_b = s_b * S_t >= 2^-109, so its reciprocal is a finite normal float;
    // rounding d_b and the reciprocal add < 2^-22 relative error to it.
    const float r = __builtin_amdgcn_rcpf(e4m3_to_f32(sbyte) * st);
    const float r_lo = r * 0x1.ffffep-1f, r_hi = r * 0x1.00001p+0f;
    codes = make_uint2(nv_encode8_fast(sbyte, st, r_lo, r_hi, v0),
                       nv_encode8_fast(sbyte, st, r_lo, r_hi, v1));
  } else {
    const NvBlockEnc enc = nv_block_encoder(sbyte, st);
    codes = make_uint2(nv_encode8(enc, v0), nv_encode8(enc, v1));
  }
}

// One MXFP4 block (32 values in v[0..3]): 16 code bytes and the E8M0 byte;
// oas selects the overflow-aware block exponent.
__device__ __forceinline__ void mx_encode_block(const uint4 (&v)[4], uint4 &codes,
                                                uint32_t &sbyte, bool oas = false) {
  const uint32_t abits = max(max(absmax_bits8(v[0]), absmax_bits8(v[1])),
                             max(absmax_bits8(v[2]), absmax_bits8(v[3])));
  const int e = mx_exponent_from_bits(abits, oas);
  codes = make_uint4(mx_encode8(e, v[0]), mx_encode8(e, v[1]), mx_encode8(e, v[2]),
                     mx_encode8(e, v[3]));
  sbyte = (uint32_t)(e + 127);
}

// ---- MXFP4 macro-block scaling (MBS) ----
//
// "FP4 n'existe pas ..." (section "L'ecart de qualite - et comment il se
// reduit") adds to MXFP4 a second-level scale over a macro-block of several
// 32-value blocks. Here a macro-block is the four blocks of one 128-value
// segment of a row along K (one fragment of the tiled layout), and its scale
// is the FP32 number S_mb in [1, 2) that puts the segment's largest magnitude
// g on the top code: S_mb = RN_fp32(g / (6 * 2^j)), j = floor(log2(g / 6))
// (1 when g = 0). Each block's E8M0 exponent is the MX rule applied to its
// values divided by S_mb, and elements round against d_b = 2^e_b * S_mb.

// S_mb from the segment maximum's bf16 bits (sign clear). g / 6 is a correctly
// rounded binary64 division; it never rounds across a power of two (g has 8
// significant bits) and its binary expansion (g / 3 / 2) never lies on a
// binary32 midpoint it was not on exactly, so the binary32 rounding of it is
// that of the real quotient.
__device__ __forceinline__ float mbs_scale_from_bits(uint32_t gbits) {
  if (gbits == 0u) return 1.0f;
  const double q = (double)bf16_bits_to_f32(gbits) / 6.0;
  int e2;
  (void)frexp(q, &e2);
  return (float)ldexp(q, 1 - e2);
}

// E8M0 exponent of a block with maximum bits abits under S_mb = s:
// clamp(floor(log2(a_b / s)) - 2, -127, 127), floor(log2(a_b / s)) being
// floor(log2 a_b) or one less as a_b < s * 2^floor(log2 a_b) (an exact
// binary64 product); oas: the smallest e with a_b <= 6 * 2^e * s.
__device__ __forceinline__ int mbs_exponent(uint32_t abits, float s, bool oas) {
  if (abits == 0u) return -127;
  const double ab = (double)bf16_bits_to_f32(abits);
  int e2;
  (void)frexp(ab, &e2);
  int fl = e2 - 1;
  if (ab < (double)s * ldexp(1.0, fl)) fl -= 1;
  int e = fl - 2;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  if (oas && e < 127 && ab > 6.0 * ldexp(1.0, e) * (double)s) e += 1;
  return e;
}

// E2M1 codes of 8 bf16 values against d_b = 2^e * s (s in [1, 2)): with
// y = |x| * 2^-e (exact, or below 2^-126 where every code is 0 anyway), the
// midpoint tests compare y with t * s. Both are multiples of 2^-25 wherever
// y >= 2^-18 (t has two fraction bits, s 23; y keeps 8 significant bits), so
// the nonzero difference fma(t, s, -y) keeps its sign through the rounding;
// below that y < t * s for every t. Ties go to the even index, 6 saturates.
__device__ __forceinline__ uint32_t mbs_encode8(int e, float s, uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t b = (w[i] >> (16 * h)) & 0xFFFFu;
      const float y = ldexpf(bf16_bits_to_f32(b & 0x7FFFu), -e);
      uint32_t m = 0;
      m += (__builtin_fmaf(0.25f, s, -y) < 0.0f);
      m += (__builtin_fmaf(0.75f, s, -y) <= 0.0f);
      m += (__builtin_fmaf(1.25f, s, -y) < 0.0f);
      m += (__builtin_fmaf(1.75f, s, -y) <= 0.0f);
      m += (__builtin_fmaf(2.5f, s, -y) < 0.0f);
      m += (__builtin_fmaf(3.5f, s, -y) <= 0.0f);
      m += (__builtin_fmaf(5.0f, s, -y) < 0.0f);
      out |= (m | ((b >> 12) & 8u)) << (4 * (2 * i + h));
    }
  }
  return out;
}

// One MXFP4 block (32 values) under macro-block scale s: 16 code bytes and
// the E8M0 byte.
__device__ __forceinline__ void mbs_encode_block(const uint4 (&v)[4], float s, uint4 &codes,
                                                 uint32_t &sbyte, bool oas) {
  const uint32_t abits = max(max(absmax_bits8(v[0]), absmax_bits8(v[1])),
                             max(absmax_bits8(v[2]), absmax_bits8(v[3])));
  const int e = mbs_exponent(abits, s, oas);
  codes = make_uint4(mbs_encode8(e, s, v[0]), mbs_encode8(e, s, v[1]), mbs_encode8(e, s, v[2]),
                     mbs_encode8(e, s, v[3]));
  sbyte = (uint32_t)(e + 127);
}

// ---- block rotation ----
//
// y_i = RN_bf16(c * sum_j H[i][j] x_j) over one block of B bf16 values, H_B
// the Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i & j)) and
// c = RN_fp32(1/sqrt(B)) (1/4 for B = 16, 0xB504F3 * 2^-26 for B = 32), as
// the MXFP4 path of "FP4 on a consumer RTX 5090: the Blackwell headline loses
// to plain int4" (section "Finding 3") rotates activations before quantizing
// them; the rotation size is the block, so every rotation stays inside the
// block it feeds. The sum and the product are exact and the bf16 rounding
// (nearest, ties to even) is the only one, so the result does not depend on
// the order of the additions; an exact zero gives +0.
//
// Fast path: every value is a multiple of the smallest quantum q_min in the
// block and every partial sum of a Walsh-Hadamard transform is below
// B * 2^(e_max + 1), so the binary64 transform is exact when the nonzero
// values' exponent fields differ by at most 45 - log2(B) (41 or 40 binades;
// wider only for crafted inputs); c * S is then split exactly into
// hi = RN(c S) and lo = fma(c, S, -hi). Other blocks take an exact integer
// path (rot_exact_one).

// bf16 bits of the real h + l rounded to nearest, ties to even, where
// h = RN_fp64(h + l) and l is the exact remainder (0 when h is exact). A
// binary64 bf16 midpoint h is decided by the sign of l. |h| >= 2^-137 or 0.
__device__ __forceinline__ uint32_t bf16_of_exact(double h, double l) {
  const uint64_t u = (uint64_t)__double_as_longlong(h);
  const uint32_t neg = (uint32_t)(u >> 63);
  const int ef = (int)((u >> 52) & 0x7FFu);
  if (ef == 0) return 0u;                              // exact zero: +0
  const int e = ef - 1023;                             // floor(log2 |h|)
  const uint64_t sig = (u & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int q = e - 7 > -133 ? e - 7 : -133;           // exponent of the bf16 quantum
  int drop = 52 - e + q;                               // 45 (normal) .. 56 (subnormal)
  if (drop > 62) drop = 62;
  uint64_t r = sig >> drop;
  const uint64_t rem = sig & ((1ull << drop) - 1ull), half = 1ull << (drop - 1);
  const bool tie_up = l != 0.0 ? ((l < 0.0) == (neg != 0u)) : (r & 1ull) != 0ull;
  if (rem > half || (rem == half && tie_up)) r += 1ull;
  // r * 2^q as bf16: exponent field q + 134 over the 8-bit significand r
  // (a carry to 256, or a subnormal r, land in the right fields by themselves)
  return (((uint32_t)(q + 133) << 7) + (uint32_t)r) | (neg << 15);
}

// The same from an FP32 pair: h = RN_fp32 of the exact value (or the value
// itself), l the exact residual. A bf16 midpoint is an FP32 number, so h lies
// on the exact value's side of every midpoint unless it is one; then l's sign
// decides (none: ties to even).
__device__ __forceinline__ uint32_t bf16_of_exact32(float h, float l) {
  const uint32_t b = __float_as_uint(h);
  if ((b & 0x7FFFFFFFu) == 0u) return 0u;             // exact zero: +0
  const uint32_t neg = b >> 31, rem = b & 0xFFFFu;
  uint32_t r = b >> 16;
  const bool tie_up = l != 0.0f ? ((l < 0.0f) == (neg != 0u)) : (r & 1u) != 0u;
  if (rem > 0x8000u || (rem == 0x8000u && tie_up)) r += 1u;
  return r;
}

// Exact rotation output i of a block (bf16 bits in vals[0 .. B-1]) with
// integer arithmetic: |x| = n * 2^-133 with n < 2^261, the signed sum in a
// 320-bit two's complement integer (ten 32-bit words), multiplied by the
// norm's integer significand cint and rounded to bf16 with the value's scale
// 2^sexp. Kept out of line: only blocks with a wide magnitude range get here.
__device__ __attribute__((noinline)) uint32_t rot_exact_one(const uint32_t *vals, int nvals, int i,
                                                            uint32_t cint, int sexp) {
  constexpr int NW = 10;
  uint32_t a[NW];
  for (int t = 0; t < NW; ++t) a[t] = 0u;
  for (int j = 0; j < nvals; ++j) {
    const uint32_t b = vals[j], f = (b >> 7) & 0xFFu, m = b & 0x7Fu;
    if (f == 0u && m == 0u) continue;
    const uint32_t sig = f ? (m | 0x80u) : m;
    const int sh = f ? (int)f - 1 : 0;
    const bool sub = ((b >> 15) ^ (uint32_t)(__popc((uint32_t)(i & j)) & 1)) != 0u;
    const int w0 = sh >> 5, off = sh & 31;
    uint64_t t = (uint64_t)sig << off;                // <= 40 bits over words w0, w0 + 1
    uint32_t carry = 0u;
    for (int w = w0; w < NW; ++w) {
      const uint64_t part = t & 0xFFFFFFFFull;
      t >>= 32;
      uint64_t r;
      if (!sub) {
        r = (uint64_t)a[w] + part + carry;
        carry = (uint32_t)(r >> 32);
      } else {
        r = (uint64_t)a[w] - part - carry;
        carry = (uint32_t)((r >> 63) & 1ull);
      }
      a[w] = (uint32_t)r;
      if (t == 0ull && carry == 0u) break;
    }
  }
  const uint32_t neg = a[NW - 1] >> 31;
  if (neg) {                                          // magnitude of a negative sum
    uint32_t c = 1u;
    for (int w = 0; w < NW; ++w) {
      const uint64_t r = (uint64_t)(~a[w]) + c;
      a[w] = (uint32_t)r;
      c = (uint32_t)(r >> 32);
    }
  }
  {
    uint64_t c = 0ull;                                // times the norm (< 2^24)
    for (int w = 0; w < NW; ++w) {
      const uint64_t r = (uint64_t)a[w] * cint + c;
      a[w] = (uint32_t)r;
      c = r >> 32;
    }
  }
  int top = NW - 1;
  while (top >= 0 && a[top] == 0u) --top;
  if (top < 0) return 0u;                             // exact zero: +0
  const int len = 32 * top + 32 - __clz(a[top]);
  const int q = len - 1 + sexp - 7 > -133 ? len - 1 + sexp - 7 : -133;
  const int drop = q - sexp;                          // >= 1: bits below the quantum
  auto bit = [&](int p) -> uint32_t { return p < 0 ? 0u : (a[p >> 5] >> (p & 31)) & 1u; };
  uint32_t r = 0u;
  for (int p = drop + 8; p >= drop; --p) r = (r << 1) | bit(p);
  const uint32_t half = bit(drop - 1);
  bool sticky = false;
  const int lim = drop - 1;                           // bits [0, lim) decide a tie
  for (int w = 0; w < NW && 32 * w < lim; ++w) {
    const uint32_t mask = 32 * w + 32 <= lim ? 0xFFFFFFFFu : ((1u << (lim - 32 * w)) - 1u);
    sticky |= (a[w] & mask) != 0u;
  }
  if (half && (sticky || (r & 1u))) r += 1u;
  return (((uint32_t)(q + 133) << 7) + r) | (neg << 15);
}

template <int B>
__device__ __forceinline__ void hadamard_block(uint4 (&v)[B / 8]) {
  static_assert(B == 16 || B == 32, "rotation size is a block: 16 or 32 values");
  constexpr int kLog2B = B == 16 ? 4 : 5;
  uint32_t w[B / 2];
#pragma unroll
  for (int i = 0; i < B / 8; ++i) {
    w[4 * i] = v[i].x; w[4 * i + 1] = v[i].y; w[4 * i + 2] = v[i].z; w[4 * i + 3] = v[i].w;
  }
  // exponent fields of the nonzero values (subnormals count as field 1: the
  // same quantum, 2^-133)
  int fmax = 0, fmin = 255;
#pragma unroll
  for (int j = 0; j < B / 2; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t b = (w[j] >> (16 * h)) & 0xFFFFu;
      const int f = max((int)((b >> 7) & 0xFFu), 1);
      if (b & 0x7FFFu) {
        fmax = max(fmax, f);
        fmin = min(fmin, f);
      }
    }
  uint32_t out[B / 2];
  // Three ways to the same result. FP32: every value is a multiple of the
  // smallest one's quantum 2^(fmin-134) below 2^(fmax-126), so every partial
  // sum of the transform is one below 2^(fmax-fmin+8+log2 B) quanta: exact in
  // FP32 when that is at most 2^24, with no overflow (fmax <= 245); for
  // B = 32 the product with c is split exactly into RN + FMA residual when
  // no nonzero sum is below 2^-100 (fmin >= 34). Binary64: the same with 53
  // bits, exact wherever FP32 is. Otherwise integers. A wave takes the FP32
  // way only when all its lanes can (a wave runs every way any lane takes,
  // and a binary64 block sits in most waves of 32-value blocks of normal
  // data).
  const bool f32_ok = fmax - fmin <= 16 - kLog2B && fmax <= 245 && (B == 16 || fmin >= 34);
  if (__all(f32_ok)) {
    float y[B];
#pragma unroll
    for (int j = 0; j < B / 2; ++j) {
      y[2 * j] = __uint_as_float(w[j] << 16);
      y[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
#pragma unroll
    for (int span = 1; span < B; span *= 2)
#pragma unroll
      for (int i = 0; i < B; ++i)
        if ((i & span) == 0) {
          const float lo = y[i], hi = y[i + span];
          y[i] = lo + hi;
          y[i + span] = lo - hi;
        }
    uint32_t r[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if constexpr (B == 16) {
        r[i] = bf16_of_exact32(y[i] * 0.25f, 0.0f);      // exact product
      } else {
        const float c = 0x1.6a09e6p-3f;                  // RN_fp32(1/sqrt(32))
        const float hi = y[i] * c;
        r[i] = bf16_of_exact32(hi, __builtin_fmaf(y[i], c, -hi));
      }
    }
#pragma unroll
    for (int j = 0; j < B / 2; ++j) out[j] = r[2 * j] | (r[2 * j + 1] << 16);
  } else if (fmax - fmin <= 45 - kLog2B) {
    double y[B];
#pragma unroll
    for (int j = 0; j < B / 2; ++j) {
      y[2 * j] = (double)__uint_as_float(w[j] << 16);
      y[2 * j + 1] = (double)__uint_as_float(w[j] & 0xFFFF0000u);
    }
#pragma unroll
    for (int span = 1; span < B; span *= 2)
#pragma unroll
      for (int i = 0; i < B; ++i)
        if ((i & span) == 0) {
          const double lo = y[i], hi = y[i + span];
          y[i] = lo + hi;
          y[i + span] = lo - hi;
        }
    uint32_t r[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if constexpr (B == 16) {
        r[i] = bf16_of_exact(y[i] * 0.25, 0.0);          // exact product
      } else {
        const double c = (double)0x1.6a09e6p-3f;         // RN_fp32(1/sqrt(32))
        const double hi = y[i] * c;
        r[i] = bf16_of_exact(hi, __builtin_fma(y[i], c, -hi));
      }
    }
#pragma unroll
    for (int j = 0; j < B / 2; ++j) out[j] = r[2 * j] | (r[2 * j + 1] << 16);
  } else {
    uint32_t vals[B];
#pragma unroll
    for (int j = 0; j < B / 2; ++j) {
      vals[2 * j] = w[j] & 0xFFFFu;
      vals[2 * j + 1] = w[j] >> 16;
    }
    // value = n * cint * 2^sexp: 2^-135 * n (B = 16), 0xB504F3 * 2^-159 * n (B = 32)
    const uint32_t cint = B == 16 ? 1u : 0xB504F3u;
    const int sexp = B == 16 ? -135 : -159;
    for (int j = 0; j < B / 2; ++j)
      out[j] = rot_exact_one(vals, B, 2 * j, cint, sexp) |
               (rot_exact_one(vals, B, 2 * j + 1, cint, sexp) << 16);
  }
#pragma unroll
  for (int i = 0; i < B / 8; ++i)
    v[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

// ---- decode side ----

// Two FP4 codes (byte b of q) -> two f16 values q * 2^8 (exact).
__device__ __forceinline__ h2v fp4x2_to_h2_times256(uint32_t q, int b) {
  switch (b) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 256.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 256.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 256.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 256.0f, 3);
  }
}

// E4M3 scale byte -> f16 bits of s_b * 2^-8 in both halves (exact: the E4M3
// exponent and mantissa fields land in the f16 fields with a bias offset of 8).
__device__ __forceinline__ h2v e4m3_scaled_h2(uint32_t byte) {
  uint32_t h = (byte & 0x7Fu) << 7;
  return __builtin_bit_cast(h2v, h | (h << 16));
}

// Dequantize one lane's 32 NVFP4 codes (4 dwords, value j in nibble j) with
// two E4M3 scales (byte 0: values 0-15, byte 1: values 16-31) into exact f16
// values q * s_b, returned as four groups of 8 values (group g = values 8g..8g+7).
// The convert applies only the exponent of its scale (2^8 here); the E4M3
// mantissa is applied by an exact f16 multiply by s_b * 2^-8.
__device__ __forceinline__ void nv_dequant32(uint4 q, uint32_t s2, h8v out[4]) {
  h2v sc0 = e4m3_scaled_h2(s2 & 0xFFu), sc1 = e4m3_scaled_h2((s2 >> 8) & 0xFFu);
  uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    h2v sc = d < 2 ? sc0 : sc1;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      // the byte-select operand picks byte b (values 2b, 2b+1 of this dword)
      h2v v = fp4x2_to_h2_times256(w[d], b) * sc;
      out[d][2 * b] = v[0];
      out[d][2 * b + 1] = v[1];
    }
  }
}

// Dequantize 8 NVFP4 codes (one dword, value j in nibble j) with E4M3 scale
// byte sbyte into 8 exact f16 values q * s_b (returned as a uint4).
__device__ __forceinline__ uint4 nv_dequant8_u4(uint32_t q, uint32_t sbyte) {
  const h2v sc = e4m3_scaled_h2(sbyte);
  uint32_t r[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    h2v v = fp4x2_to_h2_times256(q, b) * sc;
    r[b] = __builtin_bit_cast(uint32_t, v);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ v8i frag_v8i(uint4 q) {
  v8i r;
  r[0] = (int)q.x; r[1] = (int)q.y; r[2] = (int)q.z; r[3] = (int)q.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

}  // namespace fp4d
