// api.hip -- host implementation of the C ABI declared in include/fp4.h.
//
// Validation happens here, on the host, before any launch; every launch is
// asynchronous on the caller's stream. The library allocates nothing: all
// scratch comes from caller-provided workspaces whose sizes these functions
// report.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/fp4.h"
#include "fp4_internal.h"

#include <algorithm>

using namespace fp4i;

namespace {

thread_local std::string g_last_error;

fp4_status fail(fp4_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fp4_status ok() {
  g_last_error.clear();
  return FP4_OK;
}

fp4_status hip_fail(hipError_t e, const char *what) {
  return fail(FP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Per-device "is gfx950" cache.
std::mutex g_dev_mu;
int g_dev_state[64];  // 0 unknown, 1 ok, 2 wrong arch

fp4_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(FP4_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    g_dev_state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  if (g_dev_state[dev] != 1) return fail(FP4_ERR_DEVICE, "device %d is not gfx950", dev);
  return FP4_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// A format value is a base format (low byte) with optional recipe flags.
int base_fmt(int32_t f) { return f & 0xFF; }
uint32_t recipe_of(int32_t f) {
  return ((f & FP4_ROTATE) ? kRecipeRotate : 0u) | ((f & FP4_MX_OAS) ? kRecipeOas : 0u) |
         ((f & FP4_MX_MBS) ? kRecipeMbs : 0u);
}
bool has_mbs(int32_t f) { return (f & FP4_MX_MBS) != 0; }
bool valid_fmt(int32_t f) {
  const int b = base_fmt(f);
  if (b != FP4_NVFP4 && b != FP4_MXFP4) return false;
  if (f & ~(0xFF | FP4_ROTATE | FP4_MX_OAS | FP4_MX_MBS)) return false;
  return !(f & (FP4_MX_OAS | FP4_MX_MBS)) || b == FP4_MXFP4;
}
// Operands of one product: same base format, both rotated or neither, both
// with macro-block scales or neither (the block exponent rule may differ).
bool same_product_fmt(int32_t a, int32_t w) {
  return base_fmt(a) == base_fmt(w) && (a & FP4_ROTATE) == (w & FP4_ROTATE) &&
         has_mbs(a) == has_mbs(w);
}

// Macro-block scales (MXFP4 with MBS) follow a tensor's E8M0 bytes in its
// scales buffer: tiled, 16 floats per fragment after the fragments' E8M0
// bytes; canonical, [rows][K_pad / 128] floats from the first 16-byte
// boundary past rows * scales_pitch bytes.
int64_t macro_pitch(int64_t k) { return k_pad(k) / kFragK; }
size_t macro_offset(int32_t layout, int64_t rows, int64_t k, int64_t scales_pitch) {
  if (layout == FP4_LAYOUT_TILED)
    return (size_t)(round_up(rows, 16) / 16 * (k_pad(k) / kFragK) * 64);
  return (size_t)round_up(rows * scales_pitch, 16);
}
float *macro_of(const fp4_tensor *t) {
  if (!has_mbs(t->fmt)) return nullptr;
  return (float *)((uint8_t *)t->scales + macro_offset(t->layout, t->rows, t->cols, t->scales_pitch));
}
bool valid_layout(int32_t l) { return l == FP4_LAYOUT_CANONICAL || l == FP4_LAYOUT_TILED; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

fp4_status check_shape(int32_t fmt, int64_t rows, int64_t k) {
  if (!valid_fmt(fmt)) return fail(FP4_ERR_INVALID_ARG, "unknown format %d", (int)fmt);
  if (rows <= 0 || k <= 0) return fail(FP4_ERR_INVALID_ARG, "rows and k must be positive");
  if (rows > (int64_t)1 << 30 || k > (int64_t)1 << 30)
    return fail(FP4_ERR_SHAPE, "rows or k too large");
  const int bs = block_of(base_fmt(fmt));
  if (k % bs != 0)
    return fail(FP4_ERR_SHAPE, "k=%lld is not a multiple of the block size %d", (long long)k, bs);
  return FP4_OK;
}

// Validate a tensor descriptor's self-consistency.
fp4_status check_tensor(const fp4_tensor *t, const char *name) {
  if (!t) return fail(FP4_ERR_INVALID_ARG, "%s is null", name);
  fp4_status st = check_shape(t->fmt, t->rows, t->cols);
  if (st != FP4_OK) return st;
  if (!valid_layout(t->layout)) return fail(FP4_ERR_INVALID_ARG, "%s: unknown layout", name);
  if (!t->codes || !t->scales) return fail(FP4_ERR_INVALID_ARG, "%s: null buffer", name);
  if (!aligned16(t->codes) || !aligned16(t->scales))
    return fail(FP4_ERR_ALIGNMENT, "%s: buffers must be 16-byte aligned", name);
  const int base = base_fmt(t->fmt);
  if (base == FP4_NVFP4 && !t->tensor_scale)
    return fail(FP4_ERR_INVALID_ARG, "%s: NVFP4 needs a tensor_scale pointer", name);
  if (t->layout == FP4_LAYOUT_CANONICAL) {
    int64_t kp = k_pad(t->cols);
    if (t->codes_pitch < kp / 2 || t->scales_pitch < kp / block_of(base))
      return fail(FP4_ERR_SHAPE, "%s: pitch smaller than K_pad", name);
    if (t->codes_pitch % 16 != 0 || (base == FP4_NVFP4 && t->scales_pitch % 2 != 0))
      return fail(FP4_ERR_ALIGNMENT, "%s: codes pitch must be a multiple of 16 bytes and "
                  "NVFP4 scales pitch even", name);
  }
  return FP4_OK;
}

// The fused skinny linear repeats the activation quantization in every
// weight tile's workgroup; with the (exact) rotation that repeated work never
// pays off (decode shapes at M = 1: 17.8 - 40.7 us fused against 13.5 - 20.9
// us for the separate quantizer plus the skinny GEMM at M = 8).
bool use_fused(int32_t fmt, int64_t m, int64_t n, int64_t k) {
  return linear_fused_ok(base_fmt(fmt), m, n, k) && !(fmt & FP4_ROTATE) && !has_mbs(fmt);
}

size_t quant_ws(int32_t fmt) { return base_fmt(fmt) == FP4_NVFP4 ? kQuantScratchBytes : 0; }

// Everything fp4_linear keeps in its workspace: the quantizer's scratch (its
// exchange words persist from call to call) at offset 0 whatever the call's
// shape, so that one workspace can serve calls of different shapes; then the
// tensor scale, the activations quantized into the tiled layout and, for
// 33-128 rows, the mid-size GEMM's partial sums (`splits` slices of K).
struct LinearLayout {
  size_t codes, scales, ts, scratch, part, total;
  int splits;
};

// Bytes of a tiled tensor's scales buffer (with the macro-block scales).
size_t tiled_scales_bytes(int32_t fmt, int64_t rows, int64_t k) {
  const int64_t mp = round_up(rows, 16), kp = k_pad(k);
  return (size_t)(mp * kp / block_of(base_fmt(fmt))) + (has_mbs(fmt) ? (size_t)(mp * kp / 32) : 0);
}

// Partial sums of the mid-size GEMM take at most kMidPartBytes, and never
// push a linear that fits the allocation-free entry point's array past it.
constexpr int64_t kMidPartBytes = 12 << 20;
int mid_splits(int32_t fmt, int64_t m, int64_t n, int64_t k, size_t other_bytes) {
  if (has_mbs(fmt)) return 0;
  const int64_t room = (int64_t)FP4_NOALLOC_SCRATCH_BYTES - (int64_t)other_bytes;
  const int64_t cap = room >= 0 ? std::min(kMidPartBytes, room) : kMidPartBytes;
  return gemm_mid_splits(m, n, k, cap);
}

size_t mid_part_bytes(int splits, int64_t m, int64_t n) {
  return align256((size_t)splits * (size_t)(m * n) * sizeof(float));
}

LinearLayout linear_layout(int32_t fmt, int64_t m, int64_t n, int64_t k) {
  LinearLayout L;
  const int64_t mp = round_up(m, 16), kp = k_pad(k);
  size_t off = 0;
  L.scratch = off; off = align256(off + kQuantScratchBytes);
  L.ts = off; off = align256(off + sizeof(float));
  L.codes = off; off = align256(off + (size_t)(mp * kp / 2));
  L.scales = off; off = align256(off + tiled_scales_bytes(fmt, m, k));
  L.part = off;
  L.splits = mid_splits(fmt, m, n, k, off);
  if (L.splits > 1) off += mid_part_bytes(L.splits, m, n);
  L.total = off;
  return L;
}

fp4_status run_quant(int32_t fmt, int tiled, const void *x, int64_t rows, int64_t k,
                     const float *static_scale, const fp4_tensor *out, void *scratch,
                     hipStream_t stream) {
  const int base = base_fmt(fmt);
  hipError_t e = launch_quantize(base, recipe_of(fmt), tiled, (const uint16_t *)x, rows, k,
                                 static_scale, (uint8_t *)out->codes, out->codes_pitch,
                                 (uint8_t *)out->scales, out->scales_pitch, macro_of(out),
                                 macro_pitch(k), base == FP4_NVFP4 ? out->tensor_scale : nullptr,
                                 (uint32_t *)scratch, stream);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return FP4_OK;
}

// fp4_gemm's workspace: canonical activations with M > kDecodeMaxM are
// copied into the tiled layout there, so that the LDS-staged tile kernel runs.
struct RetileLayout {
  size_t codes, scales, total;
};
RetileLayout retile_layout(int32_t fmt, int64_t m, int64_t k) {
  RetileLayout L{0, 0, 0};
  if (m <= kDecodeMaxM) return L;
  const int64_t mp = round_up(m, 16), kp = k_pad(k);
  L.codes = 0;
  L.scales = align256((size_t)(mp * kp / 2));
  L.total = align256(L.scales + tiled_scales_bytes(fmt, m, k));
  return L;
}

// part / splits: the mid-size GEMM's partial-sum buffer and slice count
// (splits 0: the shape or the caller's workspace does not allow it).
fp4_status run_gemm(const fp4_tensor *a, const fp4_tensor *w, void *c, int64_t ldc, float *part,
                    int splits, hipStream_t stream) {
  GemmArgs g;
  g.fmt = base_fmt(a->fmt);
  g.a_tiled = a->layout == FP4_LAYOUT_TILED;
  g.a_codes = (const uint8_t *)a->codes; g.a_cpitch = a->codes_pitch;
  g.a_scales = (const uint8_t *)a->scales; g.a_spitch = a->scales_pitch;
  g.a_ts = a->tensor_scale;
  g.w_codes = (const uint8_t *)w->codes; g.w_scales = (const uint8_t *)w->scales;
  g.w_ts = w->tensor_scale;
  g.m = a->rows; g.n = w->rows; g.k = a->cols;
  g.c = (uint16_t *)c; g.ldc = ldc;
  g.a_ms = macro_of(a); g.a_mpitch = macro_pitch(a->cols);
  g.w_ms = macro_of(w);
  // skinny M: stream W once; large M with tiled activations: LDS-staged
  // tiles; large M with canonical activations (or macro-block scales):
  // direct-load tiles
  const bool mid = splits > 0 && mid_gemm() && g.a_tiled && !has_mbs(a->fmt) &&
                   (splits == 1 || part);
  hipError_t e = mid                          ? launch_gemm_mid(g, splits, part, stream)
                 : g.m <= kDecodeMaxM           ? launch_gemm_decode(g, stream)
                 : g.a_tiled && !has_mbs(a->fmt) ? launch_gemm_tile(g, 0, stream)
                                              : launch_gemm_prefill(g, stream);
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return FP4_OK;
}

// ---- allocation-free linear: the workspace is a device array of the library
//
// One copy per GPU (the code object is loaded on every device it runs on),
// held until the process ends. In host code `scratch` only names the array:
// its device address on the current device comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// handed to kernels.
static __device__ __align__(256) uint8_t scratch[FP4_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64];  // per device: the address of `scratch` there

__global__ __launch_bounds__(256) void k_zero_words(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The array's address on the current device (validated as gfx950). The first
// call on a device also clears, on `stream`, the words that persist from call
// to call (the quantizer's exchange words and flags), with a kernel rather than
// a memset so that it may be captured.
fp4_status noalloc_scratch(hipStream_t stream, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255u)) return fail(FP4_ERR_HIP, "scratch array has no aligned address");
    const int64_t words = (int64_t)(kQuantScratchBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(k_zero_words, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       (uint32_t *)p, words);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "scratch clear launch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FP4_OK;
}

// Arguments of a linear call (everything but the workspace).
fp4_status linear_check(const void *x_bf16, int64_t m, const fp4_tensor *w,
                        const float *static_scale, const void *y_bf16) {
  fp4_status st;
  if ((st = check_tensor(w, "w")) != FP4_OK) return st;
  if (w->layout != FP4_LAYOUT_TILED)
    return fail(FP4_ERR_FORMAT_MISMATCH, "w must be in the TILED layout");
  if ((st = check_shape(w->fmt, m, w->cols)) != FP4_OK) return st;
  if (!x_bf16 || !y_bf16) return fail(FP4_ERR_INVALID_ARG, "null input or output");
  if (!aligned16(x_bf16)) return fail(FP4_ERR_ALIGNMENT, "input must be 16-byte aligned");
  if (((uintptr_t)y_bf16 & 1u) != 0) return fail(FP4_ERR_ALIGNMENT, "output must be 2-byte aligned");
  if (base_fmt(w->fmt) == FP4_MXFP4 && static_scale)
    return fail(FP4_ERR_INVALID_ARG, "MXFP4 has no per-tensor scale");
  return FP4_OK;
}

// The linear's launches, with a workspace of linear_layout(...).total bytes.
fp4_status linear_run(const void *x_bf16, int64_t m, const fp4_tensor *w,
                      const float *static_scale, void *y_bf16, void *workspace,
                      hipStream_t stream) {
  const int32_t fmt = w->fmt;
  const int64_t k = w->cols, n = w->rows;
  const int base = base_fmt(fmt);
  if (use_fused(fmt, m, n, k)) {
    hipError_t e = launch_linear_fused(base, recipe_of(fmt), (const uint16_t *)x_bf16, m, k,
                                       static_scale,
                                       (const uint8_t *)w->codes, (const uint8_t *)w->scales,
                                       w->tensor_scale, n, (uint16_t *)y_bf16, n, stream);
    if (e != hipSuccess) return hip_fail(e, "fused linear launch");
    return FP4_OK;
  }
  const LinearLayout L = linear_layout(fmt, m, n, k);
  char *ws = (char *)workspace;
  fp4_tensor a;
  a.fmt = fmt;
  a.layout = FP4_LAYOUT_TILED;
  a.rows = m;
  a.cols = k;
  a.codes_pitch = 0;
  a.scales_pitch = 0;
  a.codes = ws + L.codes;
  a.scales = ws + L.scales;
  a.tensor_scale = (float *)(ws + L.ts);
  if (linear_fused_decode_ok(base, recipe_of(fmt), m, n, k)) {
    // one launch: quantization by the first workgroups of the skinny GEMM
    GemmArgs g;
    g.fmt = base;
    g.a_tiled = 1;
    g.a_codes = (const uint8_t *)a.codes; g.a_cpitch = 0;
    g.a_scales = (const uint8_t *)a.scales; g.a_spitch = 0;
    g.a_ts = static_scale ? static_scale : a.tensor_scale;
    g.w_codes = (const uint8_t *)w->codes; g.w_scales = (const uint8_t *)w->scales;
    g.w_ts = w->tensor_scale;
    g.m = m; g.n = n; g.k = k;
    g.c = (uint16_t *)y_bf16; g.ldc = n;
    hipError_t e = launch_linear_fused_decode(g, (const uint16_t *)x_bf16, static_scale,
                                              recipe_of(fmt), (uint32_t *)(ws + L.scratch), stream);
    if (e != hipSuccess) return hip_fail(e, "fused decode linear launch");
    return FP4_OK;
  }
  if (linear_fused_large_ok(base, recipe_of(fmt), m, n, k, static_scale != nullptr)) {
    // one launch: quantization by the first workgroups, tiles by the rest
    GemmArgs g;
    g.fmt = base;
    g.a_tiled = 1;
    g.a_codes = (const uint8_t *)a.codes; g.a_cpitch = 0;
    g.a_scales = (const uint8_t *)a.scales; g.a_spitch = 0;
    g.a_ts = static_scale;
    g.w_codes = (const uint8_t *)w->codes; g.w_scales = (const uint8_t *)w->scales;
    g.w_ts = w->tensor_scale;
    g.m = m; g.n = n; g.k = k;
    g.c = (uint16_t *)y_bf16; g.ldc = n;
    hipError_t e = launch_linear_fused_large(g, (const uint16_t *)x_bf16, static_scale,
                                             recipe_of(fmt), (uint32_t *)(ws + L.scratch), stream);
    if (e != hipSuccess) return hip_fail(e, "fused large linear launch");
    return FP4_OK;
  }
  fp4_status st = run_quant(fmt, 1, x_bf16, m, k, static_scale, &a, ws + L.scratch, stream);
  if (st != FP4_OK) return st;
  return run_gemm(&a, w, y_bf16, n, (float *)(ws + L.part), L.splits, stream);
}

}  // namespace

extern "C" {

int32_t fp4_block_size(int32_t fmt) { return valid_fmt(fmt) ? block_of(base_fmt(fmt)) : 0; }

size_t fp4_codes_bytes(int32_t fmt, int32_t layout, int64_t rows, int64_t k) {
  if (!valid_fmt(fmt) || !valid_layout(layout) || rows <= 0 || k <= 0) return 0;
  int64_t r = layout == FP4_LAYOUT_TILED ? round_up(rows, 16) : rows;
  return (size_t)(r * (k_pad(k) / 2));
}

size_t fp4_scales_bytes(int32_t fmt, int32_t layout, int64_t rows, int64_t k) {
  if (!valid_fmt(fmt) || !valid_layout(layout) || rows <= 0 || k <= 0) return 0;
  if (layout == FP4_LAYOUT_TILED) return tiled_scales_bytes(fmt, rows, k);
  const int64_t pitch = k_pad(k) / block_of(base_fmt(fmt));
  if (!has_mbs(fmt)) return (size_t)(rows * pitch);
  return macro_offset(layout, rows, k, pitch) + (size_t)(rows * macro_pitch(k)) * sizeof(float);
}

fp4_status fp4_tensor_init(fp4_tensor *t, int32_t fmt, int32_t layout, int64_t rows, int64_t k,
                           void *codes, void *scales, float *tensor_scale) {
  if (!t) return fail(FP4_ERR_INVALID_ARG, "tensor descriptor is null");
  fp4_status st = check_shape(fmt, rows, k);
  if (st != FP4_OK) return st;
  if (!valid_layout(layout)) return fail(FP4_ERR_INVALID_ARG, "unknown layout %d", (int)layout);
  t->fmt = fmt;
  t->layout = layout;
  t->rows = rows;
  t->cols = k;
  t->codes_pitch = layout == FP4_LAYOUT_CANONICAL ? k_pad(k) / 2 : 0;
  t->scales_pitch = layout == FP4_LAYOUT_CANONICAL ? k_pad(k) / block_of(base_fmt(fmt)) : 0;
  t->codes = codes;
  t->scales = scales;
  t->tensor_scale = tensor_scale;
  return ok();
}

size_t fp4_quantize_workspace_bytes(int32_t fmt, int64_t rows, int64_t k) {
  (void)rows;
  (void)k;
  return valid_fmt(fmt) ? quant_ws(fmt) : 0;
}

fp4_status fp4_quantize_weight(int32_t fmt, const void *w_bf16, int64_t n, int64_t k,
                               fp4_tensor *out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  fp4_status st = check_shape(fmt, n, k);
  if (st != FP4_OK) return st;
  if (!w_bf16) return fail(FP4_ERR_INVALID_ARG, "weight pointer is null");
  if (!aligned16(w_bf16)) return fail(FP4_ERR_ALIGNMENT, "weight must be 16-byte aligned");
  if ((st = check_tensor(out, "out")) != FP4_OK) return st;
  if (out->layout != FP4_LAYOUT_TILED)
    return fail(FP4_ERR_FORMAT_MISMATCH, "weights are stored in the TILED layout");
  if (out->fmt != fmt || out->rows != n || out->cols != k)
    return fail(FP4_ERR_FORMAT_MISMATCH, "out descriptor does not match format/shape");
  if (workspace_bytes < quant_ws(fmt) || (quant_ws(fmt) && !workspace))
    return fail(FP4_ERR_WORKSPACE, "workspace needs %zu bytes", quant_ws(fmt));
  if (workspace && !aligned16(workspace))
    return fail(FP4_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  if ((st = check_device()) != FP4_OK) return st;
  st = run_quant(fmt, 1, w_bf16, n, k, nullptr, out, workspace, stream);
  return st == FP4_OK ? ok() : st;
}

fp4_status fp4_quantize_act(int32_t fmt, const void *a_bf16, int64_t m, int64_t k,
                            const float *static_scale, fp4_tensor *out, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  fp4_status st = check_shape(fmt, m, k);
  if (st != FP4_OK) return st;
  if (!a_bf16) return fail(FP4_ERR_INVALID_ARG, "activation pointer is null");
  if (!aligned16(a_bf16)) return fail(FP4_ERR_ALIGNMENT, "activations must be 16-byte aligned");
  if ((st = check_tensor(out, "out")) != FP4_OK) return st;
  if (out->fmt != fmt || out->rows != m || out->cols != k)
    return fail(FP4_ERR_FORMAT_MISMATCH, "out descriptor does not match format/shape");
  if (base_fmt(fmt) == FP4_MXFP4 && static_scale)
    return fail(FP4_ERR_INVALID_ARG, "MXFP4 has no per-tensor scale");
  size_t need = static_scale ? 0 : quant_ws(fmt);
  if (workspace_bytes < need || (need && !workspace))
    return fail(FP4_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (workspace && !aligned16(workspace))
    return fail(FP4_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  if ((st = check_device()) != FP4_OK) return st;
  st = run_quant(fmt, out->layout == FP4_LAYOUT_TILED, a_bf16, m, k, static_scale, out,
                 workspace, stream);
  return st == FP4_OK ? ok() : st;
}

size_t fp4_gemm_workspace_bytes(int32_t fmt, int64_t m, int64_t n, int64_t k) {
  if (!valid_fmt(fmt) || m <= 0 || n <= 0 || k <= 0) return 0;
  if (m > kDecodeMaxM) return retile_layout(fmt, m, k).total;
  const int splits = has_mbs(fmt) ? 0 : gemm_mid_splits(m, n, k, kMidPartBytes);
  return splits > 1 ? mid_part_bytes(splits, m, n) : 0;
}

fp4_status fp4_gemm(const fp4_tensor *a, const fp4_tensor *w, void *c_bf16, int64_t ldc,
                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  fp4_status st;
  if ((st = check_tensor(a, "a")) != FP4_OK) return st;
  if ((st = check_tensor(w, "w")) != FP4_OK) return st;
  if (w->layout != FP4_LAYOUT_TILED)
    return fail(FP4_ERR_FORMAT_MISMATCH, "w must be in the TILED layout");
  if (!same_product_fmt(a->fmt, w->fmt))
    return fail(FP4_ERR_FORMAT_MISMATCH, "a and w differ in format, rotation or macro-block scaling");
  if (a->cols != w->cols) return fail(FP4_ERR_SHAPE, "a and w differ in K");
  if (!c_bf16) return fail(FP4_ERR_INVALID_ARG, "output pointer is null");
  if (ldc < w->rows) return fail(FP4_ERR_SHAPE, "ldc smaller than N");
  if (((uintptr_t)c_bf16 & 1u) != 0) return fail(FP4_ERR_ALIGNMENT, "output must be 2-byte aligned");
  if (a->rows > INT32_MAX || w->rows > INT32_MAX) return fail(FP4_ERR_SHAPE, "too many rows");
  // the skinny kernels address canonical activation rows with 32-bit offsets
  if (a->rows <= kDecodeMaxM && a->layout == FP4_LAYOUT_CANONICAL &&
      a->rows * std::max(a->codes_pitch, a->scales_pitch) >= (int64_t(1) << 31))
    return fail(FP4_ERR_SHAPE, "a: rows * pitch must stay below 2^31 bytes for M <= %d", kDecodeMaxM);
  if (workspace && !aligned16(workspace))
    return fail(FP4_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  if ((st = check_device()) != FP4_OK) return st;
  const RetileLayout R = retile_layout(a->fmt, a->rows, a->cols);
  if (a->layout == FP4_LAYOUT_CANONICAL && R.total && workspace && workspace_bytes >= R.total) {
    // canonical activations of a large M: tiled copy in the workspace, then
    // the tile kernel (without the workspace: the direct-load kernel)
    char *ws = (char *)workspace;
    fp4_tensor t = *a;
    t.layout = FP4_LAYOUT_TILED;
    t.codes_pitch = t.scales_pitch = 0;
    t.codes = ws + R.codes;
    t.scales = ws + R.scales;
    hipError_t e = launch_import_tiled(base_fmt(a->fmt), (const uint8_t *)a->codes, a->codes_pitch,
                                       (const uint8_t *)a->scales, a->scales_pitch, macro_of(a),
                                       macro_pitch(a->cols), a->rows, a->cols,
                                       (uint8_t *)t.codes, (uint8_t *)t.scales, macro_of(&t),
                                       stream);
    if (e != hipSuccess) return hip_fail(e, "activation re-tiling launch");
    st = run_gemm(&t, w, c_bf16, ldc, nullptr, 0, stream);
    return st == FP4_OK ? ok() : st;
  }
  // 33-128 tiled rows: the mid-size GEMM, its partial sums in the workspace
  // when it is large enough (else the skinny kernel, unless one slice does)
  int splits = a->layout == FP4_LAYOUT_TILED ? gemm_mid_splits(a->rows, w->rows, a->cols, kMidPartBytes) : 0;
  if (splits > 1 && (!workspace || workspace_bytes < mid_part_bytes(splits, a->rows, w->rows)))
    splits = 0;
  st = run_gemm(a, w, c_bf16, ldc, (float *)workspace, splits, stream);
  return st == FP4_OK ? ok() : st;
}

size_t fp4_linear_workspace_bytes(int32_t fmt, int64_t m, int64_t n, int64_t k) {
  if (!valid_fmt(fmt) || m <= 0 || n <= 0 || k <= 0) return 0;
  return linear_layout(fmt, m, n, k).total;
}

fp4_status fp4_linear(const void *x_bf16, int64_t m, const fp4_tensor *w,
                      const float *static_scale, void *y_bf16, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  fp4_status st;
  if ((st = linear_check(x_bf16, m, w, static_scale, y_bf16)) != FP4_OK) return st;
  const LinearLayout L = linear_layout(w->fmt, m, w->rows, w->cols);
  if (!workspace || workspace_bytes < L.total)
    return fail(FP4_ERR_WORKSPACE, "workspace needs %zu bytes", L.total);
  if (!aligned16(workspace)) return fail(FP4_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  if ((st = check_device()) != FP4_OK) return st;
  st = linear_run(x_bf16, m, w, static_scale, y_bf16, workspace, stream);
  return st == FP4_OK ? ok() : st;
}

fp4_status fp4_linear_noalloc(const void *x_bf16, int64_t m, const fp4_tensor *w,
                              const float *static_scale, void *y_bf16, hipStream_t stream) {
  fp4_status st;
  if ((st = linear_check(x_bf16, m, w, static_scale, y_bf16)) != FP4_OK) return st;
  const LinearLayout L = linear_layout(w->fmt, m, w->rows, w->cols);
  if (L.total > FP4_NOALLOC_SCRATCH_BYTES)
    return fail(FP4_ERR_WORKSPACE,
                "this call needs %zu bytes of workspace; the library's device array holds %zu "
                "(use fp4_linear with a workspace)", L.total, (size_t)FP4_NOALLOC_SCRATCH_BYTES);
  if ((st = check_device()) != FP4_OK) return st;
  void *ws = nullptr;
  if ((st = noalloc_scratch(stream, &ws)) != FP4_OK) return st;
  st = linear_run(x_bf16, m, w, static_scale, y_bf16, ws, stream);
  return st == FP4_OK ? ok() : st;
}

fp4_status fp4_linear_w4a16(const void *x_bf16, int64_t m, const fp4_tensor *w, void *y_bf16,
                            int64_t ldy, hipStream_t stream) {
  fp4_status st;
  if ((st = check_tensor(w, "w")) != FP4_OK) return st;
  if (w->layout != FP4_LAYOUT_TILED)
    return fail(FP4_ERR_FORMAT_MISMATCH, "w must be in the TILED layout");
  if (w->fmt & FP4_ROTATE)
    return fail(FP4_ERR_FORMAT_MISMATCH,
                "a rotated weight needs rotated activations: use fp4_linear");
  if (has_mbs(w->fmt))
    return fail(FP4_ERR_FORMAT_MISMATCH,
                "the weight-only linear takes no macro-block scales: use fp4_linear");
  const int64_t k = w->cols, n = w->rows;
  if ((st = check_shape(w->fmt, m, k)) != FP4_OK) return st;
  if (!x_bf16 || !y_bf16) return fail(FP4_ERR_INVALID_ARG, "null input or output");
  if (!aligned16(x_bf16)) return fail(FP4_ERR_ALIGNMENT, "input must be 16-byte aligned");
  if (((uintptr_t)y_bf16 & 1u) != 0) return fail(FP4_ERR_ALIGNMENT, "output must be 2-byte aligned");
  if (ldy < n) return fail(FP4_ERR_SHAPE, "ldy smaller than N");
  if (m > INT32_MAX || n > INT32_MAX) return fail(FP4_ERR_SHAPE, "too many rows");
  if ((st = check_device()) != FP4_OK) return st;
  hipError_t e = launch_linear_w4a16(base_fmt(w->fmt), (const uint16_t *)x_bf16, k, m, k,
                                     (const uint8_t *)w->codes, (const uint8_t *)w->scales,
                                     w->tensor_scale, n, (uint16_t *)y_bf16, ldy, stream);
  if (e != hipSuccess) return hip_fail(e, "w4a16 launch");
  return ok();
}

int32_t fp4_linear_launches(int32_t fmt, int64_t m, int64_t n, int64_t k, int32_t static_scale) {
  if (!valid_fmt(fmt) || m <= 0 || n <= 0 || k <= 0) return 0;
  const int base = base_fmt(fmt);
  if (k % block_of(base) != 0) return 0;
  if (use_fused(fmt, m, n, k)) return 1;
  if (linear_fused_decode_ok(base, recipe_of(fmt), m, n, k)) return 1;
  if (linear_fused_large_ok(base, recipe_of(fmt), m, n, k, static_scale != 0)) return 1;
  const int gemm = mid_gemm() && linear_layout(fmt, m, n, k).splits > 1 ? 2 : 1;
  if (base == FP4_NVFP4 && !static_scale && !quant_fits_small(base, m, k, 1) &&
      !quant_fits_mid(base, recipe_of(fmt), m, k, 1))
    return 2 + gemm;
  return 1 + gemm;
}

fp4_status fp4_export_canonical(const fp4_tensor *tiled, fp4_tensor *canonical,
                                hipStream_t stream) {
  fp4_status st;
  if ((st = check_tensor(tiled, "tiled")) != FP4_OK) return st;
  if ((st = check_tensor(canonical, "canonical")) != FP4_OK) return st;
  if (tiled->layout != FP4_LAYOUT_TILED || canonical->layout != FP4_LAYOUT_CANONICAL)
    return fail(FP4_ERR_FORMAT_MISMATCH, "expected a TILED source and CANONICAL target");
  if (tiled->fmt != canonical->fmt || tiled->rows != canonical->rows ||
      tiled->cols != canonical->cols)
    return fail(FP4_ERR_FORMAT_MISMATCH, "descriptors differ in format or shape");
  if ((st = check_device()) != FP4_OK) return st;
  const int base = base_fmt(tiled->fmt);
  hipError_t e = launch_export_canonical(
      base, (const uint8_t *)tiled->codes, (const uint8_t *)tiled->scales, macro_of(tiled),
      tiled->rows, tiled->cols, (uint8_t *)canonical->codes, canonical->codes_pitch,
      (uint8_t *)canonical->scales, canonical->scales_pitch, macro_of(canonical),
      macro_pitch(canonical->cols), base == FP4_NVFP4 ? tiled->tensor_scale : nullptr,
      base == FP4_NVFP4 ? canonical->tensor_scale : nullptr, stream);
  if (e != hipSuccess) return hip_fail(e, "export launch");
  return ok();
}

fp4_status fp4_dequantize(const fp4_tensor *t, float *out_f32, int64_t ldo, hipStream_t stream) {
  fp4_status st;
  if ((st = check_tensor(t, "t")) != FP4_OK) return st;
  if (!out_f32) return fail(FP4_ERR_INVALID_ARG, "output pointer is null");
  if (ldo < t->cols) return fail(FP4_ERR_SHAPE, "ldo smaller than K");
  if (((uintptr_t)out_f32 & 3u) != 0) return fail(FP4_ERR_ALIGNMENT, "output must be 4-byte aligned");
  if ((st = check_device()) != FP4_OK) return st;
  const int base = base_fmt(t->fmt);
  hipError_t e = launch_dequant(base, t->layout == FP4_LAYOUT_TILED,
                                (const uint8_t *)t->codes, t->codes_pitch,
                                (const uint8_t *)t->scales, t->scales_pitch, macro_of(t),
                                macro_pitch(t->cols), base == FP4_NVFP4 ? t->tensor_scale : nullptr,
                                t->rows, t->cols, out_f32, ldo, stream);
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  return ok();
}

fp4_status fp4_workspace_flags(const void *workspace, size_t workspace_bytes, uint32_t *flags,
                               int32_t clear, hipStream_t stream) {
  if (!workspace || !flags) return fail(FP4_ERR_INVALID_ARG, "null workspace or flags pointer");
  if (workspace_bytes < kQuantScratchBytes)
    return fail(FP4_ERR_WORKSPACE, "workspace smaller than the %zu bytes that hold the flags",
                kQuantScratchBytes);
  fp4_status st_check;
  if ((st_check = check_device()) != FP4_OK) return st_check;
  uint32_t *word = (uint32_t *)workspace + kErrWord;
  uint32_t host = 0;
  hipError_t e = hipMemcpyAsync(&host, word, sizeof host, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "reading the workspace flags");
  *flags = host;
  if (clear && host) {
    const uint32_t zero = 0;
    e = hipMemcpyAsync(word, &zero, sizeof zero, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "clearing the workspace flags");
  }
  return ok();
}

uint32_t fp4_set_exchange_spin_limit(uint32_t polls) { return set_exchange_spin_limit(polls); }

int32_t fp4_set_mid_gemm(int32_t on) { return set_mid_gemm(on); }

int32_t fp4_linear_mid_splits(int32_t fmt, int64_t m, int64_t n, int64_t k) {
  if (!valid_fmt(fmt) || m <= 0 || n <= 0 || k <= 0 || k % block_of(base_fmt(fmt)) != 0) return 0;
  if (use_fused(fmt, m, n, k) || linear_fused_decode_ok(base_fmt(fmt), recipe_of(fmt), m, n, k) ||
      !mid_gemm())
    return 0;
  return linear_layout(fmt, m, n, k).splits;
}

int32_t fp4_set_large_linear_fusion(int32_t on) { return set_large_linear_fusion(on); }

int32_t fp4_set_decode_linear_fusion(int32_t on) { return set_decode_linear_fusion(on); }

int32_t fp4_set_nvfp4_tile_mode(int32_t mode) {
  if (mode != 0 && mode != 1) return -1;
  return set_nvfp4_tile_mode(mode);
}

const char *fp4_status_string(int32_t s) {
  switch (s) {
    case FP4_OK: return "FP4_OK";
    case FP4_ERR_INVALID_ARG: return "FP4_ERR_INVALID_ARG";
    case FP4_ERR_SHAPE: return "FP4_ERR_SHAPE";
    case FP4_ERR_ALIGNMENT: return "FP4_ERR_ALIGNMENT";
    case FP4_ERR_WORKSPACE: return "FP4_ERR_WORKSPACE";
    case FP4_ERR_FORMAT_MISMATCH: return "FP4_ERR_FORMAT_MISMATCH";
    case FP4_ERR_DEVICE: return "FP4_ERR_DEVICE";
    case FP4_ERR_HIP: return "FP4_ERR_HIP";
    default: return "FP4_ERR_UNKNOWN";
  }
}

const char *fp4_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
