// C ABI of the MXFP8 o_proj chain library: argument validation, device check, dispatch.
//
// Every argument is checked on the host before the first HIP call, so argument
// errors are reported the same way on a machine without a GPU.  The library
// allocates nothing, never synchronizes, and keeps no state besides a per-device
// cache of the architecture check.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/mxfp8.h"
#include "launch.hpp"

#define MX_API extern "C" __attribute__((visibility("default")))

namespace {

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi) in bytes; empty when lo == hi
};

Range range2d(const void* base, int64_t rows, int64_t cols, int64_t ld, int64_t esize) {
  Range r;
  if (!base || rows <= 0 || cols <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(base);
  r.hi = r.lo + (uintptr_t)(((rows - 1) * ld + cols) * esize);
  return r;
}

bool overlaps(const Range& a, const Range& b) {
  return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

std::atomic<int> g_arch_cache[256];  // 0 = unknown, 1 = gfx950, 2 = other

int device_check() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MXFP8_ERR_DEVICE;
  if (dev < 256) {
    const int c = g_arch_cache[dev].load(std::memory_order_relaxed);
    if (c == 1) return MXFP8_OK;
    if (c == 2) return MXFP8_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXFP8_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 256) g_arch_cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MXFP8_OK : MXFP8_ERR_DEVICE;
}

// The GEMM kernels address one tile of up to 256 rows with 32-bit byte offsets:
// row strides and the reduction depth are capped so that 256 rows always fit.
constexpr int64_t kMaxRowBytes = int64_t(1) << 23;     // activation row stride, bytes
constexpr int64_t kMaxDepth = int64_t(1) << 22;         // K of one group

// Activation operand: rows [0, M), `cols` columns.
int check_act(int kind, const void* x, int64_t ld_x, const int32_t* x_sf, int64_t ld_xsf, int64_t M,
              int64_t cols) {
  if (kind != MXFP8_ACT_BF16 && kind != MXFP8_ACT_MXFP8) return MXFP8_ERR_UNSUPPORTED;
  if (ld_x < cols) return MXFP8_ERR_SHAPE;
  const int64_t esize = kind == MXFP8_ACT_BF16 ? 2 : 1;
  if (ld_x * esize > kMaxRowBytes) return MXFP8_ERR_SHAPE;
  if (kind == MXFP8_ACT_MXFP8 && ld_xsf * 4 > kMaxRowBytes / 128) return MXFP8_ERR_SHAPE;
  if ((ld_x * esize) % 16) return MXFP8_ERR_ALIGN;
  if (kind == MXFP8_ACT_MXFP8 && ld_xsf < cols / 128) return MXFP8_ERR_SHAPE;
  if (M == 0) return MXFP8_OK;
  if (!x || (kind == MXFP8_ACT_MXFP8 && !x_sf)) return MXFP8_ERR_NULL;
  if (!aligned(x, 16)) return MXFP8_ERR_ALIGN;
  if (kind == MXFP8_ACT_MXFP8 && !aligned(x_sf, 4)) return MXFP8_ERR_ALIGN;
  return MXFP8_OK;
}

Range act_range(int kind, const void* x, int64_t ld_x, int64_t M, int64_t cols) {
  return range2d(x, M, cols, ld_x, kind == MXFP8_ACT_BF16 ? 2 : 1);
}

Range act_sf_range(int kind, const int32_t* x_sf, int64_t ld_xsf, int64_t M, int64_t cols) {
  if (kind != MXFP8_ACT_MXFP8) return Range{};
  return range2d(x_sf, M, cols / 128, ld_xsf, 4);
}

// Checks the caller's workspace against the plan and points the kernel arguments into it.
int bind_workspace(const mx::GemmPlan& plan, void* ws, int64_t ws_bytes, mx::GemmArgs& p, Range& r) {
  r = Range{};
  if (plan.workspace_bytes == 0) return MXFP8_OK;
  if (!ws || ws_bytes < plan.workspace_bytes || !aligned(ws, 256)) return MXFP8_ERR_WORKSPACE;
  if (plan.counter_bytes) {
    p.ws_counters = static_cast<uint32_t*>(ws);
    p.ws_partials = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + plan.counter_bytes);
  }
  r.lo = reinterpret_cast<uintptr_t>(ws);
  r.hi = r.lo + (uintptr_t)plan.workspace_bytes;
  return MXFP8_OK;
}

// Launches the GEMM of p.  BF16 activations that the plan routes to the tile kernel
// (or to the whole-K kernel beyond its in-kernel quantization) are first quantized
// with the standalone quantizer into the workspace
// (codes [M][kt], scales [M][kt/128]); the tile kernel then reads those, so the
// result is the one pre-quantized activations give.
hipError_t launch(mx::GemmArgs p, const mx::GemmPlan& plan, int64_t G, bool x_bf16, int out, void* ws,
                  hipStream_t stream) {
  if (x_bf16 && (!plan.skinny || (plan.whole_k && !plan.whole_k_bf16))) {
    const int64_t kt = G * p.K;
    uint8_t* q = static_cast<uint8_t*>(ws) + plan.stage_offset;
    int32_t* sf = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + plan.stage_sf_offset);
    const hipError_t e = mx::launch_quantize(p.x, p.M, kt, p.ld_x, q, kt, sf, kt / 128, stream);
    if (e != hipSuccess) return e;
    p.x = q; p.ld_x = kt; p.x_sf = sf; p.ld_xsf = kt / 128;
    x_bf16 = false;
  }
  return mx::launch_gemm(p, G, x_bf16, out, stream);
}

}  // namespace

MX_API const char* mxfp8_status_string(int status) {
  switch (status) {
    case MXFP8_OK: return "ok";
    case MXFP8_ERR_NULL: return "a required pointer is NULL";
    case MXFP8_ERR_SHAPE: return "a size or stride is out of range or not a required multiple";
    case MXFP8_ERR_ALIGN: return "a pointer or row stride breaks the alignment rules";
    case MXFP8_ERR_UNSUPPORTED: return "unsupported activation kind or no output requested";
    case MXFP8_ERR_ALIAS: return "an output overlaps an input or another output";
    case MXFP8_ERR_DEVICE: return "the current HIP device is missing or is not gfx950";
    case MXFP8_ERR_LAUNCH: return "kernel launch failed";
    case MXFP8_ERR_WORKSPACE: return "workspace missing, too small, or misaligned";
    case MXFP8_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point's fixed buffer";
    default: return "unknown status";
  }
}

MX_API int mxfp8_version(void) { return 100; }

MX_API int mxfp8_device_check(void) { return device_check(); }

MX_API int mxfp8_quantize(const void* x, int64_t M, int64_t K, int64_t ld_x, void* q, int64_t ld_q,
                          int32_t* sf, int64_t ld_sf, void* stream) {
  if (M < 0 || K <= 0 || K % 128) return MXFP8_ERR_SHAPE;
  if (ld_x < K || ld_q < K || ld_sf < K / 128) return MXFP8_ERR_SHAPE;
  if ((ld_x * 2) % 16 || ld_q % 16) return MXFP8_ERR_ALIGN;
  if (M == 0) return MXFP8_OK;
  if (!x || !q || !sf) return MXFP8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(sf, 4)) return MXFP8_ERR_ALIGN;
  const Range rx = range2d(x, M, K, ld_x, 2), rq = range2d(q, M, K, ld_q, 1),
              rs = range2d(sf, M, K / 128, ld_sf, 4);
  if (overlaps(rq, rx) || overlaps(rs, rx) || overlaps(rq, rs)) return MXFP8_ERR_ALIAS;
  if (const int d = device_check(); d != MXFP8_OK) return d;
  const hipError_t e = mx::launch_quantize(x, M, K, ld_x, q, ld_q, sf, ld_sf, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MXFP8_OK : MXFP8_ERR_LAUNCH;
}

MX_API int mxfp8_rmsnorm_quantize(const void* x, int64_t M, int64_t K, int64_t ld_x, const void* gamma, float eps,
                                  void* y, int64_t ld_y, void* q, int64_t ld_q, int32_t* sf, int64_t ld_sf,
                                  void* stream) {
  if (M < 0 || K <= 0 || K % 128) return MXFP8_ERR_SHAPE;
  if (M > INT32_MAX) return MXFP8_ERR_SHAPE;
  if (!(eps > 0.0f) || !(eps < 3.4e38f)) return MXFP8_ERR_SHAPE;   // positive and finite (NaN fails too)
  const bool want_mx = q != nullptr || sf != nullptr;
  if (!want_mx && !y) return MXFP8_ERR_UNSUPPORTED;                 // no output requested
  if (want_mx && (ld_q < K || ld_sf < K / 128)) return MXFP8_ERR_SHAPE;
  if (ld_x < K || (y && ld_y < K)) return MXFP8_ERR_SHAPE;
  if ((ld_x * 2) % 16 || (want_mx && ld_q % 16) || (y && (ld_y * 2) % 16)) return MXFP8_ERR_ALIGN;
  if (M == 0) return MXFP8_OK;
  if (!x || !gamma || (want_mx && (!q || !sf))) return MXFP8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(gamma, 16) || (want_mx && (!aligned(q, 16) || !aligned(sf, 4))) ||
      (y && !aligned(y, 16)))
    return MXFP8_ERR_ALIGN;
  const Range rx = range2d(x, M, K, ld_x, 2), rg = range2d(gamma, 1, K, K, 2),
              rq = want_mx ? range2d(q, M, K, ld_q, 1) : Range{},
              rs = want_mx ? range2d(sf, M, K / 128, ld_sf, 4) : Range{}, ry = y ? range2d(y, M, K, ld_y, 2) : Range{};
  const Range outs[3] = {rq, rs, ry};
  for (const Range& o : outs)
    if (overlaps(o, rx) || overlaps(o, rg)) return MXFP8_ERR_ALIAS;
  if (overlaps(rq, rs) || overlaps(rq, ry) || overlaps(rs, ry)) return MXFP8_ERR_ALIAS;
  if (const int d = device_check(); d != MXFP8_OK) return d;
  const hipError_t e = mx::launch_rmsnorm_quantize(x, M, K, ld_x, gamma, eps, y, ld_y, q, ld_q, sf, ld_sf,
                                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MXFP8_OK : MXFP8_ERR_LAUNCH;
}

namespace {

int einsum_impl(int splitk_mode, int x_kind, const void* x, int64_t ld_x, const int32_t* x_sf, int64_t ld_xsf,
                int64_t M, int64_t G, int64_t K, int64_t N, const void* w, const int32_t* w_sf, void* z_q,
                int64_t ld_z, int32_t* z_sf, int64_t ld_zsf, void* z_bf16, int64_t ld_zb, void* workspace,
                int64_t workspace_bytes, void* stream) {
  if (splitk_mode < mx::SPLITK_LOCAL || splitk_mode > mx::SPLITK_RECOMPUTE) return MXFP8_ERR_UNSUPPORTED;
  if (M < 0 || G < 1 || K <= 0 || K % 128 || N <= 0 || N % 128) return MXFP8_ERR_SHAPE;
  if (G > 65535 || K > kMaxDepth || M > INT32_MAX || G * N > INT32_MAX) return MXFP8_ERR_SHAPE;
  const int64_t cols_in = G * K, cols_out = G * N;
  if (int s = check_act(x_kind, x, ld_x, x_sf, ld_xsf, M, cols_in); s != MXFP8_OK) return s;
  const bool want_mx = z_q != nullptr || z_sf != nullptr;
  const bool want_bf = z_bf16 != nullptr;
  if (!want_mx && !want_bf) return MXFP8_ERR_UNSUPPORTED;
  if (want_mx && (!z_q || !z_sf)) return MXFP8_ERR_NULL;
  if (want_mx && (ld_z < cols_out || ld_zsf < cols_out / 128)) return MXFP8_ERR_SHAPE;
  if (want_mx && ld_z % 16) return MXFP8_ERR_ALIGN;
  if (want_bf && ld_zb < cols_out) return MXFP8_ERR_SHAPE;
  if (want_bf && (ld_zb * 2) % 16) return MXFP8_ERR_ALIGN;
  if (!w || !w_sf) return MXFP8_ERR_NULL;
  if (!aligned(w, 16) || !aligned(w_sf, 4)) return MXFP8_ERR_ALIGN;
  if (M == 0) return MXFP8_OK;
  if (want_mx && (!aligned(z_q, 16) || !aligned(z_sf, 4))) return MXFP8_ERR_ALIGN;
  if (want_bf && !aligned(z_bf16, 16)) return MXFP8_ERR_ALIGN;

  const Range ins[4] = {act_range(x_kind, x, ld_x, M, cols_in), act_sf_range(x_kind, x_sf, ld_xsf, M, cols_in),
                        range2d(w, G * N, K, K, 1), range2d(w_sf, G * N, K / 128, K / 128, 4)};
  const Range outs[3] = {want_mx ? range2d(z_q, M, cols_out, ld_z, 1) : Range{},
                         want_mx ? range2d(z_sf, M, cols_out / 128, ld_zsf, 4) : Range{},
                         want_bf ? range2d(z_bf16, M, cols_out, ld_zb, 2) : Range{}};
  for (const Range& o : outs) {
    for (const Range& in : ins)
      if (overlaps(o, in)) return MXFP8_ERR_ALIAS;
  }
  if (overlaps(outs[0], outs[1]) || overlaps(outs[0], outs[2]) || overlaps(outs[1], outs[2]))
    return MXFP8_ERR_ALIAS;
  mx::GemmArgs p{};
  p.splitk_mode = splitk_mode;
  Range rw;
  const mx::GemmPlan plan = mx::plan_gemm(M, G, N, K, x_kind == MXFP8_ACT_BF16);
  if (int s = bind_workspace(plan, workspace, workspace_bytes, p, rw); s != MXFP8_OK) return s;
  for (const Range& o : outs)
    if (overlaps(rw, o)) return MXFP8_ERR_ALIAS;
  for (const Range& in : ins)
    if (overlaps(rw, in)) return MXFP8_ERR_ALIAS;
  if (const int d = device_check(); d != MXFP8_OK) return d;

  p.x = x; p.ld_x = ld_x; p.x_sf = x_sf; p.ld_xsf = ld_xsf;
  p.w = static_cast<const uint8_t*>(w); p.w_sf = w_sf;
  p.M = M; p.N = N; p.K = K;
  p.zq = static_cast<uint8_t*>(z_q); p.ld_zq = ld_z;
  p.zsf = reinterpret_cast<uint8_t*>(z_sf); p.ld_zsf_bytes = ld_zsf * 4;
  p.zb = static_cast<uint16_t*>(z_bf16); p.ld_zb = ld_zb;
  p.split_act = true;       // the activations carry rare large outliers (see gemm_common.hpp)
  const int out = (want_bf ? 1 : 0) | (want_mx ? 2 : 0);
  const hipError_t e = launch(p, plan, G, x_kind == MXFP8_ACT_BF16, out, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MXFP8_OK : MXFP8_ERR_LAUNCH;
}

}  // namespace

namespace mx {

int gemm_entry(int splitk_mode, int a_kind, const void* a, int64_t ld_a, const int32_t* a_sf, int64_t ld_asf,
               int64_t M, int64_t N, int64_t K, const void* b, const int32_t* b_sf, void* d, int64_t ld_d,
               void* workspace, int64_t workspace_bytes, void* stream, ScratchSource scratch,
               int64_t scratch_bytes) {
  if (splitk_mode < mx::SPLITK_LOCAL || splitk_mode > mx::SPLITK_RECOMPUTE) return MXFP8_ERR_UNSUPPORTED;
  if (M < 0 || K <= 0 || K % 128 || N <= 0 || N % 128) return MXFP8_ERR_SHAPE;
  if (K > kMaxDepth || M > INT32_MAX || N > INT32_MAX) return MXFP8_ERR_SHAPE;
  if (int s = check_act(a_kind, a, ld_a, a_sf, ld_asf, M, K); s != MXFP8_OK) return s;
  if (ld_d < N) return MXFP8_ERR_SHAPE;
  if ((ld_d * 2) % 16) return MXFP8_ERR_ALIGN;
  if (!b || !b_sf) return MXFP8_ERR_NULL;
  if (!aligned(b, 16) || !aligned(b_sf, 4)) return MXFP8_ERR_ALIGN;
  if (M == 0) return MXFP8_OK;
  if (!d) return MXFP8_ERR_NULL;
  if (!aligned(d, 16)) return MXFP8_ERR_ALIGN;
  const Range out = range2d(d, M, N, ld_d, 2);
  const Range ins[4] = {act_range(a_kind, a, ld_a, M, K), act_sf_range(a_kind, a_sf, ld_asf, M, K),
                        range2d(b, N, K, K, 1), range2d(b_sf, N, K / 128, K / 128, 4)};
  for (const Range& in : ins)
    if (overlaps(out, in)) return MXFP8_ERR_ALIAS;
  mx::GemmArgs p{};
  p.splitk_mode = splitk_mode;
  Range rw;
  const mx::GemmPlan plan = mx::plan_gemm(M, 1, N, K, a_kind == MXFP8_ACT_BF16);
  if (scratch && plan.workspace_bytes > 0) {
    // the caller's fixed scratch array stands in for the workspace (every argument is checked by now)
    if (plan.workspace_bytes > scratch_bytes) return MXFP8_ERR_SCRATCH;
    if (const int dc = device_check(); dc != MXFP8_OK) return dc;
    workspace = scratch(static_cast<hipStream_t>(stream));
    if (!workspace) return MXFP8_ERR_LAUNCH;
    workspace_bytes = scratch_bytes;
  }
  if (int s = bind_workspace(plan, workspace, workspace_bytes, p, rw); s != MXFP8_OK) return s;
  if (overlaps(rw, out)) return MXFP8_ERR_ALIAS;
  for (const Range& in : ins)
    if (overlaps(rw, in)) return MXFP8_ERR_ALIAS;
  if (const int dc = device_check(); dc != MXFP8_OK) return dc;

  p.x = a; p.ld_x = ld_a; p.x_sf = a_sf; p.ld_xsf = ld_asf;
  p.w = static_cast<const uint8_t*>(b); p.w_sf = b_sf;
  p.M = M; p.N = N; p.K = K;
  p.zb = static_cast<uint16_t*>(d); p.ld_zb = ld_d;
  const hipError_t e = launch(p, plan, 1, a_kind == MXFP8_ACT_BF16, 1, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MXFP8_OK : MXFP8_ERR_LAUNCH;
}

}  // namespace mx

MX_API int grouped_fp8_einsum(int x_kind, const void* x, int64_t ld_x, const int32_t* x_sf, int64_t ld_xsf,
                              int64_t M, int64_t G, int64_t K, int64_t N, const void* w, const int32_t* w_sf,
                              void* z_q, int64_t ld_z, int32_t* z_sf, int64_t ld_zsf, void* z_bf16, int64_t ld_zb,
                              void* workspace, int64_t workspace_bytes, void* stream) {
  return einsum_impl(mx::SPLITK_LOCAL, x_kind, x, ld_x, x_sf, ld_xsf, M, G, K, N, w, w_sf, z_q, ld_z, z_sf, ld_zsf,
                     z_bf16, ld_zb, workspace, workspace_bytes, stream);
}

MX_API int fp8_gemm_nt(int a_kind, const void* a, int64_t ld_a, const int32_t* a_sf, int64_t ld_asf, int64_t M,
                       int64_t N, int64_t K, const void* b, const int32_t* b_sf, void* d, int64_t ld_d,
                       void* workspace, int64_t workspace_bytes, void* stream) {
  return mx::gemm_entry(mx::SPLITK_LOCAL, a_kind, a, ld_a, a_sf, ld_asf, M, N, K, b, b_sf, d, ld_d, workspace,
                        workspace_bytes, stream, nullptr, 0);
}

// Test-only forms (include/mxfp8_testing.h): the same calls with the split-K combine chosen per call.
MX_API int mxfp8_testing_grouped_fp8_einsum(int splitk_combine, int x_kind, const void* x, int64_t ld_x,
                                            const int32_t* x_sf, int64_t ld_xsf, int64_t M, int64_t G, int64_t K,
                                            int64_t N, const void* w, const int32_t* w_sf, void* z_q, int64_t ld_z,
                                            int32_t* z_sf, int64_t ld_zsf, void* z_bf16, int64_t ld_zb,
                                            void* workspace, int64_t workspace_bytes, void* stream) {
  return einsum_impl(splitk_combine, x_kind, x, ld_x, x_sf, ld_xsf, M, G, K, N, w, w_sf, z_q, ld_z, z_sf, ld_zsf,
                     z_bf16, ld_zb, workspace, workspace_bytes, stream);
}

MX_API int mxfp8_testing_fp8_gemm_nt(int splitk_combine, int a_kind, const void* a, int64_t ld_a,
                                     const int32_t* a_sf, int64_t ld_asf, int64_t M, int64_t N, int64_t K,
                                     const void* b, const int32_t* b_sf, void* d, int64_t ld_d, void* workspace,
                                     int64_t workspace_bytes, void* stream) {
  return mx::gemm_entry(splitk_combine, a_kind, a, ld_a, a_sf, ld_asf, M, N, K, b, b_sf, d, ld_d, workspace,
                        workspace_bytes, stream, nullptr, 0);
}

MX_API int64_t grouped_fp8_einsum_workspace_size(int x_kind, int64_t M, int64_t G, int64_t K, int64_t N) {
  if (x_kind != MXFP8_ACT_BF16 && x_kind != MXFP8_ACT_MXFP8) return -1;
  if (M < 0 || G < 1 || G > 65535 || K <= 0 || K % 128 || N <= 0 || N % 128) return -1;
  if (K > kMaxDepth || M > INT32_MAX || G * N > INT32_MAX) return -1;
  return mx::plan_gemm(M, G, N, K, x_kind == MXFP8_ACT_BF16).workspace_bytes;
}

MX_API int64_t fp8_gemm_nt_workspace_size(int a_kind, int64_t M, int64_t N, int64_t K) {
  if (a_kind != MXFP8_ACT_BF16 && a_kind != MXFP8_ACT_MXFP8) return -1;
  if (M < 0 || K <= 0 || K % 128 || N <= 0 || N % 128) return -1;
  if (K > kMaxDepth || M > INT32_MAX || N > INT32_MAX) return -1;
  return mx::plan_gemm(M, 1, N, K, a_kind == MXFP8_ACT_BF16).workspace_bytes;
}
