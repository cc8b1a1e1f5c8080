// Block-scaled FP8 GEMM, LDS-tiled variant for many tokens, on gfx950's
// V_MFMA_SCALE_F32_32X32X64_F8F6F4.
//
// One kernel family serves both projections of the o_proj chain:
//   * grouped_fp8_einsum (wo_a): G groups, z[m, g*N+n] = sum_k x[m, g*K+k] w[g,n,k],
//     epilogue writes z as BF16 and/or MXFP8 (vLLM PR #60118 "[Perf][DSv4.1]
//     MegaAttn: wo_a writes wo_b's MXFP8 input", Overview and Claims);
//   * fp8_gemm_nt (wo_b): G = 1, BF16 output, recipe (1,1,32) (vLLM PR #57977
//     "[Perf][DSv4.1] Keep activations MXFP8 between DeepGEMM kernels", Pieces).
// Activations arrive either pre-quantized (codes + packed scales) or as BF16,
// which the load path quantizes with the same rule as mxfp8_quantize (PR #57977,
// Test Result: pre-quantized input is bit-identical to in-kernel quantization).
//
// MFMA roles and lane layout: see gemm_common.hpp.
//
// Tiles: a block owns BN weight rows x BM tokens and walks K in steps of 128
// (exactly one packed scale word per row).  Both operand tiles are staged in
// LDS, 128 bytes per row with the 16-byte chunks XOR-swizzled by row to spread
// the MFMA fragment reads over the banks; the scale words are staged beside them.
#include "gemm_common.hpp"

namespace mx {

__device__ __forceinline__ int swz(int row, int chunk) { return (row * 8 + (chunk ^ (row & 7))) * 16; }

// The 32-byte fragment of LDS tile row `row` for 64-deep half KS and lane half q.
template <int KS>
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int q) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + swz(row, 4 * KS + q));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + swz(row, 4 * KS + 2 + q));
  return frag(lo, hi);
}

template <int BN_, int BM_, int WN_, int WM_>
struct TileCfg {
  static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_;
  static constexpr int TN = WN / 32, TM = WM / 32;
  static constexpr int WAVES_N = BN / WN, WAVES_M = BM / WM;
  static_assert(WAVES_N * WAVES_M == 4, "four waves per block");
  static_assert(BN % 32 == 0 && BM % 32 == 0, "32-row MFMA tiles");
};

template <class C, bool X_BF16, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t sW[C::BN * 128];
  __shared__ __attribute__((aligned(16))) uint8_t sX[C::BM * 128];
  __shared__ uint32_t sWs[C::BN];
  __shared__ uint32_t sXs[C::BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % C::WAVES_N, wm = wave / C::WAVES_N;
  const int i = lane & 31, q = lane >> 5;

  const int64_t g = blockIdx.z;
  const int64_t n0 = (int64_t)blockIdx.x * C::BN;         // within the group
  const int64_t m0 = (int64_t)blockIdx.y * C::BM;
  const int64_t ksteps = p.K / 128;

  const uint8_t* wbase = p.w + (g * p.N + n0) * p.K;
  const int32_t* wsf = p.w_sf + (g * p.N + n0) * ksteps;

  v16f acc[C::TN][C::TM];
#pragma unroll
  for (int a = 0; a < C::TN; ++a)
#pragma unroll
    for (int b = 0; b < C::TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  for (int64_t kt = 0; kt < ksteps; ++kt) {
    // ---- stage the weight tile: BN rows x 128 bytes, 16 bytes per thread-iteration
#pragma unroll
    for (int c = tid; c < C::BN * 8; c += kThreads) {
      const int row = c >> 3, ch = c & 7;
      const uint4 v = *reinterpret_cast<const uint4*>(wbase + (int64_t)row * p.K + kt * 128 + ch * 16);
      *reinterpret_cast<uint4*>(sW + swz(row, ch)) = v;
    }
    for (int r = tid; r < C::BN; r += kThreads) sWs[r] = (uint32_t)wsf[(int64_t)r * ksteps + kt];

    // ---- stage the activation tile
    if constexpr (!X_BF16) {
      const uint8_t* xq = static_cast<const uint8_t*>(p.x);
#pragma unroll
      for (int c = tid; c < C::BM * 8; c += kThreads) {
        const int row = c >> 3, ch = c & 7;
        const int64_t m = m0 + row;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (m < p.M) v = *reinterpret_cast<const uint4*>(xq + m * p.ld_x + g * p.K + kt * 128 + ch * 16);
        *reinterpret_cast<uint4*>(sX + swz(row, ch)) = v;
      }
      for (int r = tid; r < C::BM; r += kThreads) {
        const int64_t m = m0 + r;
        sXs[r] = m < p.M ? (uint32_t)p.x_sf[m * p.ld_xsf + g * ksteps + kt] : 0u;
      }
    } else {
      // BF16 rows: 256 bytes per row = 16 lanes x 16 bytes; the lane quad 4b..4b+3 of a
      // row owns 32-element block b and quantizes it like mxfp8_quantize does.
      const uint16_t* xb = static_cast<const uint16_t*>(p.x);
#pragma unroll
      for (int c = tid; c < C::BM * 16; c += kThreads) {
        const int row = c >> 4, jj = c & 15, b = jj >> 2, part = jj & 3;
        const int64_t m = m0 + row;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (m < p.M) v = *reinterpret_cast<const uint4*>(xb + m * p.ld_x + g * p.K + kt * 128 + jj * 8);
        uint32_t am = fold_pair(amax_pair(amax_pair(amax_pair(amax_pair(0u, v.x), v.y), v.z), v.w));
        am = max(am, (uint32_t)__shfl_xor((int)am, 1, 4));
        am = max(am, (uint32_t)__shfl_xor((int)am, 2, 4));
        const int e = scale_exp_from_amax(am);
        const float scale = exp2_int(e);
        const uint2 codes = make_uint2(encode4(v.x, v.y, scale), encode4(v.z, v.w, scale));
        const int ch = 2 * b + (part >> 1);
        *reinterpret_cast<uint2*>(sX + swz(row, ch) + (part & 1) * 8) = codes;
        if (part == 0) reinterpret_cast<uint8_t*>(sXs)[row * 4 + b] = (uint8_t)(e + 127);
      }
    }
    __syncthreads();

    // ---- MFMA over the two 64-deep halves of the step
    {
      v8i fw[C::TN], fx[C::TM];
      int sw[C::TN], sx[C::TM];
#pragma unroll
      for (int a = 0; a < C::TN; ++a) {
        const int row = wn * C::WN + a * 32 + i;
        fw[a] = read_frag<0>(sW, row, q);
        sw[a] = (int)(sWs[row] >> (8 * q));
      }
#pragma unroll
      for (int b = 0; b < C::TM; ++b) {
        const int row = wm * C::WM + b * 32 + i;
        fx[b] = read_frag<0>(sX, row, q);
        sx[b] = (int)(sXs[row] >> (8 * q));
      }
#pragma unroll
      for (int a = 0; a < C::TN; ++a)
#pragma unroll
        for (int b = 0; b < C::TM; ++b) acc[a][b] = mfma_scaled<0>(fw[a], fx[b], acc[a][b], sw[a], sx[b]);
#pragma unroll
      for (int a = 0; a < C::TN; ++a) fw[a] = read_frag<1>(sW, wn * C::WN + a * 32 + i, q);
#pragma unroll
      for (int b = 0; b < C::TM; ++b) fx[b] = read_frag<1>(sX, wm * C::WM + b * 32 + i, q);
#pragma unroll
      for (int a = 0; a < C::TN; ++a)
#pragma unroll
        for (int b = 0; b < C::TM; ++b) acc[a][b] = mfma_scaled<2>(fw[a], fx[b], acc[a][b], sw[a], sx[b]);
    }
    __syncthreads();
  }

  // ---- epilogue
#pragma unroll
  for (int b = 0; b < C::TM; ++b) {
    const int64_t m = m0 + wm * C::WM + b * 32 + i;
#pragma unroll
    for (int a = 0; a < C::TN; ++a)
      store_tile<OUT>(p, acc[a][b], m, m < p.M, g * p.N + n0 + wn * C::WN + a * 32, q);
  }
}

// Tile configurations.  The choice depends only on (M, G, N, K), never on the
// activation kind or the output mode, so every variant of one shape shares the
// accumulation order.
using CfgLarge = TileCfg<128, 128, 64, 64>;  // many tokens: 2 x 2 waves, 64 x 64 each

template <class C, bool X_BF16, int OUT>
static hipError_t launch_cfg(const GemmArgs& p, int64_t G, hipStream_t stream) {
  const dim3 grid((unsigned)(p.N / C::BN), (unsigned)((p.M + C::BM - 1) / C::BM), (unsigned)G);
  hipLaunchKernelGGL((gemm_kernel<C, X_BF16, OUT>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <class C>
static hipError_t dispatch_kind_out(const GemmArgs& p, int64_t G, bool x_bf16, int out, hipStream_t s) {
  if (x_bf16) {
    if (out == OUT_BF16) return launch_cfg<C, true, OUT_BF16>(p, G, s);
    if (out == OUT_MX) return launch_cfg<C, true, OUT_MX>(p, G, s);
    return launch_cfg<C, true, OUT_BOTH>(p, G, s);
  }
  if (out == OUT_BF16) return launch_cfg<C, false, OUT_BF16>(p, G, s);
  if (out == OUT_MX) return launch_cfg<C, false, OUT_MX>(p, G, s);
  return launch_cfg<C, false, OUT_BOTH>(p, G, s);
}

hipError_t launch_gemm_tiled(const GemmArgs& p, int64_t G, bool x_bf16, int out, hipStream_t stream) {
  return dispatch_kind_out<CfgLarge>(p, G, x_bf16, out, stream);
}

// Kernel choice: a pure function of (M, G, N, K) -- never of the activation kind
// or the output mode -- so those variants share one accumulation order.
constexpr int64_t kSkinnyMaxTokens = 256;
constexpr int64_t kSliceSteps = 8;            // 128-K steps per K slice of the skinny kernel
// The workspace always starts with this many bytes of arrival counters, whatever the
// shape, so one shape's partial tiles never land on another shape's counters when
// calls share a workspace.
constexpr int64_t kCounterBytes = 65536;

GemmPlan plan_gemm(int64_t M, int64_t G, int64_t N, int64_t K) {
  GemmPlan pl{};
  const int mt = M <= 32 ? 1 : 2;
  const int chunks = (int)((M + 32 * mt - 1) / (32 * mt));
  const int64_t tiles = G * (N / 64) * chunks;
  pl.skinny = M <= kSkinnyMaxTokens && tiles * 4 <= kCounterBytes;
  if (!pl.skinny) {
    pl.workgroups = G * (N / CfgLarge::BN) * ((M + CfgLarge::BM - 1) / CfgLarge::BM);
    return pl;
  }
  pl.mt = mt;
  pl.chunks = chunks;
  pl.n_tiles = (int)(N / 64);
  pl.splits = (int)((K / 128 + kSliceSteps - 1) / kSliceSteps);
  pl.workgroups = tiles * pl.splits;
  if (pl.splits > 1 && M > 0) {
    pl.counter_bytes = kCounterBytes;
    pl.workspace_bytes = pl.counter_bytes + tiles * pl.splits * (int64_t)(2 * pl.mt * 16 * 64) * 4;
  }
  return pl;
}

hipError_t launch_gemm(const GemmArgs& p, int64_t G, bool x_bf16, int out, hipStream_t stream) {
  if (p.N % 128 != 0 || p.K % 128 != 0) return hipErrorInvalidValue;
  const GemmPlan plan = plan_gemm(p.M, G, p.N, p.K);
  if (plan.skinny) return launch_gemm_skinny(p, plan, G, x_bf16, out, stream);
  return launch_gemm_tiled(p, G, x_bf16, out, stream);
}

}  // namespace mx
