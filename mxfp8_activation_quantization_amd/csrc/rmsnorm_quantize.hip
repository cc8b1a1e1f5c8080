// RMS normalization of BF16 rows with an MXFP8 output: the producer-side fusion
// in front of the fused wqa/wkv projection.
//
// vLLM PR #57977 ("[Perf][DSv4.1] Keep activations MXFP8 between DeepGEMM
// kernels", the before/after diagrams and Pieces): the normalizing producer at
// the top of the attention sublayer emits the MXFP8 input of the fused wqa/wkv
// GEMM (codes plus packed UE8M0 scales) itself, next to its BF16 output, so no
// standalone quantize launch sits between them.  The normalization is the RMS
// form: y = x / sqrt(mean(x^2) + eps) * gamma per row, computed in fp32 and
// rounded to BF16 (nearest even); the MXFP8 output is the quantization of that
// BF16 y by the rule of mxfp8_quantize, so it holds exactly the bytes a
// standalone quantize of the BF16 output would make.
//
// One workgroup per row.  The row is walked in 128-element spans (one packed
// scale word), sixteen lanes per span as in the standalone quantizer: pass 1
// sums the squares in fp32 (lanes, then waves through LDS), pass 2 scales the
// row, rounds it to BF16 and quantizes each 32-element block.  Rows of up to
// 8192 values stay in registers between the passes (the row is read from memory
// once, non-temporally, as every output is written); longer rows are read again
// from cache.
#include "launch.hpp"
#include "mx_device.hpp"

namespace mx {

namespace {

constexpr int kRmsThreads = 256;
constexpr int kRmsGroups = kRmsThreads / 16;     // spans in flight per workgroup

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace

// Quantizes one 128-element span whose BF16 y (four words per lane) is ready.
__device__ __forceinline__ void rms_store_span(const uint32_t (&yw)[4], int j, uint16_t* yrow, uint8_t* qrow,
                                               int32_t* sfrow, int s) {
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  if (yrow) {
    const v4u yv = {yw[0], yw[1], yw[2], yw[3]};
    __builtin_nontemporal_store(yv, reinterpret_cast<v4u*>(yrow + s * 128 + j * 8));
  }
  if (!qrow) return;                                // BF16 output only
  uint32_t m = amax_pair(amax_pair(amax_pair(amax_pair(0u, yw[0]), yw[1]), yw[2]), yw[3]);
  m = fold_pair(m);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, 16));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2, 16));
  const int e = scale_exp_from_amax(m);
  const float scale = exp2_int(e);
  const v2u cv = {encode4(yw[0], yw[1], scale), encode4(yw[2], yw[3], scale)};
  const uint32_t sb = (uint32_t)(e + 127);
  const uint32_t s1 = (uint32_t)__shfl((int)sb, 4, 16);
  const uint32_t s2 = (uint32_t)__shfl((int)sb, 8, 16);
  const uint32_t s3 = (uint32_t)__shfl((int)sb, 12, 16);
  __builtin_nontemporal_store(cv, reinterpret_cast<v2u*>(qrow + s * 128 + j * 8));
  if (j == 0) sfrow[s] = (int32_t)(sb | (s1 << 8) | (s2 << 16) | (s3 << 24));
}

// SPG spans per 16-lane group held in registers (K <= SPG * 2048): the row is
// read from memory once.  SPG = 0: any K, pass 2 reads the row again from cache.
template <int SPG>
__global__ __launch_bounds__(kRmsThreads) void rmsnorm_quantize_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const uint16_t* __restrict__ gamma, float eps, int64_t K,
    uint16_t* __restrict__ y, int64_t ld_y, uint8_t* __restrict__ q, int64_t ld_q, int32_t* __restrict__ sf,
    int64_t ld_sf) {
  __shared__ float s_part[kRmsThreads / 64];
  const int64_t row = blockIdx.x;
  const int j = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int spans = (int)(K / 128);
  const uint16_t* xr = x + row * ld_x;

  // pass 1: sum of squares of the row (each lane over its spans in order, then a
  // fixed tree over lanes and waves)
  auto add_sq = [&](float& ss, const v4u& v) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = bf16_lo(v[k]), b = bf16_hi(v[k]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  };
  auto row_scale = [&](float ss) -> float {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kRmsThreads / 64; ++w) tot += s_part[w];
    return 1.0f / sqrtf(tot / (float)K + eps);
  };
  // pass 2 of one span: y = bf16((x * r) * gamma), then the MXFP8 blocks of the BF16 y.
  // The output rows are addressed here, after the reduction: addressed up front, their
  // pointers and strides put four rounds of kernel-argument loads ahead of the row's first
  // load (measured: 0.13-0.18 us per launch more at 1-300 rows, 0.3-0.7 us at 8192 rows).
  auto do_span = [&](const v4u& v, const v4u& g, float r, int s) {
    uint32_t yw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      yw[k] = bf16x2_rne((bf16_lo(v[k]) * r) * bf16_lo(g[k]), (bf16_hi(v[k]) * r) * bf16_hi(g[k]));
    }
    rms_store_span(yw, j, y ? y + row * ld_y : nullptr, q ? q + row * ld_q : nullptr,
                   q ? sf + row * ld_sf : nullptr, s);
  };

  if constexpr (SPG > 0) {
    v4u xv[SPG], gv[SPG];
#pragma unroll
    for (int u = 0; u < SPG; ++u) {
      const int sp = grp + u * kRmsGroups;
      xv[u] = sp < spans ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(xr + sp * 128 + j * 8))
                         : v4u{0, 0, 0, 0};
    }
    // gamma for pass 2, in flight across the reduction (14 KB, shared by every row: from cache)
#pragma unroll
    for (int u = 0; u < SPG; ++u) {
      const int sp = grp + u * kRmsGroups;
      gv[u] = sp < spans ? *reinterpret_cast<const v4u*>(gamma + sp * 128 + j * 8) : v4u{0, 0, 0, 0};
    }
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < SPG; ++u) add_sq(ss, xv[u]);
    const float r = row_scale(ss);
#pragma unroll
    for (int u = 0; u < SPG; ++u) {
      const int sp = grp + u * kRmsGroups;
      if (sp < spans) do_span(xv[u], gv[u], r, sp);
    }
  } else {
    float ss = 0.f;
    for (int sp = grp; sp < spans; sp += kRmsGroups)
      add_sq(ss, *reinterpret_cast<const v4u*>(xr + sp * 128 + j * 8));     // cached: pass 2 reads it again
    const float r = row_scale(ss);
    for (int sp = grp; sp < spans; sp += kRmsGroups)
      do_span(*reinterpret_cast<const v4u*>(xr + sp * 128 + j * 8),
              *reinterpret_cast<const v4u*>(gamma + sp * 128 + j * 8), r, sp);
  }
}

hipError_t launch_rmsnorm_quantize(const void* x, int64_t M, int64_t K, int64_t ld_x, const void* gamma, float eps,
                                   void* y, int64_t ld_y, void* q, int64_t ld_q, int32_t* sf, int64_t ld_sf,
                                   hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  if (M > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int64_t spg = (K / 128 + kRmsGroups - 1) / kRmsGroups;       // spans per 16-lane group
  auto* xp = static_cast<const uint16_t*>(x);
  auto* gp = static_cast<const uint16_t*>(gamma);
  auto* yp = static_cast<uint16_t*>(y);
  auto* qp = static_cast<uint8_t*>(q);
  const dim3 grid((unsigned)M), block(kRmsThreads);
#define MX_RMS_LAUNCH(S) \
  hipLaunchKernelGGL(rmsnorm_quantize_kernel<S>, grid, block, 0, stream, xp, ld_x, gp, eps, K, yp, ld_y, qp, ld_q, sf, ld_sf)
  if (spg <= 1) MX_RMS_LAUNCH(1);
  else if (spg <= 2) MX_RMS_LAUNCH(2);
  else if (spg <= 4) MX_RMS_LAUNCH(4);
  else MX_RMS_LAUNCH(0);
#undef MX_RMS_LAUNCH
  return hipGetLastError();
}

}  // namespace mx
