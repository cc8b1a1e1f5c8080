// Standalone dynamic MXFP8 quantization of BF16 rows (HBM-bound streaming kernel).
//
// The quantize launch that vLLM PR #57977 ("[Perf][DSv4.1] Keep activations
// MXFP8 between DeepGEMM kernels", Purpose) counts per decode step and that
// PR #60118 ("[Perf][DSv4.1] MegaAttn: wo_a writes wo_b's MXFP8 input",
// Claims) removes from the o_proj chain; here it also prepares the weights.
//
// Work unit: a 128-element span of one row (four 32-element blocks = one packed
// scale word).  Sixteen consecutive lanes own a span; lane j = 4b + p loads the
// 16 bytes holding elements [32b + 8p, 32b + 8p + 8), so a wave reads 1 KB of
// contiguous BF16 per load.  The four lanes of a block combine their largest
// magnitudes with two xor-shuffles, derive the block's scale, convert their
// eight values and store 8 code bytes; lanes 0, 4, 8, 12 of the span hold the
// four scale bytes, which lane 0 assembles into the packed word.
#include "launch.hpp"
#include "mx_device.hpp"

namespace mx {

constexpr int kQuantThreads = 256;
// Grid cap: enough resident waves to cover HBM latency; the rest loops.  Measured (BF16 [4096 | 16384,
// 32768]): 256 x 64 blocks 63.4 / 266 us against 64.6 / 274 for 256 x 32.
constexpr int64_t kQuantMaxBlocks = 256 * 64;
// Grids of two spans per trip below this many blocks (half of the 256 CUs) take one span per trip.
constexpr int64_t kQuantNarrowBelow = 128;

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// SPI spans per 16-lane group and loop trip (loads in flight per lane).  Each
// byte is read or written exactly once, so loads and stores are marked
// non-temporal: measured on MI355X they stream 10-14% faster than plain ones
// (BF16 [4096, 32768]: 73 -> 64 us).
template <int SPI>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ q, int64_t ld_q,
    int32_t* __restrict__ sf, int64_t ld_sf, int64_t spans_per_row, int64_t total_spans) {
  const int j = threadIdx.x & 15;
  const int64_t groups = (int64_t)gridDim.x * (kQuantThreads / 16);
  int64_t g = (int64_t)blockIdx.x * (kQuantThreads / 16) + (threadIdx.x >> 4);

  for (int64_t s0 = g * SPI; s0 < total_spans; s0 += groups * SPI) {
    uint4 v[SPI];
    int64_t row[SPI], w[SPI];
#pragma unroll
    for (int u = 0; u < SPI; ++u) {
      const int64_t s = s0 + u;
      row[u] = s / spans_per_row;
      w[u] = s - row[u] * spans_per_row;
      v4u t = {0, 0, 0, 0};
      if (s < total_spans)
        t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(x + row[u] * ld_x + w[u] * 128 + j * 8));
      v[u] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int u = 0; u < SPI; ++u) {
      uint32_t m = amax_pair(amax_pair(amax_pair(amax_pair(0u, v[u].x), v[u].y), v[u].z), v[u].w);
      m = fold_pair(m);
      m = max(m, (uint32_t)__shfl_xor((int)m, 1, 16));
      m = max(m, (uint32_t)__shfl_xor((int)m, 2, 16));
      const int e = scale_exp_from_amax(m);
      const float scale = exp2_int(e);
      const uint32_t c0 = encode4(v[u].x, v[u].y, scale);
      const uint32_t c1 = encode4(v[u].z, v[u].w, scale);
      const uint32_t sb = (uint32_t)(e + 127);
      const uint32_t s1 = (uint32_t)__shfl((int)sb, 4, 16);
      const uint32_t s2 = (uint32_t)__shfl((int)sb, 8, 16);
      const uint32_t s3 = (uint32_t)__shfl((int)sb, 12, 16);
      if (s0 + u < total_spans) {
        const v2u cv = {c0, c1};
        __builtin_nontemporal_store(cv, reinterpret_cast<v2u*>(q + row[u] * ld_q + w[u] * 128 + j * 8));
        if (j == 0) sf[row[u] * ld_sf + w[u]] = (int32_t)(sb | (s1 << 8) | (s2 << 16) | (s3 << 24));
      }
    }
  }
}

hipError_t launch_quantize(const void* x, int64_t M, int64_t K, int64_t ld_x, void* q, int64_t ld_q,
                           int32_t* sf, int64_t ld_sf, hipStream_t stream) {
  const int64_t spans_per_row = K / 128;
  const int64_t total = M * spans_per_row;
  const int64_t per_block = kQuantThreads / 16;
  // two spans per trip while that fills the grid; four once the grid is at its cap; one
  // while two would leave more than half the CUs without a workgroup.  Measured (BF16
  // [M, 32768], alternated on one box): one span per trip at 1 / 8 tokens 2.75 / 2.67 us
  // against 2.82 / 3.10 with two, but 3.9 / 4.6 / 6.9 against 3.6 / 4.3 / 6.3 at 64 / 128 / 256
  // tokens; four spans per trip were slower at every size up to 256 tokens.
  const int64_t blocks2 = (total + 2 * per_block - 1) / (2 * per_block);
  const bool wide = blocks2 > kQuantMaxBlocks;
  const bool narrow = blocks2 < kQuantNarrowBelow;
  int64_t blocks = wide ? (total + 4 * per_block - 1) / (4 * per_block)
                        : (narrow ? (total + per_block - 1) / per_block : blocks2);
  if (blocks > kQuantMaxBlocks) blocks = kQuantMaxBlocks;
  if (blocks < 1) blocks = 1;
  auto* xp = static_cast<const uint16_t*>(x);
  auto* qp = static_cast<uint8_t*>(q);
  if (narrow)
    hipLaunchKernelGGL(quantize_kernel<1>, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, xp, ld_x, qp, ld_q,
                       sf, ld_sf, spans_per_row, total);
  else if (wide)
    hipLaunchKernelGGL(quantize_kernel<4>, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, xp, ld_x, qp, ld_q,
                       sf, ld_sf, spans_per_row, total);
  else
    hipLaunchKernelGGL(quantize_kernel<2>, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, xp, ld_x, qp, ld_q,
                       sf, ld_sf, spans_per_row, total);
  return hipGetLastError();
}

}  // namespace mx
