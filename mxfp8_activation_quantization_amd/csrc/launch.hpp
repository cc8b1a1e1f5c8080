// Internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// One GEMM launch: G groups of D[m, g*N + n] = sum_k X[m, g*K + k] * W[g][n][k].
// Strides are in elements of each array (bytes for codes and scale bytes, 2-byte
// units for BF16, int32 words for packed input scales).
struct GemmArgs {
  const void* x;          // activations: BF16 or E4M3 codes, rows m, ld_x elements apart
  int64_t ld_x;
  const int32_t* x_sf;    // packed scales of E4M3 activations (unused for BF16)
  int64_t ld_xsf;
  const uint8_t* w;       // weights E4M3 [G][N][K]
  const int32_t* w_sf;    // packed scales [G][N][K/128]
  int64_t M, N, K;
  uint8_t* zq;            // MXFP8 output codes [M][ld_zq] (or null)
  int64_t ld_zq;
  uint8_t* zsf;           // MXFP8 output scales as bytes [M][ld_zsf_bytes] (or null)
  int64_t ld_zsf_bytes;
  uint16_t* zb;           // BF16 output [M][ld_zb] (or null)
  int64_t ld_zb;
};

hipError_t launch_quantize(const void* x, int64_t M, int64_t K, int64_t ld_x, void* q, int64_t ld_q,
                           int32_t* sf, int64_t ld_sf, hipStream_t stream);

// out: 1 = BF16 only, 2 = MXFP8 only, 3 = both.
hipError_t launch_gemm(const GemmArgs& p, int64_t G, bool x_bf16, int out, hipStream_t stream);

}  // namespace mx
