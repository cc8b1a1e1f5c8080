// Internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// One GEMM launch: G groups of D[m, g*N + n] = sum_k X[m, g*K + k] * W[g][n][k].
// Strides are in elements of each array (bytes for codes and scale bytes, 2-byte
// units for BF16, int32 words for packed input scales).
// How the decode kernels combine split-K partial tiles (all give the same bits):
// through the L2 of one XCD when every split of a tile ran there (checked at run
// time, with recomputation of the other splits as the fallback), always through
// memory, or -- to test the fallback -- always by recomputation.
enum SplitKMode { SPLITK_LOCAL = 0, SPLITK_THROUGH = 1, SPLITK_RECOMPUTE = 2 };

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
  uint32_t* ws_counters;  // split-K arrival counters (zero between calls), or null
  float* ws_partials;     // split-K fp32 partial tiles, or null
  int splitk_mode;        // how split-K partials are combined (SplitKMode)
  bool split_act;         // feed the activation codes >= 0x68 and the rest as two MFMA operands (the einsum)
};

enum TileCfg { TILE_BIG = 0, TILE_MID = 1 };

// Kernel choice and scratch needs of one GEMM launch: a pure function of
// (M, G, N, K, activation kind).  Workspace layout, each part 256-byte aligned:
// split-K arrival counters, split-K fp32 partial tiles, then -- BF16 activations
// with many tokens -- the activations quantized to MXFP8 (codes [M][G*K], scales
// [M][G*K/128]).  `workspace_bytes` is 0 when nothing is needed.
struct GemmPlan {
  bool skinny;
  bool whole_k;           // skinny, at most 64 tokens: 32 weight rows x whole K per workgroup, no split
  bool whole_k_bf16;      // whole_k with BF16 activations quantized in the kernel's load path
  int mt;                 // token tiles of 32 per workgroup (skinny)
  int chunks;             // token chunks (skinny)
  int n_tiles;            // weight tiles per group (skinny: 64 rows; whole_k: 32 rows)
  int splits;             // K splits (skinny)
  int64_t workgroups;
  int tile_cfg;           // many tokens: TILE_BIG (rows of 256 tokens: 256- and 128-wide weight tiles)
                          //   or TILE_MID (rows of 128 tokens: 128- and 64-wide weight tiles)
  int full_rows;          // many tokens: rows of tokens done as wide weight tiles ...
  int rows;               //   ... of all ceil(M / row height) rows; the rest as half-width tiles
  int64_t counter_bytes;  // leading part of the workspace: one 64-bit counter per (tile, chunk)
  int64_t stage_offset;   // BF16 activations, many tokens: codes [M][G*K] at this offset
  int64_t stage_sf_offset;//   and packed scales [M][G*K/128] at this one (0 when unused)
  int64_t workspace_bytes;
};

GemmPlan plan_gemm(int64_t M, int64_t G, int64_t N, int64_t K, bool x_bf16);

hipError_t launch_quantize(const void* x, int64_t M, int64_t K, int64_t ld_x, void* q, int64_t ld_q,
                           int32_t* sf, int64_t ld_sf, hipStream_t stream);

// RMS normalization of BF16 rows, BF16 output (optional) and MXFP8 output.
hipError_t launch_rmsnorm_quantize(const void* x, int64_t M, int64_t K, int64_t ld_x, const void* gamma, float eps,
                                   void* y, int64_t ld_y, void* q, int64_t ld_q, int32_t* sf, int64_t ld_sf,
                                   hipStream_t stream);

// fp8_gemm_nt with every argument check, the split-K combine chosen per call, and --
// when `scratch` is given and the plan needs scratch -- the workspace taken from
// scratch(stream) (at most scratch_bytes, MXFP8_ERR_SCRATCH beyond) instead of the
// workspace arguments, after the argument checks and the device check.
using ScratchSource = void* (*)(hipStream_t stream);
int gemm_entry(int splitk_mode, int a_kind, const void* a, int64_t ld_a, const int32_t* a_sf, int64_t ld_asf,
               int64_t M, int64_t N, int64_t K, const void* b, const int32_t* b_sf, void* d, int64_t ld_d,
               void* workspace, int64_t workspace_bytes, void* stream, ScratchSource scratch,
               int64_t scratch_bytes);

// out: 1 = BF16 only, 2 = MXFP8 only, 3 = both.  p.ws_* must point into a
// workspace of at least plan_gemm(...).workspace_bytes when that is non-zero.
hipError_t launch_gemm(const GemmArgs& p, int64_t G, bool x_bf16, int out, hipStream_t stream);

}  // namespace mx
