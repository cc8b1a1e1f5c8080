// Tile configurations of the many-token GEMM kernel (gemm_tiled_kernel.hpp) and its launcher.  The
// launcher is explicitly instantiated once per configuration, output form and activation split, each
// instance in an object of its own (gemm_tiled_inst.hip, built once per instance), so that the heavy
// kernel bodies compile in parallel; the plan and dispatch (gemm_tiled.hip) see only this declaration.
#pragma once

#include "launch.hpp"

namespace mx {

// BN weight rows x BM tokens per workgroup, WAVES_N x WAVES_M waves, NB K-step
// buffers in LDS (loads run NB - 1 steps ahead of the multiplications).
template <int BN_, int BM_, int WAVES_N_, int WAVES_M_, int NB_ = 2>
struct BigCfg {
  static constexpr int BN = BN_, BM = BM_, WAVES_N = WAVES_N_, WAVES_M = WAVES_M_, NB = NB_;
  static_assert(NB == 2 || NB == 4, "step buffers cycle within the eight unrolled K-steps");
  static constexpr int NW = WAVES_N * WAVES_M, THREADS = 64 * NW;
  static constexpr int WN = BN / WAVES_N, WM = BM / WAVES_M;
  static constexpr int TN = WN / 32, TM = WM / 32;
  static_assert(WN % 32 == 0 && WM % 32 == 0, "32-row MFMA tiles");
};

// Tile configurations.  Many tokens: 256 weight rows x 256 tokens, 128 x 256 when
// N is not a multiple of 256 and for the last rows of tokens (below); two step
// buffers.  Fewer tokens (too few 256 x 256 tiles for 256 CUs): 128 x 128 and
// 64 x 128 tiles with four step buffers, three steps of loads in flight.
using Cfg256 = BigCfg<256, 256, 2, 2>;      // 128 x 128 per wave
using Cfg128 = BigCfg<128, 256, 1, 4>;      // 128 x 64 per wave
using Mid128 = BigCfg<128, 128, 2, 2, 4>;   // 64 x 64 per wave
using Mid64 = BigCfg<64, 128, 1, 4, 4>;     // 64 x 32 per wave
// Split activations (the einsum): 256 x 256 tiles as 1 x 4 waves of 256 x 64, so that each wave splits
// two activation fragments per half step instead of four (the same bits as the 2 x 2 waves); likewise
// 128 x 128 tiles as 1 x 4 waves of 128 x 32 (one fragment per half step instead of two).  Measured,
// alternated on one box: einsum at 4096 tokens 202.5 -> 194.2 us, at 384 / 512 tokens 32.2 / 34.9 ->
// 29.1 / 32.0 us.
using Cfg256s = BigCfg<256, 256, 1, 4>;     // 256 x 64 per wave
using Mid128s = BigCfg<128, 128, 1, 4, 4>;  // 128 x 32 per wave

// Launches the tile kernel for the plan: CF tiles for the first plan.full_rows rows of tokens, CT
// tiles for the rest.
template <class CF, class CT, int OUT, bool SPLIT>
hipError_t launch_dl(const GemmArgs& p, const GemmPlan& plan, int64_t G, hipStream_t stream);

}  // namespace mx
