// Explicit instances of the tile kernel's launcher (gemm_tiled.hpp), one per object: the build compiles
// this file once for each TILE_INST in 0 .. 11.  The list is every launcher that the dispatch in
// gemm_tiled.hip can call: fp8_gemm_nt (BF16 out, activations whole) and grouped_fp8_einsum (each output
// form, activations split), for each tile family.
#include "gemm_tiled_kernel.hpp"

#ifndef TILE_INST
#error "TILE_INST selects the launcher instance this object holds"
#endif

namespace mx {

#define MX_TILE_INSTANCE(CF, CT, OUT, SPLIT) \
  template hipError_t launch_dl<CF, CT, OUT, SPLIT>(const GemmArgs&, const GemmPlan&, int64_t, hipStream_t)

#if TILE_INST == 0
MX_TILE_INSTANCE(Cfg256, Cfg128, OUT_BF16, false);
#elif TILE_INST == 1
MX_TILE_INSTANCE(Cfg256s, Cfg128, OUT_BF16, true);
#elif TILE_INST == 2
MX_TILE_INSTANCE(Cfg256s, Cfg128, OUT_MX, true);
#elif TILE_INST == 3
MX_TILE_INSTANCE(Cfg256s, Cfg128, OUT_BOTH, true);
#elif TILE_INST == 4
MX_TILE_INSTANCE(Cfg128, Cfg128, OUT_BF16, false);
#elif TILE_INST == 5
MX_TILE_INSTANCE(Cfg128, Cfg128, OUT_BF16, true);
#elif TILE_INST == 6
MX_TILE_INSTANCE(Cfg128, Cfg128, OUT_MX, true);
#elif TILE_INST == 7
MX_TILE_INSTANCE(Cfg128, Cfg128, OUT_BOTH, true);
#elif TILE_INST == 8
MX_TILE_INSTANCE(Mid128, Mid64, OUT_BF16, false);
#elif TILE_INST == 9
MX_TILE_INSTANCE(Mid128s, Mid64, OUT_BF16, true);
#elif TILE_INST == 10
MX_TILE_INSTANCE(Mid128s, Mid64, OUT_MX, true);
#elif TILE_INST == 11
MX_TILE_INSTANCE(Mid128s, Mid64, OUT_BOTH, true);
#else
#error "TILE_INST out of range"
#endif

}  // namespace mx
