// Plan and dispatch of the block-scaled FP8 GEMM: for each launch, a pure function of the shape
// chooses the few-token kernels (gemm_skinny.hip) or the tile kernel (gemm_tiled_kernel.hpp) with its
// tile configuration, and the launcher instance for the output form and activation split.
#include <map>

#include "gemm_common.hpp"
#include "gemm_tiled.hpp"

namespace mx {

template <class CF, class CT>
static hipError_t dispatch_out(const GemmArgs& p, const GemmPlan& plan, int64_t G, int out, hipStream_t s) {
  return with_variant(p.split_act, out, [&](auto out_tag, auto split_tag) -> hipError_t {
    return launch_dl<CF, CT, decltype(out_tag)::value, decltype(split_tag)::value>(p, plan, G, s);
  });
}

hipError_t launch_gemm_tiled(const GemmArgs& p, const GemmPlan& plan, int64_t G, int out, hipStream_t stream) {
  if (plan.tile_cfg == TILE_MID) {                     // N % 128 == 0
    if (p.split_act) return dispatch_out<Mid128s, Mid64>(p, plan, G, out, stream);
    return dispatch_out<Mid128, Mid64>(p, plan, G, out, stream);
  }
  if (p.N % 256 == 0) {
    if (p.split_act) return dispatch_out<Cfg256s, Cfg128>(p, plan, G, out, stream);
    return dispatch_out<Cfg256, Cfg128>(p, plan, G, out, stream);
  }
  return dispatch_out<Cfg128, Cfg128>(p, plan, G, out, stream);
}

// Few-token plan (the streaming kernel)
constexpr int64_t kSkinnyMaxTokens = 256;
// The few-token kernels are sized for one resident round: one workgroup per CU.
constexpr int64_t kSkinnyTargetWorkgroups = 256;
constexpr int64_t kSkinnyMaxSteps = 32;       // 128-deep steps per split (the streaming kernel's scale tables)
// Few tokens: a workgroup owns 32 weight rows over the whole K range (no split)
// when K fits its scale tables and the grid is wide enough -- at least 128
// workgroups up to 32 tokens, 256 (every CU) from 33 to 64, where each workgroup
// also takes in twice the activation bytes (wo_b's 160 workgroups stay on the
// split-K kernel there: 15.7-16.0 us against 18.6-18.9), and 128 again from 65
// to 128 tokens, where the split-K kernel streams every weight row once per 64
// tokens (o_proj chain: 39.9 / 42.8 / 47.4 us against 52.3 / 53.4 / 55.8 at
// 65 / 96 / 128 tokens, alternated on one box).  BF16 activations are quantized
// into the workspace first, except where the whole-K kernel quantizes them itself.
constexpr int64_t kWholeKMaxSteps = 64;
constexpr int64_t kSkinnyTileMinTokens = 128;

static bool whole_k_fits(int64_t M, int64_t G, int64_t N, int64_t K) {
  if (N % 32 != 0 || K / 128 > kWholeKMaxSteps) return false;
  const int64_t workgroups = G * (N / 32);
  if (M <= 32) return workgroups >= 128;
  if (M <= 64) return workgroups >= 256;
  return M <= 128 && workgroups >= 128;
}
// The workspace always starts with this many bytes of arrival counters, whatever the
// shape, so one shape's partial tiles never land on another shape's counters when
// calls share a workspace.
constexpr int64_t kCounterBytes = 65536;
// Many-token tiles: one resident workgroup per CU on MI355X's 256 CUs; a
// half-width tile takes about this fraction of a wide tile's time.
constexpr int64_t kTileCUs = 256;
constexpr double kNarrowTileCost = 0.65;

// Time until the last of n1 items of cost c1, then n2 items of cost c2, finishes
// when they are dealt in order to `cus` identical workers, each item to the worker
// free first.  Workers free at equal times are kept together, so this takes a
// handful of steps per round however many items there are.
static double dealt_makespan(int64_t n1, double c1, int64_t n2, double c2, int64_t cus) {
  std::map<double, int64_t> free_at;
  free_at[0.0] = cus;
  auto deal = [&](int64_t n, double c) {
    while (n > 0) {
      auto it = free_at.begin();
      const double t = it->first;
      const int64_t k = it->second < n ? it->second : n;
      it->second -= k;
      if (it->second == 0) free_at.erase(it);
      free_at[t + c] += k;
      n -= k;
    }
  };
  deal(n1, c1);
  deal(n2, c2);
  return free_at.rbegin()->first;
}

// The tile and whole-K kernels read E4M3 activations: BF16 ones are quantized
// first, into the workspace: codes [M][kt], then packed scales [M][kt/128] (after
// the counter region, so a workspace shared with split-K calls keeps its counters).
static void stage_bf16(GemmPlan& pl, int64_t M, int64_t kt) {
  pl.stage_offset = kCounterBytes;
  pl.stage_sf_offset = pl.stage_offset + (M * kt + 255) / 256 * 256;
  pl.workspace_bytes = pl.stage_sf_offset + (M * (kt / 32) + 255) / 256 * 256;
}

GemmPlan plan_gemm(int64_t M, int64_t G, int64_t N, int64_t K, bool x_bf16) {
  GemmPlan pl{};
  const int mt = M <= 32 ? 1 : 2;
  const int64_t chunks = (M + 63) / 64;
  const int64_t tiles = G * (N / 64) * chunks;
  // The few-token kernels up to 128 tokens (one row of 128-token tiles leaves wo_b
  // 80 workgroups); from 129 to 256 tokens only while the grid of 64 x 128 tiles
  // would stay under a quarter of the CUs.  Measured, o_proj chain with the
  // einsum and wo_b on 128 x 128 tiles against the split-K kernel: 50.4 / 53.9 /
  // 57.7 us against 52.3 / 53.9 / 55.6 at 65 / 96 / 128 tokens (the whole-K
  // kernel now takes those: 39.9 / 42.8 / 47.4), 55.2 / 57.0 against 69.2 / 71.6
  // at 160 / 192.
  const bool few_tiles = G * (N / 64) * ((M + 127) / 128) < kTileCUs / 4;
  pl.skinny = (M <= kSkinnyTileMinTokens || (M <= kSkinnyMaxTokens && few_tiles)) &&
              tiles * 8 <= kCounterBytes;     // one 64-bit counter per tile
  if (!pl.skinny) {
    // Tile family: 128-token rows of 128 x 128 / 64 x 128 tiles while the 256 x 256
    // grid would cover at most a quarter of the CUs, else 256-token rows of
    // 256 x 256 / 128 x 256 tiles.  Measured (einsum 8 x 4096 -> 1024; wo_b
    // 8192 -> 5120): the smaller tiles are 1.25-1.8x faster up to 512 / 768 tokens
    // (64 / 60 big tiles) and 0.63-0.87x from 640 / 1024 tokens (96 / 80) on.
    const int64_t big_tiles = G * (N / 256 > 0 ? N / 256 : 1) * ((M + 255) / 256);
    const bool mid = big_tiles <= kTileCUs / 4;
    pl.tile_cfg = mid ? TILE_MID : TILE_BIG;
    const int64_t bm = mid ? 128 : 256, bn = mid ? 128 : 256;
    const int64_t rows = (M + bm - 1) / bm;
    pl.rows = (int)rows;
    pl.full_rows = (int)rows;
    if (N % bn == 0) {
      // How many rows of tokens get wide tiles: the split that finishes first
      // when the tiles are dealt in order to kTileCUs CUs, one each, a half-width
      // tile costing kNarrowTileCost of a wide one (fewest narrow tiles among
      // equal estimates).  Many rounds leave little to gain: skip.
      const int64_t per_row = G * (N / bn);
      if (per_row * rows < 4 * kTileCUs) {
        double best = 1e30;
        for (int64_t r = rows; r >= 0; --r) {
          const double t = dealt_makespan(per_row * r, 1.0, 2 * per_row * (rows - r), kNarrowTileCost, kTileCUs);
          if (t < best * 0.99) {
            best = t;
            pl.full_rows = (int)r;
          }
        }
      }
      pl.workgroups = per_row * pl.full_rows + 2 * per_row * (rows - pl.full_rows);
    } else {
      pl.full_rows = 0;
      pl.workgroups = G * (N / (bn / 2)) * rows;
    }
    if (x_bf16 && M > 0) stage_bf16(pl, M, G * K);
    return pl;
  }
  const int64_t ksteps = K / 128;
  if (whole_k_fits(M, G, N, K)) {
    pl.whole_k = true;
    pl.mt = M <= 32 ? 1 : 2;
    pl.chunks = 1;
    pl.n_tiles = (int)(N / 32);
    pl.splits = 1;
    pl.workgroups = G * (N / 32);
    // BF16 activations: quantized in the load path up to 16 tokens with K of 32 or 64
    // steps (the decode shapes); otherwise by the standalone quantizer into the workspace.
    // Measured (wo_a, 8 x 4096 -> 1024): in the load path 9.2 / 9.4 / 10.7 / 14.7 us at
    // 1 / 8 / 16 / 32 tokens against quantize + kernel 10.6 / 11.0 / 11.4 / 12.0.
    pl.whole_k_bf16 = x_bf16 && M <= 16 && (ksteps == 32 || ksteps == 64);
    if (x_bf16 && M > 0 && !pl.whole_k_bf16) stage_bf16(pl, M, G * K);
    return pl;
  }
  int64_t splits = kSkinnyTargetWorkgroups / (tiles > 0 ? tiles : 1);
  const int64_t max_splits = ksteps / 4 > 1 ? ksteps / 4 : 1;     // at least two super-steps per split
  const int64_t min_splits = (ksteps + kSkinnyMaxSteps - 1) / kSkinnyMaxSteps;   // scale tables hold 32 steps
  splits = splits < 1 ? 1 : (splits > max_splits ? max_splits : splits);
  splits = splits < min_splits ? min_splits : splits;
  pl.mt = mt;
  pl.chunks = (int)chunks;
  pl.n_tiles = (int)(N / 64);
  pl.splits = (int)splits;
  pl.workgroups = tiles * splits;
  if (splits > 1 && M > 0) {
    pl.counter_bytes = kCounterBytes;
    pl.workspace_bytes = pl.counter_bytes + tiles * splits * (int64_t)(2 * mt * 16 * 64) * 4;
  }
  return pl;
}

hipError_t launch_gemm(const GemmArgs& p, int64_t G, bool x_bf16, int out, hipStream_t stream) {
  if (p.N % 128 != 0 || p.K % 128 != 0) return hipErrorInvalidValue;
  const GemmPlan plan = plan_gemm(p.M, G, p.N, p.K, x_bf16);
  if (plan.skinny) return launch_gemm_skinny(p, plan, G, x_bf16, out, stream);
  if (x_bf16) return hipErrorInvalidValue;        // the caller quantizes into the workspace first
  return launch_gemm_tiled(p, plan, G, out, stream);
}

}  // namespace mx
