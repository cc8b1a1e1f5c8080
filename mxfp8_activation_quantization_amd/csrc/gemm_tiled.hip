// Block-scaled FP8 GEMM for many tokens (prefill) on gfx950's
// V_MFMA_SCALE_F32_32X32X64_F8F6F4, both operands direct to LDS.
//
// One kernel serves both projections of the o_proj chain:
//   * grouped_fp8_einsum (wo_a): G groups, z[m, g*N+n] = sum_k x[m, g*K+k] w[g,n,k],
//     epilogue writes z as BF16 and/or MXFP8 (vLLM PR #60118 "[Perf][DSv4.1]
//     MegaAttn: wo_a writes wo_b's MXFP8 input", Overview and Claims);
//   * fp8_gemm_nt (wo_b): G = 1, BF16 output, recipe (1,1,32) (vLLM PR #57977
//     "[Perf][DSv4.1] Keep activations MXFP8 between DeepGEMM kernels", Pieces).
// The kernel reads E4M3 activations (codes + packed scales); the library
// quantizes BF16 activations with mxfp8_quantize first (into the caller's
// workspace), so both kinds give identical bits (PR #57977, Test Result).
//
// Tiling.  A workgroup of four waves owns BN weight rows x BM tokens and walks K
// in 64-deep half steps.  Wave (wn, wm) owns a (BN / WAVES_N) x (BM / WAVES_M)
// sub-tile of 32 x 32 MFMA tiles, TN x TM of them.
//
// Token rows past M: the row part of every activation offset is in the per-lane
// register, which the buffer range check covers (the scalar offset is not
// checked), and the range ends at row M, so those rows arrive as zeros.
#include <map>
#include <type_traits>

#include "gemm_common.hpp"

namespace mx {

template <int BN_, int BM_, int WAVES_N_, int WAVES_M_>
struct BigCfg {
  static constexpr int BN = BN_, BM = BM_, WAVES_N = WAVES_N_, WAVES_M = WAVES_M_;
  static constexpr int NW = WAVES_N * WAVES_M, THREADS = 64 * NW;
  static constexpr int WN = BN / WAVES_N, WM = BM / WAVES_M;
  static constexpr int TN = WN / 32, TM = WM / 32;
  static_assert(WN % 32 == 0 && WM % 32 == 0, "32-row MFMA tiles");
};

// ---------------------------------------------------------------------------
// Both operands are codes, so they go from memory straight into LDS
// (buffer_load_dwordx4 ... lds: lane l of an instruction writes 16 bytes at
// LDS base + 16 l) and no registers stage them.  That frees enough LDS to keep
// four half-step stages (64-deep: 256 rows x 64 bytes per operand = 16 KB), so
// the loads of stage t+3 are issued while stage t is multiplied -- three stages
// of latency cover instead of one.
//
// Stage layout of one operand: row tile T (32 rows) is a 2 KB block of 128
// 16-byte slots; chunk cc (0..3, = 2h + q) of row r sits in slot
//     4r + (cc ^ g(r)),   g(r) = ((r >> 1) ^ (r >> 3)) & 1 | ((r >> 2) & 1) << 1,
// so one load instruction (64 lanes = 16 rows x 4 chunks, row-contiguous 64 bytes
// each) fills 1 KB of consecutive slots, and the 16 lanes of one fragment read
// (16 rows, one chunk) hit 16 different 16-byte bank groups (8 for any 8 rows).
// The fragment of lane (i, q) is chunk q (dwords 0-3) and chunk 2 + q (dwords
// 4-7) of row i: operand bytes 16q .. 16q+15 and 32+16q .. 32+16q+15 of the half
// step, the MFMA's lane layout.
__device__ __forceinline__ int dl_g(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1); }

// LDS of the direct-to-LDS kernel: four half-step stages of operand data, then
// two buffers of scale words.  A scale buffer holds the words of four K-steps
// (eight stages) for every row of both operands, 16 bytes per row, so the scale
// loads touch each row once per four K-steps instead of once per stage: loads of
// one word per row cost an L2 request per row, as many as the operand data.
// Stages 0-1 and 2-3 each fit one 64 KB window of the LDS instruction offset
// field, so one per-lane base address per window serves every fragment read.
template <class C>
struct DlLds {
  static constexpr int DATA = (C::BN + C::BM) * 64;
  static constexpr int W = 0, X = C::BN * 64;              // within a stage's data
  static constexpr int SROWS = C::BN + C::BM;              // weight rows, then token rows
  static constexpr int SBUF = SROWS * 16;
  static constexpr int SCALES = 4 * DATA;
  static constexpr int BYTES = 4 * DATA + 2 * SBUF;
  static_assert(2 * DATA <= 65536, "two stages per 64 KB window");
  static_assert(BYTES <= 160 * 1024, "LDS of one CU");
};

// One output tile: weight rows n0 .. n0 + BN - 1 of group g x tokens m0 .. m0 + BM - 1,
// the whole K range.  `smem` is the workgroup's LDS (at least DlLds<C>::BYTES).
template <class C, int OUT>
__device__ __forceinline__ void dl_tile(const GemmArgs& p, uint8_t* smem, int g, int64_t n0, int64_t m0) {
  static_assert(C::NW == 4, "four waves");
  constexpr int WI = C::BN / 64;                 // weight load instructions per wave and stage
  constexpr int XI = C::BM / 64;                 // activation load instructions per wave and stage
  constexpr int L = WI + XI;                     // loads per wave and stage
  constexpr int SI = (C::BN + C::BM) / 64;       // scale-word load instructions per wave and scale group
  using Lds = DlLds<C>;

  // the wave index is uniform: keep it in a scalar register (load offsets and LDS bases derive from it)
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 5, i = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % C::WAVES_N, wm = wave / C::WAVES_N;
  const int ksteps = (int)(p.K / 128);
  const int nst = 2 * ksteps;                    // half-step stages, 64 deep
  const int64_t rows_left = p.M - m0;
  const int64_t m_rows = rows_left < C::BM ? rows_left : C::BM;
  const int ldw = (int)p.K, ldx = (int)p.ld_x, ldxs = (int)(p.ld_xsf * 4);
  const Rsrc rw = make_rsrc_sgpr(p.w + ((int64_t)g * p.N + n0) * p.K, (int64_t)C::BN * p.K);
  const Rsrc rws = make_rsrc_sgpr(p.w_sf + ((int64_t)g * p.N + n0) * ksteps, (int64_t)C::BN * ksteps * 4);
  const Rsrc rnull = make_rsrc_sgpr(p.w, 0);
  // Activations: every load instruction covers 16 token rows and gets its own
  // buffer resource starting at its first row and ending at row m_rows; the
  // per-lane offset holds the row within the instruction, and the range check --
  // which sees the per-lane offset only -- turns rows past M into zeros without
  // reading them.
  const int xcol0 = (int)((int64_t)g * p.K);
  const int xsfcol0 = g * ksteps * 4;
  const uint8_t* x_tile = static_cast<const uint8_t*>(p.x) + m0 * ldx;
  const int32_t* xsf_tile = p.x_sf + m0 * p.ld_xsf;
  auto x_rsrc = [&](int row0) {
    const int64_t rows = m_rows - row0;
    return make_rsrc_sgpr(x_tile + (int64_t)row0 * ldx, rows > 0 ? rows * ldx : 0);
  };
  auto xs_rsrc = [&](int row0) {
    const int64_t rows = m_rows - row0;
    return make_rsrc_sgpr(xsf_tile + (int64_t)row0 * p.ld_xsf, rows > 0 ? rows * ldxs : 0);
  };

  // per-lane parts of the load offsets (the same for every stage and instruction)
  const int lr = lane >> 2, lc = (lane & 3) ^ dl_g(lane >> 2);
  const int vw = lr * ldw + lc * 16, vx = lr * ldx + lc * 16;
  // scale words: lane l reads word l % 4 of the group's four in row l / 4 of the instruction's 16 rows
  const int vws = lr * ksteps * 4 + (lane & 3) * 4, vxs = lr * ldxs + xsfcol0 + (lane & 3) * 4;

  // Load instruction d (< WI: weights, then tokens) of stage t into stage buffer
  // b (= t % 4).  With `on` false the instruction gets a resource of zero bytes:
  // every lane is out of range, nothing is read and the buffer receives zeros --
  // a no-op for a buffer nobody reads, issued without a branch.
  auto issue_one = [&](auto d_tag, int b, int t, bool on) {
    constexpr int d = decltype(d_tag)::value;
    uint8_t* data = smem + b * Lds::DATA;
    const int kt = t >> 1, ks = t & 1;
    if constexpr (d < WI) {
      const int n = 4 * d + wave;                 // rows 16n .. 16n+15
      dl_load16(on ? rw : rnull, data + Lds::W + n * 1024, vw, 16 * n * ldw + kt * 128 + ks * 64);
    } else {
      const int n = 4 * (d - WI) + wave;
      dl_load16(on ? x_rsrc(16 * n) : rnull, data + Lds::X + n * 1024, vx, xcol0 + kt * 128 + ks * 64);
    }
  };
  auto issue = [&](int b, int t) { static_for<L>([&](auto d_tag) { issue_one(d_tag, b, t, t < nst); }); };
  // scale words of group s (K-steps 4s .. 4s+3) into scale buffer s % 2.  Words
  // past the end of a row (last group of a K range that is not a multiple of
  // four steps) are never used; the whole offset is in voffset, so the range
  // check also covers them.  With `on` false: zero-byte resources, as above.
  auto issue_scales = [&](int s, bool on) {
    uint8_t* sc = smem + Lds::SCALES + (s & 1) * Lds::SBUF;
    static_for<SI>([&](auto j_tag) {
      constexpr int j = decltype(j_tag)::value;
      const int n = 4 * j + wave;                 // rows 16n .. 16n+15 of the weight-then-token row list
      if constexpr (4 * j < C::BN / 16) dl_load4(on ? rws : rnull, sc + n * 256, vws + 16 * n * ksteps * 4 + 16 * s, 0);
      else dl_load4(on ? xs_rsrc(16 * n - C::BN) : rnull, sc + n * 256, vxs + 16 * s, 0);
    });
  };

  v16f acc[C::TN][C::TM];
#pragma unroll
  for (int a = 0; a < C::TN; ++a)
#pragma unroll
    for (int b = 0; b < C::TM; ++b) acc[a][b] = zero16();

  // MFMA operands of one stage, held in registers: while the MFMAs of stage t run
  // on one set, the LDS reads of stage t+1 fill the other.
  struct Frags {
    v8i fw[C::TN], fx[C::TM];
    int sw[C::TN], sx[C::TM];
  };
  // The fragment reads are inline assembly with explicit base registers and
  // constant offsets: a handful of per-lane bases serve every stage and tile (left
  // to itself the compiler keeps one address register per stage and tile, runs
  // out of registers and spills -- and a spill reload in this loop would wait for
  // every load in flight).  The compiler does not see these reads complete, so
  // wait_early() and wait_late() wait for them and tie the registers to those waits.
  const int gi = dl_g(i);
  const int off_lo = 64 * i + 16 * (q ^ gi), off_hi = 64 * i + 16 * ((2 + q) ^ gi);
  const int base = (int)lds_addr(smem);
  constexpr int WIN = 2 * Lds::DATA;              // stages 2-3 start here
  const int aw_lo = base + wn * C::TN * 2048 + off_lo, aw_hi = base + wn * C::TN * 2048 + off_hi;
  const int ax_lo = base + wm * C::TM * 2048 + off_lo, ax_hi = base + wm * C::TM * 2048 + off_hi;
  const int aw_lo1 = aw_lo + WIN, aw_hi1 = aw_hi + WIN, ax_lo1 = ax_lo + WIN, ax_hi1 = ax_hi + WIN;
  const int aws = base + Lds::SCALES + (wn * C::TN * 32 + i) * 16;
  const int axs = base + Lds::SCALES + (C::BN + wm * C::TM * 32 + i) * 16;
  // Fragment read r of stage J (mod 16) of the unrolled loop: r < TN is weight
  // tile r, then token tile r - TN; each is a scale word and two 16-byte halves.
  // Stage J lives in data buffer J % 4 and scale buffer J / 8, scale word (J % 8) / 2.
  auto read_tile = [&](auto r_tag, auto stage_tag, Frags& F) {
    constexpr int r = decltype(r_tag)::value, J = decltype(stage_tag)::value;
    constexpr int B = J % 4, SB = (J / 8) * Lds::SBUF + ((J % 8) / 2) * 4;
    constexpr int D = (B & 1) * Lds::DATA;              // within the 64 KB window of stage buffer B
    if constexpr (r < C::TN) {
      const int wl = (B >> 1) ? aw_lo1 : aw_lo, wh = (B >> 1) ? aw_hi1 : aw_hi;
      F.sw[r] = lds_read4<SB + r * 512>(aws);
      F.fw[r] = join8(lds_read16<D + Lds::W + r * 2048>(wl), lds_read16<D + Lds::W + r * 2048>(wh));
    } else {
      constexpr int c = r - C::TN;
      const int xl = (B >> 1) ? ax_lo1 : ax_lo, xh = (B >> 1) ? ax_hi1 : ax_hi;
      F.sx[c] = lds_read4<SB + c * 512>(axs);
      F.fx[c] = join8(lds_read16<D + Lds::X + c * 2048>(xl), lds_read16<D + Lds::X + c * 2048>(xh));
    }
  };
  // Read order of a stage's tiles: what the first half of the MFMAs needs (weight
  // tiles 0 .. TN/2-1 and every token tile, in the order those MFMAs use them)
  // first, the weight tiles of the second half last; a step then waits only for
  // the first group before it starts, and for the rest before its second half.
  constexpr auto order = [](int k) constexpr {
    if (k == 0) return 0;                                   // W0
    if (k <= C::TM) return C::TN + k - 1;                   // X0 .. X(TM-1)
    return k - C::TM;                                       // W1 .. W(TN-1)
  };
  constexpr int LATE_LDS_OPS = 3 * (C::TN / 2);             // scale word + two halves per late tile
  auto read = [&](auto stage_tag, Frags& F) {
    static_for<C::TN + C::TM>([&](auto k_tag) {
      read_tile(std::integral_constant<int, order(decltype(k_tag)::value)>{}, stage_tag, F);
    });
  };
  // waits for the tiles of the first half (all but the last LATE_LDS_OPS LDS reads),
  // then for the rest; each ties the registers it covers to its wait
  auto wait_early = [&](Frags& F) {
    static_assert(C::TN == 4 && C::TM <= 4, "register ties below list the tiles by name");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(F.fw[0]), "+v"(F.fw[1]) : "n"(LATE_LDS_OPS));
    asm volatile("" : "+v"(F.sw[0]), "+v"(F.sw[1]));
    if constexpr (C::TM == 4)
      asm volatile("" : "+v"(F.fx[0]), "+v"(F.fx[1]), "+v"(F.fx[2]), "+v"(F.fx[3]), "+v"(F.sx[0]), "+v"(F.sx[1]),
                   "+v"(F.sx[2]), "+v"(F.sx[3]));
    else
      asm volatile("" : "+v"(F.fx[0]), "+v"(F.fx[1]), "+v"(F.sx[0]), "+v"(F.sx[1]));
#pragma unroll
    for (int a = 0; a < C::TN / 2; ++a) F.sw[a] = (int)((uint32_t)F.sw[a] >> (8 * q));
#pragma unroll
    for (int c = 0; c < C::TM; ++c) F.sx[c] = (int)((uint32_t)F.sx[c] >> (8 * q));
  };
  auto wait_late = [&](Frags& F) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(F.fw[2]), "+v"(F.fw[3]), "+v"(F.sw[2]), "+v"(F.sw[3]));
#pragma unroll
    for (int a = C::TN / 2; a < C::TN; ++a) F.sw[a] = (int)((uint32_t)F.sw[a] >> (8 * q));
  };
  // half H (0, 1) of the TN x TM MFMAs of a stage; KS = stage parity (which 64 bytes of the K-step)
  auto mma = [&](const Frags& F, auto ks_tag, auto half_tag) {
    constexpr int KS = decltype(ks_tag)::value, H = decltype(half_tag)::value;
#pragma unroll
    for (int a = H * C::TN / 2; a < (H + 1) * C::TN / 2; ++a)
#pragma unroll
      for (int b = 0; b < C::TM; ++b) acc[a][b] = mfma_scaled<2 * KS>(F.fw[a], F.fx[b], acc[a][b], F.sw[a], F.sx[b]);
  };

  // Stage t lives in data buffer t % 4, its scale words in scale buffer (t / 8) % 2,
  // and its operands in Frags t % 2.  One step: first half of stage t's MFMAs; then
  // -- once this wave's loads of stage t+1 are complete (stages t+2, t+3 may still
  // be in flight) -- a barrier makes every wave's stage t+1 visible and, since
  // every wave has consumed its stage-t operands by then, frees data buffer t % 4
  // for the loads of stage t+4 (and, at t = 8s, scale buffer (s+1) % 2, last used
  // by stages up to 8s-1, for scale group s+1).  The second half of stage t's
  // MFMAs follows, with the LDS reads of stage t+1 and the loads of stage t+4
  // slotted between them: a wave issues in order, so a load instruction that has
  // to wait for the memory pipeline then holds up at most one MFMA's worth of
  // issue, not a whole half-stage.
  //
  // A step has no branches: a branch would split the scheduling region and let
  // the compiler regroup the MFMAs.  Every step issues the loads of stage t+4 and,
  // at t = 8s, of scale group s+1 -- switched off (zero-byte resources) where
  // those do not exist -- so the number of loads issued after stage t+1's is the
  // same constant at every step, and the last step's reads fetch a buffer that
  // is never used.
  using H0 = std::integral_constant<int, 0>;
  constexpr int NMF = C::TN / 2 * C::TM;             // MFMAs per half-stage
  static_assert(C::TN + C::TM == L, "one fragment read per load instruction");
  constexpr int PER = (2 * L + NMF - 1) / NMF;       // reads and loads slotted after each MFMA
  auto step = [&](Frags& cur, Frags& nxt, auto stage_tag, int t) {
    constexpr int J = decltype(stage_tag)::value;     // t % 16
    constexpr int KS = J & 1;
    wait_early(cur);
    mma(cur, std::integral_constant<int, KS>{}, H0{});
    __builtin_amdgcn_sched_barrier(0);
    // loads issued after stage t+1's: stages t+2 and t+3, plus scale group s+1
    // when it went out with stage 8s+4, one of those two
    wait_vmcnt<2 * L + ((J % 8 == 1 || J % 8 == 2) ? SI : 0)>();
    asm volatile("s_barrier" ::: "memory");
    if constexpr (J % 8 == 0) issue_scales(t / 8 + 1, 8 * (t / 8 + 1) < nst);
    const bool refill = t + 4 < nst;
    wait_late(cur);
    __builtin_amdgcn_sched_barrier(0);
    static_for<NMF>([&](auto m_tag) {
      constexpr int m = decltype(m_tag)::value;
      constexpr int a = C::TN / 2 + m / C::TM, b = m % C::TM;
      acc[a][b] = mfma_scaled<2 * KS>(cur.fw[a], cur.fx[b], acc[a][b], cur.sw[a], cur.sx[b]);
      __builtin_amdgcn_sched_barrier(0);
      static_for<PER>([&](auto k_tag) {
        constexpr int o = m * PER + decltype(k_tag)::value;   // even: read o/2, odd: load o/2
        if constexpr (o < 2 * L) {
          if constexpr (o % 2 == 0)
            read_tile(std::integral_constant<int, order(o / 2)>{}, std::integral_constant<int, (J + 1) % 16>{}, nxt);
          else
            issue_one(std::integral_constant<int, o / 2>{}, J % 4, t + 4, refill);
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  Frags f0, f1;
  issue_scales(0, true);
  static_for<4>([&](auto b_tag) { issue(decltype(b_tag)::value, decltype(b_tag)::value); });   // off past nst
  wait_vmcnt<3 * L>();
  asm volatile("s_barrier" ::: "memory");
  read(std::integral_constant<int, 0>{}, f0);
  for (int t0 = 0; t0 < nst; t0 += 16) {
    static_for<8>([&](auto pair_tag) {           // stages come in pairs: nst is even
      constexpr int P = decltype(pair_tag)::value;
      if (P == 0 || t0 + 2 * P < nst) {
        step(f0, f1, std::integral_constant<int, 2 * P>{}, t0 + 2 * P);
        step(f1, f0, std::integral_constant<int, 2 * P + 1>{}, t0 + 2 * P + 1);
      }
    });
  }

  // Epilogue through LDS, one 32-token block at a time.  Every wave has waited
  // for its last fragment reads before this barrier, so the stage buffers are free.
  // The lane's row i and half q (and so the lane index) are taken back from a base
  // address that lives through the loop anyway, so that nothing the epilogue
  // derives from them is computed early and kept alive across the loop.
  __syncthreads();
  int aw = aw_lo;
  asm volatile("" : "+v"(aw));                     // opaque: keeps the compiler from reusing the original i
  const int i_e = (aw - base - wn * C::TN * 2048) >> 6;
  const int q_e = ((aw >> 4) & 3) ^ dl_g(i_e);
  static_assert(4 * EpiLds<C::TN>::BYTES <= Lds::BYTES, "epilogue blocks of the four waves");
  uint8_t* chunk = smem + wave * EpiLds<C::TN>::BYTES;
  const int64_t nb = (int64_t)g * p.N + n0 + wn * C::TN * 32;
#pragma unroll
  for (int b = 0; b < C::TM; ++b) {
#pragma unroll
    for (int a = 0; a < C::TN; ++a) {
      epi_write_tile<C::TN>(chunk, acc[a][b], a, i_e, q_e);
      __builtin_amdgcn_sched_barrier(0);
    }
    epi_store_rows<OUT, C::TN>(p, chunk, m0 + (wm * C::TM + b) * 32, nb, i_e + 32 * q_e);
  }
}

// Tile configurations: 256 weight rows x 256 tokens; 128 x 256 when N is not a
// multiple of 256 and for the last rows of tokens (below).
using Cfg256 = BigCfg<256, 256, 2, 2>;   // 128 x 128 per wave
using Cfg128 = BigCfg<128, 256, 1, 4>;   // 128 x 64 per wave

// The kernel: rows of 256 tokens [0, full_rows) as CF tiles, the remaining rows
// as CT tiles (narrower: more of them, so a short last round of the machine is
// spread over more CUs).  Each output element is one whole-K accumulation in
// both, with the same operand bytes in the same order, so the tile shape never
// changes a result.
template <class CF, class CT, int OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dl_gemm_kernel(GemmArgs p, int G, int full_rows, int rows) {
  static_assert(CF::BM == 256 && CT::BM == 256, "rows of 256 tokens");
  constexpr int BYTES = DlLds<CF>::BYTES > DlLds<CT>::BYTES ? DlLds<CF>::BYTES : DlLds<CT>::BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[BYTES];
  const int nf = (int)(p.N / CF::BN), ntl = (int)(p.N / CT::BN);
  const int F = G * nf * full_rows;
  if ((int)blockIdx.x < F) {
    const int wi = xcd_work_index((int)blockIdx.x, F);
    const int nt = wi % nf, rest = wi / nf, mt = rest % full_rows, g = rest / full_rows;
    dl_tile<CF, OUT>(p, smem, g, (int64_t)nt * CF::BN, (int64_t)mt * 256);
  } else {
    const int tr = rows - full_rows;
    const int wi = xcd_work_index((int)blockIdx.x - F, G * ntl * tr);
    const int nt = wi % ntl, rest = wi / ntl, mt = full_rows + rest % tr, g = rest / tr;
    dl_tile<CT, OUT>(p, smem, g, (int64_t)nt * CT::BN, (int64_t)mt * 256);
  }
}

template <class CF, class CT, int OUT>
static hipError_t launch_dl(const GemmArgs& p, const GemmPlan& plan, int64_t G, hipStream_t stream) {
  hipLaunchKernelGGL((dl_gemm_kernel<CF, CT, OUT>), dim3((unsigned)plan.workgroups), dim3(256), 0, stream, p, (int)G,
                     plan.full_rows, plan.rows);
  return hipGetLastError();
}

template <class CF, class CT>
static hipError_t dispatch_out(const GemmArgs& p, const GemmPlan& plan, int64_t G, int out, hipStream_t s) {
  if (out == OUT_BF16) return launch_dl<CF, CT, OUT_BF16>(p, plan, G, s);
  if (out == OUT_MX) return launch_dl<CF, CT, OUT_MX>(p, plan, G, s);
  return launch_dl<CF, CT, OUT_BOTH>(p, plan, G, s);
}

hipError_t launch_gemm_tiled(const GemmArgs& p, const GemmPlan& plan, int64_t G, int out, hipStream_t stream) {
  if (p.N % 256 == 0) return dispatch_out<Cfg256, Cfg128>(p, plan, G, out, stream);
  return dispatch_out<Cfg128, Cfg128>(p, plan, G, out, stream);
}

// Few-token plan (the streaming kernel)
constexpr int64_t kSkinnyMaxTokens = 256;
// The few-token kernels are sized for one resident round: one workgroup per CU.
constexpr int64_t kSkinnyTargetWorkgroups = 256;
constexpr int64_t kSkinnyMaxSteps = 32;       // 128-deep steps per split (the streaming kernel's scale tables)
// Few tokens: a workgroup owns 32 weight rows over the whole K range (no split)
// when K fits its scale tables and the grid is wide enough -- at least 128
// workgroups up to 32 tokens, 256 (every CU) up to 64, where each workgroup also
// takes in twice the activation bytes.  BF16 activations are quantized into the
// workspace first.
constexpr int64_t kWholeKMaxSteps = 64;

static bool whole_k_fits(int64_t M, int64_t G, int64_t N, int64_t K) {
  if (N % 32 != 0 || K / 128 > kWholeKMaxSteps) return false;
  const int64_t workgroups = G * (N / 32);
  return M <= 32 ? workgroups >= 128 : (M <= 64 && workgroups >= 256);
}
// The workspace always starts with this many bytes of arrival counters, whatever the
// shape, so one shape's partial tiles never land on another shape's counters when
// calls share a workspace.
constexpr int64_t kCounterBytes = 65536;
// Many-token tiles: one resident workgroup per CU on MI355X's 256 CUs; a
// 128 x 256 tile takes about this fraction of a 256 x 256 tile's time.
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
  pl.skinny = M <= kSkinnyMaxTokens && tiles * 8 <= kCounterBytes;     // one 64-bit counter per tile
  if (!pl.skinny) {
    const int64_t rows = (M + 255) / 256;
    pl.rows = (int)rows;
    pl.full_rows = (int)rows;
    if (N % 256 == 0) {
      // How many rows of 256 tokens get 256-wide tiles: the one that finishes
      // first when the tiles are dealt in order to kTileCUs CUs, one each, a
      // 128-wide tile costing kNarrowTileCost of a 256-wide one (fewest narrow
      // tiles among equal estimates).  Many rounds leave little to gain: skip.
      const int64_t per_row = G * (N / 256);
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
      pl.workgroups = G * (N / 128) * rows;
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
