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
// in 128-deep steps, each two 64-deep MFMA half steps.  Wave (wn, wm) owns a (BN / WAVES_N) x (BM / WAVES_M)
// sub-tile of 32 x 32 MFMA tiles, TN x TM of them.
//
// Token rows past M: the row part of every activation offset is in the per-lane
// register, which the buffer range check covers (the scalar offset is not
// checked), and the range ends at row M, so those rows arrive as zeros.
#pragma once

#include <type_traits>

#include "gemm_common.hpp"
#include "gemm_tiled.hpp"

namespace mx {

// ---------------------------------------------------------------------------
// Both operands are codes, so they go from memory straight into LDS
// (buffer_load_dwordx4 ... lds: lane l of an instruction writes 16 bytes at
// LDS base + 16 l) and no registers stage them.  LDS holds NB K-steps
// (128-deep: 256 + 256 rows x 128 bytes = 64 KB each for the largest tile, so
// two of those; four of the 32 KB steps of a 128 x 128 tile), and the loads of
// step k+NB go out while step k is multiplied.
//
// Each load instruction covers eight rows x 128 bytes: every 128-byte line it
// touches is read whole, once.  (Four-row-per-64-byte-half layouts -- one line
// requested twice, a K half-step apart -- took the vector L1 twice the requests
// for the same bytes and ran the loads 25% slower.)
//
// Step layout of one operand: row r occupies 128 bytes (eight 16-byte slots);
// chunk c (0..7: bytes 16c .. 16c+15 of the row's 128 K values) sits in slot
//     c ^ f(r),   f(r) = (r >> 1) & 7,
// so one load instruction (64 lanes = 8 rows x 8 slots) fills 1 KB of
// consecutive slots, and the 16 lanes of one fragment read (16 rows, one chunk)
// hit 16 different 16-byte bank groups.  The fragment of lane (i, q) for half step
// h is chunk 4h + q (dwords 0-3) and chunk 4h + 2 + q (dwords 4-7) of row i:
// operand bytes 16q .. 16q+15 and 32+16q .. 32+16q+15 of the half step, the
// MFMA's lane layout.  Since f(r) < 8, the two halves of a step differ by
// address bit 6 only (slot bit 2).
__device__ __forceinline__ int dl_f(int r) { return (r >> 1) & 7; }

// LDS of the direct-to-LDS kernel: NB K-step buffers of operand data (weight
// rows, then token rows), then two buffers of scale words.  A scale buffer holds
// the words of four K-steps for every row of both operands, 16 bytes per row, so
// the scale loads touch each row once per four K-steps instead of once per step:
// loads of one word per row cost an L2 request per row, as many as the operand
// data.  Each K-step buffer gets its own per-lane read bases (the LDS instruction
// offset field spans 64 KB).
template <class C>
struct DlLds {
  static constexpr int DATA = (C::BN + C::BM) * 128;
  static constexpr int W = 0, X = C::BN * 128;            // within a step's data
  static constexpr int SROWS = C::BN + C::BM;              // weight rows, then token rows
  static constexpr int SBUF = SROWS * 16;
  static constexpr int SCALES = C::NB * DATA;
  static constexpr int BYTES = C::NB * DATA + 2 * SBUF;
  static_assert(DATA <= 65536, "tile offsets of a step within one LDS offset window");
  static_assert(BYTES <= 160 * 1024, "LDS of one CU");
};

// One output tile: weight rows n0 .. n0 + BN - 1 of group g x tokens m0 .. m0 + BM - 1,
// the whole K range.  `smem` is the workgroup's LDS (at least DlLds<C>::BYTES).
template <class C, int OUT, bool SPLIT>
__device__ __forceinline__ void dl_tile(const GemmArgs& p, uint8_t* smem, int g, int64_t n0, int64_t m0) {
  static_assert(C::NW == 4, "four waves");
  constexpr int WI = C::BN / 32;                 // weight load instructions per wave and K-step (8 rows each)
  constexpr int XI = C::BM / 32;                 // activation load instructions per wave and K-step
  constexpr int L = WI + XI;                     // loads per wave and K-step
  constexpr int SI = (C::BN + C::BM) / 64;       // scale-word load instructions per wave and scale group
  constexpr int NT = C::TN + C::TM;              // fragment tiles per half step
  using Lds = DlLds<C>;

  // the wave index is uniform: keep it in a scalar register (load offsets and LDS bases derive from it)
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 5, i = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % C::WAVES_N, wm = wave / C::WAVES_N;
  const int ksteps = (int)(p.K / 128);
  const int64_t rows_left = p.M - m0;
  const int64_t m_rows = rows_left < C::BM ? rows_left : C::BM;
  const int ldw = (int)p.K, ldx = (int)p.ld_x, ldxs = (int)(p.ld_xsf * 4);
  const Rsrc rw = make_rsrc_sgpr(p.w + ((int64_t)g * p.N + n0) * p.K, (int64_t)C::BN * p.K);
  const Rsrc rws = make_rsrc_sgpr(p.w_sf + ((int64_t)g * p.N + n0) * ksteps, (int64_t)C::BN * ksteps * 4);
  const Rsrc rnull = make_rsrc_sgpr(p.w, 0);
  // Activations: one buffer resource from the tile's first token row to row M;
  // the row part of every activation offset is in the per-lane offset, which the
  // range check covers (the scalar offset is not checked), so rows past M arrive
  // as zeros without being read.
  const int xcol0 = (int)((int64_t)g * p.K);
  const int xsfcol0 = g * ksteps * 4;
  const uint8_t* x_tile = static_cast<const uint8_t*>(p.x) + m0 * ldx;
  const int32_t* xsf_tile = p.x_sf + m0 * p.ld_xsf;
  const Rsrc rx = make_rsrc_sgpr(x_tile, m_rows * ldx);
  const Rsrc rxs = make_rsrc_sgpr(xsf_tile, m_rows * ldxs);

  // Per-lane parts of the load offsets (the same for every step and instruction):
  // instruction d of a wave covers rows 8n .. 8n+7, n = 4d + wave, so its offset is
  // the wave's base (rows 8 wave + l / 8) plus d x 32 rows.  Lane l fills slot l % 8
  // of its row, so it reads chunk (l % 8) ^ f(row); f's top bit is the parity of n,
  // which is the wave's parity.
  const int lr = lane >> 3;
  const int lc = (lane & 7) ^ (((wave & 1) << 2) | (lr >> 1));
  const int vw = (8 * wave + lr) * ldw + lc * 16, vx = (8 * wave + lr) * ldx + lc * 16;
  const int sw_step = 32 * ldw, sx_step = 32 * ldx;
  const int lds_ops = (int)lds_addr(smem) + wave * 1024;
  // scale words: instruction j covers rows 16n .. 16n+15 (n = 4j + wave) of the
  // weight-then-token row list; lane l reads word l % 4 of the group's four in row l / 4
  const int slr = lane >> 2;
  const int vws = (16 * wave + slr) * ksteps * 4 + (lane & 3) * 4;
  const int vxs = (16 * wave + slr) * ldxs + xsfcol0 + (lane & 3) * 4;
  const int sws_step = 64 * ksteps * 4, sxs_step = 64 * ldxs;
  const int lds_sc = (int)lds_addr(smem) + Lds::SCALES + wave * 256;

  // Load instruction d (< WI: weights, then tokens) of K-step k into step buffer
  // B.  With `on` false the instruction gets a resource of zero bytes: every lane
  // is out of range, nothing is read and the buffer receives zeros -- a no-op for
  // a buffer nobody reads, issued without a branch.
  auto issue_one = [&](auto d_tag, auto b_tag, int k, bool on) {
    constexpr int d = decltype(d_tag)::value, B = decltype(b_tag)::value;
    if constexpr (d < WI)
      dl_load16_idx<d, B * Lds::DATA + Lds::W + 4096 * d>(on ? rw : rnull, lds_ops, vw, sw_step, k * 128);
    else
      dl_load16_idx<d - WI, B * Lds::DATA + Lds::X + 4096 * (d - WI)>(on ? rx : rnull, lds_ops, vx, sx_step,
                                                                       xcol0 + k * 128);
  };
  // scale words of group s (K-steps 4s .. 4s+3) into scale buffer SB = s % 2.
  // Words past the end of a row (last group of a K range that is not a multiple
  // of four steps) are never used; the whole offset is per-lane, so the range
  // check also covers them.  With `on` false: zero-byte resources, as above.
  auto issue_scales = [&](auto sb_tag, int s, bool on) {
    constexpr int SB = decltype(sb_tag)::value;
    static_for<SI>([&](auto j_tag) {
      constexpr int j = decltype(j_tag)::value;
      constexpr int LO = SB * Lds::SBUF + 1024 * j;
      if constexpr (4 * j < C::BN / 16)
        dl_load4_idx<j, LO>(on ? rws : rnull, lds_sc, vws, sws_step, 16 * s);
      else
        dl_load4_idx<j - C::BN / 64, LO>(on ? rxs : rnull, lds_sc, vxs, sxs_step, 16 * s);
    });
  };

  v16f acc[C::TN][C::TM];
#pragma unroll
  for (int a = 0; a < C::TN; ++a)
#pragma unroll
    for (int b = 0; b < C::TM; ++b) acc[a][b] = zero16();

  // MFMA operands of the two half steps of a K-step, held in registers: f0 (first
  // half) and f1 (second half).  With SPLIT, fx holds an activation fragment's small
  // codes and fxh its large ones (split once the fragment's read has completed).
  struct Frags {
    v8i fw[C::TN], fx[C::TM];
    v8i fxh[SPLIT ? C::TM : 1];
    int sw[C::TN], sx[C::TM];
  };
  // The fragment reads are inline assembly with explicit base registers and
  // constant offsets: a handful of per-lane bases serve every step and tile (left
  // to itself the compiler keeps one address register per step and tile, runs
  // out of registers and spills -- and a spill reload in this loop would wait for
  // every load in flight).  The compiler does not see these reads complete, so
  // the waits below wait for them and tie the registers to those waits.
  const int fi = dl_f(i);
  const int base = (int)lds_addr(smem);
  // read bases per step buffer: chunk q of row i (lo, first half step); chunk
  // 2 + q is that address ^ 32, and the second half step's chunks are ^ 64
  int aw0[C::NB], ax0[C::NB];
#pragma unroll
  for (int b = 0; b < C::NB; ++b) {
    aw0[b] = base + b * Lds::DATA + Lds::W + wn * C::TN * 4096 + 128 * i + 16 * (q ^ fi);
    ax0[b] = base + b * Lds::DATA + Lds::X + wm * C::TM * 4096 + 128 * i + 16 * (q ^ fi);
  }
  const int aws = base + Lds::SCALES + (wn * C::TN * 32 + i) * 16;
  const int axs = base + Lds::SCALES + (C::BN + wm * C::TM * 32 + i) * 16;
  // Fragment read r of half step H of K-step J (mod 8) of the unrolled loop: r < TN
  // is weight tile r, then token tile r - TN; each is a scale word and two 16-byte
  // halves.  K-step J lives in step buffer J % NB and scale buffer J / 4, scale word J % 4.
  auto read_tile = [&](auto r_tag, auto j_tag, auto h_tag, Frags& F) {
    constexpr int r = decltype(r_tag)::value, J = decltype(j_tag)::value, H = decltype(h_tag)::value;
    constexpr int B = J % C::NB, SB = (J / 4) * Lds::SBUF + (J % 4) * 4;
    if constexpr (r < C::TN) {
      F.sw[r] = lds_read4<SB + r * 512>(aws);
      F.fw[r] = join8(lds_read16_xor<r * 4096, 64 * H>(aw0[B]), lds_read16_xor<r * 4096, 64 * H + 32>(aw0[B]));
    } else {
      constexpr int c = r - C::TN;
      F.sx[c] = lds_read4<SB + c * 512>(axs);
      F.fx[c] = join8(lds_read16_xor<c * 4096, 64 * H>(ax0[B]), lds_read16_xor<c * 4096, 64 * H + 32>(ax0[B]));
    }
  };
  // Read order of a half step's tiles: what the first half of its MFMAs needs
  // (weight tiles 0 .. TN/2-1 and every token tile, in the order those MFMAs use
  // them) first, the weight tiles of the second half last.
  constexpr auto order = [](int k) constexpr {
    if (k == 0) return 0;                                   // W0
    if (k <= C::TM) return C::TN + k - 1;                   // X0 .. X(TM-1)
    return k - C::TM;                                       // W1 .. W(TN-1)
  };
  // SPLIT reads a half step's activation tiles first: B2 splits them while the weight reads finish
  constexpr auto order_split = [](int k) constexpr { return k < C::TM ? C::TN + k : k - C::TM; };
  static_assert(C::TN % 2 == 0, "weight tiles split evenly over the two halves of a half step");
  constexpr int LATE_LDS_OPS = 3 * (C::TN / 2);             // scale word + two halves per late tile
  auto shift_scales = [&](Frags& F, int a0, int a1, bool x) {
    for (int a = a0; a < a1; ++a) F.sw[a] = (int)((uint32_t)F.sw[a] >> (8 * q));
    if (x)
      for (int c = 0; c < C::TM; ++c) F.sx[c] = (int)((uint32_t)F.sx[c] >> (8 * q));
  };
  // register ties: each placed right after the s_waitcnt that covers the reads
  // (volatile asm statements keep their order)
  auto tie_w = [&](Frags& F, int a0, int a1) {
#pragma unroll
    for (int a = a0; a < a1; ++a) asm volatile("" : "+v"(F.fw[a]), "+v"(F.sw[a]));
  };
  auto tie_x = [&](Frags& F) {
#pragma unroll
    for (int c = 0; c < C::TM; ++c) asm volatile("" : "+v"(F.fx[c]), "+v"(F.sx[c]));
  };
  // f0 of a K-step is read last (end of the previous K-step), its late weight
  // tiles last of all: wait for all but those
  auto wait_f0_early = [&](Frags& F) {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(LATE_LDS_OPS));
    tie_w(F, 0, C::TN / 2);
    tie_x(F);
    shift_scales(F, 0, C::TN / 2, true);
  };
  // everything: f0's late tiles and all of f1
  auto wait_f0_late_f1 = [&](Frags& F0, Frags& F1) {
    asm volatile("s_waitcnt lgkmcnt(0)");
    tie_w(F0, C::TN / 2, C::TN);
    tie_w(F1, 0, C::TN);
    tie_x(F1);
    shift_scales(F0, C::TN / 2, C::TN, false);
    shift_scales(F1, 0, C::TN, true);
  };

  // One K-step k (J = k % 8) in four quarters of NMF MFMAs each, f0's weight tiles
  // 0 .. TN/2-1, then TN/2 .. TN-1, then f1's likewise:
  //   A1: f0's first MFMAs; reads of all of f1 (step buffer k % NB, already visible)
  //       slotted between them.  Then every wave waits for its reads and a barrier
  //       frees step buffer k % NB for the loads of step k+NB (and, at k = 4s, scale
  //       buffer (s+1) % 2, last used by steps up to 4s-1, for scale group s+1).
  //   A2, B1, B2: the rest of the MFMAs with the L loads of step k+NB spread evenly
  //       between them (one memory pipeline per CU: loads issued in a burst queue
  //       faster than it accepts them, and a wave waiting to issue a load issues no
  //       MFMA either).
  //   Before B2, each wave waits for its loads of step k+1 (the ones issued in the
  //       three quarters before the previous B2 ended), and a barrier makes every
  //       wave's step k+1 visible; B2 then also reads f0 of step k+1.
  // A step has no branches: a branch would split the scheduling region and let the
  // compiler regroup the MFMAs.  Every step issues the loads of step k+NB and, at
  // k = 4s, of scale group s+1 -- switched off (zero-byte resources) where those do
  // not exist -- so the number of loads issued after step k+1's is a constant, and
  // the last step's reads fetch a buffer that is never used.
  // With SPLIT every (weight tile, token tile) pair takes two MFMAs, one per part of the
  // activation fragment: a quarter issues all its small-code MFMAs, then all its large-code
  // ones (no two consecutive MFMAs on one accumulator), and the first quarter of each half
  // step splits each activation fragment just ahead of its first MFMA, so the bit operations
  // overlap the MFMAs already in the pipeline.
  constexpr int NMF = C::TN / 2 * C::TM;             // (weight tile, token tile) pairs per quarter
  constexpr int NM = SPLIT ? 2 * NMF : NMF;          // MFMA slots per quarter
  constexpr auto load_slot = [](int d) constexpr { return d * 3 * NM / L; };   // MFMA of A2, B1, B2 it follows
  constexpr int P12 = (2 * L + 2) / 3;               // loads in A2 and B1: load_slot(d) < 2 NM <=> 3d < 2L
  Frags f0, f1;
  auto mfma_q = [&](auto j_tag, auto quarter_tag, int k) {
    constexpr int J = decltype(j_tag)::value, Q = decltype(quarter_tag)::value;   // Q: 0 = A1 .. 3 = B2
    constexpr int H = Q / 2;
    Frags& F = H == 0 ? f0 : f1;
    const bool on = k + C::NB < ksteps;
    // SPLIT: f1's activation fragments (read in A1) are split during A2, which multiplies f0;
    // f0's for the next step (read in B1) during B2, which multiplies f1, once their reads
    // are done -- so the bit operations overlap MFMAs on other registers.
    // the TM fragments' 8 TM dwords spread evenly over the quarter's NM slots (in-order issue: a burst of
    // bit operations after one MFMA would hold back the next MFMA's issue while the pipe drains)
    constexpr int SPLIT_DW = 8 * C::TM;
    constexpr int SPLIT_PER_SLOT = (SPLIT_DW + NM - 1) / NM;
    if constexpr (SPLIT && Q == 3) {
      // B1 read the activation tiles first (order_split): at most the weight tiles' reads may
      // still be in flight (the counter holds 15 at most; waiting for more is only earlier)
      asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(3 * C::TN < 15 ? 3 * C::TN : 15));
      tie_x(f0);
      shift_scales(f0, 0, 0, true);
    }
    static_for<NM>([&](auto m_tag) {
      constexpr int m = decltype(m_tag)::value;
      constexpr int mm = m % NMF;
      constexpr int a = (Q % 2) * (C::TN / 2) + mm / C::TM, b = mm % C::TM;
      if constexpr (m < NMF)
        acc[a][b] = mfma_scaled<2 * H>(F.fw[a], F.fx[b], acc[a][b], F.sw[a], F.sx[b]);
      else
        acc[a][b] = mfma_scaled<2 * H>(F.fw[a], F.fxh[b], acc[a][b], F.sw[a], F.sx[b]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (SPLIT && (Q == 1 || Q == 3)) {
        Frags& S = Q == 1 ? f1 : f0;
        static_for<SPLIT_PER_SLOT>([&](auto j_tag) {
          constexpr int w = m * SPLIT_PER_SLOT + decltype(j_tag)::value;
          if constexpr (w < SPLIT_DW) split_large_dword<w % 8>(S.fx[w / 8], S.fxh[w / 8]);
        });
      }
      if constexpr (Q == 0 || Q == (SPLIT ? 2 : 3)) {
        static_for<NT>([&](auto t_tag) {
          constexpr int t = decltype(t_tag)::value;
          if constexpr (t * NM / NT == m) {
            if constexpr (Q == 0)
              read_tile(std::integral_constant<int, order(t)>{}, j_tag, std::integral_constant<int, 1>{}, f1);
            else if constexpr (SPLIT)
              read_tile(std::integral_constant<int, order_split(t)>{}, std::integral_constant<int, (J + 1) % 8>{},
                        std::integral_constant<int, 0>{}, f0);
            else
              read_tile(std::integral_constant<int, order(t)>{}, std::integral_constant<int, (J + 1) % 8>{},
                        std::integral_constant<int, 0>{}, f0);
          }
        });
      }
      if constexpr (Q > 0) {
        static_for<L>([&](auto d_tag) {
          constexpr int d = decltype(d_tag)::value;
          if constexpr (load_slot(d) == (Q - 1) * NM + m)
            issue_one(d_tag, std::integral_constant<int, J % C::NB>{}, k + C::NB, on);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto kstep = [&](auto j_tag, int k) {
    constexpr int J = decltype(j_tag)::value;
    wait_f0_early(f0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_q(j_tag, std::integral_constant<int, 0>{}, k);
    wait_f0_late_f1(f0, f1);
    asm volatile("s_barrier" ::: "memory");
    if constexpr (J % 4 == 0)      // group k/4 + 1 = k0/4 + J/4 + 1, k0 a multiple of 8
      issue_scales(std::integral_constant<int, (J / 4 + 1) % 2>{}, k / 4 + 1, 4 * (k / 4 + 1) < ksteps);
    __builtin_amdgcn_sched_barrier(0);
    mfma_q(j_tag, std::integral_constant<int, 1>{}, k);
    mfma_q(j_tag, std::integral_constant<int, 2>{}, k);
    // loads issued after step k+1's last one (which went out in step k+1-NB): the
    // loads of steps k+2 .. k+NB-1 (steps k+2-NB .. k-1), A2 and B1 of this step,
    // and a scale group if one went out in steps k+2-NB .. k (at steps 4s)
    wait_vmcnt<(C::NB - 2) * L + P12 + (J % 4 <= C::NB - 2 ? SI : 0)>();
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    mfma_q(j_tag, std::integral_constant<int, 3>{}, k);
  };

  // SPLIT: the barrier that publishes step k+1 comes before B1 (one quarter earlier), so that B1
  // can read f0 of step k+1 and B2 split it; the loads outstanding at that wait are those of
  // steps k+2 .. k+NB-1, A2's of this step, and the scale groups as above.
  constexpr int P1 = (L + 2) / 3;                    // loads in A2: load_slot(d) < NM <=> 3d < L
  auto kstep_split = [&](auto j_tag, int k) {
    constexpr int J = decltype(j_tag)::value;
    asm volatile("s_waitcnt lgkmcnt(0)");          // f0's weight tiles, read in the previous step's B1
    tie_w(f0, 0, C::TN);
    shift_scales(f0, 0, C::TN, false);
    __builtin_amdgcn_sched_barrier(0);
    mfma_q(j_tag, std::integral_constant<int, 0>{}, k);
    asm volatile("s_waitcnt lgkmcnt(0)");          // f1, read in A1
    tie_w(f1, 0, C::TN);
    tie_x(f1);
    shift_scales(f1, 0, C::TN, true);
    asm volatile("s_barrier" ::: "memory");
    if constexpr (J % 4 == 0)
      issue_scales(std::integral_constant<int, (J / 4 + 1) % 2>{}, k / 4 + 1, 4 * (k / 4 + 1) < ksteps);
    __builtin_amdgcn_sched_barrier(0);
    mfma_q(j_tag, std::integral_constant<int, 1>{}, k);
    wait_vmcnt<(C::NB - 2) * L + P1 + (J % 4 <= C::NB - 2 ? SI : 0)>();
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    mfma_q(j_tag, std::integral_constant<int, 2>{}, k);
    mfma_q(j_tag, std::integral_constant<int, 3>{}, k);
  };

  issue_scales(std::integral_constant<int, 0>{}, 0, true);
  static_for<C::NB>([&](auto b_tag) {
    constexpr int b = decltype(b_tag)::value;
    static_for<L>([&](auto d_tag) { issue_one(d_tag, b_tag, b, b < ksteps); });
  });
  wait_vmcnt<(C::NB - 1) * L>();                   // scale group 0 and step 0
  asm volatile("s_barrier" ::: "memory");
  static_for<NT>([&](auto t_tag) {
    read_tile(std::integral_constant<int, order(decltype(t_tag)::value)>{}, std::integral_constant<int, 0>{},
              std::integral_constant<int, 0>{}, f0);
  });
  if constexpr (SPLIT) {
    asm volatile("s_waitcnt lgkmcnt(0)");
    tie_x(f0);
    shift_scales(f0, 0, 0, true);
#pragma unroll
    for (int c = 0; c < C::TM; ++c) split_large_codes(f0.fx[c], f0.fxh[c]);
  }
  for (int k0 = 0; k0 < ksteps; k0 += 8) {
    static_for<8>([&](auto j_tag) {
      constexpr int J = decltype(j_tag)::value;
      if (J == 0 || k0 + J < ksteps) {
        if constexpr (SPLIT) kstep_split(j_tag, k0 + J);
        else kstep(j_tag, k0 + J);
      }
    });
  }
  // The last step's reads of f0 (of a step that does not exist; f1's reads were
  // waited for within the step) and the switched-off loads -- which still write zeros into the step buffers that the
  // epilogue reuses -- have all landed before the barrier below.
  wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)");
  tie_w(f0, 0, C::TN);
  tie_x(f0);

  // Epilogue through LDS, one 32-token block at a time.
  // The lane's row i and half q (and so the lane index) are taken back from a base
  // address that lives through the loop anyway, so that nothing the epilogue
  // derives from them is computed early and kept alive across the loop.
  __syncthreads();
  int aw = aw0[0];
  asm volatile("" : "+v"(aw));                     // opaque: keeps the compiler from reusing the original i
  const int i_e = ((aw - base - wn * C::TN * 4096) >> 7) & 31;
  const int q_e = ((aw >> 4) & 7) ^ dl_f(i_e);
  static_assert(4 * EpiLds<C::TN>::BYTES <= Lds::BYTES, "epilogue blocks of the four waves");
  uint8_t* chunk = smem + wave * EpiLds<C::TN>::BYTES;
  const int64_t nb = (int64_t)g * p.N + n0 + wn * C::TN * 32;
#pragma unroll
  for (int b = 0; b < C::TM; ++b) {
#pragma unroll
    for (int a = 0; a < C::TN; ++a) {
      // each tile stays in accumulator registers until its turn (copied out all at
      // once, the tiles would not fit the general registers)
      asm volatile("" : "+a"(acc[a][b]));
      epi_write_tile<C::TN>(chunk, acc[a][b], a, i_e, q_e);
      __builtin_amdgcn_sched_barrier(0);
    }
    epi_store_rows<OUT, C::TN>(p, chunk, m0 + (wm * C::TM + b) * 32, nb, i_e + 32 * q_e);
  }
}

// Tile (group g, weight tile nt, token row mt) of work index wi, for nf weight
// tiles x R token rows per group: groups in turn, each walked in panels of PW
// weight tiles (the last panel may be narrower), every panel down all its token
// rows.  The work indices of one XCD are consecutive (xcd_work_index), so the
// 32 tiles an XCD runs at once form a block about PW weight tiles wide and 32/PW
// token rows deep, whose operand rows its L2 shares: for 256 x 256 tiles at
// PW = 4, 384 KB of distinct operand bytes per K-step against 704 KB for rows
// of 20 weight tiles (wo_b).
__device__ __forceinline__ void panel_tile(int wi, int nf, int R, int PW, int& g, int& nt, int& mt) {
  const int per_group = nf * R;
  g = wi / per_group;
  const int j = wi - g * per_group;
  const int panel = j / (PW * R);
  const int w = min(PW, nf - panel * PW);                 // width of this panel
  const int k = j - panel * PW * R;
  mt = k / w;
  nt = panel * PW + k % w;
}

template <class CF, class CT, int OUT, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dl_gemm_kernel(GemmArgs p, int G, int full_rows, int rows) {
  static_assert(CF::BM == CT::BM, "rows of BM tokens");
  constexpr int BM = CF::BM;
  constexpr int BYTES = DlLds<CF>::BYTES > DlLds<CT>::BYTES ? DlLds<CF>::BYTES : DlLds<CT>::BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[BYTES];
  const int nf = (int)(p.N / CF::BN), ntl = (int)(p.N / CT::BN);
  const int F = G * nf * full_rows;
  if ((int)blockIdx.x < F) {
    int g, nt, mt;
    panel_tile(xcd_work_index((int)blockIdx.x, F), nf, full_rows, 4, g, nt, mt);
    dl_tile<CF, OUT, SPLIT>(p, smem, g, (int64_t)nt * CF::BN, (int64_t)mt * BM);
  } else {
    const int tr = rows - full_rows;
    int g, nt, mt;
    panel_tile(xcd_work_index((int)blockIdx.x - F, G * ntl * tr), ntl, tr, 8, g, nt, mt);
    dl_tile<CT, OUT, SPLIT>(p, smem, g, (int64_t)nt * CT::BN, (int64_t)(full_rows + mt) * BM);
  }
}

template <class CF, class CT, int OUT, bool SPLIT>
hipError_t launch_dl(const GemmArgs& p, const GemmPlan& plan, int64_t G, hipStream_t stream) {
  hipLaunchKernelGGL((dl_gemm_kernel<CF, CT, OUT, SPLIT>), dim3((unsigned)plan.workgroups), dim3(256), 0, stream, p,
                     (int)G, plan.full_rows, plan.rows);
  return hipGetLastError();
}

}  // namespace mx
