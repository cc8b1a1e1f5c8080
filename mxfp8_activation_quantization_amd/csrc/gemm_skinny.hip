// Block-scaled FP8 GEMM for few tokens (decode): split-K weight streaming.
//
// With at most a few hundred tokens the o_proj chain is bound by reading its
// weights from HBM once (vLLM PR #60118 "[Perf][DSv4.1] MegaAttn: wo_a writes
// wo_b's MXFP8 input", Claims: the decode range is 1-256 tokens).  HBM streams
// near its peak only when every CU keeps many reads in flight for the whole
// kernel, so the grid is sized to be resident in one round (one workgroup per
// CU) and every workgroup streams a long K range through a software pipeline.
//
// Work item: 64 weight rows (two MFMA row tiles) x one chunk of up to 64 tokens
// x one K range (split s of S).  Four waves: wave (rt, tt) owns the 32 x 32
// output tile of row tile rt and token tile tt.
//
// Split K: with S > 1 every work item writes its fp32 partial tile to the
// caller's workspace, and the last of the S items of a tile to arrive (an atomic
// counter) adds the partials in split order 0, 1, ..., S-1 and runs the
// epilogue, so the result does not depend on arrival order.  The counter is
// reset to zero for the next call.
#include "gemm_common.hpp"

namespace mx {

namespace {

constexpr uint32_t kRsrcFlags = 0x00020000;   // raw buffer, 32-bit dwords, range-checked
constexpr int kUncached = 0x11;              // sc0 | sc1: bypass L1 and L2 (partials cross XCDs)
constexpr int kL2 = 0x01;                    // sc0: through L1 to the XCD's L2 (partials stay on one XCD)
constexpr int kLocalMaxSplits = 16;          // per-XCD arrival counts are 4-bit fields
constexpr int kTileRows = 64;                // weight rows per work item
constexpr int kChunkTokens = 64;             // tokens per work item (two token tiles)

}  // namespace

// The end of a work item: with one split the tile goes straight to the epilogue.
// Otherwise the item publishes its partial tile and the last of the S items of
// the tile to arrive adds the partials in split order 0, 1, ..., S-1 and runs the
// epilogue.  The items of a tile may run on different XCDs, whose L2 caches are
// not coherent with each other, so partials move with 16-byte buffer accesses
// that bypass L1 and L2 (sc0 sc1) and the counter with a relaxed system-scope
// atomic: a writer waits until its stores are complete before it bumps the
// counter, and the last one reads the partials from memory.  Partial layout per
// split: [rt][tt][lane][16 floats].  All threads of the workgroup must call this.
template <int MT, int OUT>
__device__ __forceinline__ void finish_tile(const GemmArgs& p, const v16f& acc, int tc, int s, int S, int rt, int tt,
                                            int lane, int tid, int64_t nb, int64_t m, bool computes, int* s_last) {
  const int q = lane >> 5;
  if (S == 1) {
    if (computes) store_tile<OUT>(p, acc, m, m < p.M, nb, q);
    return;
  }
  constexpr int TILE_FLOATS = 2 * MT * 16 * 64;
  constexpr int TILE_BYTES = TILE_FLOATS * 4;
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      p.ws_partials + (int64_t)tc * S * TILE_FLOATS, 0, S * TILE_BYTES, kRsrcFlags);
  const int my_off = ((rt * MT + tt) * 64 + lane) * 64;     // bytes within a split's tile
  if (computes) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const v4i v = {__float_as_int(acc[4 * k]), __float_as_int(acc[4 * k + 1]), __float_as_int(acc[4 * k + 2]),
                     __float_as_int(acc[4 * k + 3])};
      __builtin_amdgcn_raw_buffer_store_b128(v, rp, s * TILE_BYTES + my_off + 16 * k, 0, kUncached);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    *s_last = __hip_atomic_fetch_add(&p.ws_counters[tc], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
              (uint32_t)(S - 1);
  __syncthreads();
  if (!*s_last || !computes) return;

  // the last item: each wave sums its own 32 x 32 tile over the splits, in split order
  v16f tot = zero16();
  for (int s0 = 0; s0 < S; s0 += 2) {
    v4i ld[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        ld[u][k] = s0 + u < S ? __builtin_amdgcn_raw_buffer_load_b128(rp, (s0 + u) * TILE_BYTES + my_off + 16 * k, 0,
                                                                      kUncached)
                              : v4i{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (s0 + u < S) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          tot[4 * k] += __int_as_float(ld[u][k].x);
          tot[4 * k + 1] += __int_as_float(ld[u][k].y);
          tot[4 * k + 2] += __int_as_float(ld[u][k].z);
          tot[4 * k + 3] += __int_as_float(ld[u][k].w);
        }
      }
    }
  }
  store_tile<OUT>(p, tot, m, m < p.M, nb, q);
  if (tid == 0) __hip_atomic_store(&p.ws_counters[tc], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------------------
// The weight-streaming kernel.
//
// E4M3 activations: both operands are codes, so every byte goes from memory straight into LDS
// (buffer_load ... lds) and the pipeline depth is bounded by LDS, not registers:
// a ring of kRingE4 stages of kStageSteps 128-deep steps (64 weight rows and 64 token
// rows x 128 bytes per step: 32 KB per stage), with the loads of stage t + kRingE4 - 1
// issued while stage t is multiplied.  One workgroup per CU keeps 32 KB of weights
// in flight per CU: with every CU streaming at once, fewer bytes in flight per CU
// finish sooner (wo_b 8192 -> 5120 at 64 tokens: 15.2 us with two stages in flight,
// 15.5 with three, alternated on one box); two steps per stage halve the barriers and
// the LDS-read -> MFMA latency each stage exposes.  The scale words of the whole K range (up
// to kMaxSteps steps) are fetched once, at the start, into two tables: per step
// they would be 64 scattered 4-byte reads per operand.
//
// Stage layout of an operand (64 rows x 8 chunks of 16 bytes): chunk c of row r
// sits in slot 8r + (c ^ g8(r)), g8(r) = ((r >> 1) & 7) ^ ((r & 1) << 2).  One
// load instruction fills 1 KB of consecutive slots = 8 whole rows (row-contiguous
// 128-byte reads), and the 16 (or 8) lanes of a fragment read -- 16 rows, one
// chunk -- hit distinct 16-byte bank groups.  Scale tables: row r holds the words
// of steps k_lo .. k_lo + 31 as eight 16-byte chunks, chunk c at position c ^ (r & 7).
// A lane's fragment is row i, chunks 4KS + q and 4KS + 2 + q.  BF16 activations
// take the same path with the activation slot of each stage filled by the
// workgroup's own threads (quantized in registers, two stages ahead: a ring of
// kRing stages), so E4M3 and BF16 activations give identical bits.
constexpr int kRing = 4;
constexpr int kRingE4 = 3;
constexpr int kStageSteps = 2;
constexpr int kMaxSteps = 32;

__device__ __forceinline__ int g8(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// K-steps of the splits: split s of S covers [split_begin(s), split_begin(s + 1)).  With two or
// three splits, when it still fits the scale tables, the last split takes about kSplitSkew steps
// more than the others, so that it usually finishes after they have published their partials and
// skips publishing its own (the combine below); otherwise the splits are equal.  Measured at 64
// tokens, alternated on one box: wo_b 8192 -> 5120 (3 splits of 64 steps) 20/20/24 saves 0.5-0.7 us
// per call against 21/21/22, where 21/21/22 with the early counter read and 19/19/26 save nothing;
// N = 5120 at K = 2048 / 4096 (3 splits) saves 0.6 / 0.4 us, N = 6144 at K = 4096 (2 splits) 0.8 us;
// with 4 or 8 splits (N = 4096, K = 4096; N = 2048, K = 8192) the longer last split cost 1.5 / 0.3 us.
constexpr int kSplitSkew = 4;
__device__ __forceinline__ bool split_skewed(int S, int ksteps) {
  const int b = (ksteps - kSplitSkew) / S;
  return S > 1 && S <= 3 && b >= 1 && ksteps - (S - 1) * b <= kMaxSteps;
}
__device__ __forceinline__ int split_begin(int s, int S, int ksteps) {
  if (s >= S) return ksteps;
  return split_skewed(S, ksteps) ? s * ((ksteps - kSplitSkew) / S) : (int)((int64_t)s * ksteps / S);
}

__device__ __forceinline__ v8i ring_frag(const uint8_t* op, int T, int KS, int lane) {
  const int i = lane & 31, q = lane >> 5, r = 32 * T + i, g = g8(r);
  const uint8_t* b = op + 128 * r;
  return frag(*reinterpret_cast<const uint4*>(b + 16 * ((4 * KS + q) ^ g)),
              *reinterpret_cast<const uint4*>(b + 16 * ((4 * KS + 2 + q) ^ g)));
}

__device__ __forceinline__ uint32_t table_word(const uint32_t* tab, int r, int j) {
  return tab[r * 32 + (((j >> 2) ^ (r & 7)) << 2) + (j & 3)];
}

struct RingStage {
  uint8_t w[kStageSteps][64 * 128];
  uint8_t x[kStageSteps][64 * 128];
};

// Waits until at most n stages of this wave's loads (L instructions each) are in flight.
template <int L>
__device__ __forceinline__ void wait_stages(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<L>(); break;
    default: wait_vmcnt<2 * L>(); break;
  }
}

template <int MT, int OUT, bool XB, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void stream_kernel(GemmArgs p, int G, int n_tiles, int chunks, int S) {
  static_assert(kRing == 4 && kRingE4 >= 2 && kRingE4 <= kRing, "wait_stages covers up to 2 stages in flight");
  constexpr int L = 4 * kStageSteps;     // load instructions per wave and stage: per step 2 weight, 2 activation
  __shared__ __attribute__((aligned(1024))) RingStage ring[kRing];
  __shared__ __attribute__((aligned(1024))) uint32_t wtab[64 * kMaxSteps];
  __shared__ __attribute__((aligned(1024))) uint32_t xtab[64 * kMaxSteps];
  __shared__ int s_last;

  const int total = G * n_tiles * chunks * S;
  const int wi = xcd_work_index((int)blockIdx.x, total);
  const int s = wi % S;
  const int rest = wi / S;
  const int chunk = rest % chunks;
  const int tile = rest / chunks;
  const int g = tile / n_tiles, nt = tile % n_tiles;
  const int tc = tile * chunks + chunk;

  const int tid = threadIdx.x, lane = tid & 63, i = lane & 31, q = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = wave & 1, tt = wave >> 1;
  const bool computes = tt < MT;

  const int ksteps = (int)(p.K / 128);
  const int64_t n_row0 = (int64_t)g * p.N + (int64_t)nt * kTileRows;
  const int64_t m_first = (int64_t)chunk * kChunkTokens;
  const int64_t m_rows = p.M - m_first < kChunkTokens ? p.M - m_first : kChunkTokens;
  const int ldw = (int)p.K, ldx = (int)p.ld_x, ldxs = (int)(p.ld_xsf * 4);
  const int xcol0 = (int)((int64_t)g * p.K), xsfcol0 = g * ksteps * 4;
  const Rsrc rw = make_rsrc_sgpr(p.w + n_row0 * p.K, (int64_t)kTileRows * p.K);
  const Rsrc rws = make_rsrc_sgpr(p.w_sf + n_row0 * ksteps, (int64_t)kTileRows * ksteps * 4);
  // Activation ranges end at row m_rows and the row part of every activation
  // offset is in the per-lane register (the part the range check covers), so rows
  // past M arrive as zeros and nothing past row M is read.  The scale tables may
  // read up to 31 words past a row's K range: the next row's words (unused), or
  // zeros past the end of the buffer.
  const Rsrc rx = make_rsrc_sgpr(static_cast<const uint8_t*>(p.x) + m_first * ldx * (XB ? 2 : 1),
                                 m_rows * ldx * (XB ? 2 : 1));
  const Rsrc rxs = make_rsrc_sgpr(XB ? nullptr : p.x_sf + m_first * p.ld_xsf, XB ? 0 : m_rows * ldxs);
  const Rsrc rnull = make_rsrc_sgpr(p.w, 0);       // zero bytes: every lane out of range, nothing read

  // BF16 activations (quantized here): thread -> token row xr, 32-element block xb of
  // each step; its 64 bytes per step are four 16-byte loads at vxb + 16 u (row part in
  // the per-lane register, so rows past M read as zeros), step k at scalar offset 256 k.
  const int xr = tid >> 2, xb = tid & 3, gxr = g8(xr);
  const int vxb = xr * ldx * 2 + xcol0 * 2 + xb * 64;

  // per-lane offsets: instruction j of this wave covers rows 8n .. 8n+7, n = 4j + wave
  int vw[2], vx[2], vts0[2], vtx0[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = 4 * j + wave, r = 8 * n + (lane >> 3), c = (lane & 7) ^ g8(r), ct = (lane & 7) ^ (r & 7);
    vw[j] = r * ldw + c * 16;
    vx[j] = r * ldx + c * 16;
    // scale table chunk ct = steps 4ct .. 4ct+3 of the range (plus 4 k_lo bytes below);
    // the whole offset is in the per-lane register so that the range check sees it
    // (no read past a buffer's end)
    vts0[j] = r * ksteps * 4 + ct * 16;
    vtx0[j] = r * ldxs + xsfcol0 + ct * 16;
  }

  // The K range of split s_ through the pipeline, into a fresh accumulator.  All
  // threads take part (loads and barriers); waves that own no token tile return zeros.
  auto run_split = [&](int s_) -> v16f {
    const int k_lo = split_begin(s_, S, ksteps);
    const int k_hi = split_begin(s_ + 1, S, ksteps);
    const int nsteps = k_hi - k_lo;               // <= kMaxSteps (the plan and split_skewed guarantee it)
    const int nst = (nsteps + kStageSteps - 1) / kStageSteps;
    __syncthreads();                              // LDS of a previous run is no longer read

    // scale tables first (they complete before any stage: loads finish in issue order)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = 4 * j + wave;
      dl_load16(rws, wtab + n * 256, vts0[j] + k_lo * 4, 0);
      if constexpr (!XB) dl_load16(rxs, xtab + n * 256, vtx0[j] + k_lo * 4, 0);
    }

    // multiplies stage t (all threads call it; waves without a token tile skip)
    auto mma_stage = [&](int t, v16f& acc, int ring_len) {
      if (computes) {
        const RingStage& st = ring[t % ring_len];
#pragma unroll
        for (int h = 0; h < kStageSteps; ++h) {
          const int j = kStageSteps * t + h;
          if (j < nsteps) {
            const int sw = (int)(table_word(wtab, rt * 32 + i, j) >> (8 * q));
            const int sx = (int)(table_word(xtab, tt * 32 + i, j) >> (8 * q));
            acc = mfma_act<0, SPLIT>(ring_frag(st.w[h], rt, 0, lane), ring_frag(st.x[h], tt, 0, lane), acc, sw, sx);
            acc = mfma_act<2, SPLIT>(ring_frag(st.w[h], rt, 1, lane), ring_frag(st.x[h], tt, 1, lane), acc, sw, sx);
          }
        }
      }
    };

    if constexpr (XB) {
      // BF16 activations.  Weights stream into the ring as with E4M3 activations;
      // each thread loads its token's 32-element block of the two steps of a stage
      // into registers two stages ahead, then quantizes it (its own amax: the
      // quantizer's rule) into the stage's activation slot and the scale table.  Two
      // register sets alternate, so the loop is unrolled by two.  Every step issues
      // the same loads -- switched off (zero-byte resource) past the last stage --
      // so the wait counts are constants: a step needs the activation registers of
      // stage t+2, after which only the previous step's batch (4 weight + 8
      // activation loads) may still be in flight.
      struct XRegs { v4i v[8]; };
      auto load_x = [&](XRegs& X, int t) {
#pragma unroll
        for (int h = 0; h < kStageSteps; ++h) {
          const int k = k_lo + kStageSteps * t + h;
          const bool on = t < nst && k < k_hi;
#pragma unroll
          for (int u = 0; u < 4; ++u) X.v[4 * h + u] = buf_load16(on ? rx : rnull, vxb + 16 * u, k * 256);
        }
      };
      auto issue_w = [&](int t) {
        RingStage& st = ring[t % kRing];
        const bool on = t < nst;
#pragma unroll
        for (int h = 0; h < kStageSteps; ++h) {
          const int kk = k_lo + kStageSteps * t + h, k = kk < k_hi ? kk : k_hi - 1;
#pragma unroll
          for (int j = 0; j < 2; ++j) dl_load16(on ? rw : rnull, st.w[h] + (4 * j + wave) * 1024, vw[j], k * 128);
        }
      };
      auto quantize_x = [&](XRegs& X, int t) {
#pragma unroll
        for (int u = 0; u < 8; ++u) tie_after_wait(X.v[u]);
        RingStage& st = ring[t % kRing];
        uint8_t* xt = reinterpret_cast<uint8_t*>(xtab);
#pragma unroll
        for (int h = 0; h < kStageSteps; ++h) {
          uint32_t w[16];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            w[4 * u] = (uint32_t)X.v[4 * h + u].x;
            w[4 * u + 1] = (uint32_t)X.v[4 * h + u].y;
            w[4 * u + 2] = (uint32_t)X.v[4 * h + u].z;
            w[4 * u + 3] = (uint32_t)X.v[4 * h + u].w;
          }
          uint32_t am = 0;
#pragma unroll
          for (int k = 0; k < 16; ++k) am = amax_pair(am, w[k]);
          const int e = scale_exp_from_amax(fold_pair(am));
          const float sc = exp2_int(e);
          uint32_t c[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) c[k] = encode4(w[2 * k], w[2 * k + 1], sc);
          *reinterpret_cast<uint4*>(st.x[h] + 16 * (8 * xr + ((2 * xb) ^ gxr))) = make_uint4(c[0], c[1], c[2], c[3]);
          *reinterpret_cast<uint4*>(st.x[h] + 16 * (8 * xr + ((2 * xb + 1) ^ gxr))) = make_uint4(c[4], c[5], c[6], c[7]);
          const int j = kStageSteps * t + h;
          xt[4 * (xr * 32 + (((j >> 2) ^ (xr & 7)) << 2) + (j & 3)) + xb] = (uint8_t)(e + 127);
        }
      };

      v16f acc = zero16();
      XRegs A, B;
      load_x(A, 0);
      load_x(B, 1);
      issue_w(0);
      issue_w(1);
      issue_w(2);
      wait_vmcnt<0>();
      quantize_x(A, 0);
      quantize_x(B, 1);
      load_x(A, 2);
      load_x(B, 3);
      // step t: stage t+2's registers are set (t & 1); loads after them: one batch
      auto step = [&](XRegs& X, int t, bool first) {
        if (first) wait_vmcnt<8>();
        else wait_vmcnt<12>();
        asm volatile("s_barrier" ::: "memory");     // stage t landed everywhere; stages t-1, t-2 are free
        if (t + 2 < nst) quantize_x(X, t + 2);
        issue_w(t + 3);
        load_x(X, t + 4);
        mma_stage(t, acc, kRing);
      };
      for (int t = 0; t < nst; t += 2) {
        step(A, t, t == 0);
        if (t + 1 < nst) step(B, t + 1, false);
      }
      wait_vmcnt<0>();                               // the switched-off loads of the last steps
      // Those loads still write A and B when they return: the registers stay
      // allocated (tied here) until the wait above, so nothing else lives in them.
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        tie_after_wait(A.v[u]);
        tie_after_wait(B.v[u]);
      }
      return acc;
    }

    // A stage's second step past the range (odd step count) loads the last step
    // again -- valid addresses -- and is not multiplied.
    auto issue = [&](int t) {
      RingStage& st = ring[t % kRingE4];
#pragma unroll
      for (int h = 0; h < kStageSteps; ++h) {
        const int kk = k_lo + kStageSteps * t + h, k = kk < k_hi ? kk : k_hi - 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = 4 * j + wave;
          dl_load16(rw, st.w[h] + n * 1024, vw[j], k * 128);
          dl_load16(rx, st.x[h] + n * 1024, vx[j], xcol0 + k * 128);
        }
      }
    };

    v16f acc = zero16();
    const int pre = nst < kRingE4 - 1 ? nst : kRingE4 - 1;
    for (int t = 0; t < pre; ++t) issue(t);
    for (int t = 0; t < nst; ++t) {
      // stage t's loads are done when at most the later issued stages remain in flight
      const int later = (nst - 1 - t) < (kRingE4 - 2) ? (nst - 1 - t) : (kRingE4 - 2);
      wait_stages<L>(later);
      asm volatile("s_barrier" ::: "memory");       // every wave's loads of stage t landed; stage t-1 is free
      if (t + kRingE4 - 1 < nst) issue(t + kRingE4 - 1);
      mma_stage(t, acc, kRingE4);
    }
    return acc;
  };

  const v16f acc = run_split(s);
  const int64_t nb = n_row0 + rt * 32, m = m_first + tt * 32 + i;
  if (S == 1) {
    if (computes) store_tile<OUT>(p, acc, m, m < p.M, nb, q);
    return;
  }
  if (p.splitk_mode == SPLITK_THROUGH || S > kLocalMaxSplits) {
    finish_tile<MT, OUT>(p, acc, tc, s, S, rt, tt, lane, tid, nb, m, computes, &s_last);
    return;
  }

  // Split K through the XCD's L2.  The S items of a tile are consecutive work
  // items, which the XCD-aware numbering places on one XCD when workgroups are
  // dealt to the XCDs in turn; their L2 is then shared, and a partial tile needs
  // to reach L2 only, not memory (measured: the write acknowledgement then takes
  // about a third as long).  The arrival counter is 64 bits, updated by coherent
  // system-scope atomics: the low word counts arrivals, the high word holds a
  // 4-bit count per XCD.  The last arriver adds the partials in split order when
  // every other split ran on its own XCD; otherwise -- workgroups dealt some
  // other way -- a partial may sit in another XCD's L2, and the last arriver
  // computes those splits again itself.  Either way the sum is the same.
  constexpr int TILE_FLOATS = 2 * MT * 16 * 64;
  constexpr int TILE_BYTES = TILE_FLOATS * 4;
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      p.ws_partials + (int64_t)tc * S * TILE_FLOATS, 0, S * TILE_BYTES, kRsrcFlags);
  const int my_off = ((rt * MT + tt) * 64 + lane) * 64;     // bytes within a split's tile
  unsigned long long* cnt = reinterpret_cast<unsigned long long*>(p.ws_counters) + tc;
  // The longer last split of a skewed split first reads the counter: when every other split has
  // arrived it is the last arriver and keeps its partial in registers (the counter is not
  // incremented, so no other split can take the combine).  Otherwise it takes the usual path.
  bool kept = false;
  if (s == S - 1 && split_skewed(S, ksteps)) {
    if (tid == 0) {
      unsigned xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      xcc &= 7;
      const unsigned long long cur = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      const bool all_in = (unsigned)cur == (unsigned)(S - 1);
      const bool here = ((cur >> (32 + 4 * xcc)) & 15ull) == (unsigned long long)(S - 1) &&
                        p.splitk_mode != SPLITK_RECOMPUTE;
      s_last = all_in ? (1 | (here ? 2 : 0)) : 0;
    }
    __syncthreads();
    kept = s_last != 0;
    __syncthreads();                                // every thread has read s_last before it is written again
  }
  if (!kept) {
    if (computes) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const v4i v = {__float_as_int(acc[4 * k]), __float_as_int(acc[4 * k + 1]), __float_as_int(acc[4 * k + 2]),
                       __float_as_int(acc[4 * k + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, rp, s * TILE_BYTES + my_off + 16 * k, 0, kL2);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      unsigned xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      xcc &= 7;
      const unsigned long long old =
          __hip_atomic_fetch_add(cnt, 1ull | (1ull << (32 + 4 * xcc)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      const bool last = (unsigned)old == (unsigned)(S - 1);
      const bool here = ((old >> (32 + 4 * xcc)) & 15ull) == (unsigned long long)(S - 1) &&
                        p.splitk_mode != SPLITK_RECOMPUTE;
      s_last = (last ? 1 : 0) | (here ? 2 : 0);
    }
    __syncthreads();
  }
  const int fl = s_last;
  if (!(fl & 1)) return;
  v16f tot = zero16();
  for (int s2 = 0; s2 < S; ++s2) {
    v16f part = acc;
    if (s2 != s) {
      if (fl & 2) {
        if (computes) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rp, s2 * TILE_BYTES + my_off + 16 * k, 0, kL2);
            part[4 * k] = __int_as_float(v.x);
            part[4 * k + 1] = __int_as_float(v.y);
            part[4 * k + 2] = __int_as_float(v.z);
            part[4 * k + 3] = __int_as_float(v.w);
          }
        }
      } else {
        part = run_split(s2);
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) tot[e] += part[e];
  }
  if (computes) store_tile<OUT>(p, tot, m, m < p.M, nb, q);
  if (tid == 0) __hip_atomic_store(cnt, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------------------
// At most 128 tokens: whole K per workgroup, no split.
//
// With few tokens the activation bytes per weight row are small, so a workgroup
// can own 32 weight rows over the whole K range and the grid still covers most of
// the machine (wo_a: 256 workgroups, wo_b: 160); no partial tile leaves the
// workgroup.  Up to 32 tokens (one token tile) the four waves take the 128-deep
// steps in turn (step j: wave j % 4), each into its own accumulator; with 33 to 64
// tokens (two token tiles) waves 2 tt and 2 tt + 1 take the even and odd steps of
// token tile tt; with 65 to 128 (four token tiles) wave tt takes every step of
// token tile tt.  At the end the partial tiles of a token tile are added in wave
// order through LDS and the first wave of the tile stores it.
//
// Ring: NS stages of SS steps (SS = the waves per token tile, so every wave
// multiplies one step of every stage); per step 32 weight rows and 8 XG token
// rows x 128 bytes (XG = 1, 2, 4, 8 or 16 groups of 8 token rows, the fewest that
// hold M), the slot layout of the streaming kernel above.  The ring is shallow on
// purpose: with every CU streaming at once, deeper rings (8 to 12 stages of two
// steps were measured) finished later; kGvStages = 4 stages, or 3 where up to 32
// tokens run on a grid that holds every CU (the launcher below), and kXbStages = 3
// for the BF16-activation variant at up to 16 tokens (0.7 to 0.8 us less than 4 on
// the 256-workgroup wo_a einsum at 1 to 16 tokens, 0.2 us less on the 8192 -> 5120
// GEMM, equal on 32- and 64-tile grids).  Token
// rows past M arrive as zeros or are not loaded at all; MFMA lanes of tokens past
// the loaded rows read a loaded row again.  Those output columns are never
// stored.  Scale tables for up to kGvMaxSteps steps are fetched once, at the start.
constexpr int kGvMaxSteps = 64;
constexpr int kGvStages = 4;
constexpr int kXbStages = 3;
constexpr int64_t kWholeKShallowMinWorkgroups = 256;

template <int XG>
struct GvCfg {
  static constexpr int MT = XG > 8 ? 4 : (XG > 4 ? 2 : 1);   // token tiles
  static constexpr int SS = 4 / MT;               // steps per stage = waves per token tile
  static constexpr int XR = 8 * XG;               // token rows in a stage
  static constexpr int XI = MT;                   // activation loads per wave and step, at most
  static_assert(XG <= 16 && XR <= 32 * MT, "token rows of the token tiles");
};

template <int XG>
struct GvStage {
  uint8_t w[GvCfg<XG>::SS][32 * 128];
  uint8_t x[GvCfg<XG>::SS][GvCfg<XG>::XR * 128];
};

// Scale table of rows x kGvMaxSteps words: word j of row r in 16-byte chunk
// (j / 4) ^ (r % 16) of the row's 256 bytes (16 consecutive rows read one word
// from 16 different chunk positions).
__device__ __forceinline__ uint32_t gv_table_word(const uint32_t* tab, int r, int j) {
  return tab[r * kGvMaxSteps + (((j >> 2) ^ (r & 15)) << 2) + (j & 3)];
}

// MFMA fragment of row r of a stage slot (chunks 4KS + q and 4KS + 2 + q).
__device__ __forceinline__ v8i gv_frag(const uint8_t* op, int r, int KS, int q) {
  const int g = g8(r);
  const uint8_t* b = op + 128 * r;
  return frag(*reinterpret_cast<const uint4*>(b + 16 * ((4 * KS + q) ^ g)),
              *reinterpret_cast<const uint4*>(b + 16 * ((4 * KS + 2 + q) ^ g)));
}

// Waits until at most n stages (L loads each) of this wave's loads are in flight, n <= N.
template <int L, int N>
__device__ __forceinline__ void gv_wait(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N) wait_vmcnt<N * L>();
    else gv_wait<L, N - 1>(n);
  }
}

template <int OUT, int XG, int NS, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void whole_k_kernel(GemmArgs p, int G, int n_tiles) {
  using C = GvCfg<XG>;
  constexpr int SS = C::SS, XR = C::XR;
  static_assert(NS >= 3 && SS * (1 + C::XI) * (NS - 2) <= 63, "ring depth within the vmcnt range");
  __shared__ __attribute__((aligned(1024))) GvStage<XG> ring[NS];
  __shared__ __attribute__((aligned(1024))) uint32_t wtab[32 * kGvMaxSteps];
  __shared__ __attribute__((aligned(1024))) uint32_t xtab[XR * kGvMaxSteps];

  const int total = G * n_tiles;
  const int wi = xcd_work_index((int)blockIdx.x, total);
  const int g = wi / n_tiles, nt = wi % n_tiles;
  const int tid = threadIdx.x, lane = tid & 63, i = lane & 31, q = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tt = wave / SS, par = wave % SS;       // token tile, step parity

  const int ksteps = (int)(p.K / 128);             // <= kGvMaxSteps (the plan guarantees it)
  const int nst = (ksteps + SS - 1) / SS;
  const int64_t n_row0 = (int64_t)g * p.N + (int64_t)nt * 32;
  const int64_t m_rows = p.M < XR ? p.M : XR;     // the launch picks XG with M <= 8 XG
  const int ldw = (int)p.K, ldx = (int)p.ld_x, ldxs = (int)(p.ld_xsf * 4);
  const int xcol0 = (int)((int64_t)g * p.K), xsfcol0 = g * ksteps * 4;
  const Rsrc rw = make_rsrc_sgpr(p.w + n_row0 * p.K, (int64_t)32 * p.K);
  const Rsrc rws = make_rsrc_sgpr(p.w_sf + n_row0 * ksteps, (int64_t)32 * ksteps * 4);
  // The row part of every activation offset is in the per-lane register (the part
  // the range check covers): rows past M arrive as zeros and nothing past row M is read.
  const Rsrc rx = make_rsrc_sgpr(p.x, m_rows * ldx);
  const Rsrc rxs = make_rsrc_sgpr(p.x_sf, m_rows * ldxs);

  // Load instruction n of an operand and step fills rows 8n .. 8n+7 (1 KB): the weights'
  // instruction n = wave, the activations' n = wave + 4u (u < XI) while 8n < M.
  const int lr = lane >> 3, lc = lane & 7;
  const int vw = (8 * wave + lr) * ldw + (lc ^ g8(8 * wave + lr)) * 16;
  int vx[C::XI];
#pragma unroll
  for (int u = 0; u < C::XI; ++u) {
    const int r = 8 * (wave + 4 * u) + lr;
    vx[u] = r * ldx + (lc ^ g8(r)) * 16;
  }
  int nx = 0;                                       // activation loads of this wave and step
#pragma unroll
  for (int u = 0; u < C::XI; ++u) nx += 8 * (wave + 4 * u) < m_rows ? 1 : 0;

  // scale tables: instruction n covers rows 4n .. 4n+3; lane l loads chunk l % 16 of row
  // 4n + l / 16 into position (l % 16) ^ (row % 16).  The whole offset is in the per-lane
  // register (range-checked): a row's last chunks may read the next row's words (unused)
  // or zeros past the end of the buffer.
#pragma unroll
  for (int n = wave; n < 8; n += 4) {
    const int tr = 4 * n + (lane >> 4), ch = (lane & 15) ^ (tr & 15);
    dl_load16(rws, wtab + n * 256, tr * ksteps * 4 + ch * 16, 0);
  }
#pragma unroll
  for (int n = wave; n < XR / 4; n += 4) {
    const int tr = 4 * n + (lane >> 4), ch = (lane & 15) ^ (tr & 15);
    dl_load16(rxs, xtab + n * 256, tr * ldxs + xsfcol0 + ch * 16, 0);
  }

  // stage t: steps SS t .. SS t + SS - 1 (past the last step a stage loads the last step
  // again: valid addresses, not multiplied)
  auto issue = [&](int t) {
    GvStage<XG>& st = ring[t % NS];
#pragma unroll
    for (int h = 0; h < SS; ++h) {
      const int kk = SS * t + h, k = kk < ksteps ? kk : ksteps - 1;
      dl_load16(rw, st.w[h] + wave * 1024, vw, k * 128);
#pragma unroll
      for (int u = 0; u < C::XI; ++u)
        if (u < nx) dl_load16(rx, st.x[h] + (wave + 4 * u) * 1024, vx[u], xcol0 + k * 128);
    }
  };

  const int xi = C::MT >= 2 ? 32 * tt + i : (i & (XR - 1));   // the token row this lane reads
  v16f acc = zero16();
  auto loop = [&](auto l_tag) {
    constexpr int L = decltype(l_tag)::value;       // this wave's loads per stage
    const int pre = nst < NS - 1 ? nst : NS - 1;
    for (int t = 0; t < pre; ++t) issue(t);
    for (int t = 0; t < nst; ++t) {
      const int later = nst - 1 - t;                // stages issued after t (at most NS - 2 in flight)
      gv_wait<L, NS - 2>(later);
      asm volatile("s_barrier" ::: "memory");     // stage t landed everywhere; stage t-1 is free
      if (t + NS - 1 < nst) issue(t + NS - 1);
      const GvStage<XG>& st = ring[t % NS];
      const int j = SS * t + par;                   // this wave's step of the stage
      if (j < ksteps) {
        const int sw = (int)(gv_table_word(wtab, i, j) >> (8 * q));
        const int sx = (int)(gv_table_word(xtab, xi, j) >> (8 * q));
        acc = mfma_act<0, SPLIT>(gv_frag(st.w[par], i, 0, q), gv_frag(st.x[par], xi, 0, q), acc, sw, sx);
        acc = mfma_act<2, SPLIT>(gv_frag(st.w[par], i, 1, q), gv_frag(st.x[par], xi, 1, q), acc, sw, sx);
      }
    }
  };
  static_for<C::XI + 1>([&](auto n_tag) {
    constexpr int n = decltype(n_tag)::value;
    if (nx == n) loop(std::integral_constant<int, (1 + n) * SS>{});
  });

  // the partial tiles of each token tile, added in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(&ring[0]);  // 16 KB of the ring, no longer read
  static_assert(sizeof(ring) >= 4 * 16 * 64 * 4, "reduction buffer fits the ring");
  if (par > 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) red[(wave * 16 + e) * 64 + lane] = acc[e];
  }
  __syncthreads();
  if (par == 0) {
    for (int w = 1; w < SS; ++w)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += red[((wave + w) * 16 + e) * 64 + lane];
    const int64_t m = 32 * tt + i;
    store_tile<OUT>(p, acc, m, m < p.M, n_row0, q);
  }
}

// BF16 activations, at most 16 tokens, K of 32 or 64 steps: the whole-K kernel with
// the activations quantized in its load path instead of by a separate launch.
// Each thread owns BPT 32-element blocks of a stage's activation slot (step h,
// token row r, block b), loads their BF16 bytes into registers two stages ahead,
// and quantizes them by the quantizer's rule into the slot (codes) and the scale
// table (scale bytes) -- the same bytes the standalone quantizer writes, so the
// result is the one pre-quantized activations give.  The stage count is a
// compile-time constant: every register set, load and wait below is static.
template <int OUT, int XG, int NST, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void whole_k_xb_kernel(GemmArgs p, int G, int n_tiles) {
  using C = GvCfg<XG>;
  static_assert(XG <= 2, "at most 16 tokens");
  constexpr int NS = kXbStages, SS = C::SS, XR = C::XR;
  static_assert(NS >= 3, "weights of stage t+NS-1 go into the slot stage t-1 freed");
  constexpr int KSTEPS = SS * NST;
  static_assert(KSTEPS <= kGvMaxSteps, "scale tables hold kGvMaxSteps steps");
  constexpr int BLK = SS * XR * 4;                 // activation blocks per stage
  constexpr int BPT = BLK >= kThreads ? BLK / kThreads : 1;
  static_assert((BLK % kThreads == 0 || BLK < kThreads) && BLK % 64 == 0, "whole blocks per thread and wave");
  __shared__ __attribute__((aligned(1024))) GvStage<XG> ring[NS];
  __shared__ __attribute__((aligned(1024))) uint32_t wtab[32 * kGvMaxSteps];
  __shared__ __attribute__((aligned(1024))) uint32_t xtab[XR * kGvMaxSteps];

  const int total = G * n_tiles;
  const int wi = xcd_work_index((int)blockIdx.x, total);
  const int g = wi / n_tiles, nt = wi % n_tiles;
  const int tid = threadIdx.x, lane = tid & 63, i = lane & 31, q = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int par = wave % SS;                       // this wave's step of each stage

  const int64_t n_row0 = (int64_t)g * p.N + (int64_t)nt * 32;
  const int64_t m_rows = p.M < XR ? p.M : XR;
  const int ldw = KSTEPS * 128, ldx2 = (int)p.ld_x * 2;
  const int xcol0b = g * KSTEPS * 256;             // first BF16 byte of the group's columns
  const Rsrc rw = make_rsrc_sgpr(p.w + n_row0 * ldw, (int64_t)32 * ldw);
  const Rsrc rws = make_rsrc_sgpr(p.w_sf + n_row0 * KSTEPS, (int64_t)32 * KSTEPS * 4);
  // BF16 rows: the row part of the offset is in the per-lane register, so rows past M read as zeros
  const Rsrc rx = make_rsrc_sgpr(p.x, m_rows * ldx2);
  const Rsrc rnull = make_rsrc_sgpr(p.w, 0);
  const int lr = lane >> 3, lc = lane & 7;
  const int vw = (8 * wave + lr) * ldw + (lc ^ g8(8 * wave + lr)) * 16;

#pragma unroll
  for (int n = wave; n < 8; n += 4) {
    const int tr = 4 * n + (lane >> 4), ch = (lane & 15) ^ (tr & 15);
    dl_load16(rws, wtab + n * 256, tr * KSTEPS * 4 + ch * 16, 0);
  }

  // this thread's blocks: index tid + kThreads u -> step h, token row r, block b of the stage
  int bh[BPT], br[BPT], bb[BPT], vxo[BPT];
  bool has[BPT];
#pragma unroll
  for (int u = 0; u < BPT; ++u) {
    const int bi = tid + kThreads * u;
    has[u] = 64 * wave + kThreads * u < BLK;        // BLK is a multiple of 64: uniform per wave
    bh[u] = (bi / (XR * 4)) % SS;
    br[u] = (bi % (XR * 4)) / 4;
    bb[u] = bi % 4;
    // per-lane part (range-checked): row, then step and block within the stage's 4 x 256 bytes
    // of the row -- at most 1 KB past the row start, less than a row stride (ld_x >= 4096)
    vxo[u] = br[u] * ldx2 + bh[u] * 256 + bb[u] * 64;
  }
  struct XRegs { v4i v[4 * BPT]; };
  auto load_x = [&](XRegs& X, int t) {
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const bool on = has[u] && t < NST;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        X.v[4 * u + c] = buf_load16(on ? rx : rnull, vxo[u] + 16 * c, xcol0b + SS * t * 256);
    }
  };
  auto quantize_x = [&](XRegs& X, int t) {
    GvStage<XG>& st = ring[t % NS];
    uint8_t* xt = reinterpret_cast<uint8_t*>(xtab);
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      if (!has[u]) continue;
      uint32_t w[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        w[4 * c] = (uint32_t)X.v[4 * u + c].x;
        w[4 * c + 1] = (uint32_t)X.v[4 * u + c].y;
        w[4 * c + 2] = (uint32_t)X.v[4 * u + c].z;
        w[4 * c + 3] = (uint32_t)X.v[4 * u + c].w;
      }
      uint32_t am = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) am = amax_pair(am, w[k]);
      const int e = scale_exp_from_amax(fold_pair(am));
      const float sc = exp2_int(e);
      uint32_t cd[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) cd[k] = encode4(w[2 * k], w[2 * k + 1], sc);
      const int r = br[u], b = bb[u], gr = g8(r);
      uint8_t* slot = st.x[bh[u]];
      *reinterpret_cast<uint4*>(slot + 16 * (8 * r + ((2 * b) ^ gr))) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
      *reinterpret_cast<uint4*>(slot + 16 * (8 * r + ((2 * b + 1) ^ gr))) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
      const int j = SS * t + bh[u];
      xt[4 * (r * kGvMaxSteps + (((j >> 2) ^ (r & 15)) << 2) + (j & 3)) + b] = (uint8_t)(e + 127);
    }
  };
  // weights of stage t (one 1 KB load per wave and step), switched off past the last stage
  auto issue_w = [&](int t) {
    GvStage<XG>& st = ring[t % NS];
    const bool on = t < NST;
#pragma unroll
    for (int h = 0; h < SS; ++h) dl_load16(on ? rw : rnull, st.w[h] + wave * 1024, vw, (SS * t + h) * 128);
  };

  const int xi = i & (XR - 1);                     // the token row this lane reads
  v16f acc = zero16();
  XRegs A, B;
  load_x(A, 0);
  load_x(B, 1);
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) issue_w(t);
  wait_vmcnt<0>();
#pragma unroll
  for (int u = 0; u < 4 * BPT; ++u) {
    tie_after_wait(A.v[u]);
    tie_after_wait(B.v[u]);
  }
  quantize_x(A, 0);
  quantize_x(B, 1);
  load_x(A, 2);
  load_x(B, 3);
  // iteration t: the weights of stage t (issued NS-1 iterations earlier) and the
  // registers of stage t+2 (set t % 2) are complete once only the previous
  // iteration's batch (SS weight loads, and 4 BPT activation loads while stage t+3
  // exists) is in flight.  Both writes of stage t+2 and the weights of stage
  // t+NS-1 go into slots that stage t-1 or earlier freed.  Activation loads past the last stage are not
  // issued at all: a load whose registers the compiler takes as dead would still
  // write them when it returns.
  static_for<NST>([&](auto t_tag) {
    constexpr int t = decltype(t_tag)::value;
    XRegs& X = (t % 2 == 0) ? A : B;
    if constexpr (t == 0) wait_vmcnt<4 * BPT>();
    else wait_vmcnt<SS + (t + 3 < NST ? 4 * BPT : 0)>();
#pragma unroll
    for (int u = 0; u < 4 * BPT; ++u) tie_after_wait(X.v[u]);
    lds_barrier();                                  // stage t landed and quantized everywhere; t-1 is free
    if constexpr (t + 2 < NST) quantize_x(X, t + 2);
    issue_w(t + NS - 1);
    if constexpr (t + 4 < NST) load_x(X, t + 4);
    const GvStage<XG>& st = ring[t % NS];
    const int j = SS * t + par;
    const int sw = (int)(gv_table_word(wtab, i, j) >> (8 * q));
    const int sx = (int)(gv_table_word(xtab, xi, j) >> (8 * q));
    acc = mfma_act<0, SPLIT>(gv_frag(st.w[par], i, 0, q), gv_frag(st.x[par], xi, 0, q), acc, sw, sx);
    acc = mfma_act<2, SPLIT>(gv_frag(st.w[par], i, 1, q), gv_frag(st.x[par], xi, 1, q), acc, sw, sx);
  });
  wait_vmcnt<0>();                                  // the switched-off weight loads of the last iterations

  // the partial tiles of the four waves, added in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(&ring[0]);
  static_assert(sizeof(ring) >= 4 * 16 * 64 * 4, "reduction buffer fits the ring");
  if (par > 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) red[(wave * 16 + e) * 64 + lane] = acc[e];
  }
  __syncthreads();
  if (par == 0) {
    for (int w = 1; w < SS; ++w)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += red[((wave + w) * 16 + e) * 64 + lane];
    const int64_t m = i;
    store_tile<OUT>(p, acc, m, m < p.M, n_row0, q);
  }
}

template <int OUT, int XG, bool SPLIT>
static hipError_t launch_whole_k_xb(const GemmArgs& p, const GemmPlan& plan, int64_t G, hipStream_t stream) {
  const dim3 grid((unsigned)plan.workgroups), block(kThreads);
  if (p.K == 32 * 128)
    hipLaunchKernelGGL((whole_k_xb_kernel<OUT, XG, 32 / GvCfg<XG>::SS, SPLIT>), grid, block, 0, stream, p, (int)G,
                       plan.n_tiles);
  else if (p.K == 64 * 128)
    hipLaunchKernelGGL((whole_k_xb_kernel<OUT, XG, 64 / GvCfg<XG>::SS, SPLIT>), grid, block, 0, stream, p, (int)G,
                       plan.n_tiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int OUT, bool SPLIT>
static hipError_t launch_whole_k_bf16(const GemmArgs& p, const GemmPlan& plan, int64_t G, hipStream_t stream) {
  if (p.M <= 8) return launch_whole_k_xb<OUT, 1, SPLIT>(p, plan, G, stream);
  if (p.M <= 16) return launch_whole_k_xb<OUT, 2, SPLIT>(p, plan, G, stream);
  return hipErrorInvalidValue;
}

template <int OUT, int XG, bool SPLIT>
static hipError_t launch_whole_k_xg(const GemmArgs& p, const GemmPlan& plan, int64_t G, hipStream_t stream) {
  // Ring depth: with up to 32 tokens on a grid that holds every CU, three stages (two in flight)
  // instead of four.  Measured, alternated on one box: einsum 8 x 4096 -> 1024 (256 workgroups) at
  // 8 / 20 / 32 tokens 9.18 / 9.27 / 9.55 -> 8.55 / 8.89 / 9.21 us; wo_b 8192 -> 5120 (160 workgroups)
  // 10.95 / 12.1 -> 11.44 / 12.35 us with three, so smaller grids keep four.
  if (XG <= 4 && plan.workgroups >= kWholeKShallowMinWorkgroups)
    hipLaunchKernelGGL((whole_k_kernel<OUT, XG, 3, SPLIT>), dim3((unsigned)plan.workgroups), dim3(kThreads), 0,
                       stream, p, (int)G, plan.n_tiles);
  else
    hipLaunchKernelGGL((whole_k_kernel<OUT, XG, kGvStages, SPLIT>), dim3((unsigned)plan.workgroups), dim3(kThreads),
                       0, stream, p, (int)G, plan.n_tiles);
  return hipGetLastError();
}

template <int OUT, bool SPLIT>
static hipError_t launch_whole_k(const GemmArgs& p, const GemmPlan& plan, int64_t G, hipStream_t stream) {
  if (p.M <= 8) return launch_whole_k_xg<OUT, 1, SPLIT>(p, plan, G, stream);
  if (p.M <= 16) return launch_whole_k_xg<OUT, 2, SPLIT>(p, plan, G, stream);
  if (p.M <= 32) return launch_whole_k_xg<OUT, 4, SPLIT>(p, plan, G, stream);
  if (p.M <= 64) return launch_whole_k_xg<OUT, 8, SPLIT>(p, plan, G, stream);
  if (p.M <= 128) return launch_whole_k_xg<OUT, 16, SPLIT>(p, plan, G, stream);
  return hipErrorInvalidValue;
}

template <int MT, int OUT, bool XB, bool SPLIT>
static hipError_t launch_stream(const GemmArgs& p, const GemmPlan& plan, int64_t G, hipStream_t stream) {
  hipLaunchKernelGGL((stream_kernel<MT, OUT, XB, SPLIT>), dim3((unsigned)plan.workgroups), dim3(kThreads), 0, stream,
                     p, (int)G, plan.n_tiles, plan.chunks, plan.splits);
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const GemmArgs& p, const GemmPlan& plan, int64_t G, bool x_bf16, int out,
                              hipStream_t stream) {
  return with_variant(p.split_act, out, [&](auto out_tag, auto split_tag) -> hipError_t {
    constexpr int OUT = decltype(out_tag)::value;
    constexpr bool SPLIT = decltype(split_tag)::value;
    if (plan.whole_k) {
      if (x_bf16) {
        if (!plan.whole_k_bf16) return hipErrorInvalidValue;   // the caller quantizes into the workspace first
        return launch_whole_k_bf16<OUT, SPLIT>(p, plan, G, stream);
      }
      return launch_whole_k<OUT, SPLIT>(p, plan, G, stream);
    }
    if (plan.mt == 1) {
      return x_bf16 ? launch_stream<1, OUT, true, SPLIT>(p, plan, G, stream)
                    : launch_stream<1, OUT, false, SPLIT>(p, plan, G, stream);
    }
    return x_bf16 ? launch_stream<2, OUT, true, SPLIT>(p, plan, G, stream)
                  : launch_stream<2, OUT, false, SPLIT>(p, plan, G, stream);
  });
}

}  // namespace mx
