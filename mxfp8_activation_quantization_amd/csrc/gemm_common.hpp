// Pieces shared by the GEMM kernels: the scaled MFMA, fragment assembly, and the
// output epilogue of one 32 x 32 accumulator tile.
//
// gfx950 lane layout of V_MFMA_SCALE_F32_32X32X64_F8F6F4 (checked on the device):
//   operands: lane l = i + 32q holds row i, K bytes [16q, 16q+16) in dwords 0-3
//             and [32+16q, 32+16q+16) in dwords 4-7 of a 64-deep K step, so
//             bytes 0-15 of every lane belong to the step's first 32-block and
//             bytes 16-31 to its second;
//   scales:   the scale of (row i, 32-block b) is byte `opsel` of lane i + 32b;
//   result:   lane l holds column l % 32, rows 8*(r/4) + 4*(l/32) + r%4, r < 16.
// With the packed word of a row's four 128-K blocks shifted right by 8q, opsel 0
// serves the first 64-deep half of a 128-K step and opsel 2 the second.
//
// The weights are always the A operand (rows = output columns n) and the
// activations the B operand (columns = tokens m): a lane's 16 results then lie in
// one 32-wide block of n for one token, shared with the partner lane l ^ 32.
#pragma once

#include <type_traits>

#include "launch.hpp"
#include "mx_device.hpp"

namespace mx {

constexpr int kThreads = 256;  // four waves per workgroup

enum OutMode { OUT_BF16 = 1, OUT_MX = 2, OUT_BOTH = 3 };

template <int OPSEL>
__device__ __forceinline__ v16f mfma_scaled(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, sa, OPSEL, sb);
}

// Accumulation precision of the scaled FP8 MFMA (measured on gfx950, and reproduced bit for bit by an
// emulation of the instruction on the o_proj einsum's data): the 64 products of one instruction are
// summed in groups of 8 consecutive K; within a group every product is cut toward zero to a multiple
// of 2^(E - 13), E being the largest sum of the two operands' exponents in the group, and the group sums
// and the fp32 accumulator are then added without further loss.  An activation value a hundred times
// its neighbours (the 0.1% x100 entries of the attention output) therefore takes six or seven bits off
// each of the seven products it shares a group with, and the einsum's BF16 z then differs from the
// correctly rounded value in about 2.6% of its elements (0.24% of the E4M3 codes).  The einsum hands
// the instruction its activation fragment as two operands instead -- the codes of magnitude >= 64
// (0x68: within a factor of seven of the block maximum, which lies in (224, 448]) and the rest -- into
// the same accumulator, so that no group mixes a large code with small ones: 0.24% of z's BF16 values
// and 0.017% of its codes differ from the correctly rounded ones (emulated on the decode configuration),
// and the chain's output error falls to that of rounding the exact result to BF16.
constexpr uint32_t kSplitBias = 0x80u - 0x68u;   // per byte: (|code| + bias) has bit 7 set iff |code| >= 0x68

// Dword D of a fragment: its codes of magnitude >= 0x68 into hi (others zero), the rest stay in lo.
template <int D>
__device__ __forceinline__ void split_large_dword(v8i& lo, v8i& hi) {
  const uint32_t u = (uint32_t)lo[D];
  // bit 7 of each byte of t: |code| >= 0x68 ((0x80 | c) - 0x68 borrows from no other byte)
  const uint32_t t = (u | 0x80808080u) - (0x80u - kSplitBias) * 0x01010101u;
  // v_perm_b32 selectors 8-11 give 0xFF or 0x00 from bit 7 of bytes 1, 3, 5, 7 of {src0, src1}:
  // with src1 = t and src0 = t << 8 those are t's bytes 1, 3, 0, 2
  const uint32_t mask = __builtin_amdgcn_perm(t << 8, t, 0x090B080Au);
  hi[D] = (int)(u & mask);
  lo[D] = (int)(u ^ (u & mask));
}

// The codes of magnitude >= 0x68 of a fragment (others zero) and the remaining codes (those zero).
__device__ __forceinline__ void split_large_codes(v8i& lo, v8i& hi) {
  split_large_dword<0>(lo, hi); split_large_dword<1>(lo, hi); split_large_dword<2>(lo, hi);
  split_large_dword<3>(lo, hi); split_large_dword<4>(lo, hi); split_large_dword<5>(lo, hi);
  split_large_dword<6>(lo, hi); split_large_dword<7>(lo, hi);
}

// acc + W . X with the activation operand X split as above when SPLIT (the small codes first, then the
// large ones, both into the same accumulator).
template <int OPSEL, bool SPLIT>
__device__ __forceinline__ v16f mfma_act(const v8i& w, const v8i& x, const v16f& c, int sw, int sx) {
  if constexpr (!SPLIT) {
    return mfma_scaled<OPSEL>(w, x, c, sw, sx);
  } else {
    v8i lo = x, hi;
    split_large_codes(lo, hi);
    const v16f t = mfma_scaled<OPSEL>(w, lo, c, sw, sx);
    return mfma_scaled<OPSEL>(w, hi, t, sw, sx);
  }
}

__device__ __forceinline__ v8i frag(const uint4& lo, const uint4& hi) {
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

__device__ __forceinline__ v16f zero16() {
  v16f z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Stores one 32 (n) x 32 (m) accumulator tile: lane (i, q) holds token m and the
// 16 columns nb + 8*(r/4) + 4q + r%4.  Every fp32 sum is rounded to BF16 (nearest
// even); the MXFP8 form quantizes those BF16 values, block by 32 columns, with the
// same rule as mxfp8_quantize.  All lanes must call this (it shuffles); `live`
// gates the stores of tokens beyond M.
template <int OUT>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const v16f& acc, int64_t m, bool live, int64_t nb,
                                           int q) {
  uint32_t h2[8];                                    // BF16 pairs (r, r + 1), r even
#pragma unroll
  for (int r = 0; r < 16; r += 2) h2[r / 2] = bf16x2_rne(acc[r], acc[r + 1]);
  if constexpr (OUT & OUT_BF16) {
    if (live) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        *reinterpret_cast<uint2*>(p.zb + m * p.ld_zb + nb + 8 * r4 + 4 * q) = make_uint2(h2[2 * r4], h2[2 * r4 + 1]);
      }
    }
  }
  if constexpr (OUT & OUT_MX) {
    uint32_t am2 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) am2 = amax_pair(am2, h2[k]);
    uint32_t am = fold_pair(am2);
    am = max(am, (uint32_t)__shfl_xor((int)am, 32));
    const int e = scale_exp_from_amax(am);
    const float scale = exp2_int(e);
    if (live) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const uint32_t c = encode4(h2[2 * r4], h2[2 * r4 + 1], scale);
        *reinterpret_cast<uint32_t*>(p.zq + m * p.ld_zq + nb + 8 * r4 + 4 * q) = c;
      }
      if (q == 0) p.zsf[m * p.ld_zsf_bytes + nb / 32] = (uint8_t)(e + 127);
    }
  }
}

// Epilogue through LDS.  store_tile() above writes straight from the MFMA
// layout, where a lane holds 16 columns of one token scattered over the tile: each
// store instruction then touches 32 token rows with 8 (BF16) or 4 (E4M3) bytes
// each.  Large tiles instead pass a wave's TN x 32 columns of 32 tokens through
// LDS as BF16, token-major, and read them back along token rows, so that every
// store writes 16 contiguous bytes per lane and whole 128-byte row segments per
// group of lanes.  The arithmetic is the same as store_tile's (BF16 rounding,
// block amax of the rounded values, scale exponent, encoding), so both give the
// same bits.
//
// Row stride in LDS: TN * 64 bytes of BF16 plus 16 bytes of padding, which keeps
// the 16-byte row reads aligned and spreads the 32 token rows of a write over
// the banks.
template <int TN>
struct EpiLds {
  static constexpr int RS = TN * 64 + 16;
  static constexpr int BYTES = 32 * RS;
};

// Tile a (columns 32a .. 32a+31) of the wave's row block: lane (i, q) holds
// token i, columns 8 r4 + 4 q + (0..3) for r4 = 0..3.
template <int TN>
__device__ __forceinline__ void epi_write_tile(uint8_t* chunk, const v16f& acc, int a, int i, int q) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const uint2 v = make_uint2(bf16x2_rne(acc[4 * r4], acc[4 * r4 + 1]), bf16x2_rne(acc[4 * r4 + 2], acc[4 * r4 + 3]));
    *reinterpret_cast<uint2*>(chunk + i * EpiLds<TN>::RS + (a * 32 + 8 * r4 + 4 * q) * 2) = v;
  }
}

// Stores the 32 tokens m_base .. m_base+31 (those below M) x TN * 32 columns from
// column nb of the output row.  Call after every lane's epi_write_tile of the
// block and a wait for those LDS writes.
template <int OUT, int TN>
__device__ __forceinline__ void epi_store_rows(const GemmArgs& p, const uint8_t* chunk, int64_t m_base, int64_t nb,
                                               int lane) {
  constexpr int RS = EpiLds<TN>::RS;
  static_assert(TN == 1 || TN == 2 || TN == 4 || TN == 8, "lane split of a row");
  if constexpr (OUT & OUT_BF16) {
    constexpr int LPR = 4 * TN, RPP = 64 / LPR;      // lanes per row (8 columns each), rows per pass
#pragma unroll
    for (int pass = 0; pass < 32 / RPP; ++pass) {
      const int row = lane / LPR + pass * RPP, c8 = lane % LPR;
      const uint4 v = *reinterpret_cast<const uint4*>(chunk + row * RS + c8 * 16);
      const int64_t m = m_base + row;
      if (m < p.M) *reinterpret_cast<uint4*>(p.zb + m * p.ld_zb + nb + c8 * 8) = v;
      __builtin_amdgcn_sched_barrier(0);            // one pass at a time: bounds the registers
    }
  }
  if constexpr (OUT & OUT_MX) {
    constexpr int RPP = 64 / TN;                       // one lane per 32-column block
#pragma unroll
    for (int pass = 0; pass < 32 / RPP; ++pass) {
      const int row = lane / TN + pass * RPP, blk = lane % TN;
      const uint4* src = reinterpret_cast<const uint4*>(chunk + row * RS + blk * 64);
      uint32_t w[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 v = src[k];
        w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
      }
      uint32_t am = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) am = max(am, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
      const int e = scale_exp_from_amax(am);
      const float scale = exp2_int(e);
      uint32_t c[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) c[k] = encode4(w[2 * k], w[2 * k + 1], scale);
      const int64_t m = m_base + row;
      if (m < p.M) {
        uint8_t* dst = p.zq + m * p.ld_zq + nb + blk * 32;
        *reinterpret_cast<uint4*>(dst) = make_uint4(c[0], c[1], c[2], c[3]);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(c[4], c[5], c[6], c[7]);
        p.zsf[m * p.ld_zsf_bytes + nb / 32 + blk] = (uint8_t)(e + 127);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr uint32_t kRawBufferFlags = 0x00020000;   // raw buffer, 32-bit dwords, range-checked

// Direct-to-LDS loads are written as inline assembly on purpose: the compiler
// tracks its own LDS-DMA builtins conservatively and would wait for every one in
// flight before each LDS read, which would undo the pipeline.  The kernel does
// its own counting (s_waitcnt vmcnt) and its own barriers.  The buffer resource
// is built by hand: base address, stride 0, byte range, raw-buffer flags.
struct Rsrc {
  v4i v;
};

__device__ __forceinline__ Rsrc make_rsrc_sgpr(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  Rsrc r;
  r.v = v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, (int)kRawBufferFlags};
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// 64 lanes x 16 bytes from rsrc + voff + soff into LDS [lds, lds + 1024), lane l at lds + 16 l.
__device__ __forceinline__ void dl_load16(const Rsrc& r, const void* lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr(lds)), "v"(voff), "s"(r.v), "s"(soff) : "memory");
}

// 64 lanes x 4 bytes, lane l at lds + 4 l.
__device__ __forceinline__ void dl_load4(const Rsrc& r, const void* lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_addr(lds)), "v"(voff), "s"(r.v), "s"(soff) : "memory");
}

// Indexed forms of the LDS-DMA loads for unrolled load sequences: per-lane offset
// voff + I * vstep (+ vadd), LDS destination lds_base + LDSOFF, with every sum
// formed inside the same inline assembly, so that none of the per-instruction
// values is kept in a register across a loop (a tile's dozens of destinations
// and row offsets would otherwise be hoisted and spill).  The whole offset is
// per-lane, so the buffer range check covers it.  The scalar adds write SCC,
// which the clobber list declares.
template <int I, int LDSOFF>
__device__ __forceinline__ void dl_load16_idx(const Rsrc& r, int lds_base, int voff, int vstep, int soff) {
  int t, st;
  asm volatile("s_mul_i32 %1, %3, %4\n\t"
               "v_add_u32 %0, %1, %2\n\t"
               "s_add_u32 m0, %5, %6\n\t"
               "s_nop 0\n\t"
               "buffer_load_dwordx4 %0, %7, %8 offen lds"
               : "=&v"(t), "=&s"(st)
               : "v"(voff), "s"(vstep), "i"(I), "s"(lds_base), "i"(LDSOFF), "s"(r.v), "s"(soff)
               : "memory", "scc");
}

template <int I, int LDSOFF>
__device__ __forceinline__ void dl_load4_idx(const Rsrc& r, int lds_base, int voff, int vstep, int vadd) {
  int t, st;
  asm volatile("s_mul_i32 %1, %3, %4\n\t"
               "s_add_u32 %1, %1, %5\n\t"
               "v_add_u32 %0, %1, %2\n\t"
               "s_add_u32 m0, %6, %7\n\t"
               "s_nop 0\n\t"
               "buffer_load_dword %0, %8, 0 offen lds"
               : "=&v"(t), "=&s"(st)
               : "v"(voff), "s"(vstep), "i"(I), "s"(vadd), "s"(lds_base), "i"(LDSOFF), "s"(r.v)
               : "memory", "scc");
}

// 16 bytes per lane from memory into registers.  Inline assembly like the LDS-DMA
// loads above, for the same reason: the caller counts its loads (s_waitcnt
// vmcnt) and ties the result registers to its own wait (`tie_after_wait`); the
// compiler's own counting would not see the LDS-DMA loads in flight.
__device__ __forceinline__ v4i buf_load16(const Rsrc& r, int voff, int soff) {
  v4i v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(v) : "v"(voff), "s"(r.v), "s"(soff) : "memory");
  return v;
}

// Declares a register written by an asm load valid from here on (place it after
// the s_waitcnt that covers the load): the compiler may not move a use above it.
__device__ __forceinline__ void tie_after_wait(v4i& v) { asm volatile("" : "+v"(v)); }

// LDS reads with a constant offset (inline assembly: see the direct-to-LDS GEMM).
// The result is not valid until a later s_waitcnt lgkmcnt(0) that the caller
// ties to the result registers.
template <int OFF>
__device__ __forceinline__ v4i lds_read16(int addr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS instruction offsets are 16 bits");
  v4i v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

// As lds_read16, at address (addr ^ XOR) + OFF: the XOR is part of the same
// inline assembly, so it is computed where the read is issued and holds no
// register across a loop.
template <int OFF, int XOR>
__device__ __forceinline__ v4i lds_read16_xor(int addr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS instruction offsets are 16 bits");
  if constexpr (XOR == 0) {
    return lds_read16<OFF>(addr);
  } else {
    v4i v;
    int t;
    asm volatile("v_xor_b32 %1, %3, %2\n\tds_read_b128 %0, %1 offset:%4"
                 : "=v"(v), "=&v"(t) : "v"(addr), "i"(XOR), "i"(OFF));
    return v;
  }
}

template <int OFF>
__device__ __forceinline__ int lds_read4(int addr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS instruction offsets are 16 bits");
  int v;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

__device__ __forceinline__ v8i join8(const v4i& lo, const v4i& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// s_waitcnt vmcnt(N) for a compile-time N.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS exchange inside software pipelines: waits for this
// wave's LDS operations only, then s_barrier.  __syncthreads() would also wait
// for every global load still in flight (its release fence covers all memory),
// which would collapse a multi-stage prefetch to a single stage.  The asm is a
// compiler memory fence as well, so no LDS access moves across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Maps a flat workgroup id to a work index so that each XCD (workgroups are
// dispatched round-robin over the 8 XCDs) receives one contiguous range of work:
// neighbouring tiles, which share activation rows, then share one L2.
__device__ __forceinline__ int xcd_work_index(int id, int total) {
  if (total % 8 != 0) return id;
  return (id % 8) * (total / 8) + id / 8;
}

// Calls f(std::integral_constant<int, OUT>, std::integral_constant<bool, SPLIT>) for the output form and
// the activation split of a launch.  Only the forms the entry points use exist: fp8_gemm_nt (BF16 out, no
// split) and grouped_fp8_einsum (any output, split).
template <class F>
hipError_t with_variant(bool split, int out, F&& f) {
  using std::integral_constant;
  if (!split) {
    if (out != OUT_BF16) return hipErrorInvalidValue;
    return f(integral_constant<int, OUT_BF16>{}, integral_constant<bool, false>{});
  }
  if (out == OUT_BF16) return f(integral_constant<int, OUT_BF16>{}, integral_constant<bool, true>{});
  if (out == OUT_MX) return f(integral_constant<int, OUT_MX>{}, integral_constant<bool, true>{});
  return f(integral_constant<int, OUT_BOTH>{}, integral_constant<bool, true>{});
}

hipError_t launch_gemm_tiled(const GemmArgs& p, const GemmPlan& plan, int64_t G, int out, hipStream_t stream);
hipError_t launch_gemm_skinny(const GemmArgs& p, const GemmPlan& plan, int64_t G, bool x_bf16, int out,
                              hipStream_t stream);

}  // namespace mx
