// Block-scaled FP8 GEMM for few tokens (decode): split-K weight streaming.
//
// With at most a few hundred tokens the o_proj chain is bound by reading its
// weights from HBM once (vLLM PR #60118 "[Perf][DSv4.1] MegaAttn: wo_a writes
// wo_b's MXFP8 input", Claims: the decode range is 1-256 tokens).  HBM only
// streams near its peak when every CU keeps many reads in flight, so the work is
// cut finely: a workgroup owns 64 weight rows (two MFMA row tiles), the tokens of
// one chunk (32 or 64) and one 1024-deep K slice; wo_a at 64 tokens becomes 512
// workgroups and wo_b 640.
//
// Inside a workgroup:
//   1. each wave issues all loads of its weight fragments at once (4 K-steps of
//      its 32 rows, straight into registers in the MFMA lane layout);
//   2. all threads stage the activation slice (tokens x 1024) in LDS with
//      coalesced 16-byte loads, quantizing BF16 input per 32-block on the way
//      (four lanes per block, one amax shuffle pair, the standalone quantizer's
//      rule), so both row tiles read it from LDS;
//   3. wave (row tile rt, K half kh) runs 4 K-steps of scaled MFMAs;
//   4. the two K halves are added through LDS (kh 0 + kh 1).
// With one K slice the workgroup runs the epilogue itself.  Otherwise it writes
// its fp32 partial tile to the caller's workspace, and the last workgroup of the
// tile to arrive (an atomic counter) adds the slices in slice order 0, 1, ...,
// S-1 and runs the epilogue: the result does not depend on arrival order.  The
// counter is reset to zero for the next call.
#include "gemm_common.hpp"

namespace mx {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSplitSteps = 8;   // 128-K steps per K slice
constexpr int kHalfSteps = 4;    // steps per wave (two waves per row tile)

__device__ __forceinline__ int sswz(int row, int chunk) { return (row * 8 + (chunk ^ (row & 7))) * 16; }

template <int MT, bool X_BF16, int OUT>
__global__ __launch_bounds__(kThreads) void splitk_kernel(GemmArgs p, int G, int n_tiles, int chunks, int S) {
  constexpr int ROWS = 32 * MT;                          // token rows of the chunk
  constexpr int STEP_BYTES = ROWS * 128;
  __shared__ __attribute__((aligned(16))) uint8_t sx[kSplitSteps * STEP_BYTES];
  __shared__ uint32_t sxs[kSplitSteps][ROWS];
  __shared__ int s_last;

  const int total = G * n_tiles * chunks * S;
  const int wi = xcd_work_index((int)blockIdx.x, total);
  const int s = wi % S;
  const int rest = wi / S;
  const int chunk = rest % chunks;
  const int tile = rest / chunks;
  const int g = tile / n_tiles, nt = tile % n_tiles;
  const int tc = tile * chunks + chunk;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 31, q = lane >> 5;
  const int rt = wave & 1, kh = wave >> 1;
  const int64_t ksteps = p.K / 128;
  const int64_t kt0 = (int64_t)s * kSplitSteps;

  // 1. this wave's weight fragments: rows of row tile rt, steps kt0 + 4 kh + j
  const int64_t n_row = (int64_t)g * p.N + (int64_t)nt * 64 + rt * 32 + i;
  const uint8_t* wp = p.w + n_row * p.K + 16 * q;
  const int32_t* wsfp = p.w_sf + n_row * ksteps;
  uint4 wv[kHalfSteps][4];
  uint32_t wsw[kHalfSteps];
#pragma unroll
  for (int j = 0; j < kHalfSteps; ++j) {
    const int64_t kt = kt0 + kHalfSteps * kh + j;
    const int64_t kc = kt < ksteps ? kt : ksteps - 1;     // steps past K: loaded from a valid address, zeroed below
#pragma unroll
    for (int c = 0; c < 4; ++c) wv[j][c] = *reinterpret_cast<const uint4*>(wp + kc * 128 + 32 * c);
    wsw[j] = (uint32_t)wsfp[kc];
  }

  // 2. activation slice -> LDS (E4M3 codes, swizzled 128-byte rows per step, packed scale words)
  const int64_t m_first = (int64_t)chunk * ROWS;
  if constexpr (!X_BF16) {
    const uint8_t* xq = static_cast<const uint8_t*>(p.x);
#pragma unroll 4
    for (int c = tid; c < kSplitSteps * ROWS * 8; c += kThreads) {
      const int j = c / (ROWS * 8), rem = c % (ROWS * 8), row = rem >> 3, ch = rem & 7;
      const int64_t m = m_first + row < p.M ? m_first + row : p.M - 1;
      const int64_t kt = kt0 + j;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kt < ksteps) v = *reinterpret_cast<const uint4*>(xq + m * p.ld_x + (int64_t)g * p.K + kt * 128 + ch * 16);
      *reinterpret_cast<uint4*>(sx + j * STEP_BYTES + sswz(row, ch)) = v;
    }
    for (int c = tid; c < kSplitSteps * ROWS; c += kThreads) {
      const int j = c / ROWS, row = c % ROWS;
      const int64_t m = m_first + row < p.M ? m_first + row : p.M - 1;
      const int64_t kt = kt0 + j;
      sxs[j][row] = kt < ksteps ? (uint32_t)p.x_sf[m * p.ld_xsf + (int64_t)g * ksteps + kt] : 0u;
    }
  } else {
    // BF16: 256 bytes per row and step = 16 lanes x 16 bytes; lanes 4b..4b+3 own 32-block b
    const uint16_t* xb = static_cast<const uint16_t*>(p.x);
#pragma unroll 4
    for (int c = tid; c < kSplitSteps * ROWS * 16; c += kThreads) {
      const int j = c / (ROWS * 16), rem = c % (ROWS * 16), row = rem >> 4, jj = rem & 15;
      const int b = jj >> 2, part = jj & 3;
      const int64_t m = m_first + row < p.M ? m_first + row : p.M - 1;
      const int64_t kt = kt0 + j;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kt < ksteps) v = *reinterpret_cast<const uint4*>(xb + m * p.ld_x + (int64_t)g * p.K + kt * 128 + jj * 8);
      uint32_t am = fold_pair(amax_pair(amax_pair(amax_pair(amax_pair(0u, v.x), v.y), v.z), v.w));
      am = max(am, (uint32_t)__shfl_xor((int)am, 1, 4));
      am = max(am, (uint32_t)__shfl_xor((int)am, 2, 4));
      const int e = scale_exp_from_amax(am);
      const float sc = exp2_int(e);
      const uint2 codes = make_uint2(encode4(v.x, v.y, sc), encode4(v.z, v.w, sc));
      *reinterpret_cast<uint2*>(sx + j * STEP_BYTES + sswz(row, 2 * b + (part >> 1)) + (part & 1) * 8) = codes;
      if (part == 0) reinterpret_cast<uint8_t*>(&sxs[j][row])[b] = (uint8_t)(e + 127);
    }
  }
  __syncthreads();

  // 3. scaled MFMAs over this wave's four steps
  v16f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = zero16();
#pragma unroll
  for (int jj = 0; jj < kHalfSteps; ++jj) {
    const int j = kHalfSteps * kh + jj;
    const bool valid = kt0 + j < ksteps;
    uint4 w0 = wv[jj][0], w1 = wv[jj][1], w2 = wv[jj][2], w3 = wv[jj][3];
    if (!valid) w0 = w1 = w2 = w3 = make_uint4(0, 0, 0, 0);    // exact zero contribution
    const v8i w01 = frag(w0, w1), w23 = frag(w2, w3);
    const int sw = (int)(wsw[jj] >> (8 * q));
    const uint8_t* slab = sx + j * STEP_BYTES;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int row = 32 * t + i;
      const v8i x01 = frag(*reinterpret_cast<const uint4*>(slab + sswz(row, q)),
                           *reinterpret_cast<const uint4*>(slab + sswz(row, 2 + q)));
      const v8i x23 = frag(*reinterpret_cast<const uint4*>(slab + sswz(row, 4 + q)),
                           *reinterpret_cast<const uint4*>(slab + sswz(row, 6 + q)));
      const int sxw = (int)(sxs[j][row] >> (8 * q));
      acc[t] = mfma_scaled<0>(w01, x01, acc[t], sw, sxw);
      acc[t] = mfma_scaled<2>(w23, x23, acc[t], sw, sxw);
    }
  }

  // 4. K halves: kh 0 + kh 1, through LDS (the activation slice is no longer needed)
  __syncthreads();
  float* red = reinterpret_cast<float*>(sx);           // [rt][t][16][64]
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((rt * MT + t) * 16 + r) * 64 + lane] = acc[t][r];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] += red[((rt * MT + t) * 16 + r) * 64 + lane];
  }

  const int64_t nb = (int64_t)g * p.N + (int64_t)nt * 64 + rt * 32;
  if (S == 1) {
    if (kh == 0) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int64_t m = m_first + 32 * t + i;
        store_tile<OUT>(p, acc[t], m, m < p.M, nb, q);
      }
    }
    return;
  }

  // 5. split K: publish the partial tile; the last slice to arrive reduces in slice order.
  // The slices of a tile may run on different XCDs, whose L2 caches are not
  // coherent with each other.  Partial tiles therefore move with 16-byte buffer
  // accesses that bypass L1 and L2 (sc0 sc1), and the counter with a relaxed
  // system-scope atomic: a writer waits until its stores are complete before it
  // bumps the counter, and the last workgroup reads the partials from memory.  No
  // cache-wide writeback or invalidate is needed, so other workgroups keep their
  // cached activations.  Partial layout per slice: [rt][t][lane][16 floats].
  constexpr int TILE_FLOATS = 2 * MT * 16 * 64;
  constexpr int TILE_BYTES = TILE_FLOATS * 4;
  constexpr int kUncached = 0x11;                           // sc0 | sc1
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      p.ws_partials + (int64_t)tc * S * TILE_FLOATS, 0, S * TILE_BYTES, 0x00020000);
  if (kh == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int base = s * TILE_BYTES + ((rt * MT + t) * 64 + lane) * 64;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const v4i v = {__float_as_int(acc[t][4 * k]), __float_as_int(acc[t][4 * k + 1]),
                       __float_as_int(acc[t][4 * k + 2]), __float_as_int(acc[t][4 * k + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, base + 16 * k, 0, kUncached);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&p.ws_counters[tc], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
             (uint32_t)(S - 1);
  __syncthreads();
  if (!s_last) return;

  // every thread sums its 16-byte chunks of the tile over the slices, in slice order
  constexpr int CH = TILE_BYTES / 16 / kThreads;            // chunks per thread (2 MT)
  float4 sum[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) sum[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += 4) {
    v4i ld[4][CH];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (s0 + u < S)
          ld[u][c] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (s0 + u) * TILE_BYTES + (c * kThreads + tid) * 16,
                                                           0, kUncached);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (s0 + u < S) {
          if (s0 + u == 0) {
            sum[c] = make_float4(__int_as_float(ld[u][c].x), __int_as_float(ld[u][c].y),
                                 __int_as_float(ld[u][c].z), __int_as_float(ld[u][c].w));
          } else {
            sum[c].x += __int_as_float(ld[u][c].x);
            sum[c].y += __int_as_float(ld[u][c].y);
            sum[c].z += __int_as_float(ld[u][c].z);
            sum[c].w += __int_as_float(ld[u][c].w);
          }
        }
  }
  // back to the MFMA lane layout through LDS, then the epilogue
  float4* red4 = reinterpret_cast<float4*>(sx);
#pragma unroll
  for (int c = 0; c < CH; ++c) red4[c * kThreads + tid] = sum[c];
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float* src = reinterpret_cast<const float*>(sx) + ((rt * MT + t) * 64 + lane) * 16;
      v16f tot;
#pragma unroll
      for (int r = 0; r < 16; ++r) tot[r] = src[r];
      const int64_t m = m_first + 32 * t + i;
      store_tile<OUT>(p, tot, m, m < p.M, nb, q);
    }
  }
  if (tid == 0) __hip_atomic_store(&p.ws_counters[tc], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <int MT, bool X_BF16, int OUT>
static hipError_t launch_mt(const GemmArgs& p, const GemmPlan& plan, int64_t G, hipStream_t stream) {
  hipLaunchKernelGGL((splitk_kernel<MT, X_BF16, OUT>), dim3((unsigned)plan.workgroups), dim3(kThreads), 0, stream,
                     p, (int)G, plan.n_tiles, plan.chunks, plan.splits);
  return hipGetLastError();
}

template <int MT>
static hipError_t dispatch(const GemmArgs& p, const GemmPlan& plan, int64_t G, bool x_bf16, int out,
                           hipStream_t s) {
  if (x_bf16) {
    if (out == OUT_BF16) return launch_mt<MT, true, OUT_BF16>(p, plan, G, s);
    if (out == OUT_MX) return launch_mt<MT, true, OUT_MX>(p, plan, G, s);
    return launch_mt<MT, true, OUT_BOTH>(p, plan, G, s);
  }
  if (out == OUT_BF16) return launch_mt<MT, false, OUT_BF16>(p, plan, G, s);
  if (out == OUT_MX) return launch_mt<MT, false, OUT_MX>(p, plan, G, s);
  return launch_mt<MT, false, OUT_BOTH>(p, plan, G, s);
}

hipError_t launch_gemm_skinny(const GemmArgs& p, const GemmPlan& plan, int64_t G, bool x_bf16, int out,
                              hipStream_t stream) {
  if (plan.mt == 1) return dispatch<1>(p, plan, G, x_bf16, out, stream);
  return dispatch<2>(p, plan, G, x_bf16, out, stream);
}

}  // namespace mx
