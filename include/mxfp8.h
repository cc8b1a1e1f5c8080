/*
 * mxfp8.h -- C ABI of the MXFP8 o_proj chain library for AMD Instinct MI355X (gfx950).
 *
 * The chain (vLLM PR #60118 "[Perf][DSv4.1] MegaAttn: wo_a writes wo_b's MXFP8
 * input", sections Conversation, Overview and Claims; vLLM PR #57977
 * "[Perf][DSv4.1] Keep activations MXFP8 between DeepGEMM kernels", the
 * before/after diagrams and Pieces):
 *
 *   x (BF16) --mxfp8_quantize--> (x_q, x_sf)            [optional: the einsum can take BF16 x]
 *     --grouped_fp8_einsum (wo_a, MXFP8 epilogue)--> (z_q, z_sf)
 *     --fp8_gemm_nt (wo_b, 1x32 scale blocks on both operands)--> out (BF16)
 *
 * MXFP8 format used by every entry point: one OCP FP8 E4M3FN byte per element
 * plus one UE8M0 scale byte (value 2^(byte-127)) per 32 contiguous elements of
 * a row.  Scales are packed four to an int32, K-major: word w of a row holds
 * blocks 4w..4w+3, block 4w+j in bits [8j, 8j+8) (a little-endian byte view of
 * the words is the per-block byte array).  The scale exponent of a block is the
 * smallest e with max|x| <= 448 * 2^e, clamped to [-127, 127] (an all-zero block
 * gets byte 0x00); codes are x * 2^-e rounded to nearest even with saturation.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device memory owned by the caller; the library
 *     never frees or keeps them.  Row strides (ld*) count elements (bytes for
 *     E4M3, 2-byte units for BF16, int32 words for scales).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and returns without waiting; the call never synchronizes the device.
 *   - Arguments are validated on the host before any HIP call.  Errors are
 *     returned as mxfp8_status codes; nothing is launched on error and no
 *     output is touched.  M == 0 is a valid no-op (MXFP8_OK).
 *   - Data pointers must be 16-byte aligned and data row strides a multiple of
 *     16 bytes; scale pointers must be 4-byte aligned.
 *   - GEMM size limits (32-bit tile addressing): K of a group <= 2^22, activation
 *     row strides <= 2^23 bytes (scale rows <= 2^16 bytes); otherwise
 *     MXFP8_ERR_SHAPE.
 *   - Outputs must not overlap inputs or each other (MXFP8_ERR_ALIAS).
 *   - Workspace: the GEMM entry points may need device scratch -- split-K
 *     partial sums, and, for BF16 activations that go to a kernel reading E4M3
 *     (the tile kernels: more than 128 rows on large grids, more than 256 on
 *     small ones; the whole-K kernel: 17 to 128 rows, or fewer at K depths other
 *     than 32 or 64 steps), the activations quantized to MXFP8 (the library
 *     quantizes BF16 input with mxfp8_quantize first).  The matching
 *     *_workspace_size(kind, shape) call gives the bytes (0 = none needed,
 *     pointer may be NULL).  The caller owns it, zero-fills it once before first
 *     use (256-byte aligned).  Split-K calls keep arrival counters in its first
 *     64 KiB and leave them at zero when they complete; the rest is scratch.
 *     Calls of any shape may therefore reuse one workspace one after another
 *     (same stream), but calls that run concurrently (other streams) must not
 *     share one.
 *   - No entry point allocates, frees, synchronizes or records a memset: each
 *     call is a fixed sequence of kernel launches on `stream`, so it can be
 *     captured in a HIP graph.  A replay reuses the captured pointers, the
 *     workspace included, which must stay allocated while the graph lives.
 *   - Non-finite inputs are outside the contract (codes then unspecified).
 *   - The library keeps no mutable global state: every call's behaviour is a
 *     function of its arguments (the only cache is the per-device result of
 *     the architecture check), so calls from several threads are safe.
 *   - Results are deterministic: the same inputs give the same bytes, and BF16
 *     and pre-quantized activations give identical results (the split-K
 *     streaming kernel quantizes BF16 in its load path with the quantizer's
 *     rule and the same split plan; before the other kernels the quantizer
 *     runs first).
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXFP8_OK = 0,
  MXFP8_ERR_NULL = 1,         /* a required pointer is NULL */
  MXFP8_ERR_SHAPE = 2,        /* a size or stride is out of range or not a required multiple */
  MXFP8_ERR_ALIGN = 3,        /* a pointer or row stride breaks the alignment rules */
  MXFP8_ERR_UNSUPPORTED = 4,  /* unknown activation kind, or no output requested */
  MXFP8_ERR_ALIAS = 5,        /* an output overlaps an input or another output */
  MXFP8_ERR_DEVICE = 6,       /* the current HIP device is missing or is not gfx950 */
  MXFP8_ERR_LAUNCH = 7,       /* the kernel launch failed */
  MXFP8_ERR_WORKSPACE = 8,    /* workspace missing, too small, or misaligned */
  MXFP8_ERR_SCRATCH = 9       /* fp8_gemm_nt_noalloc: the shape needs more than its fixed scratch */
} mxfp8_status;

/* Activation kinds: the type tag of an activation operand.  A producer/consumer
 * pair exchanges MXFP8 only in the one packed K-major layout above, so the tag
 * cannot describe a foreign scale layout (vLLM PR #57977, Pieces: the typed
 * activation key that keeps producer and consumer layouts from mixing). */
typedef enum {
  MXFP8_ACT_BF16 = 0,    /* data = BF16 [rows][ld]; quantized inside the GEMM's load path; sf ignored */
  MXFP8_ACT_MXFP8 = 1    /* data = E4M3 [rows][ld] bytes; sf = packed UE8M0 [rows][ld_sf] int32 */
} mxfp8_act_kind;

/* Text for a status code (static storage; never NULL). */
const char* mxfp8_status_string(int status);

/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int mxfp8_version(void);

/* MXFP8_OK when the current HIP device is a gfx950, else MXFP8_ERR_DEVICE. */
int mxfp8_device_check(void);

/*
 * mxfp8_quantize -- dynamic MXFP8 quantization of BF16 rows
 * (the standalone quantize launch that vLLM PR #57977, section Purpose, counts
 * per decode step, and that PR #60118, Claims, removes from the o_proj chain).
 *
 *   x     BF16 [M][ld_x], row length K           (input)
 *   q     E4M3 [M][ld_q] bytes, row length K     (output)
 *   sf    int32 [M][ld_sf], K/128 words per row  (output, packed UE8M0 scales)
 *
 * K must be a positive multiple of 128; ld_x >= K, ld_q >= K, ld_sf >= K/128.
 * Bit-exact: every code and scale equals the rule in the header comment.
 */
int mxfp8_quantize(const void* x, int64_t M, int64_t K, int64_t ld_x,
                   void* q, int64_t ld_q, int32_t* sf, int64_t ld_sf, void* stream);

/*
 * mxfp8_rmsnorm_quantize -- RMS normalization of BF16 rows whose output leaves
 * as MXFP8 (and optionally BF16): the producer-side fusion of vLLM PR #57977
 * (before/after diagrams, Pieces), where the normalizing producer in front of
 * the fused wqa/wkv projection emits that GEMM's MXFP8 input (codes + packed
 * UE8M0 scales) itself instead of a standalone quantize launch.
 *
 *   x      BF16 [M][ld_x], row length K                (input)
 *   gamma  BF16 [K], the per-column weight              (input)
 *   eps    positive, finite                             (added to the mean square)
 *   y      BF16 [M][ld_y], row length K, or NULL        (output, optional)
 *   q      E4M3 [M][ld_q] bytes, row length K, or NULL  (output)
 *   sf     int32 [M][ld_sf], K/128 words per row, or NULL (output, packed UE8M0 scales)
 *
 * Per row: y = BF16_RNE((x * r) * gamma) with r = 1 / sqrt(sum(x^2) / K + eps),
 * all in fp32 (the sum of squares in a fixed order); (q, sf) = mxfp8_quantize of
 * that BF16 y, bit for bit.  q and sf come together (both or neither); at least
 * one of y and (q, sf) must be given (MXFP8_ERR_UNSUPPORTED otherwise) -- y
 * alone is the unfused producer, whose output a standalone mxfp8_quantize then
 * reads.  K must be a positive multiple of 128; ld_x, ld_q, ld_y >= K,
 * ld_sf >= K/128; row strides 16-byte aligned.  Errors: as mxfp8_quantize, plus
 * MXFP8_ERR_SHAPE for eps <= 0 or not finite and MXFP8_ERR_ALIAS when an output
 * overlaps x, gamma or another output.
 */
int mxfp8_rmsnorm_quantize(const void* x, int64_t M, int64_t K, int64_t ld_x, const void* gamma, float eps,
                           void* y, int64_t ld_y, void* q, int64_t ld_q, int32_t* sf, int64_t ld_sf,
                           void* stream);

/*
 * grouped_fp8_einsum -- the wo_a projection: G independent groups
 *     z[m, g*N + n] = sum_k x[m, g*K + k] * w[g, n, k]
 * with MXFP8 operands and fp32 accumulation (vLLM PR #60118, Validation:
 * "8 groups x 4096 -> 1024"; PR #57977, Pieces: the einsum emits (z, sf)).
 *
 *   x_kind, x, ld_x, x_sf, ld_xsf
 *           activation rows m in [0, M), G*K columns, kind MXFP8_ACT_BF16 or
 *           MXFP8_ACT_MXFP8 (then x_sf holds G*K/128 words per row)
 *   w       E4M3 [G][N][K] bytes, contiguous        w_sf  int32 [G][N][K/128], contiguous
 *   z_q, ld_z, z_sf, ld_zsf
 *           optional MXFP8 output: E4M3 [M][ld_z] (G*N columns) and packed
 *           scales int32 [M][ld_zsf] (G*N/128 words).  The epilogue rounds each
 *           fp32 sum to BF16 (nearest even) and quantizes that BF16 value, so
 *           the bytes equal mxfp8_quantize applied to the BF16 output below.
 *   z_bf16, ld_zb
 *           optional BF16 output [M][ld_zb] (G*N columns).
 * At least one of z_q / z_bf16 must be given (z_q and z_sf together).
 * Accumulation: fp32; the MFMA is handed each activation fragment as two
 * operands, its codes of magnitude >= 64 and the rest, so that a large
 * activation (the attention output's rare x100 entries) never shares one of
 * the instruction's 8-product alignment groups with small ones (which would
 * lose their low bits); fp8_gemm_nt takes its activations whole.
 *   workspace, workspace_bytes
 *           scratch, at least grouped_fp8_einsum_workspace_size(x_kind, M, G, K, N)
 *           bytes (see the conventions above).
 * K and N must be positive multiples of 128 (N % 128 == 0 keeps every scale
 * word of z inside one group: PR #60118, Details, the o_lora_rank % 128 gate).
 */
int grouped_fp8_einsum(int x_kind, const void* x, int64_t ld_x, const int32_t* x_sf, int64_t ld_xsf,
                       int64_t M, int64_t G, int64_t K, int64_t N,
                       const void* w, const int32_t* w_sf,
                       void* z_q, int64_t ld_z, int32_t* z_sf, int64_t ld_zsf,
                       void* z_bf16, int64_t ld_zb,
                       void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes grouped_fp8_einsum needs for this activation kind and shape (0 = none);
 * -1 for an invalid kind or shape. */
int64_t grouped_fp8_einsum_workspace_size(int x_kind, int64_t M, int64_t G, int64_t K, int64_t N);

/*
 * fp8_gemm_nt -- the wo_b projection, recipe (1,1,32): both operands K-contiguous
 * with 1x32 scale blocks (vLLM PR #57977, Pieces and the per-layer table):
 *     d[m, n] = bf16_rne( sum_k a[m, k] * b[n, k] )
 *
 *   a_kind, a, ld_a, a_sf, ld_asf   activation rows m in [0, M), K columns (as in the einsum)
 *   b       E4M3 [N][K] bytes, contiguous      b_sf  int32 [N][K/128], contiguous
 *   d       BF16 [M][ld_d], N columns (output)
 *   workspace, workspace_bytes   scratch, at least fp8_gemm_nt_workspace_size(a_kind, M, N, K) bytes
 * K and N must be positive multiples of 128.
 */
int fp8_gemm_nt(int a_kind, const void* a, int64_t ld_a, const int32_t* a_sf, int64_t ld_asf,
                int64_t M, int64_t N, int64_t K,
                const void* b, const int32_t* b_sf,
                void* d, int64_t ld_d,
                void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes fp8_gemm_nt needs for this activation kind and shape (0 = none);
 * -1 for an invalid kind or shape. */
int64_t fp8_gemm_nt_workspace_size(int a_kind, int64_t M, int64_t N, int64_t K);

/*
 * fp8_gemm_nt_noalloc -- fp8_gemm_nt for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, meaning, kernels and results (bit for bit)
 * as fp8_gemm_nt, without the workspace arguments: where fp8_gemm_nt needs a
 * workspace (fp8_gemm_nt_workspace_size > 0: split-K partials of the few-token
 * kernels, BF16 activations staged as MXFP8), this call uses a fixed device
 * array of MXFP8_NOALLOC_SCRATCH_BYTES inside the library instead.  It never
 * calls hipMalloc, hipFree or any allocating routine.
 *
 *   - Limit: a shape whose workspace need exceeds MXFP8_NOALLOC_SCRATCH_BYTES
 *     returns MXFP8_ERR_SCRATCH after the usual argument checks, nothing
 *     launched (e.g. BF16 activations of more than about 1900 rows at
 *     K = 8192; MXFP8 activations never stage, and the decode shapes' split-K
 *     scratch is a few MB).
 *   - The array is per GPU (each device holds its own copy, from the library's
 *     load until the process ends) and shared by every call on that GPU: calls
 *     that overlap in time on one GPU (other streams, other threads, a graph
 *     replaying while an eager call runs) race on it and must be serialized
 *     by the caller.  Calls in one stream's order are safe.
 *   - The first call on a device also enqueues, on its stream and ahead of its
 *     own kernels, a kernel that zero-fills the split-K counters (the kernels
 *     leave them at zero after every call, as with a workspace).
 */
#define MXFP8_NOALLOC_SCRATCH_BYTES ((int64_t)16 << 20)
int fp8_gemm_nt_noalloc(int a_kind, const void* a, int64_t ld_a, const int32_t* a_sf, int64_t ld_asf,
                        int64_t M, int64_t N, int64_t K,
                        const void* b, const int32_t* b_sf,
                        void* d, int64_t ld_d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H */
