/*
 * mxfp8_testing.h -- test-only entry points of libmxfp8.so.
 *
 * The few-token (decode) GEMM kernels split the K range across workgroups and
 * add the fp32 partial tiles in split order in the last workgroup to arrive.
 * Where the partials travel is an implementation choice that never changes a
 * bit of the result; these two calls let a test pick it per call, so that every
 * combine path can be checked against the others.  They take exactly the
 * arguments of grouped_fp8_einsum / fp8_gemm_nt in include/mxfp8.h (same
 * meaning, layout, ownership and error behaviour), preceded by:
 *
 *   splitk_combine
 *     0  through the L2 cache of one XCD (what grouped_fp8_einsum and
 *        fp8_gemm_nt always do): the splits of a tile are consecutive
 *        workgroups, which round-robin dispatch places on one XCD; the arrival
 *        counter records each split's XCD, and if any split ran on another XCD
 *        the last split to arrive computes the other splits again itself;
 *     1  through memory (write-through stores, read back past the caches);
 *     2  as 0, but the last split always recomputes the others (the fallback
 *        of mode 0, forced).
 *   Any other value: MXFP8_ERR_UNSUPPORTED, nothing launched.
 *
 * Production code calls the entry points of include/mxfp8.h.
 */
#ifndef MXFP8_TESTING_H
#define MXFP8_TESTING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int mxfp8_testing_grouped_fp8_einsum(int splitk_combine, int x_kind, const void* x, int64_t ld_x,
                                     const int32_t* x_sf, int64_t ld_xsf, int64_t M, int64_t G, int64_t K,
                                     int64_t N, const void* w, const int32_t* w_sf, void* z_q, int64_t ld_z,
                                     int32_t* z_sf, int64_t ld_zsf, void* z_bf16, int64_t ld_zb,
                                     void* workspace, int64_t workspace_bytes, void* stream);

int mxfp8_testing_fp8_gemm_nt(int splitk_combine, int a_kind, const void* a, int64_t ld_a,
                              const int32_t* a_sf, int64_t ld_asf, int64_t M, int64_t N, int64_t K,
                              const void* b, const int32_t* b_sf, void* d, int64_t ld_d, void* workspace,
                              int64_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_TESTING_H */
