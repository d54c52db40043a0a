/*
 * gdn_bench.h -- measurement helpers of the MI355X GDN speculative-decode
 * library: the HBM traffic of one update launch with no arithmetic, and a
 * probe of how the SIMD issues FP32 matrix and vector instructions.
 *
 * Not part of the method.  The vLLM PR #51674 report (功能与动机) measures the
 * fused decode kernel in a cold-cache microbenchmark against the unfused
 * chain; a bandwidth-bound kernel is judged against what the memory system
 * delivers for its traffic.  This call gives that ceiling for one launch:
 * the same grid, unit mapping, metadata phase and blocks per CU as
 * gdn_mixed_decode_update (num_seqs > 0) or gdn_decode_update
 * (num_seqs == 0) with the same arguments, and the same bytes moved --
 * each unit's rewind tile read once and written back UNCHANGED to each of
 * its draft-token slots, its q/k/v/z rows and gate scalars read, its out
 * rows written with the XOR of the bits it read -- but no arithmetic.
 *
 * Arguments, ownership, errors and the safety net are those of
 * gdn_mixed_decode_update (include/gdn_spec.h); with num_seqs == 0 the
 * single-token entries take their rows through non_spec_token_indx.
 * blocks_per_cu: 0 runs as many blocks per CU as the update kernel would;
 * 1..8 runs that many instead (a sweep of launch shapes for the same
 * traffic); anything else is GDN_ERR_INVALID.  The
 * pool's written slots receive copies of the rewind tiles and `out` receives
 * meaningless bits: run it on scratch copies.  One kernel on `stream`, no
 * allocation, no synchronisation.
 */
#ifndef GDN_BENCH_H
#define GDN_BENCH_H

#include "gdn_spec.h"

#ifdef __cplusplus
extern "C" {
#endif

gdn_status gdn_traffic_pattern(const gdn_layer* layer, const gdn_state_pool* pool,
                               const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_q_len,
                               const int32_t* spec_state_indices, int32_t spec_stride,
                               const int32_t* num_accepted_tokens,
                               const int32_t* spec_token_indx, const int32_t* state_indices,
                               int32_t num_tokens, const int32_t* non_spec_token_indx,
                               int32_t blocks_per_cu, hipStream_t stream);

/*
 * The issue probe: whether FP32 matrix instructions and FP32 vector
 * instructions of two waves on one SIMD execute at the same time, which
 * bounds how a kernel that mixes them (the chunkwise prefill) can overlap
 * its two kinds of work.  One launch of `blocks` 512-thread blocks: waves
 * 0-3 run two interleaved chains of n_mfma v_mfma_f32_32x32x2f32 each when
 * mode & 1, waves 4-7 (wave w + 4 shares wave w's SIMD) eight independent
 * chains of n_valu FP32 FMAs when mode & 2.  Every thread writes one float
 * of `out` (device memory, caller-owned, blocks * 512 floats) so that no
 * work is dead.  Timed by the caller in modes 1, 2 and 3: if mode 3 takes
 * the sum of modes 1 and 2, the SIMD issues the two kinds one after the
 * other.  mode 1..3, n_mfma and n_valu 0..10^6, blocks 1..65536, out
 * non-null, else GDN_ERR_INVALID.  One kernel on `stream`, no allocation,
 * no synchronisation.
 */
gdn_status gdn_issue_probe(float* out, int32_t blocks, int32_t mode, int32_t n_mfma,
                           int32_t n_valu, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_BENCH_H */
