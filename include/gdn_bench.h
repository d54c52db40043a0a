/*
 * gdn_bench.h -- measurement helper of the MI355X GDN speculative-decode
 * library: the HBM traffic of one update launch with no arithmetic.
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

#ifdef __cplusplus
}
#endif

#endif /* GDN_BENCH_H */
