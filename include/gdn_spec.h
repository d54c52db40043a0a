/*
 * gdn_spec.h -- C ABI of the MI355X (gfx950) fused Gated DeltaNet (GDN)
 * speculative-decode state update.
 *
 * The operation is the fused post-conv MTP decode step described by the vLLM
 * PR reports on prhub.com.cn:
 *   #51674 "[Kernel][Perf] Add fused CUDA post-conv MTP decode kernel for
 *          Qwen3.5 GDN", 实现拆解 (implementation breakdown) item 1: per
 *          (request, value head) rewind to the last accepted state slot, run
 *          the gated delta-rule recurrence over up to 8 draft tokens, store
 *          every post-token state, finish with a gated RMSNorm; item 2 and the
 *          vllm/_custom_ops.py excerpt: the argument list and the defaults
 *          scale = 128**-0.5, norm_eps = 1e-5.
 *   #46090 "[CPU][Spec Decode] Support DFlash speculative decoding for GDN
 *          models on CPU", 关键源码片段 (key source excerpts), fla.cpp: the
 *          variable-length batch (cu_seqlens, q_len <= 0 skipped), the clamp
 *          max(num_accepted - 1, 0), per-token slots spec_state_indices[b, t],
 *          per-tensor token/head strides, non-interleaved GQA.
 *   #52191 "[CPU] Support FP16/BF16 persisted GDN state on AMX", 实现拆解
 *          item 4: arithmetic in FP32, only slot reads and writes in the state
 *          dtype (fp32, bf16 or fp16).
 *   #51812 "[Bugfix] Align Qwen GDN gates with speculative tokens",
 *          关键源码片段: the same token index gathers q/k/v and the gates a/b.
 *
 * Per (sequence b, value head h) with L = cu_seqlens[b+1] - cu_seqlens[b] > 0:
 *   r     = spec_state_indices[b][max(num_accepted_tokens[b] - 1, 0)]
 *   S     = float(pool[r][h])                       (V x K, read once)
 *   for t < L, row = token_indx ? token_indx[cu[b]+t] : cu[b]+t:
 *     alpha = exp(-exp(A_log[h]) * softplus(a[row][h] + dt_bias[h]))
 *     beta  = sigmoid(b[row][h])
 *     k^ = k[row][kh] / sqrt(|k|^2 + 1e-6),  q^ = scale * q[row][kh] / sqrt(|q|^2 + 1e-6)
 *     S  = alpha S;  S += beta (v[row][h] - S k^) k^T;  o = S q^
 *     pool[spec_state_indices[b][t]][h] = round_to_state_dtype(S)
 *     out[row][h] = o / sqrt(mean(o^2) + norm_eps) * norm_weight * silu(z[row][h])
 *   with kh = h / (HV / HK).  The FP32 carry S is not re-rounded between
 *   tokens; rounding happens only at the slot and output stores (to nearest,
 *   ties to even).  The arithmetic is FP32; exp, log, the reciprocals and
 *   the reciprocal square roots of the gates, norms and RMSNorm come from the
 *   hardware units, each within about one ulp.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, owned by the caller.  The
 *     library allocates nothing, keeps no state between calls and never
 *     synchronises: the call enqueues one kernel on `stream` and returns.
 *     Launches are therefore capturable in a HIP graph.  Faults surface at
 *     the caller's next synchronisation.
 *   - Strides are in elements.  The innermost (head-dim) stride is 1.
 *   - Only the rows of processed tokens are written in `out`; other rows keep
 *     their contents (callers that pad batches zero-initialise `out`).
 *   - Only the slots spec_state_indices[b][t] (t < L_b), resp.
 *     state_indices[i] >= 0, change; every other byte of the pool is kept.
 *   - Host-checkable argument errors return GDN_ERR_INVALID, unsupported
 *     shapes or dtypes GDN_ERR_UNSUPPORTED, a failed launch GDN_ERR_DEVICE;
 *     each sets a thread-local reason returned by gdn_last_error().  Nothing
 *     is enqueued on any error.  There is no fallback path.
 *   - Device-side metadata is trusted, as on the pages, with one safety net:
 *     a unit whose metadata is out of range (acc < 0 or > spec_stride,
 *     L > 8 or > spec_stride, a slot outside [0, num_slots), a row outside
 *     [0, n_tok)) is skipped whole -- nothing read or written for it.
 *     Distinct write slots, and no read slot of one sequence equal to a write
 *     slot of another, are the caller's contract (data races otherwise);
 *     gdn_validate_indices_host() checks all of it on host copies.
 *   - The pool and `out` must not overlap each other or any input: the
 *     metadata, q/k/v/z/a/b and the parameters are read-only for the whole
 *     launch.
 */
#ifndef GDN_SPEC_H
#define GDN_SPEC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 5
#define GDN_MAX_DRAFT_TOKENS 8
#define GDN_HEAD_DIM 128

/* GDN_F8E4M3 (OCP FP8 E4M3 without infinities, largest finite 448) is a
 * state-pool format only: #52191 风险与影响 notes that the state type leaves
 * room for FP8, halving the state bytes again.  Stores round to nearest even
 * and saturate to +-448 (NaN stays NaN); loads are exact. */
typedef enum { GDN_F32 = 0, GDN_F16 = 1, GDN_BF16 = 2, GDN_F8E4M3 = 3 } gdn_dtype;

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID = 1,
    GDN_ERR_UNSUPPORTED = 2,
    GDN_ERR_DEVICE = 3
} gdn_status;

/* A strided 3-D (or 2-D) device tensor [n_tok][heads][dim], dim contiguous.
 * For the gates a and b ([n_tok][HV]) stride_head must be 1. */
typedef struct {
    void*   data;
    int64_t stride_tok;
    int64_t stride_head;
} gdn_view;

/* One layer's activations, parameters and output.
 *   q, k : [n_tok][num_k_heads][head_k_dim]   act_dtype, read
 *   v, z : [n_tok][num_v_heads][head_v_dim]   act_dtype, read (z = output gate)
 *   a, b : [n_tok][num_v_heads]               act_dtype, read (gate inputs)
 *   out  : [n_tok][num_v_heads][head_v_dim]   out_dtype, written
 *   A_log, dt_bias : fp32 [num_v_heads];  norm_weight : fp32 [head_v_dim]
 * A packed mixed_qkv projection is passed as three views into it.
 * With n_tok == 0 the activation/output pointers may be NULL and every call
 * is a no-op.
 * Alignment: q, k, v, z, out data pointers aligned to 2 elements and their
 * token/head strides even; A_log and dt_bias 4-byte aligned; norm_weight
 * 8-byte aligned (the kernels read it in pairs). */
typedef struct {
    gdn_view q, k, v, z, a, b, out;
    const float* A_log;
    const float* dt_bias;
    const float* norm_weight;
    int32_t act_dtype;    /* gdn_dtype */
    int32_t out_dtype;    /* gdn_dtype */
    int32_t num_k_heads;  /* HK */
    int32_t num_v_heads;  /* HV, a multiple of HK */
    int32_t head_k_dim;   /* K, must be 128 */
    int32_t head_v_dim;   /* V, must be 128 */
    int64_t n_tok;        /* rows addressable in q..out */
    float   scale;        /* applied to the normalised q; K^-0.5 by default */
    float   norm_eps;     /* RMSNorm epsilon; 1e-5 by default */
} gdn_layer;

/* The recurrent-state pool, contiguous [num_slots][num_v_heads][V][K]
 * (K innermost), updated in place.  16-byte aligned.  dtype: fp32, fp16, bf16
 * or fp8 e4m3. */
typedef struct {
    void*   data;
    int32_t dtype;        /* gdn_dtype */
    int32_t reserved;
    int64_t num_slots;
} gdn_state_pool;

/*
 * Speculative (MTP) update of num_seqs sequences, one workgroup per
 * (sequence, value head).
 *   cu_seqlens          int32 [num_seqs+1]  row offsets of each sequence in
 *                                            the (gathered) token space
 *   max_q_len           host bound on every L_b, 1..8
 *   spec_state_indices  int32 [num_seqs][spec_stride]  slot of each draft
 *                                            token's post-token state
 *   num_accepted_tokens int32 [num_seqs]    accepted tokens of the previous
 *                                            step; the state is read from slot
 *                                            [b][max(acc - 1, 0)]
 *   token_indx          int32 [cu_seqlens[num_seqs]] or NULL: row of q/k/v/z/
 *                                            a/b/out used by gathered token i
 *                                            (NULL: row = i)
 * Reads the pool at the rewind slots, writes it at the draft-token slots,
 * writes out at the processed rows.
 */
gdn_status gdn_spec_decode_update(const gdn_layer* layer,
                                  const gdn_state_pool* pool,
                                  const int32_t* cu_seqlens, int32_t num_seqs,
                                  int32_t max_q_len,
                                  const int32_t* spec_state_indices,
                                  int32_t spec_stride,
                                  const int32_t* num_accepted_tokens,
                                  const int32_t* token_indx,
                                  hipStream_t stream);

/*
 * Non-speculative decode: num_tokens single-token updates, entry i reading
 * and writing slot state_indices[i] in place (a negative slot marks padding:
 * skipped, its output row untouched).  token_indx int32 [num_tokens] or NULL
 * gives the row of entry i (NULL: row = i).  Same recurrence with L = 1.
 * Defined by: #46090 实现拆解 item 1 (a batch without speculative decoding
 * takes the non-spec path, _cpu_gdn_attention_nonspec, one state slot per
 * request) and #52191 实现拆解 item 3 (the decode kernel
 * fused_sigmoid_gating_delta_rule_update reads its slot as state_t, updates
 * in FP32 and writes the same slot back); #51812 关键源码片段 (the non-spec
 * rows are gathered by non_spec_token_indx, the gates with them).
 */
gdn_status gdn_decode_update(const gdn_layer* layer, const gdn_state_pool* pool,
                             const int32_t* state_indices, int32_t num_tokens,
                             const int32_t* token_indx, hipStream_t stream);

/*
 * A mixed batch in ONE launch: the num_seqs speculative sequences of
 * gdn_spec_decode_update (rows through spec_token_indx) and the num_tokens
 * single-token entries of gdn_decode_update (slot state_indices[i], negative
 * = padding, rows through non_spec_token_indx), one workgroup per (entry,
 * value head) of either kind.  The result equals the two calls made one
 * after the other, in either order; the two parts must touch disjoint slots
 * and rows (gdn_validate_indices_host checks both parts together).  Either
 * count may be 0.  The [51674] CUDA path gave this fusion up as low-gain
 * (实现拆解, evolution notes: it needed prefix-length metadata and slicing);
 * here the two index arrays already carry all it needs.
 */
gdn_status gdn_mixed_decode_update(const gdn_layer* layer, const gdn_state_pool* pool,
                                   const int32_t* cu_seqlens, int32_t num_seqs,
                                   int32_t max_q_len, const int32_t* spec_state_indices,
                                   int32_t spec_stride, const int32_t* num_accepted_tokens,
                                   const int32_t* spec_token_indx,
                                   const int32_t* state_indices, int32_t num_tokens,
                                   const int32_t* non_spec_token_indx, hipStream_t stream);

/*
 * Chunked prefill ([52191] 实现拆解 items 3-4): num_seqs sequences of any
 * length, rows cu_seqlens[b] .. cu_seqlens[b+1]-1 (through token_indx when
 * given), sequence b on slot state_indices[b] (negative: skipped), read at
 * the start when has_initial_state[b] != 0 (NULL: always; 0: start from a
 * zero state) and written at the end.  Every row runs the token step above
 * (same gates, norms, recurrence and gated-RMSNorm output); the carried
 * state is rounded to the pool dtype after every chunk_size-th row of the
 * call and after its last -- where the chunked kernels of the pages write
 * the state back -- and continues from the rounded value.  A call split at
 * a multiple of chunk_size therefore equals one call.  Slots distinct per
 * call (gdn_validate_prefill_indices_host checks it).  Arithmetic is FP32.
 * With chunk_size >= 16 the rows of a chunk are taken 16 at a time in the
 * chunkwise form of the same recurrence (matrix products plus a small
 * triangular solve), which differs from row-by-row evaluation only in
 * rounding order; results are deterministic for a given chunk_size.
 */
gdn_status gdn_prefill_update(const gdn_layer* layer, const gdn_state_pool* pool,
                              const int32_t* cu_seqlens, int32_t num_seqs,
                              const int32_t* state_indices,
                              const int32_t* has_initial_state, const int32_t* token_indx,
                              int32_t chunk_size, hipStream_t stream);

/*
 * Host-side check of prefill metadata on HOST copies: cu_seqlens
 * non-decreasing from 0, slots < num_slots (negative = skipped) and
 * distinct, rows inside [0, n_tok) and used once.  The prefill kernels trust
 * this metadata as the decode kernels trust theirs; #46090 评论区精华 and
 * 风险与影响 record the state-index arrays left unvalidated there, which
 * this check covers for the prefill.
 */
gdn_status gdn_validate_prefill_indices_host(int64_t num_slots, int64_t n_tok,
                                             const int32_t* cu_seqlens, int32_t num_seqs,
                                             const int32_t* state_indices,
                                             const int32_t* token_indx);

/*
 * Defined by #46090 评论区精华 and 风险与影响: static analysis of the CPU spec
 * kernel found the acc - 1 underflow (fixed by the clamp) and noted that
 * spec_state_indices is never checked for shape or range.  The kernels keep
 * trusting device metadata (and skip a unit whose metadata is out of
 * range); this is the check a caller runs on host copies instead.
 *
 * Host-side check of the metadata contract on HOST copies of the index
 * arrays (any pointer may be NULL when its count is 0; the token-index arrays
 * may be NULL for the identity).  Returns GDN_OK, or GDN_ERR_INVALID with the
 * first violation in gdn_last_error(): cu_seqlens not non-decreasing from 0,
 * L_b > max_q_len or > spec_stride, acc outside [0, spec_stride], a slot
 * outside [0, num_slots), a row outside [0, n_tok), a write slot used twice,
 * a read slot of one sequence written by another (or by a non-spec entry),
 * a row used twice.  The spec entries and the non-spec entries of one mixed
 * batch are checked together.
 */
gdn_status gdn_validate_indices_host(int64_t num_slots, int64_t n_tok,
                                     const int32_t* cu_seqlens,
                                     int32_t num_seqs, int32_t max_q_len,
                                     const int32_t* spec_state_indices,
                                     int32_t spec_stride,
                                     const int32_t* num_accepted_tokens,
                                     const int32_t* spec_token_indx,
                                     const int32_t* state_indices,
                                     int32_t num_non_spec,
                                     const int32_t* non_spec_token_indx);

/*
 * Rounds n fp32 values (device pointer src) into the state format `dtype`
 * at dst (device pointer, n elements), with the conversion every kernel of
 * this library uses at a state store: nearest even, FP8 saturating to +-448.
 * For filling a pool from FP32 states; one kernel on `stream`.
 */
gdn_status gdn_cast_to_state(const float* src, void* dst, int64_t n, int32_t dtype,
                             hipStream_t stream);

/* Reason for the last non-OK status returned on this thread ("" if none).
 * Defined by #51674 实现拆解 item 3: _fused_gdn_decode_unsupported_reason
 * gathers every constraint of the fused kernel (non-interleaved GQA,
 * K = V = 128, dtypes, at most 8 MTP tokens) into one reason string, and an
 * explicit request that fails them raises instead of falling back.  Here a
 * call that fails a check returns GDN_ERR_UNSUPPORTED or GDN_ERR_INVALID and
 * this returns the reason; there is no fallback path. */
const char* gdn_last_error(void);

/* Static name of a status code (the same #51674 passage: the status is the
 * raise-or-proceed decision, this is its name for logs). */
const char* gdn_status_string(gdn_status status);

/* GDN_ABI_VERSION of the built library, and the sizes of the argument
 * structs it was built with, so bindings can check their layout. */
int32_t gdn_abi_version(void);
void gdn_abi_struct_sizes(size_t* view, size_t* layer, size_t* pool);

#ifdef __cplusplus
}
#endif

#endif /* GDN_SPEC_H */
