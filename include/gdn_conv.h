/*
 * gdn_conv.h -- C ABI of the causal depthwise conv1d update with rewind over
 * a wide rolling conv buffer: the step that turns a GDN layer's packed q/k/v
 * projection into the q, k, v that the speculative state update
 * (gdn_spec.h) consumes.
 *
 * Sources (the vLLM PR reports on prhub.com.cn):
 *   #46090 "[CPU][Spec Decode] Support DFlash speculative decoding for GDN
 *          models on CPU", 实现拆解 (implementation breakdown) items 1-2 and
 *          the gdn_attention.py excerpt under 关键源码片段: in speculative
 *          mode the conv cache holds more than width - 1 positions (a rolling
 *          buffer); each draft token convolves a width-wide view of it, and
 *          the buffer is written back.  The conv state is rewound through the
 *          wide buffer, not through per-token slots.
 *   #51674 "[Kernel][Perf] Add fused CUDA post-conv MTP decode kernel for
 *          Qwen3.5 GDN", 实现拆解 item 3: the speculative path runs the causal
 *          conv1d update with rewind, keyed by num_accepted_tokens, before the
 *          fused recurrent update; the conv state is BF16 there.
 *
 * The pages print no formula for the buffer; the reading implemented (the
 * same as the CPU oracle's) is, per sequence b with
 * L = cu_seqlens[b+1] - cu_seqlens[b] > 0 and line = conv_indices[b]:
 *   o            = max(num_accepted_tokens[b] - 1, 0)      (rewind offset)
 *   e[j]         = cache[line][o + j]     for j < width - 1 (history: inputs)
 *   e[width-1+t] = x[row_t]               for t < L
 *   out[row_t][c] = act(bias[c] + sum_{j < width} weight[c][j] * e[t + j][c])
 *   cache[line][p] = e[p + 1]             for p < width - 2 + L
 * with row_t = token_indx ? token_indx[cu[b] + t] : cu[b] + t.  The buffer
 * holds inputs, oldest first; after a step it holds the history without its
 * oldest entry followed by every draft input, so that the next step, told
 * that acc drafts were accepted, finds the width - 1 inputs preceding its
 * first token at offset acc - 1.  With acc = 1 and L = 1 this is the plain
 * shift-by-one conv state of non-speculative decode.  Arithmetic is FP32 (one
 * fused multiply-add per tap, taps in ascending j); the output is rounded to
 * out_dtype to nearest, ties to even; buffer writes copy inputs exactly.
 *
 * Conventions: as in gdn_spec.h -- device pointers owned by the caller, no
 * allocation, no synchronisation, one kernel enqueued on `stream`, strides in
 * elements, a thread-local reason for every non-OK status, nothing enqueued
 * on error, no fallback.  Positions of a line at or beyond width - 2 + L,
 * other lines, and output rows not processed keep their contents.  `out` and
 * the buffer must not overlap each other or any input.
 *
 * Device-side metadata is trusted, with the same safety net as the state
 * update: a sequence whose metadata is out of range (L > max_q_len, a line
 * outside [0, num_lines), acc < 0, o + width - 1 > state_len, a row outside
 * [0, n_tok)) is skipped whole.  Distinct lines per call are the caller's
 * contract; gdn_validate_conv_indices_host() checks it on host copies.
 */
#ifndef GDN_CONV_H
#define GDN_CONV_H

#include "gdn_spec.h"

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_CONV_MAX_WIDTH 4

typedef enum { GDN_CONV_ACT_NONE = 0, GDN_CONV_ACT_SILU = 1 } gdn_conv_activation;

/* One layer's conv inputs, parameters and outputs.
 *   x      [n_tok][channels]  x_dtype, read; channel stride 1, token stride
 *                             x_stride_tok (a view into a wider packed
 *                             projection is fine)
 *   out    [n_tok][channels]  out_dtype, written; token stride out_stride_tok
 *                             >= channels
 *   weight fp32 [channels][width], contiguous (torch's conv1d weight
 *          [channels, 1, width] of a depthwise conv)
 *   bias   fp32 [channels] or NULL (no bias)
 * With n_tok == 0, x and out may be NULL and every call is a no-op.
 * x and out are aligned to their element size; weight and bias to 4 bytes. */
typedef struct {
    const void*  x;
    int64_t      x_stride_tok;
    void*        out;
    int64_t      out_stride_tok;
    const float* weight;
    const float* bias;
    int32_t      x_dtype;      /* gdn_dtype */
    int32_t      out_dtype;    /* gdn_dtype */
    int32_t      channels;     /* C > 0 */
    int32_t      width;        /* 1 .. GDN_CONV_MAX_WIDTH */
    int32_t      activation;   /* gdn_conv_activation */
    int32_t      reserved;
    int64_t      n_tok;        /* rows addressable in x and out */
} gdn_conv_layer;

/* The rolling conv buffer: num_lines lines of state_len positions of
 * `channels` values, in the layer's x_dtype, element (line, pos, c) at
 * data[line * stride_line + pos * stride_pos + c * stride_chan].  The
 * position-major layout (stride_chan == 1) is the fast one; a channel-major
 * buffer (stride_pos == 1) is accepted and served by an element-wise path.
 * Updated in place. */
typedef struct {
    void*   data;
    int32_t dtype;        /* gdn_dtype, must equal the layer's x_dtype */
    int32_t state_len;    /* positions per line, >= width - 1 */
    int64_t num_lines;
    int64_t stride_line;
    int64_t stride_pos;
    int64_t stride_chan;
} gdn_conv_cache;

/*
 * Speculative conv update of num_seqs sequences (formula above).
 *   cu_seqlens          int32 [num_seqs+1]  row offsets (gathered token space)
 *   max_q_len           host bound on every L_b, 1..GDN_MAX_DRAFT_TOKENS;
 *                       state_len must be >= width - 2 + max_q_len
 *   conv_indices        int32 [num_seqs]    buffer line of each sequence
 *   num_accepted_tokens int32 [num_seqs]    accepted drafts of the previous
 *                                            step (rewind offset acc - 1,
 *                                            0 for acc <= 1)
 *   token_indx          int32 [cu_seqlens[num_seqs]] or NULL (row = i)
 */
gdn_status gdn_conv_spec_update(const gdn_conv_layer* layer, const gdn_conv_cache* cache,
                                const int32_t* cu_seqlens, int32_t num_seqs,
                                int32_t max_q_len, const int32_t* conv_indices,
                                const int32_t* num_accepted_tokens,
                                const int32_t* token_indx, hipStream_t stream);

/*
 * Non-speculative decode: num_tokens single-token updates, entry i on line
 * conv_indices[i] at offset 0 (a negative line marks padding: skipped, its
 * output row untouched).  token_indx int32 [num_tokens] or NULL (row = i).
 */
gdn_status gdn_conv_decode_update(const gdn_conv_layer* layer, const gdn_conv_cache* cache,
                                  const int32_t* conv_indices, int32_t num_tokens,
                                  const int32_t* token_indx, hipStream_t stream);

/*
 * Host-side check of the conv metadata on HOST copies (pointers may be NULL
 * when their count is 0; token-index arrays NULL for the identity).  Returns
 * GDN_OK, or GDN_ERR_INVALID with the first violation in gdn_last_error():
 * cu_seqlens not non-decreasing from 0, L_b > max_q_len, acc < 0 or an
 * offset acc - 1 beyond state_len - width + 1, width - 2 + L_b > state_len,
 * a line outside [0, num_lines) (negative allowed for decode padding), a row
 * outside [0, n_tok), a line used twice or a row used twice across the spec
 * and decode entries of one batch.
 */
gdn_status gdn_validate_conv_indices_host(int64_t num_lines, int32_t state_len, int32_t width,
                                          int64_t n_tok, const int32_t* cu_seqlens,
                                          int32_t num_seqs, int32_t max_q_len,
                                          const int32_t* conv_indices,
                                          const int32_t* num_accepted_tokens,
                                          const int32_t* spec_token_indx,
                                          const int32_t* decode_indices, int32_t num_decode,
                                          const int32_t* decode_token_indx);

/* Sizes of gdn_conv_layer and gdn_conv_cache as built, for bindings. */
void gdn_conv_abi_struct_sizes(size_t* layer, size_t* cache);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CONV_H */
