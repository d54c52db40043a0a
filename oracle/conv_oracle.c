/*
 * conv_oracle.c -- plain serial CPU oracle of the causal depthwise conv1d
 * update with rewind over a wide rolling conv buffer, the step that feeds
 * q/k/v to the GDN state update in speculative (MTP) decode.
 *
 * TEST INFRASTRUCTURE ONLY, like gdn_oracle.c: tests, the smoke check and
 * the CPU-baseline leg of the benchmark use it to compute expected results.
 * Nothing on the product path may link, load or call it, and it shares no
 * code with the HIP library.
 *
 * Sources (the vLLM pull-request reports on prhub.com.cn):
 *   [46090] "[CPU][Spec Decode] Support DFlash speculative decoding for GDN
 *           models on CPU", "实现拆解" (implementation breakdown) items 1-2
 *           and the gdn_attention.py excerpt under "关键源码片段": the conv
 *           cache of a speculative model is wider than width - 1 positions
 *           (a rolling buffer); each draft token takes a width-wide view of
 *           it, a plain conv1d over that view gives the token's output, and
 *           the buffer is written back.  The conv state is rewound through
 *           this wide buffer, while the recurrent state uses per-token slots.
 *   [51674] "[Kernel][Perf] Add fused CUDA post-conv MTP decode kernel for
 *           Qwen3.5 GDN", "实现拆解" item 3: the speculative path runs the
 *           causal conv1d update with rewind (driven by num_accepted_tokens)
 *           before the fused recurrent update; the conv state is BF16.
 *
 * The pages print no formula for the buffer.  Readings taken (plainest the
 * rest supports):
 *   R1  The buffer line of a sequence holds past conv INPUTS, one position
 *       per token, oldest first: a causal conv needs its last width - 1
 *       inputs, and feeding outputs back would make it a recursive filter.
 *       (The excerpt's write of the conv result into the cache is read as the
 *       cache update in general, not as storing outputs.)
 *   R2  Rewind: the previous step appended all its draft inputs, of which
 *       acc were accepted.  The width - 1 inputs that precede the new first
 *       token then start at position o = max(acc - 1, 0) of the line -- the
 *       same clamp as the recurrent-state rewind ([46090] fla.cpp excerpt),
 *       so acc = 0 behaves as acc = 1.
 *   R3  Window of token t: e[t .. t + width - 1], where e = history ++ inputs
 *       (history = line[o .. o + width - 2], inputs u_0 .. u_{L-1}).  The
 *       output is a cross-correlation as torch's conv1d computes it:
 *         y_t[c] = act(bias[c] + sum_j weight[c][j] * e[t + j][c]),
 *       weight[c][width - 1] multiplying the current token.
 *   R4  Write-back: line[p] = e[p + 1] for p < width - 2 + L (the history
 *       without its oldest entry, then every draft input); later positions
 *       keep their contents.  The next step rewinds into exactly this layout
 *       (R2), and with acc = 1 and L = 1 it is the ordinary shift-by-one
 *       conv state of non-speculative decode.
 *   R5  Activation: none or SiLU, chosen by the caller (the pages name none;
 *       the GDN layers gate with SiLU elsewhere).  Bias optional.
 *
 * Precision: double throughout; the output is rounded to its storage format
 * once (orc_round); buffer writes are copies of inputs, rounded to the
 * buffer's format (exact when it equals the input format).
 *
 * Layouts (contiguous, row major):
 *   x, out  [n_tok][C]          cache  [num_lines][state_len][C]
 *   weight  [C][width]          bias   [C] or NULL
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

double orc_round(int fmt, double x);   /* gdn_oracle.c */

enum { CONV_OK = 0, CONV_BAD_ARG = 1, CONV_BAD_INDEX = 2, CONV_NO_MEMORY = 3 };
enum { CONV_ACT_NONE = 0, CONV_ACT_SILU = 1 };

static int fmt_valid(int f) { return f >= 0 && f <= 4; }

static double activate(int act, double s)
{
    return act == CONV_ACT_SILU ? s / (1.0 + exp(-s)) : s;
}

/*
 * One sequence: L tokens at rows rows[0..L-1], buffer line `line`, rewind
 * offset o.  e holds (width - 1 + L) * C doubles of scratch.
 */
static void conv_sequence(const double *x, double *out, int out_fmt,
                          double *cache, int cache_fmt, int state_len, int C,
                          int width, const double *weight, const double *bias,
                          int act, int64_t line, int64_t o, int64_t L,
                          const int64_t *rows, double *e)
{
    double *ln = cache + line * (int64_t)state_len * C;
    int64_t p, t;
    int c, j;

    /* e = history ++ inputs; the history is read whole before any write. */
    for (p = 0; p < width - 1; ++p)
        memcpy(e + p * C, ln + (o + p) * C, sizeof(double) * (size_t)C);
    for (t = 0; t < L; ++t)
        memcpy(e + (width - 1 + t) * C, x + rows[t] * C, sizeof(double) * (size_t)C);

    for (t = 0; t < L; ++t) {
        for (c = 0; c < C; ++c) {
            double s = bias ? bias[c] : 0.0;
            for (j = 0; j < width; ++j)
                s += weight[(int64_t)c * width + j] * e[(t + j) * C + c];
            out[rows[t] * C + c] = orc_round(out_fmt, activate(act, s));
        }
    }
    for (p = 0; p < width - 2 + L; ++p)
        for (c = 0; c < C; ++c)
            ln[p * C + c] = orc_round(cache_fmt, e[(p + 1) * C + c]);
}

/*
 * Speculative update of B sequences (cu_seqlens != NULL) or non-speculative
 * decode of B single tokens (cu_seqlens == NULL: entry i is row
 * token_indx ? token_indx[i] : i, offset 0, and a negative line is padding).
 *   spec:  L_b = cu[b+1] - cu[b]; L_b <= 0 skips the sequence; rows
 *          token_indx ? token_indx[cu[b]+t] : cu[b]+t; o = max(acc_b - 1, 0).
 * Every index is checked before anything is written: a line outside
 * [0, num_lines) (spec) or >= num_lines (decode), a row outside [0, n_tok),
 * acc < 0, o + width - 1 > state_len or width - 2 + L > state_len give
 * CONV_BAD_INDEX.
 */
int orc_conv_update(const double *x, double *out, int out_fmt, double *cache,
                    int cache_fmt, int64_t num_lines, int32_t state_len,
                    int64_t n_tok, int32_t C, int32_t width,
                    const double *weight, const double *bias, int32_t act,
                    const int32_t *cu_seqlens, int32_t B,
                    const int32_t *lines, const int32_t *num_acc,
                    const int32_t *token_indx)
{
    int64_t *rows;
    double *e;
    int64_t maxlen = 1;
    int32_t bi;
    int64_t t;

    if (!x || !out || !cache || !weight || !fmt_valid(out_fmt) ||
        !fmt_valid(cache_fmt) || C <= 0 || width < 1 || state_len < width - 1 ||
        B < 0 || (B > 0 && !lines) || (cu_seqlens && B > 0 && !num_acc) ||
        (act != CONV_ACT_NONE && act != CONV_ACT_SILU))
        return CONV_BAD_ARG;

    for (bi = 0; bi < B; ++bi) {
        int64_t start = cu_seqlens ? cu_seqlens[bi] : bi;
        int64_t len = cu_seqlens ? (int64_t)cu_seqlens[bi + 1] - start : 1;
        int64_t o = 0;
        if (len <= 0)
            continue;
        if (!cu_seqlens && lines[bi] < 0)
            continue;
        if (lines[bi] < 0 || lines[bi] >= num_lines || start < 0)
            return CONV_BAD_INDEX;
        if (cu_seqlens) {
            if (num_acc[bi] < 0)
                return CONV_BAD_INDEX;
            o = num_acc[bi] - 1 > 0 ? num_acc[bi] - 1 : 0;
        }
        if (o + width - 1 > state_len || width - 2 + len > state_len)
            return CONV_BAD_INDEX;
        for (t = 0; t < len; ++t) {
            int64_t row = token_indx ? token_indx[start + t] : start + t;
            if (row < 0 || row >= n_tok)
                return CONV_BAD_INDEX;
        }
        if (len > maxlen)
            maxlen = len;
    }

    rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)maxlen);
    e = (double *)malloc(sizeof(double) * (size_t)(width - 1 + maxlen) * (size_t)C);
    if (!rows || !e) {
        free(rows);
        free(e);
        return CONV_NO_MEMORY;
    }
    for (bi = 0; bi < B; ++bi) {
        int64_t start = cu_seqlens ? cu_seqlens[bi] : bi;
        int64_t len = cu_seqlens ? (int64_t)cu_seqlens[bi + 1] - start : 1;
        int64_t o = 0;
        if (len <= 0 || lines[bi] < 0)
            continue;
        if (cu_seqlens)
            o = num_acc[bi] - 1 > 0 ? num_acc[bi] - 1 : 0;
        for (t = 0; t < len; ++t)
            rows[t] = token_indx ? token_indx[start + t] : start + t;
        conv_sequence(x, out, out_fmt, cache, cache_fmt, state_len, C, width,
                      weight, bias, act, lines[bi], o, len, rows, e);
    }
    free(rows);
    free(e);
    return CONV_OK;
}
