/*
 * gdn_oracle.c -- plain serial CPU oracle of the fused sigmoid-gated
 * delta-rule state update used by Gated DeltaNet (GDN) layers in
 * speculative (MTP) decode.
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists so that tests, the smoke check
 * and the CPU-baseline leg of the benchmark can compute the expected result
 * of the GPU path.  Nothing on the product path may link, load or call it.
 * It shares no code, header, table or constant generator with the HIP
 * library; the two only ever meet on inputs produced by the seeded workload
 * generator.
 *
 * Sources (the vLLM pull-request reports on prhub.com.cn):
 *   [46090] "[CPU][Spec Decode] Support DFlash speculative decoding for GDN
 *           models on CPU" -- the spec kernel excerpt under "关键源码片段"
 *           (key source excerpts, csrc/cpu/sgl-kernels/fla.cpp) fixes the
 *           (sequence, v-head) decomposition, the GQA head map, the q_len<=0
 *           skip, the clamped rewind slot and the per-token slot store.
 *   [51674] "[Kernel][Perf] Add fused CUDA post-conv MTP decode kernel for
 *           Qwen3.5 GDN" -- "实现拆解" (implementation breakdown) item 1:
 *           gating, rewind, serial recurrence over <= 8 draft tokens, store of
 *           every post-token state, gated RMSNorm epilogue; item 2 and the
 *           _custom_ops.py excerpt: scale = 128**-0.5, norm_eps = 1e-5.
 *   [52191] "[CPU] Support FP16/BF16 persisted GDN state on AMX" --
 *           "实现拆解" item 4: all arithmetic is wide, only slot reads and
 *           writes go through the narrow state type.
 *   [51812] "[Bugfix] Align Qwen GDN gates with speculative tokens" --
 *           "关键源码片段": one gather index selects q/k/v *and* the gates.
 *
 * The pages name the steps and their arguments but print no equation.  The
 * readings taken where they are silent (gate formula, softplus threshold,
 * L2-norm epsilon, where `scale` applies, decay-before-delta, output after the
 * token's update, RMSNorm axis and order, wide carry across tokens) are stated
 * at each function below.
 *
 * Precision: every input is upcast exactly to double and every operation is
 * done in double.  The pages compute in FP32 on their kernels; the oracle
 * computes the same definition more accurately, and rounds to the narrow
 * storage type at exactly the points the method stores: each slot write and
 * each output write.
 *
 * Layouts (all contiguous, row major):
 *   q, k        [n_tok][HK][K]          v, z, out  [n_tok][HV][V]
 *   a, b        [n_tok][HV]             pool       [num_slots][HV][V][K]
 *   A_log, dt_bias [HV]                 norm_weight [V]
 * The pool holds values already representable in its storage format; after a
 * write each stored value is again representable (orc_round).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Storage formats understood by orc_round. */
enum { ORC_FMT_F32 = 0, ORC_FMT_F16 = 1, ORC_FMT_BF16 = 2, ORC_FMT_F64 = 3,
       ORC_FMT_F8E4M3 = 4 };

/* Return codes. */
enum { ORC_OK = 0, ORC_BAD_ARG = 1, ORC_BAD_INDEX = 2, ORC_NO_MEMORY = 3 };

/*
 * Nearest value to x that the binary format `fmt` can hold, ties to even
 * (IEEE 754 roundTiesToEven), with gradual underflow and overflow to +-inf.
 * The reports fix only that arithmetic is wide and storage narrow ([52191]
 * 实现拆解 4);
 * round-to-nearest-even is the IEEE default and the plainest reading.
 *
 *   format  significant bits  smallest normal  subnormal spacing  largest finite
 *   f32     24                2^-126           2^-149             (2-2^-23)*2^127
 *   f16     11                2^-14            2^-24              65504
 *   bf16     8                2^-126           2^-133             (2-2^-7)*2^127
 *   fp8 e4m3 4                2^-6             2^-9               448
 * The FP8 state format is OCP E4M3 without infinities; the reports only say
 * the state type leaves room for FP8, so the plainest reading is taken:
 * nearest-even, and values beyond 448 (infinities included) saturate to
 * +-448 rather than becoming NaN, which a recurrent state would never shed.
 */
double orc_round(int fmt, double x)
{
    int p, emin;          /* precision, exponent of the smallest normal */
    double maxfin;
    int e, q;
    double r;

    switch (fmt) {
    case ORC_FMT_F64: return x;
    case ORC_FMT_F32: p = 24; emin = -126; maxfin = ldexp(2.0 - ldexp(1.0, -23), 127); break;
    case ORC_FMT_F16: p = 11; emin = -14;  maxfin = 65504.0; break;
    case ORC_FMT_BF16: p = 8; emin = -126; maxfin = ldexp(2.0 - ldexp(1.0, -7), 127); break;
    case ORC_FMT_F8E4M3: p = 4; emin = -6; maxfin = 448.0; break;
    default: return NAN;
    }
    if (fmt == ORC_FMT_F8E4M3 && isinf(x))
        return x > 0 ? maxfin : -maxfin;
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    /* x = m * 2^e with 0.5 <= |m| < 1, so |x| lies in [2^(e-1), 2^e). */
    (void)frexp(x, &e);
    /* Spacing of representable numbers around x is 2^q. */
    q = e - p;
    if (q < emin - p + 1)
        q = emin - p + 1;
    /* Scaling by a power of two is exact; nearbyint rounds ties to even in
     * the default rounding mode. */
    r = ldexp(nearbyint(ldexp(x, -q)), q);
    if (fabs(r) > maxfin) {
        if (fmt == ORC_FMT_F8E4M3)
            return x > 0 ? maxfin : -maxfin;
        return x > 0 ? INFINITY : -INFINITY;
    }
    return r;
}

/* softplus with the threshold the CPU kernel takes as an argument
 * ([46090] 关键源码片段, `softplus_threshold`); its value is not printed, 20
 * is taken: above it softplus(x) equals x to far below double resolution. */
static double softplus(double x)
{
    return x > 20.0 ? x : log1p(exp(x));
}

static double sigmoid(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

static double silu(double x)
{
    return x / (1.0 + exp(-x));
}

/*
 * Gate scalars for one (token row, v-head).
 * [46090] passes A_log, a, dt_bias, b and a softplus threshold to the fused
 * sigmoid-gating update; [52191] 实现拆解 4 scales the state by exp(g).
 * Reading: g = -exp(A_log) * softplus(a + dt_bias) so alpha = exp(g) is a
 * decay in (0, 1]; beta = sigmoid(b) is the write strength in (0, 1).
 */
static void gates(double a, double b, double A_log, double dt_bias,
                  double *alpha, double *beta)
{
    double g = -exp(A_log) * softplus(a + dt_bias);
    *alpha = exp(g);
    *beta = sigmoid(b);
}

/*
 * In-kernel q/k L2 normalisation (use_qk_l2norm_in_kernel=True, [51812]
 * 关键源码片段; the body is elided in [46090]).  Reading: x / sqrt(sum x^2 +
 * 1e-6) over the head dimension, then `scale` applied to q only
 * ([51674] 实现拆解 2: scale = 128**-0.5).
 */
static void l2norm_scaled(const double *x, int n, double scale, double *y)
{
    double ss = 0.0;
    int i;
    for (i = 0; i < n; ++i)
        ss += x[i] * x[i];
    for (i = 0; i < n; ++i)
        y[i] = x[i] * (scale / sqrt(ss + 1e-6));
}

/* Scratch for one (sequence, v-head) unit. */
typedef struct {
    double *S;   /* V x K carry, row v holds S[v][0..K-1] */
    double *kn;  /* K: normalised key */
    double *qn;  /* K: normalised, scaled query */
    double *d;   /* V: delta */
    double *o;   /* V: read-out */
} unit_scratch;

static int scratch_alloc(unit_scratch *w, int K, int V)
{
    w->S = (double *)malloc(sizeof(double) * (size_t)V * (size_t)K);
    w->kn = (double *)malloc(sizeof(double) * (size_t)K);
    w->qn = (double *)malloc(sizeof(double) * (size_t)K);
    w->d = (double *)malloc(sizeof(double) * (size_t)V);
    w->o = (double *)malloc(sizeof(double) * (size_t)V);
    return w->S && w->kn && w->qn && w->d && w->o;
}

static void scratch_free(unit_scratch *w)
{
    free(w->S); free(w->kn); free(w->qn); free(w->d); free(w->o);
}

typedef struct {
    const double *q, *k, *v, *z, *a, *b;
    const double *A_log, *dt_bias, *norm_weight;
    double *out;
    int out_fmt;
    double *pool;
    int state_fmt;
    int64_t num_slots;
    int HK, HV, K, V;
    double scale, norm_eps;
} layer_t;

/*
 * One draft token of the recurrence for the unit (head h) whose carry is
 * w->S, followed by the slot store and the gated-RMSNorm epilogue.
 *
 * Order ([51674] 实现拆解 1; [46090] spec kernel excerpt, whose per-token
 * steps update the state, produce the output, then store the state in the
 * token's own slot):
 *   S <- alpha * S                      decay first (reading: only this order
 *                                       makes beta=1 retrieve v exactly)
 *   d <- beta * (v - S k^)              delta toward v along k^
 *   S <- S + d k^T                      rank-1 write
 *   o <- S q^                           read-out after the token's update
 *   pool[wslot, h] <- round(S)          every post-token state to its slot
 *                                       (skipped for wslot < 0: the prefill
 *                                       loop stores at chunk ends itself)
 *   out[row, h] <- round(RMSNorm(o) * w * silu(z))   gated RMSNorm over V
 * The carry S itself stays in double: rounding happens only in the store
 * ([52191] 实现拆解 4: only slot reads/writes go through the state type).
 */
static void token_step(const layer_t *L, unit_scratch *w, int h, int64_t row,
                       int64_t wslot)
{
    const int K = L->K, V = L->V;
    const int kh = h / (L->HV / L->HK);  /* non-interleaved GQA ([46090]) */
    double alpha, beta, ms, rr;
    int i, vv;

    gates(L->a[row * L->HV + h], L->b[row * L->HV + h], L->A_log[h],
          L->dt_bias[h], &alpha, &beta);
    l2norm_scaled(L->k + (row * L->HK + kh) * K, K, 1.0, w->kn);
    l2norm_scaled(L->q + (row * L->HK + kh) * K, K, L->scale, w->qn);

    for (vv = 0; vv < V; ++vv)
        for (i = 0; i < K; ++i)
            w->S[vv * K + i] *= alpha;

    for (vv = 0; vv < V; ++vv) {
        double u = 0.0;
        for (i = 0; i < K; ++i)
            u += w->S[vv * K + i] * w->kn[i];
        w->d[vv] = beta * (L->v[(row * L->HV + h) * V + vv] - u);
    }
    for (vv = 0; vv < V; ++vv)
        for (i = 0; i < K; ++i)
            w->S[vv * K + i] += w->d[vv] * w->kn[i];

    for (vv = 0; vv < V; ++vv) {
        double acc = 0.0;
        for (i = 0; i < K; ++i)
            acc += w->S[vv * K + i] * w->qn[i];
        w->o[vv] = acc;
    }

    if (wslot >= 0) {
        double *dst = L->pool + (wslot * L->HV + h) * (int64_t)V * K;
        for (i = 0; i < V * K; ++i)
            dst[i] = orc_round(L->state_fmt, w->S[i]);
    }

    /* Gated RMSNorm, one (token, v-head) over its V outputs ([51674]
     * 实现拆解 1 and 3: one block owns one v-head; "SiLU gating";
     * norm_eps=1e-5).  Normalise, then weight, then gate. */
    ms = 0.0;
    for (vv = 0; vv < V; ++vv)
        ms += w->o[vv] * w->o[vv];
    ms /= V;
    rr = 1.0 / sqrt(ms + L->norm_eps);
    for (vv = 0; vv < V; ++vv) {
        double y = w->o[vv] * rr * L->norm_weight[vv] *
                   silu(L->z[(row * L->HV + h) * V + vv]);
        L->out[(row * L->HV + h) * V + vv] = orc_round(L->out_fmt, y);
    }
}

static int layer_ok(const layer_t *L)
{
    if (!L->q || !L->k || !L->v || !L->z || !L->a || !L->b || !L->A_log ||
        !L->dt_bias || !L->norm_weight || !L->out || !L->pool)
        return 0;
    if (L->HK <= 0 || L->HV <= 0 || L->K <= 0 || L->V <= 0 || L->HV % L->HK)
        return 0;
    return 1;
}

static int fmt_ok(int f)
{
    return f == ORC_FMT_F32 || f == ORC_FMT_F16 || f == ORC_FMT_BF16 ||
           f == ORC_FMT_F64 || f == ORC_FMT_F8E4M3;
}

/*
 * Speculative update.  For every sequence b with L_b = cu[b+1]-cu[b] > 0 and
 * every v-head h ([46090] spec kernel; [51674] 实现拆解 1):
 *   r = spec_idx[b*spec_stride + max(acc_b - 1, 0)]   clamped rewind slot
 *   S = pool[r, h]                                    whole tile, read first
 *   for t < L_b: token row = token_indx ? token_indx[cu[b]+t] : cu[b]+t
 *                ([51812]: one index gathers q/k/v and the gates a/b; the
 *                output goes back to the same row), token_step(), store to
 *                slot spec_idx[b*spec_stride + t].
 * Output rows of skipped sequences are left untouched.
 *
 * Every index is checked before anything is written: out-of-range slots or
 * rows, 0 > acc or acc > spec_stride, L_b > spec_stride return ORC_BAD_INDEX.
 */
int orc_spec_update(const double *q, const double *k, const double *v,
                    const double *z, const double *a, const double *b,
                    const double *A_log, const double *dt_bias,
                    const double *norm_weight, double *out, int out_fmt,
                    double *pool, int state_fmt, int64_t num_slots,
                    int64_t n_tok, const int32_t *cu_seqlens, int32_t B,
                    const int32_t *spec_idx, int64_t spec_stride,
                    const int32_t *num_acc, const int32_t *token_indx,
                    int32_t HK, int32_t HV, int32_t K, int32_t V,
                    double scale, double norm_eps)
{
    layer_t L = {q, k, v, z, a, b, A_log, dt_bias, norm_weight, out, out_fmt,
                 pool, state_fmt, num_slots, HK, HV, K, V, scale, norm_eps};
    unit_scratch w;
    int32_t bi;
    int h, t;

    if (!layer_ok(&L) || !fmt_ok(out_fmt) || !fmt_ok(state_fmt) || B < 0 ||
        !cu_seqlens || (B > 0 && (!spec_idx || !num_acc)) || spec_stride <= 0)
        return ORC_BAD_ARG;

    /* Validate every index the computation will use. */
    for (bi = 0; bi < B; ++bi) {
        int64_t len = (int64_t)cu_seqlens[bi + 1] - cu_seqlens[bi];
        int64_t acc = num_acc[bi], j;
        if (len <= 0)
            continue;
        if (cu_seqlens[bi] < 0 || len > spec_stride || acc < 0 ||
            acc > spec_stride)
            return ORC_BAD_INDEX;
        j = acc - 1 > 0 ? acc - 1 : 0;
        if (spec_idx[bi * spec_stride + j] < 0 ||
            spec_idx[bi * spec_stride + j] >= num_slots)
            return ORC_BAD_INDEX;
        for (t = 0; t < len; ++t) {
            int64_t g = (int64_t)cu_seqlens[bi] + t;
            int64_t row = token_indx ? token_indx[g] : g;
            int32_t ws = spec_idx[bi * spec_stride + t];
            if (row < 0 || row >= n_tok || ws < 0 || ws >= num_slots)
                return ORC_BAD_INDEX;
        }
    }

    if (!scratch_alloc(&w, K, V)) {
        scratch_free(&w);
        return ORC_NO_MEMORY;
    }
    for (bi = 0; bi < B; ++bi) {
        int64_t start = cu_seqlens[bi];
        int64_t len = (int64_t)cu_seqlens[bi + 1] - start;
        int64_t acc = num_acc[bi];
        int64_t r;
        if (len <= 0)
            continue;  /* q_len <= 0: nothing read, written or output */
        r = spec_idx[bi * spec_stride + (acc - 1 > 0 ? acc - 1 : 0)];
        for (h = 0; h < HV; ++h) {
            const double *src = pool + (r * HV + h) * (int64_t)V * K;
            memcpy(w.S, src, sizeof(double) * (size_t)V * (size_t)K);
            for (t = 0; t < len; ++t) {
                int64_t g = start + t;
                int64_t row = token_indx ? token_indx[g] : g;
                token_step(&L, &w, h, row, spec_idx[bi * spec_stride + t]);
            }
        }
    }
    scratch_free(&w);
    return ORC_OK;
}

/*
 * Non-speculative decode: one token per entry i, state read from and written
 * back to the same slot state_indices[i] (in place).  A negative slot marks a
 * padded entry, which is skipped.  Row = token_indx ? token_indx[i] : i.
 */
int orc_decode_update(const double *q, const double *k, const double *v,
                      const double *z, const double *a, const double *b,
                      const double *A_log, const double *dt_bias,
                      const double *norm_weight, double *out, int out_fmt,
                      double *pool, int state_fmt, int64_t num_slots,
                      int64_t n_tok, const int32_t *state_indices, int32_t N,
                      const int32_t *token_indx, int32_t HK, int32_t HV,
                      int32_t K, int32_t V, double scale, double norm_eps)
{
    layer_t L = {q, k, v, z, a, b, A_log, dt_bias, norm_weight, out, out_fmt,
                 pool, state_fmt, num_slots, HK, HV, K, V, scale, norm_eps};
    unit_scratch w;
    int32_t i;
    int h;

    if (!layer_ok(&L) || !fmt_ok(out_fmt) || !fmt_ok(state_fmt) || N < 0 ||
        (N > 0 && !state_indices))
        return ORC_BAD_ARG;
    for (i = 0; i < N; ++i) {
        int64_t row = token_indx ? token_indx[i] : i;
        if (state_indices[i] < 0)
            continue;
        if (state_indices[i] >= num_slots || row < 0 || row >= n_tok)
            return ORC_BAD_INDEX;
    }
    if (!scratch_alloc(&w, K, V)) {
        scratch_free(&w);
        return ORC_NO_MEMORY;
    }
    for (i = 0; i < N; ++i) {
        int64_t s = state_indices[i];
        int64_t row = token_indx ? token_indx[i] : i;
        if (s < 0)
            continue;
        for (h = 0; h < HV; ++h) {
            memcpy(w.S, pool + (s * HV + h) * (int64_t)V * K,
                   sizeof(double) * (size_t)V * (size_t)K);
            token_step(&L, &w, h, row, s);
        }
    }
    scratch_free(&w);
    return ORC_OK;
}

/*
 * Chunked prefill of B sequences, rows cu[b] .. cu[b+1]-1 (or
 * token_indx[cu[b] + t]), one state slot per sequence, state_indices[b]
 * (negative: skipped).  [52191] 实现拆解 3-4 and its test notes: the
 * inter-chunk kernel expands the narrow state into an FP32 buffer, runs the
 * chunk in FP32 and writes the buffer back to the slot at the chunk's end, so
 * the state is rounded once per chunk; the reference recurrence it is tested
 * against takes a state dtype and a write interval to reproduce exactly that.
 * Reading: per (sequence, v-head)
 *   S = has_initial_state[b] ? pool[s, h] : 0       (NULL: every sequence has one)
 *   for t < L_b: token_step() without a slot store; then, after every
 *     chunk_size-th token of the call and after its last token:
 *     pool[s, h] <- round(S) and S <- that rounded value
 * Token semantics, the gated-RMSNorm output and the GQA map are those of the
 * decode step, so a chunk of one token is one decode call (pinned).
 */
int orc_prefill_update(const double *q, const double *k, const double *v,
                       const double *z, const double *a, const double *b,
                       const double *A_log, const double *dt_bias,
                       const double *norm_weight, double *out, int out_fmt,
                       double *pool, int state_fmt, int64_t num_slots,
                       int64_t n_tok, const int32_t *cu_seqlens, int32_t B,
                       const int32_t *state_indices,
                       const int32_t *has_initial_state,
                       const int32_t *token_indx, int32_t chunk_size,
                       int32_t HK, int32_t HV, int32_t K, int32_t V,
                       double scale, double norm_eps)
{
    layer_t L = {q, k, v, z, a, b, A_log, dt_bias, norm_weight, out, out_fmt,
                 pool, state_fmt, num_slots, HK, HV, K, V, scale, norm_eps};
    unit_scratch w;
    int32_t bi;
    int h;
    int64_t t, i;

    if (!layer_ok(&L) || !fmt_ok(out_fmt) || !fmt_ok(state_fmt) || B < 0 ||
        chunk_size < 1 || (B > 0 && (!cu_seqlens || !state_indices)))
        return ORC_BAD_ARG;
    for (bi = 0; bi < B; ++bi) {
        int64_t start = cu_seqlens[bi];
        int64_t len = (int64_t)cu_seqlens[bi + 1] - start;
        if (len <= 0 || state_indices[bi] < 0)
            continue;
        if (start < 0 || state_indices[bi] >= num_slots)
            return ORC_BAD_INDEX;
        for (t = 0; t < len; ++t) {
            int64_t row = token_indx ? token_indx[start + t] : start + t;
            if (row < 0 || row >= n_tok)
                return ORC_BAD_INDEX;
        }
    }
    if (!scratch_alloc(&w, K, V)) {
        scratch_free(&w);
        return ORC_NO_MEMORY;
    }
    for (bi = 0; bi < B; ++bi) {
        int64_t start = cu_seqlens[bi];
        int64_t len = (int64_t)cu_seqlens[bi + 1] - start;
        int64_t s = state_indices[bi];
        if (len <= 0 || s < 0)
            continue;
        for (h = 0; h < HV; ++h) {
            double *slot = pool + (s * HV + h) * (int64_t)V * K;
            if (!has_initial_state || has_initial_state[bi])
                memcpy(w.S, slot, sizeof(double) * (size_t)V * (size_t)K);
            else
                memset(w.S, 0, sizeof(double) * (size_t)V * (size_t)K);
            for (t = 0; t < len; ++t) {
                int64_t row = token_indx ? token_indx[start + t] : start + t;
                token_step(&L, &w, h, row, -1);
                if ((t + 1) % chunk_size == 0 || t == len - 1)
                    for (i = 0; i < (int64_t)V * K; ++i)
                        slot[i] = w.S[i] = orc_round(state_fmt, w.S[i]);
            }
        }
    }
    scratch_free(&w);
    return ORC_OK;
}
