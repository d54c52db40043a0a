// Host-side half of the C ABI: argument checks, the thread-local error
// reason, status names and the metadata validator.  No device calls here;
// the launchers in gdn_kernels.hip call check_layer/check_pool first and
// enqueue nothing when they fail.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "gdn_internal.h"

namespace gdn {

static thread_local char g_err[512] = "";

gdn_status fail(gdn_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() { g_err[0] = '\0'; }

int dtype_size(int32_t dt)
{
    switch (dt) {
    case GDN_F32: return 4;
    case GDN_F16: return 2;
    case GDN_BF16: return 2;
    case GDN_F8E4M3: return 1;
    default: return 0;
    }
}

static bool aligned(const void* p, int64_t bytes)
{
    return (reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(bytes)) == 0;
}

// A q/k/v/z/out view: non-null (unless there are no rows at all), aligned to
// two elements with even strides (the kernel moves head-dim pairs), strides
// non-negative.
static gdn_status check_pair_view(const gdn_view& v, const char* name, int esz,
                                  int64_t n_tok)
{
    if (!v.data)
        return n_tok == 0 ? GDN_OK : fail(GDN_ERR_INVALID, "%s.data is NULL", name);
    if (v.stride_tok < 0 || v.stride_head < 0)
        return fail(GDN_ERR_INVALID, "%s has a negative stride", name);
    if (!aligned(v.data, 2 * esz) || (v.stride_tok & 1) || (v.stride_head & 1))
        return fail(GDN_ERR_INVALID,
                    "%s is misaligned: data must be %d-byte aligned and strides even",
                    name, 2 * esz);
    return GDN_OK;
}

gdn_status check_layer(const gdn_layer* L)
{
    if (!L)
        return fail(GDN_ERR_INVALID, "layer is NULL");
    const int ea = L->act_dtype == GDN_F8E4M3 ? 0 : dtype_size(L->act_dtype);
    const int eo = L->out_dtype == GDN_F8E4M3 ? 0 : dtype_size(L->out_dtype);
    if (!ea)
        return fail(GDN_ERR_UNSUPPORTED, "act_dtype %d is not f32/f16/bf16", L->act_dtype);
    if (!eo)
        return fail(GDN_ERR_UNSUPPORTED, "out_dtype %d is not f32/f16/bf16", L->out_dtype);
    if (L->num_k_heads <= 0 || L->num_v_heads <= 0)
        return fail(GDN_ERR_INVALID, "head counts must be positive (HK=%d HV=%d)",
                    L->num_k_heads, L->num_v_heads);
    if (L->num_v_heads % L->num_k_heads)
        return fail(GDN_ERR_INVALID, "num_v_heads %d is not a multiple of num_k_heads %d",
                    L->num_v_heads, L->num_k_heads);
    if (L->head_k_dim != GDN_HEAD_DIM || L->head_v_dim != GDN_HEAD_DIM)
        return fail(GDN_ERR_UNSUPPORTED, "head dims must be K = V = %d (got K=%d V=%d)",
                    GDN_HEAD_DIM, L->head_k_dim, L->head_v_dim);
    if (L->n_tok < 0)
        return fail(GDN_ERR_INVALID, "n_tok is negative");
    gdn_status st;
    const int64_t n = L->n_tok;
    if ((st = check_pair_view(L->q, "q", ea, n)) || (st = check_pair_view(L->k, "k", ea, n)) ||
        (st = check_pair_view(L->v, "v", ea, n)) || (st = check_pair_view(L->z, "z", ea, n)) ||
        (st = check_pair_view(L->out, "out", eo, n)))
        return st;
    const gdn_view* gates[2] = {&L->a, &L->b};
    const char* gname[2] = {"a", "b"};
    for (int i = 0; i < 2; ++i) {
        const gdn_view& g = *gates[i];
        if (!g.data && n == 0)
            continue;
        if (!g.data)
            return fail(GDN_ERR_INVALID, "%s.data is NULL", gname[i]);
        if (g.stride_head != 1 || g.stride_tok < 0)
            return fail(GDN_ERR_INVALID, "%s must have stride_head 1 and stride_tok >= 0",
                        gname[i]);
        if (!aligned(g.data, ea))
            return fail(GDN_ERR_INVALID, "%s is misaligned", gname[i]);
    }
    if (!L->A_log || !L->dt_bias || !L->norm_weight)
        return fail(GDN_ERR_INVALID, "A_log, dt_bias and norm_weight must be non-NULL");
    if (!aligned(L->A_log, 4) || !aligned(L->dt_bias, 4))
        return fail(GDN_ERR_INVALID, "A_log and dt_bias must be 4-byte aligned");
    // the kernels read norm_weight as float pairs
    if (!aligned(L->norm_weight, 8))
        return fail(GDN_ERR_INVALID, "norm_weight must be 8-byte aligned");
    if (!(L->norm_eps >= 0.0f))
        return fail(GDN_ERR_INVALID, "norm_eps must be >= 0");
    return GDN_OK;
}

gdn_status check_pool(const gdn_state_pool* P)
{
    if (!P)
        return fail(GDN_ERR_INVALID, "pool is NULL");
    if (!dtype_size(P->dtype))
        return fail(GDN_ERR_UNSUPPORTED, "state dtype %d is not f32/f16/bf16/f8e4m3", P->dtype);
    if (!P->data)
        return fail(GDN_ERR_INVALID, "pool.data is NULL");
    if (!aligned(P->data, 16))
        return fail(GDN_ERR_INVALID, "pool.data must be 16-byte aligned");
    if (P->num_slots <= 0)
        return fail(GDN_ERR_INVALID, "pool.num_slots must be positive");
    return GDN_OK;
}

}  // namespace gdn

using gdn::fail;

extern "C" const char* gdn_last_error(void) { return gdn::g_err; }

extern "C" const char* gdn_status_string(gdn_status s)
{
    switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID: return "GDN_ERR_INVALID";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_DEVICE: return "GDN_ERR_DEVICE";
    default: return "GDN_STATUS_UNKNOWN";
    }
}

extern "C" int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

extern "C" void gdn_abi_struct_sizes(size_t* view, size_t* layer, size_t* pool)
{
    if (view) *view = sizeof(gdn_view);
    if (layer) *layer = sizeof(gdn_layer);
    if (pool) *pool = sizeof(gdn_state_pool);
}

// Closes the validation gap the CPU report (#46090, 评论区精华 / review
// highlights) leaves open: spec_state_indices is never checked there.
extern "C" gdn_status gdn_validate_indices_host(
    int64_t num_slots, int64_t n_tok, const int32_t* cu, int32_t num_seqs,
    int32_t max_q_len, const int32_t* spec_idx, int32_t spec_stride,
    const int32_t* num_acc, const int32_t* spec_tix, const int32_t* state_idx,
    int32_t num_non_spec, const int32_t* ns_tix)
{
    gdn::clear_error();
    if (num_seqs < 0 || num_non_spec < 0 || num_slots <= 0 || n_tok < 0)
        return fail(GDN_ERR_INVALID, "negative count or empty pool");
    if (num_seqs > 0) {
        if (!cu || !spec_idx || !num_acc)
            return fail(GDN_ERR_INVALID, "spec metadata pointer is NULL");
        if (spec_stride <= 0)
            return fail(GDN_ERR_INVALID, "spec_stride must be positive");
        if (max_q_len < 1 || max_q_len > GDN_MAX_DRAFT_TOKENS)
            return fail(GDN_ERR_INVALID, "max_q_len %d outside 1..%d", max_q_len,
                        GDN_MAX_DRAFT_TOKENS);
        if (cu[0] != 0)
            return fail(GDN_ERR_INVALID, "cu_seqlens[0] = %d, expected 0", cu[0]);
    }
    if (num_non_spec > 0 && !state_idx)
        return fail(GDN_ERR_INVALID, "state_indices is NULL");

    // slot -> writer (sequence id, or num_seqs + i for non-spec entry i)
    std::unordered_map<int64_t, int64_t> writer;
    std::vector<int64_t> reads(num_seqs, -1);
    std::vector<char> row_used(static_cast<size_t>(n_tok), 0);

    auto use_row = [&](int64_t row, const char* who, int64_t id) -> gdn_status {
        if (row < 0 || row >= n_tok)
            return fail(GDN_ERR_INVALID, "%s %lld: row %lld outside [0, %lld)", who,
                        (long long)id, (long long)row, (long long)n_tok);
        if (row_used[row])
            return fail(GDN_ERR_INVALID, "%s %lld: row %lld used twice", who,
                        (long long)id, (long long)row);
        row_used[row] = 1;
        return GDN_OK;
    };

    for (int32_t b = 0; b < num_seqs; ++b) {
        const int64_t len = static_cast<int64_t>(cu[b + 1]) - cu[b];
        if (len < 0)
            return fail(GDN_ERR_INVALID, "cu_seqlens decreases at sequence %d", b);
        if (len == 0)
            continue;
        if (len > max_q_len || len > spec_stride)
            return fail(GDN_ERR_INVALID, "sequence %d has %lld rows > max_q_len %d / stride %d",
                        b, (long long)len, max_q_len, spec_stride);
        const int64_t acc = num_acc[b];
        if (acc < 0 || acc > spec_stride)
            return fail(GDN_ERR_INVALID, "sequence %d: num_accepted %lld outside [0, %d]", b,
                        (long long)acc, spec_stride);
        const int64_t r = spec_idx[(int64_t)b * spec_stride + (acc > 1 ? acc - 1 : 0)];
        if (r < 0 || r >= num_slots)
            return fail(GDN_ERR_INVALID, "sequence %d: read slot %lld outside [0, %lld)", b,
                        (long long)r, (long long)num_slots);
        reads[b] = r;
        for (int64_t t = 0; t < len; ++t) {
            const int64_t w = spec_idx[(int64_t)b * spec_stride + t];
            if (w < 0 || w >= num_slots)
                return fail(GDN_ERR_INVALID, "sequence %d token %lld: slot %lld outside [0, %lld)",
                            b, (long long)t, (long long)w, (long long)num_slots);
            if (!writer.emplace(w, b).second)
                return fail(GDN_ERR_INVALID, "slot %lld is written twice", (long long)w);
            const int64_t g = static_cast<int64_t>(cu[b]) + t;
            gdn_status st = use_row(spec_tix ? spec_tix[g] : g, "sequence", b);
            if (st != GDN_OK)
                return st;
        }
    }
    for (int32_t i = 0; i < num_non_spec; ++i) {
        const int64_t s = state_idx[i];
        if (s < 0)
            continue;  // padding
        if (s >= num_slots)
            return fail(GDN_ERR_INVALID, "non-spec entry %d: slot %lld outside [0, %lld)", i,
                        (long long)s, (long long)num_slots);
        if (!writer.emplace(s, (int64_t)num_seqs + i).second)
            return fail(GDN_ERR_INVALID, "slot %lld is written twice", (long long)s);
        gdn_status st = use_row(ns_tix ? ns_tix[i] : i, "non-spec entry", i);
        if (st != GDN_OK)
            return st;
    }
    for (int32_t b = 0; b < num_seqs; ++b) {
        if (reads[b] < 0)
            continue;
        auto it = writer.find(reads[b]);
        if (it != writer.end() && it->second != b)
            return fail(GDN_ERR_INVALID,
                        "sequence %d reads slot %lld, which %s %lld writes", b,
                        (long long)reads[b],
                        it->second < num_seqs ? "sequence" : "non-spec entry",
                        (long long)(it->second < num_seqs ? it->second : it->second - num_seqs));
    }
    return GDN_OK;
}

extern "C" gdn_status gdn_validate_prefill_indices_host(int64_t num_slots, int64_t n_tok,
                                                        const int32_t* cu, int32_t num_seqs,
                                                        const int32_t* state_idx,
                                                        const int32_t* tix)
{
    gdn::clear_error();
    if (num_seqs < 0 || num_slots <= 0 || n_tok < 0)
        return fail(GDN_ERR_INVALID, "negative count or empty pool");
    if (num_seqs == 0)
        return GDN_OK;
    if (!cu || !state_idx)
        return fail(GDN_ERR_INVALID, "cu_seqlens or state_indices is NULL");
    if (cu[0] != 0)
        return fail(GDN_ERR_INVALID, "cu_seqlens[0] = %d, expected 0", cu[0]);
    std::vector<char> slot_used(static_cast<size_t>(num_slots), 0);
    std::vector<char> row_used(static_cast<size_t>(n_tok), 0);
    for (int32_t b = 0; b < num_seqs; ++b) {
        const int64_t len = static_cast<int64_t>(cu[b + 1]) - cu[b];
        if (len < 0)
            return fail(GDN_ERR_INVALID, "cu_seqlens decreases at sequence %d", b);
        const int64_t s = state_idx[b];
        if (len == 0 || s < 0)
            continue;
        if (s >= num_slots)
            return fail(GDN_ERR_INVALID, "sequence %d: slot %lld outside [0, %lld)", b,
                        (long long)s, (long long)num_slots);
        if (slot_used[s])
            return fail(GDN_ERR_INVALID, "slot %lld is used by two sequences", (long long)s);
        slot_used[s] = 1;
        for (int64_t t = 0; t < len; ++t) {
            const int64_t g = static_cast<int64_t>(cu[b]) + t;
            const int64_t row = tix ? tix[g] : g;
            if (row < 0 || row >= n_tok)
                return fail(GDN_ERR_INVALID, "sequence %d: row %lld outside [0, %lld)", b,
                            (long long)row, (long long)n_tok);
            if (row_used[row])
                return fail(GDN_ERR_INVALID, "sequence %d: row %lld used twice", b,
                            (long long)row);
            row_used[row] = 1;
        }
    }
    return GDN_OK;
}
