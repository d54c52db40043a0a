// Host-side half of the conv-update C ABI: argument checks, the metadata
// validator and the struct sizes.  No device calls; the launchers in
// conv_kernels.hip call these first and enqueue nothing when they fail.
#include <cstdint>
#include <vector>

#include "gdn_internal.h"

namespace gdn {

static bool aligned_to(const void* p, int64_t bytes)
{
    return (reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(bytes)) == 0;
}

gdn_status check_conv_layer(const gdn_conv_layer* L)
{
    if (!L)
        return fail(GDN_ERR_INVALID, "conv layer is NULL");
    const int ex = L->x_dtype == GDN_F8E4M3 ? 0 : dtype_size(L->x_dtype);
    const int eo = L->out_dtype == GDN_F8E4M3 ? 0 : dtype_size(L->out_dtype);
    if (!ex)
        return fail(GDN_ERR_UNSUPPORTED, "x_dtype %d is not f32/f16/bf16", L->x_dtype);
    if (!eo)
        return fail(GDN_ERR_UNSUPPORTED, "out_dtype %d is not f32/f16/bf16", L->out_dtype);
    if (L->channels <= 0)
        return fail(GDN_ERR_INVALID, "channels must be positive (got %d)", L->channels);
    if (L->width < 1)
        return fail(GDN_ERR_INVALID, "width must be >= 1 (got %d)", L->width);
    if (L->width > GDN_CONV_MAX_WIDTH)
        return fail(GDN_ERR_UNSUPPORTED, "width %d exceeds %d", L->width, GDN_CONV_MAX_WIDTH);
    if (L->activation != GDN_CONV_ACT_NONE && L->activation != GDN_CONV_ACT_SILU)
        return fail(GDN_ERR_INVALID, "activation %d is not NONE/SILU", L->activation);
    if (L->n_tok < 0)
        return fail(GDN_ERR_INVALID, "n_tok is negative");
    if (!L->weight)
        return fail(GDN_ERR_INVALID, "weight is NULL");
    if (!aligned_to(L->weight, 4) || (L->bias && !aligned_to(L->bias, 4)))
        return fail(GDN_ERR_INVALID, "weight and bias must be 4-byte aligned");
    if (L->n_tok == 0)
        return GDN_OK;
    if (!L->x || !L->out)
        return fail(GDN_ERR_INVALID, "x or out is NULL");
    if (L->x_stride_tok < 0)
        return fail(GDN_ERR_INVALID, "x_stride_tok is negative");
    if (L->out_stride_tok < L->channels)
        return fail(GDN_ERR_INVALID, "out_stride_tok %lld < channels %d: output rows overlap",
                    (long long)L->out_stride_tok, L->channels);
    if (!aligned_to(L->x, ex) || !aligned_to(L->out, eo))
        return fail(GDN_ERR_INVALID, "x and out must be aligned to their element size");
    return GDN_OK;
}

gdn_status check_conv_cache(const gdn_conv_cache* c, const gdn_conv_layer* L)
{
    if (!c)
        return fail(GDN_ERR_INVALID, "conv cache is NULL");
    if (!dtype_size(c->dtype))
        return fail(GDN_ERR_UNSUPPORTED, "cache dtype %d is not f32/f16/bf16", c->dtype);
    if (c->dtype != L->x_dtype)
        return fail(GDN_ERR_UNSUPPORTED,
                    "cache dtype %d differs from x_dtype %d (the buffer stores inputs as is)",
                    c->dtype, L->x_dtype);
    if (!c->data)
        return fail(GDN_ERR_INVALID, "cache.data is NULL");
    if (!aligned_to(c->data, dtype_size(c->dtype)))
        return fail(GDN_ERR_INVALID, "cache.data must be aligned to its element size");
    if (c->num_lines <= 0)
        return fail(GDN_ERR_INVALID, "cache.num_lines must be positive");
    if (c->state_len < L->width - 1 || c->state_len < 0)
        return fail(GDN_ERR_INVALID, "state_len %d < width - 1 = %d", c->state_len,
                    L->width - 1);
    if (c->stride_line < 0 || c->stride_pos < 0 || c->stride_chan < 0)
        return fail(GDN_ERR_INVALID, "cache strides must be non-negative");
    return GDN_OK;
}

}  // namespace gdn

using gdn::fail;

extern "C" void gdn_conv_abi_struct_sizes(size_t* layer, size_t* cache)
{
    if (layer) *layer = sizeof(gdn_conv_layer);
    if (cache) *cache = sizeof(gdn_conv_cache);
}

extern "C" gdn_status gdn_validate_conv_indices_host(
    int64_t num_lines, int32_t state_len, int32_t width, int64_t n_tok, const int32_t* cu,
    int32_t num_seqs, int32_t max_q_len, const int32_t* lines, const int32_t* num_acc,
    const int32_t* spec_tix, const int32_t* dec_lines, int32_t num_decode,
    const int32_t* dec_tix)
{
    gdn::clear_error();
    if (num_seqs < 0 || num_decode < 0 || num_lines <= 0 || n_tok < 0)
        return fail(GDN_ERR_INVALID, "negative count or empty buffer");
    if (width < 1 || state_len < width - 1)
        return fail(GDN_ERR_INVALID, "width %d / state_len %d inconsistent", width, state_len);
    if (num_seqs > 0) {
        if (!cu || !lines || !num_acc)
            return fail(GDN_ERR_INVALID, "spec metadata pointer is NULL");
        if (max_q_len < 1 || max_q_len > GDN_MAX_DRAFT_TOKENS)
            return fail(GDN_ERR_INVALID, "max_q_len %d outside 1..%d", max_q_len,
                        GDN_MAX_DRAFT_TOKENS);
        if (cu[0] != 0)
            return fail(GDN_ERR_INVALID, "cu_seqlens[0] = %d, expected 0", cu[0]);
    }
    if (num_decode > 0 && !dec_lines)
        return fail(GDN_ERR_INVALID, "decode line indices are NULL");

    std::vector<char> line_used(static_cast<size_t>(num_lines), 0);
    std::vector<char> row_used(static_cast<size_t>(n_tok), 0);
    auto use = [&](std::vector<char>& used, int64_t v, int64_t lim, const char* what,
                   const char* who, int64_t id) -> gdn_status {
        if (v < 0 || v >= lim)
            return fail(GDN_ERR_INVALID, "%s %lld: %s %lld outside [0, %lld)", who,
                        (long long)id, what, (long long)v, (long long)lim);
        if (used[v])
            return fail(GDN_ERR_INVALID, "%s %lld: %s %lld used twice", who, (long long)id,
                        what, (long long)v);
        used[v] = 1;
        return GDN_OK;
    };

    for (int32_t b = 0; b < num_seqs; ++b) {
        const int64_t len = static_cast<int64_t>(cu[b + 1]) - cu[b];
        if (len < 0)
            return fail(GDN_ERR_INVALID, "cu_seqlens decreases at sequence %d", b);
        if (len == 0)
            continue;
        if (len > max_q_len)
            return fail(GDN_ERR_INVALID, "sequence %d has %lld rows > max_q_len %d", b,
                        (long long)len, max_q_len);
        if (width - 2 + len > state_len)
            return fail(GDN_ERR_INVALID,
                        "sequence %d: width - 2 + %lld rows exceeds state_len %d", b,
                        (long long)len, state_len);
        const int64_t acc = num_acc[b];
        const int64_t o = acc > 1 ? acc - 1 : 0;
        if (acc < 0 || o + width - 1 > state_len)
            return fail(GDN_ERR_INVALID,
                        "sequence %d: num_accepted %lld puts the history outside the line", b,
                        (long long)acc);
        gdn_status st = use(line_used, lines[b], num_lines, "line", "sequence", b);
        if (st != GDN_OK)
            return st;
        for (int64_t t = 0; t < len; ++t) {
            const int64_t g = static_cast<int64_t>(cu[b]) + t;
            if ((st = use(row_used, spec_tix ? spec_tix[g] : g, n_tok, "row", "sequence", b)) !=
                GDN_OK)
                return st;
        }
    }
    for (int32_t i = 0; i < num_decode; ++i) {
        if (dec_lines[i] < 0)
            continue;  // padding
        gdn_status st = use(line_used, dec_lines[i], num_lines, "line", "decode entry", i);
        if (st != GDN_OK)
            return st;
        if ((st = use(row_used, dec_tix ? dec_tix[i] : i, n_tok, "row", "decode entry", i)) !=
            GDN_OK)
            return st;
    }
    return GDN_OK;
}
