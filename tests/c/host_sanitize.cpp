// host_sanitize.cpp -- the CPU oracle and the library's host-side checks
// under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// TEST INFRASTRUCTURE: built with g++/gcc -fsanitize=address,undefined by
// tests/test_host_sanitizers.py (host code only, no device code, no GPU) and
// linked from oracle/*.c and the library's host sources (gdn_host.cpp,
// conv_host.cpp).  The two sides are called separately; nothing here passes
// data from one to the other.
//
// Why: the metadata of this path is caller-supplied index arrays, read with
// no length next to them.  The one memory bug the vLLM PR #46090 report
// records on the CPU spec kernel (评论区精华: num_accepted = 0 made acc - 1
// underflow into an out-of-bounds read, found by static analysis) is of that
// kind, and the same report notes spec_state_indices is never validated.
// This driver runs every oracle entry over the edge cases of that metadata
// (acc 0 .. T, empty and full sequences, padding, gathers, chunk ends,
// rejected indices) and every validator over valid and invalid metadata,
// so that an out-of-bounds access or undefined operation aborts the run.
// Prints "HOST_SANITIZE ok" and exits 0 when every expectation holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../speculative_decode_amd/csrc/gdn_internal.h"

extern "C" {
int orc_spec_update(const double* q, const double* k, const double* v, const double* z,
                    const double* a, const double* b, const double* A_log,
                    const double* dt_bias, const double* norm_weight, double* out, int out_fmt,
                    double* pool, int state_fmt, int64_t num_slots, int64_t n_tok,
                    const int32_t* cu_seqlens, int32_t B, const int32_t* spec_idx,
                    int64_t spec_stride, const int32_t* num_acc, const int32_t* token_indx,
                    int32_t HK, int32_t HV, int32_t K, int32_t V, double scale,
                    double norm_eps);
int orc_decode_update(const double* q, const double* k, const double* v, const double* z,
                      const double* a, const double* b, const double* A_log,
                      const double* dt_bias, const double* norm_weight, double* out,
                      int out_fmt, double* pool, int state_fmt, int64_t num_slots,
                      int64_t n_tok, const int32_t* state_indices, int32_t N,
                      const int32_t* token_indx, int32_t HK, int32_t HV, int32_t K, int32_t V,
                      double scale, double norm_eps);
int orc_prefill_update(const double* q, const double* k, const double* v, const double* z,
                       const double* a, const double* b, const double* A_log,
                       const double* dt_bias, const double* norm_weight, double* out,
                       int out_fmt, double* pool, int state_fmt, int64_t num_slots,
                       int64_t n_tok, const int32_t* cu_seqlens, int32_t B,
                       const int32_t* state_indices, const int32_t* has_initial_state,
                       const int32_t* token_indx, int32_t chunk_size, int32_t HK, int32_t HV,
                       int32_t K, int32_t V, double scale, double norm_eps);
int orc_conv_update(const double* x, double* out, int out_fmt, double* cache, int cache_fmt,
                    int64_t num_lines, int32_t state_len, int64_t n_tok, int32_t C,
                    int32_t width, const double* weight, const double* bias, int32_t act,
                    const int32_t* cu_seqlens, int32_t B, const int32_t* lines,
                    const int32_t* num_acc, const int32_t* token_indx);
double orc_round(int fmt, double x);
}

namespace {

int g_fail = 0;

void expect(bool ok, const char* what)
{
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s\n", what);
        ++g_fail;
    }
}

struct Lcg {
    uint64_t s;
    double uniform()   // [0, 1)
    {
        s = s * 6364136223846793005ULL + 1442695040888963407ULL;
        return static_cast<double>(s >> 11) * (1.0 / 9007199254740992.0);
    }
    double normalish() { return 2.0 * (uniform() + uniform() + uniform() - 1.5); }
};

// Inputs of one small layer: exact-size heap arrays, so that any read past
// an end is an ASan report.
struct Layer {
    int HK, HV, K, V;
    int64_t n_tok;
    std::vector<double> q, k, v, z, a, b, A_log, dt_bias, w, out;
    Layer(int HK_, int HV_, int K_, int V_, int64_t n, Lcg& r)
        : HK(HK_), HV(HV_), K(K_), V(V_), n_tok(n)
    {
        auto fill = [&](std::vector<double>& x, size_t m, double s) {
            x.resize(m);
            for (auto& e : x) e = s * r.normalish();
        };
        fill(q, n * HK * K, 1.0);
        fill(k, n * HK * K, 1.0);
        fill(v, n * HV * V, 1.0);
        fill(z, n * HV * V, 1.0);
        fill(a, n * HV, 1.0);
        fill(b, n * HV, 1.0);
        fill(A_log, HV, 0.5);
        fill(dt_bias, HV, 0.3);
        fill(w, V, 0.2);
        for (auto& e : w) e += 1.0;
        out.assign(n * HV * V, 0.0);
    }
};

std::vector<double> make_pool(int64_t slots, const Layer& L, int fmt, Lcg& r)
{
    std::vector<double> p(static_cast<size_t>(slots) * L.HV * L.V * L.K);
    for (auto& e : p) e = orc_round(fmt, 0.1 * r.normalish());
    return p;
}

int spec(Layer& L, std::vector<double>& pool, int fmt, int64_t slots,
         const std::vector<int32_t>& cu, const std::vector<int32_t>& si, int stride,
         const std::vector<int32_t>& acc, const int32_t* tix)
{
    return orc_spec_update(L.q.data(), L.k.data(), L.v.data(), L.z.data(), L.a.data(),
                           L.b.data(), L.A_log.data(), L.dt_bias.data(), L.w.data(),
                           L.out.data(), 2, pool.data(), fmt, slots, L.n_tok, cu.data(),
                           static_cast<int32_t>(cu.size() - 1), si.data(), stride, acc.data(),
                           tix, L.HK, L.HV, L.K, L.V, 1.0 / std::sqrt(L.K), 1e-5);
}

void oracle_spec_cases(Lcg& r)
{
    // 5 sequences of up to 3 drafts, lengths 3, 0, 2, 1, 3 (9 rows); every
    // acceptance count 0..3 appears; pools with spare slots; every format.
    const std::vector<int32_t> cu = {0, 3, 3, 5, 6, 9};
    const int T = 3;
    for (int fmt : {0, 1, 2, 3, 4}) {
        for (int gather = 0; gather < 2; ++gather) {
            Layer L(1, 2, 8, 8, 9, r);
            const int64_t slots = 17;
            std::vector<double> pool = make_pool(slots, L, fmt, r);
            std::vector<int32_t> si(5 * T);
            for (int i = 0; i < 5 * T; ++i) si[i] = (7 * i + 3) % 17;   // distinct
            std::vector<int32_t> acc = {0, 3, 1, 2, 3};
            std::vector<int32_t> tix = {8, 2, 5, 0, 7, 1, 3, 6, 4};
            expect(spec(L, pool, fmt, slots, cu, si, T, acc, gather ? tix.data() : nullptr) == 0,
                   "oracle spec update on valid metadata");
            for (double e : L.out) expect(std::isfinite(e), "finite output");
            // rejected metadata: nothing written, no read past an array
            std::vector<double> before = pool;
            std::vector<int32_t> bad = si;
            bad[6] = 17;                        // slot out of range (sequence 2, token 0)
            expect(spec(L, pool, fmt, slots, cu, bad, T, acc, nullptr) != 0, "slot 17 rejected");
            std::vector<int32_t> bacc = acc;
            bacc[3] = 4;                                              // acc > stride
            expect(spec(L, pool, fmt, slots, cu, si, T, bacc, nullptr) != 0, "acc 4 rejected");
            bacc[3] = -1;
            expect(spec(L, pool, fmt, slots, cu, si, T, bacc, nullptr) != 0, "acc -1 rejected");
            std::vector<int32_t> btix = tix;
            btix[2] = 9;                                              // row out of range
            expect(spec(L, pool, fmt, slots, cu, si, T, acc, btix.data()) != 0,
                   "row 9 rejected");
            std::vector<int32_t> bcu = {0, 3, 3, 5, 6, 10};            // L = 4 > stride
            expect(spec(L, pool, fmt, slots, bcu, si, T, acc, nullptr) != 0,
                   "length 4 rejected");
            expect(std::memcmp(before.data(), pool.data(), pool.size() * sizeof(double)) == 0,
                   "a rejected call writes nothing");
        }
    }
}

void oracle_decode_and_prefill_cases(Lcg& r)
{
    for (int fmt : {0, 2, 4}) {
        Layer L(2, 4, 8, 8, 6, r);
        const int64_t slots = 9;
        std::vector<double> pool = make_pool(slots, L, fmt, r);
        const std::vector<int32_t> si = {4, -1, 0, 8, -3, 2};        // two padded entries
        const std::vector<int32_t> tix = {5, 4, 3, 2, 1, 0};
        expect(orc_decode_update(L.q.data(), L.k.data(), L.v.data(), L.z.data(), L.a.data(),
                                 L.b.data(), L.A_log.data(), L.dt_bias.data(), L.w.data(),
                                 L.out.data(), 1, pool.data(), fmt, slots, L.n_tok, si.data(), 6,
                                 tix.data(), L.HK, L.HV, L.K, L.V, 0.35, 1e-5) == 0,
               "oracle decode with padding");
        const std::vector<int32_t> bad = {4, 9, 0, 8, -3, 2};
        expect(orc_decode_update(L.q.data(), L.k.data(), L.v.data(), L.z.data(), L.a.data(),
                                 L.b.data(), L.A_log.data(), L.dt_bias.data(), L.w.data(),
                                 L.out.data(), 1, pool.data(), fmt, slots, L.n_tok, bad.data(),
                                 6, nullptr, L.HK, L.HV, L.K, L.V, 0.35, 1e-5) != 0,
               "decode slot 9 rejected");
    }
    // prefill: lengths 9, 0, 5 with chunk 4 (chunk ends inside and at the
    // end of a sequence), one sequence without an initial state, gathered.
    for (int fmt : {0, 1, 2, 4}) {
        Layer L(1, 2, 8, 8, 14, r);
        const int64_t slots = 4;
        std::vector<double> pool = make_pool(slots, L, fmt, r);
        const std::vector<int32_t> cu = {0, 9, 9, 14}, si = {3, 0, 1}, hi = {1, 1, 0};
        std::vector<int32_t> tix(14);
        for (int i = 0; i < 14; ++i) tix[i] = (5 * i + 2) % 14;
        for (int chunk : {1, 4, 64}) {
            expect(orc_prefill_update(L.q.data(), L.k.data(), L.v.data(), L.z.data(),
                                      L.a.data(), L.b.data(), L.A_log.data(), L.dt_bias.data(),
                                      L.w.data(), L.out.data(), 2, pool.data(), fmt, slots,
                                      L.n_tok, cu.data(), 3, si.data(), hi.data(), tix.data(),
                                      chunk, L.HK, L.HV, L.K, L.V, 0.35, 1e-5) == 0,
                   "oracle prefill");
        }
        const std::vector<int32_t> bsi = {3, 0, 4};
        expect(orc_prefill_update(L.q.data(), L.k.data(), L.v.data(), L.z.data(), L.a.data(),
                                  L.b.data(), L.A_log.data(), L.dt_bias.data(), L.w.data(),
                                  L.out.data(), 2, pool.data(), fmt, slots, L.n_tok, cu.data(),
                                  3, bsi.data(), nullptr, nullptr, 4, L.HK, L.HV, L.K, L.V,
                                  0.35, 1e-5) != 0,
               "prefill slot 4 rejected");
    }
}

void oracle_conv_cases(Lcg& r)
{
    // width 4, 3 sequences of up to 3 drafts (lengths 3, 0, 2) and buffer
    // lines of width - 2 + 3 positions; every acceptance from 0 to 3.
    const int C = 6, W = 4, T = 3, SL = W - 2 + T;
    const int64_t lines_n = 5, n_tok = 5;
    std::vector<double> x(n_tok * C), out(n_tok * C, 0.0), w(C * W), bias(C),
        cache(lines_n * SL * C);
    for (auto& e : x) e = r.normalish();
    for (auto& e : w) e = r.uniform() - 0.5;
    for (auto& e : bias) e = r.uniform() - 0.5;
    for (auto& e : cache) e = orc_round(2, r.normalish());
    const std::vector<int32_t> cu = {0, 3, 3, 5}, lines = {4, 0, 2}, tix = {3, 0, 4, 1, 2};
    for (int acc0 = 0; acc0 <= T; ++acc0) {
        const std::vector<int32_t> acc = {acc0, 1, T - acc0};
        expect(orc_conv_update(x.data(), out.data(), 2, cache.data(), 2, lines_n, SL, n_tok, C, W,
                               w.data(), bias.data(), 1, cu.data(), 3, lines.data(), acc.data(),
                               tix.data()) == 0,
               "oracle conv spec update");
    }
    const std::vector<int32_t> dec = {1, -1, 3, 0, -2};                // decode with padding
    expect(orc_conv_update(x.data(), out.data(), 0, cache.data(), 2, lines_n, SL, n_tok, C, W,
                           w.data(), nullptr, 0, nullptr, 5, dec.data(), nullptr, nullptr) == 0,
           "oracle conv decode");
    const std::vector<int32_t> bad = {5, 0, 2};
    const std::vector<int32_t> acc = {1, 1, 1};
    expect(orc_conv_update(x.data(), out.data(), 2, cache.data(), 2, lines_n, SL, n_tok, C, W,
                           w.data(), bias.data(), 1, cu.data(), 3, bad.data(), acc.data(),
                           nullptr) != 0,
           "conv line 5 rejected");
}

gdn_status vspec(int64_t slots, int64_t n_tok, const std::vector<int32_t>& cu, int maxq,
                 const std::vector<int32_t>& si, int stride, const std::vector<int32_t>& acc,
                 const int32_t* stix, const std::vector<int32_t>& ns, const int32_t* nstix)
{
    return gdn_validate_indices_host(slots, n_tok, cu.data(),
                                     static_cast<int32_t>(cu.size() - 1), maxq, si.data(), stride,
                                     acc.data(), stix, ns.empty() ? nullptr : ns.data(),
                                     static_cast<int32_t>(ns.size()), nstix);
}

void validator_cases()
{
    // 3 sequences of up to 4 drafts (lengths 4, 0, 2) plus 2 single tokens.
    const std::vector<int32_t> cu = {0, 4, 4, 6};
    const std::vector<int32_t> si = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11};
    const std::vector<int32_t> acc = {0, 4, 2};
    const std::vector<int32_t> stix = {7, 0, 1, 2, 3, 4};
    const std::vector<int32_t> ns = {12, -1}, nstix = {5, 6};
    expect(vspec(13, 8, cu, 4, si, 4, acc, stix.data(), ns, nstix.data()) == GDN_OK,
           "valid mixed metadata");
    struct Case {
        const char* what;
        std::vector<int32_t> cu, si, acc, stix, ns;
        int maxq;
    };
    const Case bad[] = {
        {"cu[0] != 0", {1, 4, 4, 6}, si, acc, stix, ns, 4},
        {"cu decreasing", {0, 4, 3, 6}, si, acc, stix, ns, 4},
        {"length > max_q_len", cu, si, acc, stix, ns, 3},
        {"acc > stride", cu, si, {0, 4, 5}, stix, ns, 4},
        {"acc < 0", cu, si, {0, 4, -1}, stix, ns, 4},
        {"write slot out of range", cu, {0, 1, 2, 13, 4, 5, 6, 7, 8, 9, 10, 11}, acc, stix, ns, 4},
        {"read slot out of range", cu, {0, 1, 2, 3, 4, 5, 6, 7, 8, -4, 10, 11}, {0, 4, 2}, stix,
         ns, 4},
        {"write slot twice", cu, {0, 1, 2, 3, 4, 5, 6, 7, 8, 1, 10, 11}, acc, stix, ns, 4},
        // sequence 2 (2 rows, acc 4) reads slot 11, which it does not write
        {"read slot written by another", cu, si, {0, 4, 4}, stix, {11, -1}, 4},
        {"row out of range", cu, si, acc, {7, 0, 1, 2, 3, 8}, ns, 4},
        {"row twice", cu, si, acc, {7, 0, 1, 2, 3, 7}, ns, 4},
        {"single-token slot out of range", cu, si, acc, stix, {13, -1}, 4},
    };
    for (const Case& c : bad)
        expect(vspec(13, 8, c.cu, c.maxq, c.si, 4, c.acc, c.stix.data(), c.ns, nstix.data()) ==
                   GDN_ERR_INVALID,
               c.what);
    // the single-token row is taken from the non-spec gather
    expect(vspec(13, 8, cu, 4, si, 4, acc, stix.data(), {12, 11}, std::vector<int32_t>{5, 0}.data())
               == GDN_ERR_INVALID,
           "single-token row used by a sequence");

    // prefill metadata
    const std::vector<int32_t> pcu = {0, 5, 5, 9}, psi = {2, 0, 1};
    expect(gdn_validate_prefill_indices_host(3, 9, pcu.data(), 3, psi.data(), nullptr) ==
               GDN_OK,
           "valid prefill metadata");
    const std::vector<int32_t> psi_dup = {2, 0, 2}, psi_oob = {2, 0, 3}, ptix = {0, 1, 2, 3, 4, 5,
                                                                                6, 7, 9};
    expect(gdn_validate_prefill_indices_host(3, 9, pcu.data(), 3, psi_dup.data(), nullptr) ==
               GDN_ERR_INVALID,
           "prefill slot twice");
    expect(gdn_validate_prefill_indices_host(3, 9, pcu.data(), 3, psi_oob.data(), nullptr) ==
               GDN_ERR_INVALID,
           "prefill slot out of range");
    expect(gdn_validate_prefill_indices_host(3, 9, pcu.data(), 3, psi.data(), ptix.data()) ==
               GDN_ERR_INVALID,
           "prefill row out of range");

    // conv metadata: width 4, state_len 6 (= width - 2 + 4)
    const std::vector<int32_t> ccu = {0, 4, 4, 6}, lines = {3, 0, 1}, cacc = {0, 4, 3};
    const std::vector<int32_t> dl = {2, -1}, dtix = {6, 7};
    expect(gdn_validate_conv_indices_host(4, 6, 4, 8, ccu.data(), 3, 4, lines.data(), cacc.data(),
                                          nullptr, dl.data(), 2, dtix.data()) == GDN_OK,
           "valid conv metadata");
    const std::vector<int32_t> lines_dup = {3, 0, 3}, cacc_far = {0, 4, 5}, dl_dup = {3, -1};
    expect(gdn_validate_conv_indices_host(4, 6, 4, 8, ccu.data(), 3, 4, lines_dup.data(),
                                          cacc.data(), nullptr, dl.data(), 2, dtix.data()) ==
               GDN_ERR_INVALID,
           "conv line twice");
    expect(gdn_validate_conv_indices_host(4, 6, 4, 8, ccu.data(), 3, 4, lines.data(),
                                          cacc_far.data(), nullptr, dl.data(), 2, dtix.data()) ==
               GDN_ERR_INVALID,
           "conv history outside the line");
    expect(gdn_validate_conv_indices_host(4, 6, 4, 8, ccu.data(), 3, 4, lines.data(), cacc.data(),
                                          nullptr, dl_dup.data(), 2, dtix.data()) ==
               GDN_ERR_INVALID,
           "conv decode line used by a sequence");
    expect(gdn_validate_conv_indices_host(4, 6, 4, 8, ccu.data(), 3, 4, lines.data(), cacc.data(),
                                          nullptr, dl.data(), 2, nullptr) == GDN_ERR_INVALID,
           "conv decode row used by a sequence");
    expect(gdn_validate_conv_indices_host(4, 5, 4, 8, ccu.data(), 3, 4, lines.data(), cacc.data(),
                                          nullptr, dl.data(), 2, dtix.data()) == GDN_ERR_INVALID,
           "conv buffer too short for 4 drafts");
}

void layer_check_cases()
{
    // check_layer / check_pool read only addresses and sizes: fake pointers.
    alignas(16) static char buf[1 << 12];
    gdn_layer L;
    std::memset(&L, 0, sizeof L);
    gdn_view* views[] = {&L.q, &L.k, &L.v, &L.z, &L.out};
    for (gdn_view* v : views) {
        v->data = buf;
        v->stride_tok = 256;
        v->stride_head = 128;
    }
    L.a.data = buf;
    L.a.stride_tok = 2;
    L.a.stride_head = 1;
    L.b = L.a;
    L.A_log = reinterpret_cast<const float*>(buf);
    L.dt_bias = reinterpret_cast<const float*>(buf);
    L.norm_weight = reinterpret_cast<const float*>(buf);
    L.act_dtype = GDN_BF16;
    L.out_dtype = GDN_BF16;
    L.num_k_heads = 1;
    L.num_v_heads = 2;
    L.head_k_dim = L.head_v_dim = 128;
    L.n_tok = 4;
    L.scale = 0.088f;
    L.norm_eps = 1e-5f;
    expect(gdn::check_layer(&L) == GDN_OK, "valid layer");
    gdn_layer M = L;
    M.norm_weight = reinterpret_cast<const float*>(buf + 4);
    expect(gdn::check_layer(&M) == GDN_ERR_INVALID, "norm_weight misaligned");
    M = L;
    M.num_k_heads = 2;
    M.num_v_heads = 3;
    expect(gdn::check_layer(&M) == GDN_ERR_INVALID, "HV not a multiple of HK");
    M = L;
    M.head_k_dim = 64;
    expect(gdn::check_layer(&M) == GDN_ERR_UNSUPPORTED, "K = 64 unsupported");
    expect(gdn::check_layer(nullptr) == GDN_ERR_INVALID, "NULL layer");
    gdn_state_pool P = {buf, GDN_BF16, 0, 4};
    expect(gdn::check_pool(&P) == GDN_OK, "valid pool");
    P.data = buf + 8;
    expect(gdn::check_pool(&P) == GDN_ERR_INVALID, "pool misaligned");
    expect(gdn_status_string(static_cast<gdn_status>(99)) != nullptr, "status name");
    expect(std::strlen(gdn_last_error()) > 0, "a reason is set");
}

}  // namespace

int main()
{
    Lcg r{20240601ULL};
    oracle_spec_cases(r);
    oracle_decode_and_prefill_cases(r);
    oracle_conv_cases(r);
    validator_cases();
    layer_check_cases();
    if (g_fail) {
        std::fprintf(stderr, "HOST_SANITIZE: %d expectation(s) failed\n", g_fail);
        return 1;
    }
    std::printf("HOST_SANITIZE ok\n");
    return 0;
}
