// abi_parity.cpp -- the speculative update through the C ABI alone, from a
// C++ caller with no Python, checked against the C oracle on the same inputs.
//
// TEST INFRASTRUCTURE: links the oracle (oracle/liboracle.so) next to the
// library; run by tests/test_gpu_c_abi.py.  Built in-tree by build().
//
// Batch: 3 sequences with 4, 2 and 4 draft tokens (HK = 1, HV = 4,
// K = V = 128), bf16 activations and output, a BF16 pool of 16 slots, the
// acceptances 0, 2 and 4.  Inputs come from a seeded 64-bit LCG, rounded to
// bf16 (nearest even) before either side sees them, so both sides read the
// same values.  Bars: state |gpu - oracle| <= 3e-2 + 3e-2 |oracle|; output
// relative L2 < 5e-4 over processed rows, both in bf16; untouched pool slots
// and output rows bit-identical.  Prints "ABI_PARITY ok" and exits 0 on
// success.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/gdn_spec.h"

extern "C" int orc_spec_update(const double* q, const double* k, const double* v,
                               const double* z, const double* a, const double* b,
                               const double* A_log, const double* dt_bias,
                               const double* norm_weight, double* out, int out_fmt,
                               double* pool, int state_fmt, int64_t num_slots, int64_t n_tok,
                               const int32_t* cu_seqlens, int32_t B, const int32_t* spec_idx,
                               int64_t spec_stride, const int32_t* num_acc,
                               const int32_t* token_indx, int32_t HK, int32_t HV, int32_t K,
                               int32_t V, double scale, double norm_eps);

namespace {

constexpr int B = 3, T = 4, HK = 1, HV = 4, D = 128, SLOTS = 16, ORC_BF16 = 2;

struct Lcg {
    uint64_t s;
    double uniform()  // [-1, 1)
    {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return static_cast<double>(s >> 11) * (2.0 / 9007199254740992.0) - 1.0;
    }
};

uint16_t to_bf16(float x)  // nearest even; inputs here are finite
{
    uint32_t u;
    std::memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

double from_bf16(uint16_t h)
{
    const uint32_t u = static_cast<uint32_t>(h) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// n bf16 values uniform in [-r, r): raw bits for the device, doubles for the oracle.
void draw(Lcg& g, size_t n, double r, std::vector<uint16_t>& bits, std::vector<double>& vals)
{
    bits.resize(n);
    vals.resize(n);
    for (size_t i = 0; i < n; ++i) {
        bits[i] = to_bf16(static_cast<float>(r * g.uniform()));
        vals[i] = from_bf16(bits[i]);
    }
}

template <class T_>
T_* upload(const std::vector<T_>& h)
{
    void* d = nullptr;
    if (hipMalloc(&d, h.size() * sizeof(T_)) != hipSuccess ||
        hipMemcpy(d, h.data(), h.size() * sizeof(T_), hipMemcpyHostToDevice) != hipSuccess) {
        std::printf("ABI_PARITY fail: device allocation or copy\n");
        std::exit(1);
    }
    return static_cast<T_*>(d);
}

}  // namespace

int main()
{
    if (gdn_abi_version() != GDN_ABI_VERSION) {
        std::printf("ABI_PARITY fail: library ABI %d, header %d\n", gdn_abi_version(),
                    GDN_ABI_VERSION);
        return 1;
    }
    const int32_t cu[B + 1] = {0, 4, 6, 10};
    const int32_t acc[B] = {0, 2, 4};
    const int n_tok = cu[B];
    Lcg g{20241202ull};

    std::vector<uint16_t> qb, kb, vb, zb, ab, bb, poolb, outb;
    std::vector<double> qd, kd, vd, zd, ad, bd, poold;
    draw(g, size_t(n_tok) * HK * D, 1.0, qb, qd);
    draw(g, size_t(n_tok) * HK * D, 1.0, kb, kd);
    draw(g, size_t(n_tok) * HV * D, 1.0, vb, vd);
    draw(g, size_t(n_tok) * HV * D, 1.0, zb, zd);
    draw(g, size_t(n_tok) * HV, 1.0, ab, ad);
    draw(g, size_t(n_tok) * HV, 1.0, bb, bd);
    draw(g, size_t(SLOTS) * HV * D * D, 0.1, poolb, poold);
    std::vector<float> A_log(HV), dt_bias(HV), w(D);
    std::vector<double> A_logd(HV), dt_biasd(HV), wd(D);
    for (int h = 0; h < HV; ++h) {
        A_log[h] = static_cast<float>(g.uniform());
        dt_bias[h] = static_cast<float>(0.5 * g.uniform());
        A_logd[h] = A_log[h];
        dt_biasd[h] = dt_bias[h];
    }
    for (int i = 0; i < D; ++i) {
        w[i] = static_cast<float>(1.0 + 0.5 * g.uniform());
        wd[i] = w[i];
    }
    // slots: a shuffle of 0..15; the first B*T are the draft-token slots
    int32_t perm[SLOTS];
    for (int i = 0; i < SLOTS; ++i)
        perm[i] = i;
    for (int i = SLOTS - 1; i > 0; --i) {
        const int j = static_cast<int>((g.uniform() + 1.0) * 0.5 * (i + 1)) % (i + 1);
        const int32_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
    std::vector<int32_t> sidx(perm, perm + B * T);
    outb.assign(size_t(n_tok) * HV * D, to_bf16(-3.0f));   // sentinel rows
    std::vector<double> outd(outb.size(), -3.0);

    // ---- the library, through the C ABI ----
    uint16_t* dq = upload(qb);
    uint16_t* dk = upload(kb);
    uint16_t* dv = upload(vb);
    uint16_t* dz = upload(zb);
    uint16_t* da = upload(ab);
    uint16_t* db = upload(bb);
    uint16_t* dout = upload(outb);
    uint16_t* dpool = upload(poolb);
    float* dA = upload(A_log);
    float* ddt = upload(dt_bias);
    float* dw = upload(w);
    int32_t* dcu = upload(std::vector<int32_t>(cu, cu + B + 1));
    int32_t* dacc = upload(std::vector<int32_t>(acc, acc + B));
    int32_t* dsidx = upload(sidx);

    gdn_layer L{};
    L.q = {dq, HK * D, D};
    L.k = {dk, HK * D, D};
    L.v = {dv, HV * D, D};
    L.z = {dz, HV * D, D};
    L.a = {da, HV, 1};
    L.b = {db, HV, 1};
    L.out = {dout, HV * D, D};
    L.A_log = dA;
    L.dt_bias = ddt;
    L.norm_weight = dw;
    L.act_dtype = GDN_BF16;
    L.out_dtype = GDN_BF16;
    L.num_k_heads = HK;
    L.num_v_heads = HV;
    L.head_k_dim = D;
    L.head_v_dim = D;
    L.n_tok = n_tok;
    L.scale = 1.0f / std::sqrt(static_cast<float>(D));
    L.norm_eps = 1e-5f;
    gdn_state_pool P{dpool, GDN_BF16, 0, SLOTS};
    const gdn_status st = gdn_spec_decode_update(&L, &P, dcu, B, T, dsidx, T, dacc, nullptr,
                                                 nullptr);
    if (st != GDN_OK) {
        std::printf("ABI_PARITY fail: %s: %s\n", gdn_status_string(st), gdn_last_error());
        return 1;
    }
    if (hipDeviceSynchronize() != hipSuccess) {
        std::printf("ABI_PARITY fail: device error\n");
        return 1;
    }
    std::vector<uint16_t> pool_gpu(poolb.size()), out_gpu(outb.size());
    if (hipMemcpy(pool_gpu.data(), dpool, pool_gpu.size() * 2, hipMemcpyDeviceToHost) ||
        hipMemcpy(out_gpu.data(), dout, out_gpu.size() * 2, hipMemcpyDeviceToHost)) {
        std::printf("ABI_PARITY fail: copy back\n");
        return 1;
    }

    // ---- the oracle on the same values ----
    const int rc = orc_spec_update(qd.data(), kd.data(), vd.data(), zd.data(), ad.data(),
                                   bd.data(), A_logd.data(), dt_biasd.data(), wd.data(),
                                   outd.data(), ORC_BF16, poold.data(), ORC_BF16, SLOTS, n_tok,
                                   cu, B, sidx.data(), T, acc, nullptr, HK, HV, D, D,
                                   static_cast<double>(L.scale), 1e-5);
    if (rc != 0) {
        std::printf("ABI_PARITY fail: oracle returned %d\n", rc);
        return 1;
    }

    // ---- compare ----
    const size_t tile = size_t(HV) * D * D;
    int bad_state = 0, changed_untouched = 0;
    for (int s = 0; s < SLOTS; ++s) {
        bool touched = false;
        for (int bi = 0; bi < B; ++bi)
            for (int t = 0; t < cu[bi + 1] - cu[bi]; ++t)
                touched |= sidx[bi * T + t] == s;
        for (size_t e = 0; e < tile; ++e) {
            const size_t i = s * tile + e;
            if (touched) {
                const double gv = from_bf16(pool_gpu[i]), ov = poold[i];
                bad_state += std::fabs(gv - ov) > 3e-2 + 3e-2 * std::fabs(ov);
            } else {
                changed_untouched += pool_gpu[i] != poolb[i];
            }
        }
    }
    double num = 0.0, den = 0.0;
    for (int r = 0; r < n_tok; ++r)
        for (int i = 0; i < HV * D; ++i) {
            const size_t j = size_t(r) * HV * D + i;
            const double gv = from_bf16(out_gpu[j]), ov = from_bf16(to_bf16(float(outd[j])));
            num += (gv - ov) * (gv - ov);
            den += ov * ov;
        }
    const double rel = std::sqrt(num / den);
    std::printf("ABI_PARITY state mismatches %d, untouched bytes changed %d, output rel L2 %.3e\n",
                bad_state, changed_untouched, rel);
    if (bad_state || changed_untouched || !(rel < 5e-4)) {
        std::printf("ABI_PARITY fail\n");
        return 1;
    }
    std::printf("ABI_PARITY ok\n");
    return 0;
}
