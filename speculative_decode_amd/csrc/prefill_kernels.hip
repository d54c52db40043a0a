// prefill_kernels.hip -- chunked Gated DeltaNet prefill for CDNA4 (gfx950):
// the recurrence of the speculative-decode update run over whole prompts,
// one state slot per sequence, and its C-ABI entry point.
//
// What is computed is fixed by the vLLM PR reports on prhub.com.cn: the token
// step of the decode update (#51674 实现拆解 item 1, #46090 fla.cpp excerpt),
// and the chunk semantics of #52191 (实现拆解 items 3-4): FP32 arithmetic
// throughout, the state rounded to its storage dtype once per chunk, when the
// chunk's state is written back.  gdn_spec.h spells out the formula.
//
// How it is computed here -- two kernels, one (sequence, value head) unit per
// workgroup, chosen by chunk size:
//   * chunk_size >= 16: the chunkwise form on the FP32 matrix cores
//     (gdn_prefill_mma_kernel).  Tokens go 16 at a time (never across a chunk
//     end).  Within such a sub-chunk the token recurrence unrolls into dense
//     products, S0 [k^ | q^] and the state update S <- e^{G} S + D' K^T,
//     which run on v_mfma_f32_32x32x2f32, plus a 16 x 16 triangular solve
//     per value row on the vector ALU.  The decays are carried as sums of
//     log(alpha), so no product of decays under- or overflows.  The state
//     stays transposed in the matrix-core accumulator layout, which is also
//     the operand layout S0 needs for S0 [k^ | q^]: it never moves between
//     the two products.  About 6 K V flop per token and head against the
//     recurrence's 7, at twice the rate of non-packed FP32 vector issue.
//   * chunk_size < 16: the token recurrence itself (gdn_prefill_kernel): the
//     128 x 128 state in registers with the decode kernel's lane layout
//     (each 8-lane group owns a row at a time, each lane 16 elements), over
//     eight waves -- 2 rows per lane -- so that a SIMD has more waves to hide
//     the latency of each token's LDS reads and reductions.  Tokens are
//     taken 8 at a time; their normalised q/k, v, z, gates and k^.q^ are
//     staged in LDS (double-buffered), the next step's loads issued before
//     this step's token loop.
//   * Both read the state once, round it in registers at every chunk end,
//     and write it once: intermediate chunk write-backs go to the same slot
//     and are overwritten, so only the rounding is kept, not the stores.
//   * Prefill is compute-bound (about 130 flop per byte of HBM traffic).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dtype_cvt.h"
#include "gdn_internal.h"
#include "lane_ops.h"

namespace {

using namespace gdn_dev;

constexpr int D = GDN_HEAD_DIM;
constexpr int NTHREADS = 512;
constexpr int NWAVES = NTHREADS / 64;
constexpr int ROWS_PER_WAVE = D / NWAVES;
constexpr int RPT = ROWS_PER_WAVE / 8;               // rows per thread
constexpr int NE = D / 8;                            // elements per (thread, row): 16
constexpr int NXCD = 8;
constexpr int TS = 8;                                // tokens per step
constexpr int NTW = TS / NWAVES;                     // tokens per wave per step
static_assert(TS % NWAVES == 0 && RPT >= 1, "geometry");

struct PParams {
    const void* q;
    const void* k;
    const void* v;
    const void* z;
    const void* a;
    const void* b;
    void* out;
    int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, z_st, z_sh, a_st, b_st, o_st, o_sh;
    const float* A_log;
    const float* dt_bias;
    const float* norm_weight;
    void* pool;
    int64_t num_slots;
    int64_t n_tok;
    int32_t HV;
    int32_t group;
    float scale;
    float norm_eps;
    const int32_t* cu;
    const int32_t* state_idx;
    const int32_t* has_init;
    const int32_t* tix;
    int32_t chunk;
};

// One step's staging: normalised k and q, v, z, the read-outs o, the gate
// scalars and the rows of its 8 tokens.
struct Step {
    float k[TS][D];
    float q[TS][D];
    float v[TS][D];
    float o[TS][D];
    float z[TS][D];
    float alpha[TS], beta[TS], kq[TS];
    int64_t row[TS];
};

// A block barrier that orders LDS only.  The waves of a block exchange
// everything through LDS; __syncthreads() would also wait for every global
// load still in flight, so the activation loads issued a step ahead would
// cost a full memory latency at the next barrier.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The raw activations of one step for one wave (tokens wave, wave + NWAVES, ...).
template <int ACT>
struct StepRaw {
    typename Pair<ACT>::raw q[NTW], k[NTW], v[NTW], z[NTW];
    uint32_t a[NTW], b[NTW];
    int64_t row[NTW];
};

template <int ACT>
__device__ __forceinline__ void issue_step(const PParams& p, int64_t c0, int L, int step,
                                           int wave, int lane, int h, int kh, StepRaw<ACT>& r)
{
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int t = step * TS + wave + NWAVES * i;
        const int tt = t < L ? t : L - 1;        // clamped: always a valid row
        const int64_t row = p.tix ? static_cast<int64_t>(p.tix[c0 + tt]) : c0 + tt;
        r.row[i] = row;
        r.q[i] = load_pair_raw<ACT>(p.q, row * p.q_st + kh * p.q_sh + 2 * lane);
        r.k[i] = load_pair_raw<ACT>(p.k, row * p.k_st + kh * p.k_sh + 2 * lane);
        r.v[i] = load_pair_raw<ACT>(p.v, row * p.v_st + h * p.v_sh + 2 * lane);
        r.z[i] = load_pair_raw<ACT>(p.z, row * p.z_st + h * p.z_sh + 2 * lane);
        r.a[i] = load_one_raw<ACT>(p.a, row * p.a_st + h);
        r.b[i] = load_one_raw<ACT>(p.b, row * p.b_st + h);
    }
}

template <int ACT, int ST, int OUT>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(ST == GDN_F32 ? 2 : 4)))
gdn_prefill_kernel(const PParams p)
{
    constexpr int ESZ = ST == GDN_F32 ? 4 : (ST == GDN_F8E4M3 ? 1 : 2);
    constexpr int CH = D * ESZ / 128;
    constexpr int EPC = 16 / ESZ;
    constexpr int CSTRIDE = D / CH;
    static_assert(CH * EPC == NE, "layout");
    __shared__ __attribute__((aligned(16))) Step sb[2];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 3;
    const int j = lane & 7;

    // XCD-contiguous units: the heads of a sequence share its q/k rows.
    const uint32_t nblk = gridDim.x;
    const uint32_t xcd = blockIdx.x % NXCD;
    const uint32_t per = nblk / NXCD, rem = nblk % NXCD;
    const uint32_t unit = xcd * per + (xcd < rem ? xcd : rem) + blockIdx.x / NXCD;
    const uint32_t seq32 = unit / static_cast<uint32_t>(p.HV);
    const int64_t seq = seq32;
    const int h = static_cast<int>(unit - seq32 * static_cast<uint32_t>(p.HV));
    const int kh = static_cast<int>(static_cast<uint32_t>(h) / static_cast<uint32_t>(p.group));

    // ---- metadata; a sequence with any out-of-range field is skipped whole ----
    const int64_t c0 = p.cu[seq];
    const int L = static_cast<int>(p.cu[seq + 1] - c0);
    const int64_t slot = p.state_idx[seq];
    if (L <= 0 || slot < 0)
        return;
    bool bad = slot >= p.num_slots || c0 < 0;
    for (int t = tid; t < L && !bad; t += NTHREADS) {
        const int64_t row = p.tix ? static_cast<int64_t>(p.tix[c0 + t]) : c0 + t;
        bad = row < 0 || row >= p.n_tok;
    }
    if (__syncthreads_or(bad))
        return;
    const bool init = p.has_init ? p.has_init[seq] != 0 : true;

    // ---- the state: read once (or zero), kept in registers ----
    const size_t tile = static_cast<size_t>(D) * D;
    char* sbase = static_cast<char*>(p.pool) +
                  (static_cast<size_t>(slot) * p.HV + h) * tile * ESZ;
    float S[RPT][NE];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = wave * ROWS_PER_WAVE + r * 8 + g;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            uint4 w = make_uint4(0u, 0u, 0u, 0u);
            if (init)
                w = *reinterpret_cast<const uint4*>(
                    sbase + (static_cast<size_t>(row) * D + c * CSTRIDE + j * EPC) * ESZ);
            chunk_to_f32<ST>(w, &S[r][c * EPC]);
        }
    }

    const float A = -expf(p.A_log[h]);
    const float dtb = p.dt_bias[h];
    const float2 wn = *reinterpret_cast<const float2*>(p.norm_weight + 2 * lane);
    const int nsteps = (L + TS - 1) / TS;
    StepRaw<ACT> raw;
    issue_step<ACT>(p, c0, L, 0, wave, lane, h, kh, raw);

    for (int step = 0; step < nsteps; ++step) {
        Step& B = sb[step & 1];
        const int base = step * TS;
        const int n = L - base < TS ? L - base : TS;   // tokens in this step

        // ---- prologue: gates, normalised k and q, k^.q^ into LDS ----
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            const int tl = wave + NWAVES * i;
            const float2 qv = unpack_pair<ACT>(raw.q[i]);
            const float2 kv = unpack_pair<ACT>(raw.k[i]);
            const float nq = sum64(qv.x * qv.x + qv.y * qv.y);
            const float nk = sum64(kv.x * kv.x + kv.y * kv.y);
            const float rk = frsqrt(nk + 1e-6f);
            const float rq = p.scale * frsqrt(nq + 1e-6f);
            const float2 kn = make_float2(kv.x * rk, kv.y * rk);
            const float2 qn = make_float2(qv.x * rq, qv.y * rq);
            const float kq = sum64(kn.x * qn.x + kn.y * qn.y);
            if (tl < n) {
                *reinterpret_cast<float2*>(&B.k[tl][2 * lane]) = kn;
                *reinterpret_cast<float2*>(&B.q[tl][2 * lane]) = qn;
                *reinterpret_cast<float2*>(&B.v[tl][2 * lane]) = unpack_pair<ACT>(raw.v[i]);
                *reinterpret_cast<float2*>(&B.z[tl][2 * lane]) = unpack_pair<ACT>(raw.z[i]);
                if (lane == 0) {
                    B.row[tl] = raw.row[i];
                    const float x = unpack_one<ACT>(raw.a[i]) + dtb;
                    B.alpha[tl] = fexp(A * softplus_fast(x));
                    B.beta[tl] = sigmoid_fast(unpack_one<ACT>(raw.b[i]));
                    B.kq[tl] = kq;
                }
            }
        }
        // ---- the next step's loads, in flight during this step's tokens ----
        if (step + 1 < nsteps)
            issue_step<ACT>(p, c0, L, step + 1, wave, lane, h, kh, raw);
        lds_barrier();

        // ---- the step's tokens, strictly in order ----
        for (int tl = 0; tl < n; ++tl) {
            const float alpha = B.alpha[tl];
            const float beta = B.beta[tl];
            const float kq = B.kq[tl];
            float kn[NE], qn[NE];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
#pragma unroll
                for (int m = 0; m < EPC; m += 4) {
                    const float4 k4 =
                        *reinterpret_cast<const float4*>(&B.k[tl][c * CSTRIDE + j * EPC + m]);
                    const float4 q4 =
                        *reinterpret_cast<const float4*>(&B.q[tl][c * CSTRIDE + j * EPC + m]);
                    kn[c * EPC + m + 0] = k4.x; kn[c * EPC + m + 1] = k4.y;
                    kn[c * EPC + m + 2] = k4.z; kn[c * EPC + m + 3] = k4.w;
                    qn[c * EPC + m + 0] = q4.x; qn[c * EPC + m + 1] = q4.y;
                    qn[c * EPC + m + 2] = q4.z; qn[c * EPC + m + 3] = q4.w;
                }
            }
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int row = wave * ROWS_PER_WAVE + r * 8 + g;
                float pk = 0.0f, pq = 0.0f;
#pragma unroll
                for (int e = 0; e < NE; ++e) {
                    pk = fmaf(S[r][e], kn[e], pk);
                    pq = fmaf(S[r][e], qn[e], pq);
                }
                pk = sum8(pk);
                pq = sum8(pq);
                const float d = beta * (B.v[tl][row] - alpha * pk);
                const float o = fmaf(alpha, pq, d * kq);
#pragma unroll
                for (int e = 0; e < NE; ++e)
                    S[r][e] = fmaf(d, kn[e], alpha * S[r][e]);
                if (j == 0)
                    B.o[tl][row] = o;
            }
            // chunk end: the state continues from its stored (rounded) value
            const int tg = base + tl;
            if ((tg + 1) % p.chunk == 0 && tg + 1 < L) {
#pragma unroll
                for (int r = 0; r < RPT; ++r)
#pragma unroll
                    for (int e = 0; e < NE; e += 2)
                        round_pair<ST>(S[r][e], S[r][e + 1]);
            }
        }
        lds_barrier();

        // ---- gated RMSNorm over V per (token, head) ----
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            const int tl = wave + NWAVES * i;
            if (tl < n) {
                const float2 o = *reinterpret_cast<const float2*>(&B.o[tl][2 * lane]);
                const float2 zv = *reinterpret_cast<const float2*>(&B.z[tl][2 * lane]);
                const int64_t row = B.row[tl];
                const float ms = sum64(o.x * o.x + o.y * o.y) * (1.0f / D);
                const float rr = frsqrt(ms + p.norm_eps);
                const float gx = zv.x * sigmoid_fast(zv.x);
                const float gy = zv.y * sigmoid_fast(zv.y);
                const float2 y = make_float2(o.x * rr * wn.x * gx, o.y * rr * wn.y * gy);
                store_pair<OUT>(p.out, row * p.o_st + h * p.o_sh + 2 * lane, y);
            }
        }
    }

    // ---- the final state, rounded once, written once ----
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = wave * ROWS_PER_WAVE + r * 8 + g;
#pragma unroll
        for (int c = 0; c < CH; ++c)
            __builtin_nontemporal_store(f32_to_chunk<ST>(&S[r][c * EPC]),
                reinterpret_cast<u32x4*>(
                    sbase + (static_cast<size_t>(row) * D + c * CSTRIDE + j * EPC) * ESZ));
    }
}

// ---- the chunkwise form on the FP32 matrix cores ---------------------------
// Within a sub-chunk of up to MC tokens starting from state S0, with
// G_t = sum_{j<=t} log(alpha_j) (log decays, so no product under- or
// overflows):
//   S_t      = e^{G_t} S0 + sum_{i<=t} e^{G_t - G_i} d_i k^_i^T
//   d_t      = beta_t (v_t - e^{G_t} S0 k^_t - sum_{i<t} e^{G_t-G_i} (k^_i.k^_t) d_i)
//   o_t      = e^{G_t} S0 q^_t + sum_{i<=t} e^{G_t-G_i} (k^_i.q^_t) d_i
// -- the token recurrence unrolled, the same values up to rounding order.
// The products S0 [k^ | q^] (V x K by K x 2MC) and the update
// S <- e^{G_end} S + D' K^T (D'_i = e^{G_end - G_i} d_i) run on
// v_mfma_f32_32x32x2f32, the k^ rows of the Gram matrix and the read-outs
// O = diag(e^G) S0 Q^ + Bkq D on v_mfma_f32_16x16x4f32; the MC x MC
// triangular solve for d runs on the vector ALU, one value row per lane.
//
// Layout: wave w owns value rows v = 32w..32w+31.  The state is kept
// transposed in the matrix-core accumulator layout: element r of tile kb in
// lane l is S[32w + l%32][32kb + 8(r/4) + 4(l/32) + r%4].  That is also the
// A-operand layout of S0 for S0 X (lane l supplies row l%32, and the two
// lane halves the two k of a step), so the state never moves between the
// two products.
constexpr int MC = 16;            // tokens per sub-chunk
constexpr int MT = 256;           // threads per block: 4 waves
constexpr int XP = D + 4;         // padded row stride of the staged k^ / q^ rows
constexpr int PP = 33;            // padded row stride of the 32 x 32 transposes
constexpr int MTW = MC / (MT / 64);   // tokens staged per wave

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int GP = MC + 1;        // padded row stride of the Gram tiles
constexpr int OP = D + 4;         // padded row stride of the read-outs
constexpr int DP = MC + 4;        // padded row stride of the staged d

struct MStage {
    float x[2 * MC][XP];          // rows t: k^_t, rows MC + t: q^_t (zero past the sub-chunk)
    float v[MC][D];
    float p[4][2 * MC][PP];       // per wave: S0 [k^|q^], [token column][value row]
    float gp[2][2][MC][GP];       // [K half][k^ or q^ columns][i][j]: partial k^_i . (k^|q^)_j
    float o[MC][OP];              // the read-outs, until the next sub-chunk's products ran
    float dd[4][32][DP];          // per wave: d, [value row][token], for the read-out products
    float akk[MC][MC];            // [t][i]: e^{G_t-G_i} k^_i.k^_t for i < t, else 0
    float bkq[MC][MC];            // [t][i]: e^{G_t-G_i} k^_i.q^_t for i <= t, else 0
    float gam[MC];                // e^{G_t}
    float wend[MC];               // e^{G_end - G_t}
    float g[MC];                  // log alpha_t (0 past the sub-chunk)
    float G[MC];                  // running sums of g: G_t = g_0 + ... + g_t
    float beta[MC];               // (0 past the sub-chunk)
    int32_t rows[2][MC];          // token rows of the current / previous sub-chunk
};

template <int ACT>
struct MRaw {
    typename Pair<ACT>::raw q[MTW], k[MTW], v[MTW], z[MTW];
    uint32_t a, b;     // the gates of token pos + wave + 4 (lane % MTW) ...
    int32_t row;       // ... and its row (rows fit 32 bits: they come from int32 offsets)
};

// The element idx of an activation tensor (idx wave-uniform: a scalar address).
template <int ACT>
__device__ __forceinline__ const void* elem_at(const void* base, int64_t idx)
{
    return static_cast<const char*>(base) + idx * (ACT == GDN_F32 ? 4 : 2);
}

// Tokens of one sub-chunk for this wave: t = wave + 4 i.  The row and head
// offsets are wave-uniform; only the lane's pair offset is per lane.
template <int ACT>
__device__ __forceinline__ void issue_sub(const PParams& p, int64_t c0, int L, int pos,
                                          int wave, int lane, int h, int kh, MRaw<ACT>& r)
{
    const uint32_t e = 2u * static_cast<uint32_t>(lane);
    // the token index map is read-only here: scalar loads, which the vector
    // loads below need not wait behind
    using cint = const __attribute__((address_space(4))) int32_t;
    cint* tix = (cint*)(p.tix);
    int64_t rows[MTW];
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
        const int t = pos + wave + 4 * i;
        const int tt = t < L ? t : L - 1;
        rows[i] = p.tix ? static_cast<int64_t>(tix[c0 + tt]) : c0 + tt;
    }
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
        const int64_t row = rows[i];
        r.q[i] = load_pair_raw<ACT>(elem_at<ACT>(p.q, row * p.q_st + kh * p.q_sh), e);
        r.k[i] = load_pair_raw<ACT>(elem_at<ACT>(p.k, row * p.k_st + kh * p.k_sh), e);
        r.v[i] = load_pair_raw<ACT>(elem_at<ACT>(p.v, row * p.v_st + h * p.v_sh), e);
        r.z[i] = load_pair_raw<ACT>(elem_at<ACT>(p.z, row * p.z_st + h * p.z_sh), e);
    }
    // one token's gates per lane (token pos + wave + 4 (lane % MTW)), not
    // every token's in every lane
    int64_t row = rows[0];
#pragma unroll
    for (int i = 1; i < MTW; ++i)
        row = lane % MTW == i ? rows[i] : row;
    r.row = static_cast<int32_t>(row);
    r.a = load_one_raw<ACT>(p.a, row * p.a_st + h);
    r.b = load_one_raw<ACT>(p.b, row * p.b_st + h);
}

// Tokens in the sub-chunk at pos: up to MC, never across a chunk end.
__device__ __forceinline__ int sub_len(int pos, int L, int chunk)
{
    int n = L - pos < MC ? L - pos : MC;
    const int to_end = chunk - pos % chunk;
    return n < to_end ? n : to_end;
}

// Four consecutive state elements (k contiguous) to / from fp32.
template <int ST>
__device__ __forceinline__ void load4_state(const char* base, uint32_t e, float* f)
{
    if constexpr (ST == GDN_F32) {
        const uint4 w = *reinterpret_cast<const uint4*>(base + e * 4);
        f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
        f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
    } else if constexpr (ST == GDN_F8E4M3) {
        unpack4_f8(*reinterpret_cast<const uint32_t*>(base + e), f[0], f[1], f[2], f[3]);
    } else {
        const uint2 w = *reinterpret_cast<const uint2*>(base + e * 2);
        const float2 lo = unpack_pair<ST>(w.x), hi = unpack_pair<ST>(w.y);
        f[0] = lo.x; f[1] = lo.y; f[2] = hi.x; f[3] = hi.y;
    }
}

template <int ST>
__device__ __forceinline__ void store4_state(char* base, uint32_t e, const float* f)
{
    if constexpr (ST == GDN_F32) {
        *reinterpret_cast<uint4*>(base + e * 4) =
            make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                       __float_as_uint(f[3]));
    } else if constexpr (ST == GDN_F8E4M3) {
        *reinterpret_cast<uint32_t*>(base + e) = pack4_f8(f[0], f[1], f[2], f[3]);
    } else {
        *reinterpret_cast<uint2*>(base + e * 2) =
            make_uint2(pack2<ST>(f[0], f[1]), pack2<ST>(f[2], f[3]));
    }
}

// Gated RMSNorm over V per (token, head) for this wave's tokens t = wave + 4 i
// of a sub-chunk of n tokens, from its read-outs o.
template <int ACT, int OUT>
__device__ __forceinline__ void epilogue(const PParams& p, const float (&o)[MC][OP],
                                         const typename Pair<ACT>::raw (&zr)[MTW],
                                         const int32_t (&rows)[MC], int n, int wave, int lane,
                                         int h, float2 wn)
{
    static_assert(MTW == 4, "one four-way wave sum per sub-chunk");
    float2 ov[MTW];
    float ms[MTW];
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
        // (rows past the sub-chunk are summed too: each sum is kept apart
        // from the others, and theirs go unused)
        ov[i] = *reinterpret_cast<const float2*>(&o[wave + 4 * i][2 * lane]);
        ms[i] = ov[i].x * ov[i].x + ov[i].y * ov[i].y;
    }
    sum64x4(ms[0], ms[1], ms[2], ms[3]);
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
        const int t = wave + 4 * i;
        if (t < n) {
            const float rr = frsqrt(ms[i] * (1.0f / D) + p.norm_eps);
            const float2 z = unpack_pair<ACT>(zr[i]);
            const float gx = z.x * sigmoid_fast(z.x);
            const float gy = z.y * sigmoid_fast(z.y);
            const float2 y =
                make_float2(ov[i].x * rr * wn.x * gx, ov[i].y * rr * wn.y * gy);
            store_pair<OUT>(p.out, static_cast<int64_t>(rows[t]) * p.o_st + h * p.o_sh + 2 * lane,
                            y);
        }
    }
}

template <int ACT, int ST, int OUT>
__global__ void __launch_bounds__(MT) __attribute__((amdgpu_waves_per_eu(2)))
gdn_prefill_mma_kernel(const PParams p)
{
    constexpr int ESZ = ST == GDN_F32 ? 4 : (ST == GDN_F8E4M3 ? 1 : 2);
    __shared__ __attribute__((aligned(16))) MStage sm;

    const int tid = threadIdx.x;
    // wave-uniform, and known to be: the token rows and their addresses are then
    // scalar arithmetic
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lc = lane & 31;
    const int lh = lane >> 5;

    const uint32_t nblk = gridDim.x;
    const uint32_t xcd = blockIdx.x % NXCD;
    const uint32_t per = nblk / NXCD, rem = nblk % NXCD;
    const uint32_t unit = xcd * per + (xcd < rem ? xcd : rem) + blockIdx.x / NXCD;
    const uint32_t seq32 = unit / static_cast<uint32_t>(p.HV);
    const int64_t seq = seq32;
    const int h = static_cast<int>(unit - seq32 * static_cast<uint32_t>(p.HV));
    const int kh = static_cast<int>(static_cast<uint32_t>(h) / static_cast<uint32_t>(p.group));

    const int64_t c0 = p.cu[seq];
    const int L = static_cast<int>(p.cu[seq + 1] - c0);
    const int64_t slot = p.state_idx[seq];
    if (L <= 0 || slot < 0)
        return;
    bool bad = slot >= p.num_slots || c0 < 0;
    for (int t = tid; t < L && !bad; t += MT) {
        const int64_t row = p.tix ? static_cast<int64_t>(p.tix[c0 + t]) : c0 + t;
        bad = row < 0 || row >= p.n_tok;
    }
    if (__syncthreads_or(bad))
        return;
    const bool init = p.has_init ? p.has_init[seq] != 0 : true;

    // ---- the state, transposed into the accumulator layout ----
    const size_t tile = static_cast<size_t>(D) * D;
    char* sbase = static_cast<char*>(p.pool) + (static_cast<size_t>(slot) * p.HV + h) * tile * ESZ;
    const int vrow = 32 * wave + lc;
    // (every load issued, then the zero state selected, so that the 16 loads
    // are in flight together)
    f32x16 S[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float f[4];
            load4_state<ST>(sbase, static_cast<uint32_t>(vrow * D + 32 * kb + 8 * q + 4 * lh), f);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                S[kb][4 * q + m] = init ? f[m] : 0.0f;
        }

    // head constants, wave-uniform: kept in scalar registers
    const float A =
        __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(-expf(p.A_log[h]))));
    const float dtb =
        __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(p.dt_bias[h])));
    float2 wn = *reinterpret_cast<const float2*>(p.norm_weight + 2 * lane);
    // Complete these loads before the loop: a load still pending at the loop
    // entry makes its uses inside the loop wait, conservatively, for the
    // activation loads of the sub-chunk ahead as well.
    asm volatile("" : "+v"(wn.x), "+v"(wn.y));
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            asm volatile("" : "+v"(S[kb][r]));

    // The gated RMSNorm of a sub-chunk runs while the next sub-chunk's
    // matrix products do: its tokens' rows, z and count stay in registers.
    typename Pair<ACT>::raw zc[MTW];
    int nprev = 0, par = 0;
    // The activations of a sub-chunk are loaded while the previous one is
    // processed: issued right after its staging, in every iteration (the
    // positions clamp to the last row), so that they land in the registers
    // the next iteration reads.
    MRaw<ACT> raw;
    issue_sub<ACT>(p, c0, L, 0, wave, lane, h, kh, raw);
    for (int pos = 0; pos < L;) {
        const int n = sub_len(pos, L, p.chunk);
        const int next = pos + n;
        typename Pair<ACT>::raw zn[MTW];

        // ---- stage: normalised k and q, v, gates; z stays in registers ----
        float nq[MTW], nk[MTW];
#pragma unroll
        for (int i = 0; i < MTW; ++i) {
            const float2 qv = unpack_pair<ACT>(raw.q[i]);
            const float2 kv = unpack_pair<ACT>(raw.k[i]);
            nq[i] = qv.x * qv.x + qv.y * qv.y;
            nk[i] = kv.x * kv.x + kv.y * kv.y;
        }
        sum64x4(nq[0], nq[1], nq[2], nq[3]);
        sum64x4(nk[0], nk[1], nk[2], nk[3]);
#pragma unroll
        for (int i = 0; i < MTW; ++i) {
            const int t = wave + 4 * i;
            const bool live = t < n;
            const float2 qv = unpack_pair<ACT>(raw.q[i]);
            const float2 kv = unpack_pair<ACT>(raw.k[i]);
            const float rk = live ? frsqrt(nk[i] + 1e-6f) : 0.0f;
            const float rq = live ? p.scale * frsqrt(nq[i] + 1e-6f) : 0.0f;
            const float2 vv = unpack_pair<ACT>(raw.v[i]);
            zn[i] = raw.z[i];
            *reinterpret_cast<float2*>(&sm.x[t][2 * lane]) =
                live ? make_float2(kv.x * rk, kv.y * rk) : make_float2(0.0f, 0.0f);
            *reinterpret_cast<float2*>(&sm.x[MC + t][2 * lane]) =
                live ? make_float2(qv.x * rq, qv.y * rq) : make_float2(0.0f, 0.0f);
            *reinterpret_cast<float2*>(&sm.v[t][2 * lane]) =
                live ? vv : make_float2(0.0f, 0.0f);
        }
        if (lane < MTW) {
            const int t = wave + 4 * lane;
            const bool live = t < n;
            const float x = unpack_one<ACT>(raw.a) + dtb;
            sm.g[t] = live ? A * softplus_fast(x) : 0.0f;
            sm.beta[t] = live ? sigmoid_fast(unpack_one<ACT>(raw.b)) : 0.0f;
            sm.rows[par][t] = raw.row;
        }
        issue_sub<ACT>(p, c0, L, next, wave, lane, h, kh, raw);
        lds_barrier();

        // ---- S0 [k^ | q^] and this wave's share of the Gram matrix.  The
        // matrix phases run at raised wave priority, so that the other block
        // on the SIMD fills the gaps with its vector work. ----
        __builtin_amdgcn_s_setprio(2);
        f32x16 P = {};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 xb =
                    *reinterpret_cast<const float4*>(&sm.x[lc][32 * kb + 8 * q + 4 * lh]);
                P = __builtin_amdgcn_mfma_f32_32x32x2f32(S[kb][4 * q + 0], xb.x, P, 0, 0, 0);
                P = __builtin_amdgcn_mfma_f32_32x32x2f32(S[kb][4 * q + 1], xb.y, P, 0, 0, 0);
                P = __builtin_amdgcn_mfma_f32_32x32x2f32(S[kb][4 * q + 2], xb.z, P, 0, 0, 0);
                P = __builtin_amdgcn_mfma_f32_32x32x2f32(S[kb][4 * q + 3], xb.w, P, 0, 0, 0);
            }
        // the running sums of the log decays, by one lane, while the
        // products run; the barrier below publishes them
        if (tid == 0) {
            float run = 0.0f;
#pragma unroll
            for (int j = 0; j < MC; ++j) {
                run += sm.g[j];
                sm.G[j] = run;
            }
        }
        // k^_i . k^_t and k^_i . q^_t over this wave's half of K, on the
        // 16 x 16 x 4 form: only the k^ rows of the Gram matrix are needed
        const int gcol = wave & 1, gk = 64 * (wave >> 1), l16 = lane & 15, lq = lane >> 4;
        f32x4 Gm = {};
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int k = gk + 4 * s + lq;
            Gm = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.x[l16][k], sm.x[MC * gcol + l16][k], Gm,
                                                      0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        // the previous sub-chunk's gated RMSNorm, while the products run
        epilogue<ACT, OUT>(p, sm.o, zc, sm.rows[par ^ 1], nprev, wave, lane, h, wn);
#pragma unroll
        for (int i = 0; i < MTW; ++i)
            zc[i] = zn[i];
        nprev = n;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r / 4) + 4 * lh + r % 4;
            sm.p[wave][lc][i] = P[r];          // [token column][value row]
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sm.gp[wave >> 1][gcol][4 * lq + r][l16] = Gm[r];
        lds_barrier();

        // ---- decay-weighted Gram coefficients (one (i, t) pair per thread) ----
        {
            const int i = tid / MC, t = tid % MC;
            const float Gi = sm.G[i], Gt = sm.G[t], Ge = sm.G[MC - 1];
            const float kk = sm.gp[0][0][i][t] + sm.gp[1][0][i][t];
            const float kq = sm.gp[0][1][i][t] + sm.gp[1][1][i][t];
            const float e = i <= t ? fexp(Gt - Gi) : 0.0f;
            sm.akk[t][i] = i < t ? e * kk : 0.0f;
            sm.bkq[t][i] = e * kq;
            if (i == 0) {
                sm.gam[t] = fexp(Gt);
                sm.wend[t] = fexp(Ge - Gt);
            }
        }
        lds_barrier();
        // the decay of S over the sub-chunk, ahead of the solve, whose
        // dependent chain leaves issue slots free
        {
            const float ge = sm.gam[MC - 1];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    S[kb][r] *= ge;
        }

        // ---- the triangular solve for d: value row 32 wave + lc per lane
        // (both lane halves) ----
        // Right-looking: once d_i is known it is folded into every later
        // accumulator, which keeps each sum in ascending i (the same bits as
        // summing row by row) and leaves only one FMA per step on the chain
        // from d_i to d_{i+1}.
        float d[MC], acc[MC];
#pragma unroll
        for (int t = 0; t < MC; ++t)
            acc[t] = sm.gam[t] * sm.p[wave][t][lc];
#pragma unroll
        for (int i = 0; i < MC; ++i) {
            d[i] = sm.beta[i] * (sm.v[i][vrow] - acc[i]);
#pragma unroll
            for (int t = i + 1; t < MC; ++t)
                acc[t] = fmaf(sm.akk[t][i], d[i], acc[t]);
        }
        // ---- the read-outs O = diag(e^G) (S0 q^) + Bkq D on the 16 x 16 x 4
        // form: token rows x this wave's value rows, two tiles of 16.  Step
        // s takes token i = 4 (lane / 16) + s of the contraction.  d reaches
        // the operand layout through LDS; only this wave reads its rows, and
        // one wave's LDS accesses complete in order. ----
#pragma unroll
        for (int m = 0; m < MC; m += 4)      // both lane halves write the same values
            *reinterpret_cast<float4*>(&sm.dd[wave][lc][m]) =
                make_float4(d[m], d[m + 1], d[m + 2], d[m + 3]);
        {
            const float4 a4 = *reinterpret_cast<const float4*>(&sm.bkq[l16][4 * lq]);
#pragma unroll
            for (int tile = 0; tile < 2; ++tile) {
                const int vr = 16 * tile + l16;
                const float4 b4 = *reinterpret_cast<const float4*>(&sm.dd[wave][vr][4 * lq]);
                f32x4 c;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    c[j] = sm.gam[4 * lq + j] * sm.p[wave][MC + 4 * lq + j][vr];
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, b4.x, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, b4.y, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, b4.z, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, b4.w, c, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sm.o[4 * lq + j][32 * wave + vr] = c[j];
            }
        }

        // ---- S <- (e^{G_end} S) + D' K^T ----
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int s = 0; s < MC / 2; ++s) {
            const float b = lh ? sm.wend[2 * s + 1] * d[2 * s + 1] : sm.wend[2 * s] * d[2 * s];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                S[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(sm.x[2 * s + lh][32 * kb + lc], b,
                                                             S[kb], 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        // chunk end: the state continues from its stored (rounded) value
        if (next % p.chunk == 0 && next < L) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float x0 = S[kb][r], x1 = S[kb][r + 1];
                    round_pair<ST>(x0, x1);
                    S[kb][r] = x0;
                    S[kb][r + 1] = x1;
                }
        }
        lds_barrier();

        pos = next;
        par ^= 1;
    }
    epilogue<ACT, OUT>(p, sm.o, zc, sm.rows[par ^ 1], nprev, wave, lane, h, wn);

    // ---- the final state, rounded once, written once ----
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float f[4];
#pragma unroll
            for (int m = 0; m < 4; ++m)
                f[m] = S[kb][4 * q + m];
            store4_state<ST>(sbase, static_cast<uint32_t>(vrow * D + 32 * kb + 8 * q + 4 * lh), f);
        }
}

template <int A, int S, int O>
hipError_t launch_typed(const PParams& p, int64_t grid, hipStream_t stream)
{
    PParams args = p;
    void* argv[] = {&args};
    if (p.chunk >= MC)
        return hipLaunchKernel(reinterpret_cast<const void*>(&gdn_prefill_mma_kernel<A, S, O>),
                               dim3(static_cast<uint32_t>(grid)), dim3(MT), argv, 0, stream);
    return hipLaunchKernel(reinterpret_cast<const void*>(&gdn_prefill_kernel<A, S, O>),
                           dim3(static_cast<uint32_t>(grid)), dim3(NTHREADS), argv, 0, stream);
}

template <int A, int S>
hipError_t launch_out(int out, const PParams& p, int64_t grid, hipStream_t s)
{
    switch (out) {
    case GDN_F32: return launch_typed<A, S, GDN_F32>(p, grid, s);
    case GDN_F16: return launch_typed<A, S, GDN_F16>(p, grid, s);
    default: return launch_typed<A, S, GDN_BF16>(p, grid, s);
    }
}

template <int A>
hipError_t launch_state(int st, int out, const PParams& p, int64_t grid, hipStream_t s)
{
    switch (st) {
    case GDN_F32: return launch_out<A, GDN_F32>(out, p, grid, s);
    case GDN_F16: return launch_out<A, GDN_F16>(out, p, grid, s);
    case GDN_F8E4M3: return launch_out<A, GDN_F8E4M3>(out, p, grid, s);
    default: return launch_out<A, GDN_BF16>(out, p, grid, s);
    }
}

hipError_t launch(int act, int st, int out, const PParams& p, int64_t grid, hipStream_t s)
{
    switch (act) {
    case GDN_F32: return launch_state<GDN_F32>(st, out, p, grid, s);
    case GDN_F16: return launch_state<GDN_F16>(st, out, p, grid, s);
    default: return launch_state<GDN_BF16>(st, out, p, grid, s);
    }
}

}  // namespace

extern "C" gdn_status gdn_prefill_update(const gdn_layer* layer, const gdn_state_pool* pool,
                                         const int32_t* cu_seqlens, int32_t num_seqs,
                                         const int32_t* state_indices,
                                         const int32_t* has_initial_state,
                                         const int32_t* token_indx, int32_t chunk_size,
                                         hipStream_t stream)
{
    gdn::clear_error();
    gdn_status st;
    if ((st = gdn::check_layer(layer)) != GDN_OK || (st = gdn::check_pool(pool)) != GDN_OK)
        return st;
    if (num_seqs < 0)
        return gdn::fail(GDN_ERR_INVALID, "num_seqs is negative");
    if (chunk_size < 1)
        return gdn::fail(GDN_ERR_INVALID, "chunk_size must be >= 1");
    if (num_seqs == 0 || layer->n_tok == 0)
        return GDN_OK;
    if (!cu_seqlens || !state_indices)
        return gdn::fail(GDN_ERR_INVALID, "cu_seqlens or state_indices is NULL");
    const int64_t grid = static_cast<int64_t>(num_seqs) * layer->num_v_heads;
    if (grid > 0x7fffffffLL)
        return gdn::fail(GDN_ERR_INVALID, "num_seqs * num_v_heads exceeds the grid limit");
    PParams p{};
    const gdn_layer* L = layer;
    p.q = L->q.data; p.q_st = L->q.stride_tok; p.q_sh = L->q.stride_head;
    p.k = L->k.data; p.k_st = L->k.stride_tok; p.k_sh = L->k.stride_head;
    p.v = L->v.data; p.v_st = L->v.stride_tok; p.v_sh = L->v.stride_head;
    p.z = L->z.data; p.z_st = L->z.stride_tok; p.z_sh = L->z.stride_head;
    p.a = L->a.data; p.a_st = L->a.stride_tok;
    p.b = L->b.data; p.b_st = L->b.stride_tok;
    p.out = L->out.data; p.o_st = L->out.stride_tok; p.o_sh = L->out.stride_head;
    p.A_log = L->A_log;
    p.dt_bias = L->dt_bias;
    p.norm_weight = L->norm_weight;
    p.pool = pool->data;
    p.num_slots = pool->num_slots;
    p.n_tok = L->n_tok;
    p.HV = L->num_v_heads;
    p.group = L->num_v_heads / L->num_k_heads;
    p.scale = L->scale;
    p.norm_eps = L->norm_eps;
    p.cu = cu_seqlens;
    p.state_idx = state_indices;
    p.has_init = has_initial_state;
    p.tix = token_indx;
    p.chunk = chunk_size;
    const hipError_t e = launch(L->act_dtype, pool->dtype, L->out_dtype, p, grid, stream);
    if (e != hipSuccess)
        return gdn::fail(GDN_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}
