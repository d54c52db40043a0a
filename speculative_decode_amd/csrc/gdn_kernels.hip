// gdn_kernels.hip -- fused Gated DeltaNet speculative-decode state update for
// CDNA4 (gfx950), and its C-ABI entry points (speculative, single-token,
// mixed, and the state-format cast).
//
// What is computed is fixed by the vLLM PR reports on prhub.com.cn (#51674
// 实现拆解 item 1: one block per (request, value head), rewind by
// num_accepted_tokens, serial recurrence over <= 8 draft tokens, every
// post-token state stored to its slot, gated RMSNorm epilogue; #46090 fla.cpp
// excerpt: clamp, skip, GQA map; #52191 实现拆解 item 4: FP32 arithmetic,
// state-dtype slot stores; #51812: one gather index for q/k/v and a/b).
//
// How it is computed here (not the pages' CUDA design):
//   * One 256-thread workgroup (4 wave64) per (sequence, value head); a 1-D
//     grid of num_seqs*HV workgroups, mapped so each XCD works on a
//     contiguous range of units.  Launches are capped by an LDS
//     reservation: one block per CU for 7-8 draft tokens, two for 2-6, none
//     for single tokens or an FP8 pool.
//   * The 128x128 state tile (V rows, K contiguous) lives in registers for
//     the whole draft: each 8-lane group owns one row at a time, each lane 16
//     of its elements, and every lane holds 4 rows (64 fp32 values).  A row
//     chunk moves as one 16-byte access per lane, so one wave instruction
//     covers eight full 128-byte lines.  The tile is read from HBM once and
//     written once per draft token, both with non-temporal accesses; nothing
//     else touches it.
//   * Rows of S evolve independently.  Per token and row, the two dot
//     products of the OLD row (S.k^ and S.q^) are reduced together over the
//     8 lanes with three DPP steps; then
//        d = beta (v - alpha S.k^),  o = alpha S.q^ + d (k^.q^),
//        S = alpha S + d k^
//     which is S_t q^ of the updated state without a second pass.
//   * Per-token vectors (k^, q^, v) and scalars (alpha, beta, k^.q^) are
//     computed once per workgroup in a prologue and shared through LDS; the
//     read-outs o go to LDS for the per-(token, head) RMSNorm epilogue.  The
//     scalar math of both uses the hardware exp/log/rcp/rsq units.
//   * No MFMA: a rank-1 recurrence is not a dense contraction.  The kernel is
//     bound by HBM bandwidth (8 of 9 tile transfers at T=8 are stores).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <type_traits>

#include "dtype_cvt.h"
#include "lane_ops.h"
#include "gdn_internal.h"

namespace {

using namespace gdn_dev;

constexpr int D = GDN_HEAD_DIM;          // K = V = 128
constexpr int MAXT = GDN_MAX_DRAFT_TOKENS;
constexpr int NTHREADS = 256;
constexpr int ROWS_PER_WAVE = D / (NTHREADS / 64);   // 32
constexpr int RPT = ROWS_PER_WAVE / 8;               // rows per thread: 4
constexpr int NE = D / 8;                            // elements per (thread, row): 16
constexpr int NXCD = 8;                              // accelerator complex dies on MI355X

struct KParams {
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
    int32_t group;        // HV / HK
    float scale;
    float norm_eps;
    const int32_t* cu;
    const int32_t* spec_idx;
    const int32_t* num_acc;
    const int32_t* tix;
    const int32_t* state_idx;
    const int32_t* ns_tix;    // gather of the single-token entries of a mixed launch
    int64_t num_spec;         // sequences of the spec part
    int64_t num_ns;           // single-token entries of a mixed launch (0: pure spec)
    int32_t spec_stride;
    int32_t max_writes;       // host bound on slot writes per unit (launch planning only)
    int32_t pattern_blocks_per_cu;   // traffic pattern only: 0 = as the update kernel
};

// ---- the kernel ------------------------------------------------------------
// ACT, ST, OUT: gdn_dtype of activations, state pool, output.  SPEC selects
// the speculative metadata (cu_seqlens / spec_state_indices / num_accepted)
// or the single-token in-place form (state_indices).
template <int ACT, int ST, int OUT, bool SPEC>
__global__ void __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(ST == GDN_F32 ? 1 : 4)))
gdn_update_kernel(const KParams p)
{
    constexpr int ESZ = ST == GDN_F32 ? 4 : (ST == GDN_F8E4M3 ? 1 : 2);   // state bytes
    constexpr int CH = D * ESZ / 128;              // 16-byte chunks per (thread,row): 4, 2, 1
    constexpr int EPC = 16 / ESZ;                  // elements per chunk: 4, 8, 16
    constexpr int CSTRIDE = D / CH;                // row offset between chunks: 32, 64, 128
    constexpr int NT = SPEC ? MAXT : 1;            // static bound on draft tokens
    static_assert(CH * EPC == NE, "layout");

    // 16-byte aligned: the token loop reads k^ and q^ as float4.
    __shared__ __attribute__((aligned(16))) float sK[NT][D];
    __shared__ __attribute__((aligned(16))) float sQ[NT][D];
    __shared__ __attribute__((aligned(16))) float sV[NT][D];
    __shared__ __attribute__((aligned(16))) float sO[NT][D];
    __shared__ __attribute__((aligned(16))) float sZ[NT][D];
    __shared__ float sAlpha[NT], sBeta[NT], sKQ[NT];
    __shared__ int64_t sRow[NT];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 3;   // row within the wave's 8-row band
    const int j = lane & 7;    // position within the row's 8-lane group

    // Workgroups are dealt to the 8 XCDs round robin (block b runs on XCD
    // b % 8).  Give each XCD one contiguous range of units instead, so the
    // heads of a sequence -- whose state tiles are adjacent in a slot and whose
    // q/k rows are shared -- meet in one XCD's L2.  Bijective for any grid.
    // Grid and head counts fit 32 bits (the host checks units < 2^31), so
    // the unit arithmetic stays 32-bit: no 64-bit division in the prologue.
    const uint32_t nblk = gridDim.x;
    const uint32_t xcd = blockIdx.x % NXCD;
    const uint32_t per = nblk / NXCD, rem = nblk % NXCD;
    const uint32_t unit = xcd * per + (xcd < rem ? xcd : rem) + blockIdx.x / NXCD;
    const uint32_t entry32 = unit / static_cast<uint32_t>(p.HV);
    const int64_t entry = entry32;
    const int h = static_cast<int>(unit - entry32 * static_cast<uint32_t>(p.HV));
    const int kh = static_cast<int>(static_cast<uint32_t>(h) / static_cast<uint32_t>(p.group));

    // A mixed launch interleaves its two kinds of entries in proportion, so
    // that every XCD's contiguous range gets its share of the heavier spec
    // units: entry e is spec sequence floor(e*S/E) when that count steps at
    // e, else single-token entry e - floor(e*S/E) (S spec of E entries; a
    // bijection).
    bool spec_unit = SPEC;
    int64_t seq = entry;
    if (SPEC && p.num_ns > 0) {
        const int64_t E = p.num_spec + p.num_ns;
        const int64_t before = entry * p.num_spec / E;
        const int64_t after = (entry + 1) * p.num_spec / E;
        spec_unit = after > before;
        seq = spec_unit ? before : entry - before;
    }

    // ---- unit metadata (uniform), fetched in one batch.  The single-token
    // entries of a mixed launch read and write one slot in place. ----
    int L;
    int64_t c0, rslot;
    int64_t wslot[NT];
    const int32_t* tix = p.tix;
    if (spec_unit) {
        c0 = p.cu[seq];
        L = static_cast<int>(p.cu[seq + 1] - c0);
        const int acc = p.num_acc[seq];
        if (L <= 0)
            return;  // q_len <= 0: nothing read, written or output
        if (L > MAXT || L > p.spec_stride || acc < 0 || acc > p.spec_stride)
            return;
        const int32_t* sidx = p.spec_idx + seq * p.spec_stride;
        rslot = sidx[acc > 1 ? acc - 1 : 0];
        bool bad = rslot < 0 || rslot >= p.num_slots;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int tt = t < L ? t : L - 1;
            wslot[t] = sidx[tt];
            const int64_t row = p.tix ? p.tix[c0 + tt] : c0 + tt;
            bad |= wslot[t] < 0 || wslot[t] >= p.num_slots || row < 0 || row >= p.n_tok;
        }
        if (bad)
            return;
    } else {
        const int64_t i = seq;
        tix = SPEC ? p.ns_tix : p.tix;
        rslot = p.state_idx[i];
        c0 = i;
        L = 1;
#pragma unroll
        for (int t = 0; t < NT; ++t)
            wslot[t] = rslot;
        const int64_t row = tix ? tix[i] : i;
        if (rslot < 0 || rslot >= p.num_slots || row < 0 || row >= p.n_tok)
            return;
    }

    // ---- prologue loads: this wave's tokens t = wave, wave + 4 (clamped to
    // the last token, so every lane loads a valid address and no branch
    // forces an early wait) ----
    constexpr int NTW = (NT + 3) / 4;   // tokens per wave
    typename Pair<ACT>::raw qr[NTW], kr[NTW], vr[NTW], zr[NTW];
    uint32_t ar[NTW], br[NTW];
    int64_t rowv[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int t = wave + 4 * i;
        const int tt = t < L ? t : L - 1;
        const int64_t row = tix ? tix[c0 + tt] : c0 + tt;
        rowv[i] = row;
        qr[i] = load_pair_raw<ACT>(p.q, row * p.q_st + kh * p.q_sh + 2 * lane);
        kr[i] = load_pair_raw<ACT>(p.k, row * p.k_st + kh * p.k_sh + 2 * lane);
        vr[i] = load_pair_raw<ACT>(p.v, row * p.v_st + h * p.v_sh + 2 * lane);
        zr[i] = load_pair_raw<ACT>(p.z, row * p.z_st + h * p.z_sh + 2 * lane);
        ar[i] = load_one_raw<ACT>(p.a, row * p.a_st + h);
        br[i] = load_one_raw<ACT>(p.b, row * p.b_st + h);
    }
    const float A = -expf(p.A_log[h]);
    const float dtb = p.dt_bias[h];

    // ---- the rewind tile: read once, 16 B per lane per chunk.  Streaming
    // (non-temporal) loads: nothing reads the tile again in this launch, and
    // a single-token unit rewrites these very lines, which then find no copy
    // of them in L2 to update. ----
    const size_t tile = static_cast<size_t>(D) * D;
    const char* rbase = static_cast<const char*>(p.pool) +
                        (static_cast<size_t>(rslot) * p.HV + h) * tile * ESZ;
    uint4 raw[RPT][CH];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = wave * ROWS_PER_WAVE + r * 8 + g;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                rbase + (static_cast<size_t>(row) * D + c * CSTRIDE + j * EPC) * ESZ));
            raw[r][c] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }

    // ---- prologue compute: gates, normalised k and q, k^.q^.  Everything
    // the epilogue needs (z, the token's row) is parked in LDS so that no
    // register stays live across the token loop for it. ----
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int t = wave + 4 * i;
        const float2 qv = unpack_pair<ACT>(qr[i]);
        const float2 kv = unpack_pair<ACT>(kr[i]);
        const float nq = sum64(qv.x * qv.x + qv.y * qv.y);
        const float nk = sum64(kv.x * kv.x + kv.y * kv.y);
        const float rk = frsqrt(nk + 1e-6f);
        const float rq = p.scale * frsqrt(nq + 1e-6f);
        const float2 kn = make_float2(kv.x * rk, kv.y * rk);
        const float2 qn = make_float2(qv.x * rq, qv.y * rq);
        const float kq = sum64(kn.x * qn.x + kn.y * qn.y);
        if (t < L) {
            *reinterpret_cast<float2*>(&sK[t][2 * lane]) = kn;
            *reinterpret_cast<float2*>(&sQ[t][2 * lane]) = qn;
            *reinterpret_cast<float2*>(&sV[t][2 * lane]) = unpack_pair<ACT>(vr[i]);
            *reinterpret_cast<float2*>(&sZ[t][2 * lane]) = unpack_pair<ACT>(zr[i]);
            if (lane == 0) {
                sRow[t] = rowv[i];
                const float x = unpack_one<ACT>(ar[i]) + dtb;
                sAlpha[t] = fexp(A * softplus_fast(x));
                sBeta[t] = sigmoid_fast(unpack_one<ACT>(br[i]));
                sKQ[t] = kq;
            }
        }
    }
    __syncthreads();

    // ---- tile to fp32 registers ----
    float S[RPT][NE];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int c = 0; c < CH; ++c)
            chunk_to_f32<ST>(raw[r][c], &S[r][c * EPC]);

    // ---- the draft tokens, strictly in order (unrolled: the tile stays in
    // the same registers from token to token) ----
    char* pool = static_cast<char*>(p.pool);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t >= L)
            break;
        // Keep the scheduler from hoisting the next token's LDS reads into
        // this one: that only raises register pressure.
        __builtin_amdgcn_sched_barrier(0);
        const float alpha = sAlpha[t];
        const float beta = sBeta[t];
        const float kq = sKQ[t];
        float kn[NE], qn[NE];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
#pragma unroll
            for (int m = 0; m < EPC; m += 4) {
                const float4 k4 = *reinterpret_cast<const float4*>(&sK[t][c * CSTRIDE + j * EPC + m]);
                const float4 q4 = *reinterpret_cast<const float4*>(&sQ[t][c * CSTRIDE + j * EPC + m]);
                kn[c * EPC + m + 0] = k4.x; kn[c * EPC + m + 1] = k4.y;
                kn[c * EPC + m + 2] = k4.z; kn[c * EPC + m + 3] = k4.w;
                qn[c * EPC + m + 0] = q4.x; qn[c * EPC + m + 1] = q4.y;
                qn[c * EPC + m + 2] = q4.z; qn[c * EPC + m + 3] = q4.w;
            }
        }
        char* wbase = pool + (static_cast<size_t>(wslot[t]) * p.HV + h) * tile * ESZ;
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
            const float d = beta * (sV[t][row] - alpha * pk);
            const float o = fmaf(alpha, pq, d * kq);
#pragma unroll
            for (int e = 0; e < NE; ++e)
                S[r][e] = fmaf(d, kn[e], alpha * S[r][e]);
            if (j == 0)
                sO[t][row] = o;
            if constexpr (ST != GDN_F8E4M3) {
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    // Streaming store: the tile is not read again in this
                    // launch, so it should not displace anything in L2 / MALL.
                    __builtin_nontemporal_store(f32_to_chunk<ST>(&S[r][c * EPC]),
                        reinterpret_cast<u32x4*>(
                            wbase + (static_cast<size_t>(row) * D + c * CSTRIDE + j * EPC) * ESZ));
                }
            }
        }
        if constexpr (ST == GDN_F8E4M3) {
            // One 16-byte chunk per row; encoded together so that the check
            // for saturation is taken once per token.
            u32x4 w8[RPT] = {};
            encode_f8_rows<RPT>(S, w8);
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int row = wave * ROWS_PER_WAVE + r * 8 + g;
                __builtin_nontemporal_store(w8[r], reinterpret_cast<u32x4*>(
                    wbase + (static_cast<size_t>(row) * D + j * EPC) * ESZ));
            }
        }
    }
    __syncthreads();

    // ---- gated RMSNorm over V per (token, head): y = o rsqrt(mean o^2 + eps) w silu(z)
    // The lane id is taken afresh (mbcnt) so that no prologue address is kept
    // alive across the token loop for the epilogue's benefit.
    const int el = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const float2 wn = *reinterpret_cast<const float2*>(p.norm_weight + 2 * el);
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int t = wave + 4 * i;
        if (t < L) {
            const float2 o = *reinterpret_cast<const float2*>(&sO[t][2 * el]);
            const float2 zv = *reinterpret_cast<const float2*>(&sZ[t][2 * el]);
            const int64_t row = sRow[t];
            const float ms = sum64(o.x * o.x + o.y * o.y) * (1.0f / D);
            const float rr = frsqrt(ms + p.norm_eps);
            const float gx = zv.x * sigmoid_fast(zv.x);
            const float gy = zv.y * sigmoid_fast(zv.y);
            const float2 y = make_float2(o.x * rr * wn.x * gx, o.y * rr * wn.y * gy);
            store_pair<OUT>(p.out, row * p.o_st + h * p.o_sh + 2 * el, y);
        }
    }
}

// ---- launch planning ---------------------------------------------------------
// Per-device figures the plan needs, queried once per device.
struct DeviceInfo {
    int cus = 0;
    int lds_per_cu = 0;
    int lds_per_block = 0;
};

hipError_t device_info(DeviceInfo* out)
{
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static DeviceInfo cache[MAX_DEVICES];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const bool cacheable = dev >= 0 && dev < MAX_DEVICES;
    std::lock_guard<std::mutex> lock(mu);
    if (cacheable && cache[dev].cus > 0) {
        *out = cache[dev];
        return hipSuccess;
    }
    DeviceInfo d;
    if ((e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev)) ||
        (e = hipDeviceGetAttribute(&d.lds_per_cu,
                                   hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev)) ||
        (e = hipDeviceGetAttribute(&d.lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock,
                                   dev)))
        return e;
    if (cacheable)
        cache[dev] = d;
    *out = d;
    return hipSuccess;
}

// Static LDS of one block: k^, q^, v, o, z rows plus the per-token scalars.
constexpr size_t static_lds_bytes(int nt)
{
    return size_t(5) * nt * D * sizeof(float) + size_t(3) * nt * sizeof(float) +
           size_t(nt) * sizeof(int64_t);
}

// Concurrent blocks per CU for a launch whose units write up to
// `writes` state tiles each (0: no cap).  A unit reads one tile and writes up
// to `writes`.  With many such write streams per CU, the chip's writes land
// on more DRAM rows at once than the memory keeps open, and the sustained
// rate drops: seven- and eight-token units run best one per CU, two- to
// six-token units two per CU.  Single-token units read as much as they write
// and need the concurrency to hide their read latency, so they run uncapped.
// An FP8 pool moves half the bytes of a 16-bit one for the same arithmetic,
// which then sets the pace: its launches run uncapped, so that more waves
// per SIMD hide each other's instruction latency.
int blocks_per_cu_for(int writes, int state_dtype)
{
    if (writes <= 1 || state_dtype == GDN_F8E4M3)
        return 0;
    return writes <= 6 ? 2 : 1;
}

// Dynamic LDS to reserve for a launch.  The launch reserves LDS that the
// kernel never touches -- just over 1/(n+1) of a CU's, counting the static
// LDS -- so that at most n blocks run per CU (n from blocks_per_cu_for).  The
// stores of a finishing block still drain while the CU's next block loads.
// The cap holds for small batches too: even a batch that would fit in one
// round of resident blocks runs faster with fewer concurrent write streams.
template <int NT>
hipError_t plan_lds(int writes, int state_dtype, size_t* lds)
{
    *lds = 0;
    const int n = blocks_per_cu_for(writes, state_dtype);
    if (n == 0)
        return hipSuccess;
    DeviceInfo d;
    hipError_t e = device_info(&d);
    if (e != hipSuccess)
        return e;
    const size_t share = static_cast<size_t>(d.lds_per_cu) / (n + 1) + 1;
    if (share > static_lds_bytes(NT) && share <= static_cast<size_t>(d.lds_per_block))
        *lds = share - static_lds_bytes(NT);
    return hipSuccess;
}

template <int A, int S, int O, bool SPEC>
hipError_t launch_typed(const KParams& p, int64_t grid, hipStream_t stream)
{
    size_t lds = 0;
    hipError_t e = plan_lds<SPEC ? MAXT : 1>(p.max_writes, S, &lds);
    if (e != hipSuccess)
        return e;
    KParams args = p;
    void* argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gdn_update_kernel<A, S, O, SPEC>),
                           dim3(static_cast<uint32_t>(grid)), dim3(NTHREADS), argv, lds, stream);
}

template <int A, int S, bool SPEC>
hipError_t launch_out(int out, const KParams& p, int64_t grid, hipStream_t s)
{
    switch (out) {
    case GDN_F32: return launch_typed<A, S, GDN_F32, SPEC>(p, grid, s);
    case GDN_F16: return launch_typed<A, S, GDN_F16, SPEC>(p, grid, s);
    default: return launch_typed<A, S, GDN_BF16, SPEC>(p, grid, s);
    }
}

template <int A, bool SPEC>
hipError_t launch_state(int st, int out, const KParams& p, int64_t grid, hipStream_t s)
{
    switch (st) {
    case GDN_F32: return launch_out<A, GDN_F32, SPEC>(out, p, grid, s);
    case GDN_F16: return launch_out<A, GDN_F16, SPEC>(out, p, grid, s);
    case GDN_F8E4M3: return launch_out<A, GDN_F8E4M3, SPEC>(out, p, grid, s);
    default: return launch_out<A, GDN_BF16, SPEC>(out, p, grid, s);
    }
}

template <bool SPEC>
hipError_t launch(int act, int st, int out, const KParams& p, int64_t grid, hipStream_t s)
{
    switch (act) {
    case GDN_F32: return launch_state<GDN_F32, SPEC>(st, out, p, grid, s);
    case GDN_F16: return launch_state<GDN_F16, SPEC>(st, out, p, grid, s);
    default: return launch_state<GDN_BF16, SPEC>(st, out, p, grid, s);
    }
}

KParams make_params(const gdn_layer* L, const gdn_state_pool* P)
{
    KParams p{};
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
    p.pool = P->data;
    p.num_slots = P->num_slots;
    p.n_tok = L->n_tok;
    p.HV = L->num_v_heads;
    p.group = L->num_v_heads / L->num_k_heads;
    p.scale = L->scale;
    p.norm_eps = L->norm_eps;
    return p;
}

// fp32 -> state format with the store conversion of the kernels above (for
// FP8, the same 16-element encoder as the token loop, one group per thread).
template <int DT>
__global__ void __launch_bounds__(256) cast_kernel(const float* src, void* dst, int64_t n)
{
    constexpr int G = DT == GDN_F8E4M3 ? 16 : 1;   // elements per thread and step
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * G;
    for (int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * G; i < n;
         i += stride) {
        if constexpr (DT == GDN_F8E4M3) {
            float f[1][16];
#pragma unroll
            for (int e = 0; e < 16; ++e)
                f[0][e] = i + e < n ? src[i + e] : 0.0f;
            u32x4 w[1] = {};
            encode_f8_rows<1>(f, w);
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (i + e < n)
                    static_cast<uint8_t*>(dst)[i + e] =
                        static_cast<uint8_t>(w[0][e >> 2] >> (8 * (e & 3)));
        } else {
            const float x = src[i];
            if constexpr (DT == GDN_F32)
                static_cast<float*>(dst)[i] = x;
            else
                static_cast<uint16_t*>(dst)[i] = static_cast<uint16_t>(pack2<DT>(x, 0.f) & 0xffffu);
        }
    }
}

// ---- the launch's traffic pattern, with no arithmetic ------------------------
// For measurement only.  The same grid, unit mapping, metadata phase and
// per-CU block count as gdn_update_kernel, and the same HBM traffic: the
// rewind tile read once (16-byte non-temporal loads, same lane layout) and
// written back unchanged to each draft-token slot (non-temporal stores, same
// order), the q/k/v/z rows and the gate scalars read, the out rows written
// (with the XOR of the bits read, so that no load is dead).  Nothing is
// computed, so its duration is what the memory system allows for exactly
// that traffic -- the ceiling the kernel is measured against.
// ASZ, SSZ, OSZ: bytes per activation, state and output element.
template <int ASZ, int SSZ, int OSZ, bool SPEC>
__global__ void __launch_bounds__(NTHREADS) gdn_traffic_kernel(const KParams p)
{
    constexpr int CH = D * SSZ / 128;
    constexpr int EPC = 16 / SSZ;
    constexpr int CSTRIDE = D / CH;
    constexpr int NT = SPEC ? MAXT : 1;
    constexpr int NTW = (NT + 3) / 4;
    using raw_t = typename std::conditional<ASZ == 4, uint2, uint32_t>::type;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 3;
    const int j = lane & 7;

    const uint32_t nblk = gridDim.x;
    const uint32_t xcd = blockIdx.x % NXCD;
    const uint32_t per = nblk / NXCD, rem = nblk % NXCD;
    const uint32_t unit = xcd * per + (xcd < rem ? xcd : rem) + blockIdx.x / NXCD;
    const uint32_t entry32 = unit / static_cast<uint32_t>(p.HV);
    const int64_t entry = entry32;
    const int h = static_cast<int>(unit - entry32 * static_cast<uint32_t>(p.HV));
    const int kh = static_cast<int>(static_cast<uint32_t>(h) / static_cast<uint32_t>(p.group));

    bool spec_unit = SPEC;
    int64_t seq = entry;
    if (SPEC && p.num_ns > 0) {
        const int64_t E = p.num_spec + p.num_ns;
        const int64_t before = entry * p.num_spec / E;
        const int64_t after = (entry + 1) * p.num_spec / E;
        spec_unit = after > before;
        seq = spec_unit ? before : entry - before;
    }
    int L;
    int64_t c0, rslot;
    int64_t wslot[NT];
    const int32_t* tix = p.tix;
    if (spec_unit) {
        c0 = p.cu[seq];
        L = static_cast<int>(p.cu[seq + 1] - c0);
        const int acc = p.num_acc[seq];
        if (L <= 0 || L > MAXT || L > p.spec_stride || acc < 0 || acc > p.spec_stride)
            return;
        const int32_t* sidx = p.spec_idx + seq * p.spec_stride;
        rslot = sidx[acc > 1 ? acc - 1 : 0];
        bool bad = rslot < 0 || rslot >= p.num_slots;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int tt = t < L ? t : L - 1;
            wslot[t] = sidx[tt];
            const int64_t row = p.tix ? p.tix[c0 + tt] : c0 + tt;
            bad |= wslot[t] < 0 || wslot[t] >= p.num_slots || row < 0 || row >= p.n_tok;
        }
        if (bad)
            return;
    } else {
        tix = SPEC ? p.ns_tix : p.tix;
        rslot = p.state_idx[seq];
        c0 = seq;
        L = 1;
#pragma unroll
        for (int t = 0; t < NT; ++t)
            wslot[t] = rslot;
        const int64_t row = tix ? tix[seq] : seq;
        if (rslot < 0 || rslot >= p.num_slots || row < 0 || row >= p.n_tok)
            return;
    }

    // the activation rows of this wave's tokens, as the kernel loads them
    raw_t x[NTW];
    int64_t rowv[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int t = wave + 4 * i;
        const int tt = t < L ? t : L - 1;
        const int64_t row = tix ? tix[c0 + tt] : c0 + tt;
        rowv[i] = row;
        const char* qa = static_cast<const char*>(p.q) + (row * p.q_st + kh * p.q_sh + 2 * lane) * ASZ;
        const char* ka = static_cast<const char*>(p.k) + (row * p.k_st + kh * p.k_sh + 2 * lane) * ASZ;
        const char* va = static_cast<const char*>(p.v) + (row * p.v_st + h * p.v_sh + 2 * lane) * ASZ;
        const char* za = static_cast<const char*>(p.z) + (row * p.z_st + h * p.z_sh + 2 * lane) * ASZ;
        x[i] = *reinterpret_cast<const raw_t*>(qa);
        raw_t kx = *reinterpret_cast<const raw_t*>(ka);
        raw_t vx = *reinterpret_cast<const raw_t*>(va);
        raw_t zx = *reinterpret_cast<const raw_t*>(za);
        uint32_t ab;
        if constexpr (ASZ == 4)
            ab = static_cast<const uint32_t*>(p.a)[row * p.a_st + h] ^
                 static_cast<const uint32_t*>(p.b)[row * p.b_st + h];
        else
            ab = static_cast<const uint16_t*>(p.a)[row * p.a_st + h] ^
                 static_cast<const uint16_t*>(p.b)[row * p.b_st + h];
        if constexpr (ASZ == 4) {
            x[i].x ^= kx.x ^ vx.x ^ zx.x ^ ab;
            x[i].y ^= kx.y ^ vx.y ^ zx.y;
        } else {
            x[i] ^= kx ^ vx ^ zx ^ ab;
        }
    }

    // the rewind tile, read once
    const size_t tile = static_cast<size_t>(D) * D;
    const char* rbase = static_cast<const char*>(p.pool) +
                        (static_cast<size_t>(rslot) * p.HV + h) * tile * SSZ;
    u32x4 raw[RPT][CH];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = wave * ROWS_PER_WAVE + r * 8 + g;
#pragma unroll
        for (int c = 0; c < CH; ++c)
            raw[r][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                rbase + (static_cast<size_t>(row) * D + c * CSTRIDE + j * EPC) * SSZ));
    }

    // ... written back unchanged to every draft-token slot
    char* pool = static_cast<char*>(p.pool);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t >= L)
            break;
        __builtin_amdgcn_sched_barrier(0);
        char* wbase = pool + (static_cast<size_t>(wslot[t]) * p.HV + h) * tile * SSZ;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int row = wave * ROWS_PER_WAVE + r * 8 + g;
#pragma unroll
            for (int c = 0; c < CH; ++c)
                __builtin_nontemporal_store(raw[r][c], reinterpret_cast<u32x4*>(
                    wbase + (static_cast<size_t>(row) * D + c * CSTRIDE + j * EPC) * SSZ));
        }
    }

    // the out rows
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int t = wave + 4 * i;
        if (t < L) {
            char* oa = static_cast<char*>(p.out) +
                       (rowv[i] * p.o_st + h * p.o_sh + 2 * lane) * OSZ;
            uint32_t lo;
            if constexpr (ASZ == 4)
                lo = x[i].x ^ x[i].y;
            else
                lo = x[i];
            if constexpr (OSZ == 4)
                *reinterpret_cast<uint2*>(oa) = make_uint2(lo, lo);
            else
                *reinterpret_cast<uint32_t*>(oa) = lo;
        }
    }
}

// Blocks per CU of the kernel whose traffic the pattern reproduces (or
// `blocks_per_cu` when positive), and the dynamic LDS that gives the pattern
// kernel (whose registers would allow more) that count.
template <int A, int S, int O, bool SPEC>
hipError_t traffic_lds(const KParams& p, int blocks_per_cu, size_t* lds)
{
    hipError_t e;
    int n = blocks_per_cu;
    if (n <= 0) {
        size_t real_lds = 0;
        if ((e = plan_lds<SPEC ? MAXT : 1>(p.max_writes, S, &real_lds)) != hipSuccess)
            return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&gdn_update_kernel<A, S, O, SPEC>), NTHREADS,
            real_lds);
        if (e != hipSuccess)
            return e;
    }
    DeviceInfo d;
    if ((e = device_info(&d)) != hipSuccess)
        return e;
    *lds = 0;
    const size_t share = static_cast<size_t>(d.lds_per_cu) / (n + 1) + 1;
    if (n > 0 && share <= static_cast<size_t>(d.lds_per_block))
        *lds = share;
    return hipSuccess;
}

constexpr int esize(int dt) { return dt == GDN_F32 ? 4 : (dt == GDN_F8E4M3 ? 1 : 2); }

template <int A, int S, int O, bool SPEC>
hipError_t launch_traffic_typed(const KParams& p, int64_t grid, hipStream_t stream)
{
    size_t lds = 0;
    hipError_t e = traffic_lds<A, S, O, SPEC>(p, p.pattern_blocks_per_cu, &lds);
    if (e != hipSuccess)
        return e;
    KParams args = p;
    void* argv[] = {&args};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(
            &gdn_traffic_kernel<esize(A), esize(S), esize(O), SPEC>),
        dim3(static_cast<uint32_t>(grid)), dim3(NTHREADS), argv, lds, stream);
}

template <int A, int S, bool SPEC>
hipError_t launch_traffic_out(int out, const KParams& p, int64_t grid, hipStream_t s)
{
    switch (out) {
    case GDN_F32: return launch_traffic_typed<A, S, GDN_F32, SPEC>(p, grid, s);
    case GDN_F16: return launch_traffic_typed<A, S, GDN_F16, SPEC>(p, grid, s);
    default: return launch_traffic_typed<A, S, GDN_BF16, SPEC>(p, grid, s);
    }
}

template <int A, bool SPEC>
hipError_t launch_traffic_state(int st, int out, const KParams& p, int64_t grid, hipStream_t s)
{
    switch (st) {
    case GDN_F32: return launch_traffic_out<A, GDN_F32, SPEC>(out, p, grid, s);
    case GDN_F16: return launch_traffic_out<A, GDN_F16, SPEC>(out, p, grid, s);
    case GDN_F8E4M3: return launch_traffic_out<A, GDN_F8E4M3, SPEC>(out, p, grid, s);
    default: return launch_traffic_out<A, GDN_BF16, SPEC>(out, p, grid, s);
    }
}

template <bool SPEC>
hipError_t launch_traffic(int act, int st, int out, const KParams& p, int64_t grid,
                          hipStream_t s)
{
    switch (act) {
    case GDN_F32: return launch_traffic_state<GDN_F32, SPEC>(st, out, p, grid, s);
    case GDN_F16: return launch_traffic_state<GDN_F16, SPEC>(st, out, p, grid, s);
    default: return launch_traffic_state<GDN_BF16, SPEC>(st, out, p, grid, s);
    }
}

gdn_status device_status(hipError_t e)
{
    if (e == hipSuccess)
        return GDN_OK;
    return gdn::fail(GDN_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
}

}  // namespace

extern "C" gdn_status gdn_spec_decode_update(const gdn_layer* layer,
                                             const gdn_state_pool* pool,
                                             const int32_t* cu_seqlens, int32_t num_seqs,
                                             int32_t max_q_len,
                                             const int32_t* spec_state_indices,
                                             int32_t spec_stride,
                                             const int32_t* num_accepted_tokens,
                                             const int32_t* token_indx, hipStream_t stream)
{
    gdn::clear_error();
    gdn_status st;
    if ((st = gdn::check_layer(layer)) != GDN_OK || (st = gdn::check_pool(pool)) != GDN_OK)
        return st;
    if (num_seqs < 0)
        return gdn::fail(GDN_ERR_INVALID, "num_seqs is negative");
    if (max_q_len < 1)
        return gdn::fail(GDN_ERR_INVALID, "max_q_len must be >= 1");
    if (max_q_len > GDN_MAX_DRAFT_TOKENS)
        return gdn::fail(GDN_ERR_UNSUPPORTED, "max_q_len %d exceeds %d draft tokens",
                         max_q_len, GDN_MAX_DRAFT_TOKENS);
    if (spec_stride < 1)
        return gdn::fail(GDN_ERR_INVALID, "spec_stride must be >= 1");
    if (num_seqs == 0 || layer->n_tok == 0)
        return GDN_OK;  // no sequence, or no row any sequence could use
    if (!cu_seqlens || !spec_state_indices || !num_accepted_tokens)
        return gdn::fail(GDN_ERR_INVALID, "spec metadata pointer is NULL");
    const int64_t grid = static_cast<int64_t>(num_seqs) * layer->num_v_heads;
    if (grid > 0x7fffffffLL)
        return gdn::fail(GDN_ERR_INVALID, "num_seqs * num_v_heads exceeds the grid limit");
    KParams p = make_params(layer, pool);
    p.cu = cu_seqlens;
    p.spec_idx = spec_state_indices;
    p.num_acc = num_accepted_tokens;
    p.tix = token_indx;
    p.spec_stride = spec_stride;
    p.num_spec = num_seqs;
    p.max_writes = max_q_len;
    return device_status(
        launch<true>(layer->act_dtype, pool->dtype, layer->out_dtype, p, grid, stream));
}

extern "C" gdn_status gdn_mixed_decode_update(const gdn_layer* layer,
                                              const gdn_state_pool* pool,
                                              const int32_t* cu_seqlens, int32_t num_seqs,
                                              int32_t max_q_len,
                                              const int32_t* spec_state_indices,
                                              int32_t spec_stride,
                                              const int32_t* num_accepted_tokens,
                                              const int32_t* spec_token_indx,
                                              const int32_t* state_indices, int32_t num_tokens,
                                              const int32_t* non_spec_token_indx,
                                              hipStream_t stream)
{
    gdn::clear_error();
    gdn_status st;
    if ((st = gdn::check_layer(layer)) != GDN_OK || (st = gdn::check_pool(pool)) != GDN_OK)
        return st;
    if (num_seqs < 0 || num_tokens < 0)
        return gdn::fail(GDN_ERR_INVALID, "num_seqs or num_tokens is negative");
    if (max_q_len < 1)
        return gdn::fail(GDN_ERR_INVALID, "max_q_len must be >= 1");
    if (max_q_len > GDN_MAX_DRAFT_TOKENS)
        return gdn::fail(GDN_ERR_UNSUPPORTED, "max_q_len %d exceeds %d draft tokens",
                         max_q_len, GDN_MAX_DRAFT_TOKENS);
    if (spec_stride < 1)
        return gdn::fail(GDN_ERR_INVALID, "spec_stride must be >= 1");
    if ((num_seqs == 0 && num_tokens == 0) || layer->n_tok == 0)
        return GDN_OK;
    if (num_seqs > 0 && (!cu_seqlens || !spec_state_indices || !num_accepted_tokens))
        return gdn::fail(GDN_ERR_INVALID, "spec metadata pointer is NULL");
    if (num_tokens > 0 && !state_indices)
        return gdn::fail(GDN_ERR_INVALID, "state_indices is NULL");
    const int64_t grid =
        (static_cast<int64_t>(num_seqs) + num_tokens) * layer->num_v_heads;
    if (grid > 0x7fffffffLL)
        return gdn::fail(GDN_ERR_INVALID, "(num_seqs + num_tokens) * num_v_heads exceeds the "
                                          "grid limit");
    KParams p = make_params(layer, pool);
    p.cu = cu_seqlens;
    p.spec_idx = spec_state_indices;
    p.num_acc = num_accepted_tokens;
    p.tix = spec_token_indx;
    p.spec_stride = spec_stride;
    p.num_spec = num_seqs;
    p.state_idx = state_indices;
    p.ns_tix = non_spec_token_indx;
    p.num_ns = num_tokens;
    p.max_writes = num_seqs > 0 ? max_q_len : 1;
    return device_status(
        launch<true>(layer->act_dtype, pool->dtype, layer->out_dtype, p, grid, stream));
}

extern "C" gdn_status gdn_decode_update(const gdn_layer* layer, const gdn_state_pool* pool,
                                        const int32_t* state_indices, int32_t num_tokens,
                                        const int32_t* token_indx, hipStream_t stream)
{
    gdn::clear_error();
    gdn_status st;
    if ((st = gdn::check_layer(layer)) != GDN_OK || (st = gdn::check_pool(pool)) != GDN_OK)
        return st;
    if (num_tokens < 0)
        return gdn::fail(GDN_ERR_INVALID, "num_tokens is negative");
    if (num_tokens == 0 || layer->n_tok == 0)
        return GDN_OK;
    if (!state_indices)
        return gdn::fail(GDN_ERR_INVALID, "state_indices is NULL");
    const int64_t grid = static_cast<int64_t>(num_tokens) * layer->num_v_heads;
    if (grid > 0x7fffffffLL)
        return gdn::fail(GDN_ERR_INVALID, "num_tokens * num_v_heads exceeds the grid limit");
    KParams p = make_params(layer, pool);
    p.state_idx = state_indices;
    p.tix = token_indx;
    p.spec_stride = 1;
    p.max_writes = 1;
    return device_status(
        launch<false>(layer->act_dtype, pool->dtype, layer->out_dtype, p, grid, stream));
}

extern "C" gdn_status gdn_cast_to_state(const float* src, void* dst, int64_t n, int32_t dtype,
                                        hipStream_t stream)
{
    gdn::clear_error();
    if (n < 0)
        return gdn::fail(GDN_ERR_INVALID, "n is negative");
    if (!gdn::dtype_size(dtype))
        return gdn::fail(GDN_ERR_UNSUPPORTED, "dtype %d is not f32/f16/bf16/f8e4m3", dtype);
    if (n == 0)
        return GDN_OK;
    if (!src || !dst)
        return gdn::fail(GDN_ERR_INVALID, "src or dst is NULL");
    const int64_t per_thread = dtype == GDN_F8E4M3 ? 16 : 1;
    const int64_t blocks = (n + 256 * per_thread - 1) / (256 * per_thread);
    const uint32_t grid = static_cast<uint32_t>(blocks < 65536 ? blocks : 65536);
    void* argv[] = {&src, &dst, &n};
    const void* fn;
    switch (dtype) {
    case GDN_F32: fn = reinterpret_cast<const void*>(&cast_kernel<GDN_F32>); break;
    case GDN_F16: fn = reinterpret_cast<const void*>(&cast_kernel<GDN_F16>); break;
    case GDN_BF16: fn = reinterpret_cast<const void*>(&cast_kernel<GDN_BF16>); break;
    default: fn = reinterpret_cast<const void*>(&cast_kernel<GDN_F8E4M3>); break;
    }
    return device_status(hipLaunchKernel(fn, dim3(grid), dim3(256), argv, 0, stream));
}

extern "C" gdn_status gdn_traffic_pattern(const gdn_layer* layer, const gdn_state_pool* pool,
                                          const int32_t* cu_seqlens, int32_t num_seqs,
                                          int32_t max_q_len, const int32_t* spec_state_indices,
                                          int32_t spec_stride,
                                          const int32_t* num_accepted_tokens,
                                          const int32_t* spec_token_indx,
                                          const int32_t* state_indices, int32_t num_tokens,
                                          const int32_t* non_spec_token_indx,
                                          int32_t blocks_per_cu, hipStream_t stream)
{
    gdn::clear_error();
    gdn_status st;
    if ((st = gdn::check_layer(layer)) != GDN_OK || (st = gdn::check_pool(pool)) != GDN_OK)
        return st;
    if (num_seqs < 0 || num_tokens < 0)
        return gdn::fail(GDN_ERR_INVALID, "num_seqs or num_tokens is negative");
    if (max_q_len < 1)
        return gdn::fail(GDN_ERR_INVALID, "max_q_len must be >= 1");
    if (max_q_len > GDN_MAX_DRAFT_TOKENS)
        return gdn::fail(GDN_ERR_UNSUPPORTED, "max_q_len %d exceeds %d draft tokens",
                         max_q_len, GDN_MAX_DRAFT_TOKENS);
    if (spec_stride < 1)
        return gdn::fail(GDN_ERR_INVALID, "spec_stride must be >= 1");
    if ((num_seqs == 0 && num_tokens == 0) || layer->n_tok == 0)
        return GDN_OK;
    if (num_seqs > 0 && (!cu_seqlens || !spec_state_indices || !num_accepted_tokens))
        return gdn::fail(GDN_ERR_INVALID, "spec metadata pointer is NULL");
    if (num_tokens > 0 && !state_indices)
        return gdn::fail(GDN_ERR_INVALID, "state_indices is NULL");
    const int64_t grid =
        (static_cast<int64_t>(num_seqs) + num_tokens) * layer->num_v_heads;
    if (grid > 0x7fffffffLL)
        return gdn::fail(GDN_ERR_INVALID, "(num_seqs + num_tokens) * num_v_heads exceeds the "
                                          "grid limit");
    if (blocks_per_cu < 0 || blocks_per_cu > 8)
        return gdn::fail(GDN_ERR_INVALID, "blocks_per_cu %d outside 0..8", blocks_per_cu);
    KParams p = make_params(layer, pool);
    p.spec_stride = spec_stride;
    p.pattern_blocks_per_cu = blocks_per_cu;
    if (num_seqs == 0) {
        // the single-token launch of gdn_decode_update
        p.state_idx = state_indices;
        p.tix = non_spec_token_indx;
        p.spec_stride = 1;
        p.max_writes = 1;
        return device_status(launch_traffic<false>(layer->act_dtype, pool->dtype,
                                                   layer->out_dtype, p, grid, stream));
    }
    p.cu = cu_seqlens;
    p.spec_idx = spec_state_indices;
    p.num_acc = num_accepted_tokens;
    p.tix = spec_token_indx;
    p.num_spec = num_seqs;
    p.state_idx = state_indices;
    p.ns_tix = non_spec_token_indx;
    p.num_ns = num_tokens;
    p.max_writes = max_q_len;
    return device_status(launch_traffic<true>(layer->act_dtype, pool->dtype, layer->out_dtype,
                                              p, grid, stream));
}
