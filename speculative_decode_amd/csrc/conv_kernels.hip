// conv_kernels.hip -- causal depthwise conv1d update with rewind over the wide
// rolling conv buffer, for CDNA4 (gfx950), and its two C-ABI entry points.
//
// What is computed is fixed by the vLLM PR reports on prhub.com.cn (#46090
// 实现拆解 items 1-2 and the gdn_attention.py excerpt: a speculative conv
// cache wider than width - 1, a width-wide view per draft token, the buffer
// written back; #51674 实现拆解 item 3: the conv update with rewind keyed by
// num_accepted_tokens runs before the fused recurrent update).  The buffer
// reading -- inputs oldest first, history at offset max(acc - 1, 0), write-back
// of the history without its oldest entry followed by every draft input -- is
// spelled out in gdn_conv.h.
//
// How it is computed here:
//   * Width 4 on the vector path (the conv width of the GDN layers, channel
//     counts a multiple of 8, channel-contiguous buffer): one wave per
//     (sequence, 512 channels), each lane a run of 8 channels, so every
//     buffer position, input row and output row of the run is one 16-byte
//     access per lane (two for fp32) and a wave moves coalesced 1 KiB rows.
//     The wave issues every load of its window at once -- width - 1 history
//     positions, then the draft inputs -- with the weights and bias of its
//     channels, keeps the window in registers, writes the buffer back from
//     the loaded bits and then computes and stores its outputs.  No LDS and
//     no barrier: there is one round of load latency per wave, and with
//     1,280 waves at B = 128, C = 5120 every wave is resident at once.
//     In-place safety: each buffer store waits for its own data, which was
//     loaded after every history position that store may overwrite, and no
//     two waves share a channel of a line.
//   * Other widths and layouts (width 1-3, channel-major buffers, odd
//     channel counts, unaligned views) take a block-staged kernel: one block
//     per (sequence, block of channels) -- 8 token slots x 64 runs of 8
//     channels, or one channel per thread with arbitrary strides -- stages
//     the window in LDS as fp32, each position loaded once, and after one
//     barrier each token slot computes its outputs from LDS and writes back
//     its buffer positions.  All reads of a line precede the barrier and all
//     writes follow it.
//   * Sequence metadata is uniform per wave and read with scalar loads; a
//     sequence with any out-of-range field is skipped before anything is
//     read or written.
//   * The kernels are HBM-bound: per active sequence they read width - 1
//     history positions and L inputs and write L outputs and width - 2 + L
//     positions, about 4 flop per byte.  Buffer stores are non-temporal (the
//     next read is one decode step away); output stores are not (the
//     recurrent update reads them next).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dtype_cvt.h"
#include "gdn_internal.h"

namespace {

using namespace gdn_dev;

constexpr int MAXW = GDN_CONV_MAX_WIDTH;     // 4
constexpr int MAXT = GDN_MAX_DRAFT_TOKENS;   // 8
constexpr int WAVE = 64;
constexpr int VEC_EPT = 8;                   // channels per lane, fast path

// Block geometry: one wave per token slot (TOK waves), each lane a run of
// EPT channels, so a block covers CB = 64 * EPT channels of one sequence.
// The vector path moves whole 16-byte chunks; the element-wise path EPT = 1.
template <bool SPEC, bool VEC>
struct Geo {
    static constexpr int TOK = SPEC ? MAXT : 1;
    static constexpr int EPT = VEC ? VEC_EPT : 1;
    static constexpr int THREADS = TOK * WAVE;
    static constexpr int CB = WAVE * EPT;
};

struct ConvParams {
    const void* x;
    int64_t x_st;
    void* out;
    int64_t o_st;
    const float* weight;
    const float* bias;
    void* cache;
    int64_t c_line, c_pos, c_chan;
    int64_t num_lines;
    int64_t n_tok;
    int32_t state_len;
    int32_t C;
    int32_t W;
    int32_t act;
    const int32_t* cu;
    const int32_t* lines;
    const int32_t* acc;
    const int32_t* tix;
    int32_t num_seqs;
    int32_t max_q_len;
    int32_t nblk;         // channel blocks per sequence
};

// The raw bits of EPT consecutive elements at byte address b (EPT a
// multiple of 8: contiguous, 16-byte aligned, moved in 16-byte chunks; EPT ==
// 1: one element).  Loads into it do not wait; unpack_run converts once
// every load of a phase has been issued.
template <int DT, int EPT>
struct RawRun {
    static constexpr int ESZ = DT == GDN_F32 ? 4 : 2;
    static constexpr int CHUNKS = EPT == 1 ? 0 : EPT * ESZ / 16;
    static constexpr int N = EPT == 1 ? 1 : 4 * CHUNKS;    // dwords
    uint32_t d[N];
};

template <int DT, int EPT>
__device__ __forceinline__ void load_raw(const char* b, RawRun<DT, EPT>& r)
{
    if constexpr (EPT == 1) {
        r.d[0] = load_one_raw<DT>(b, 0);
    } else {
#pragma unroll
        for (int c = 0; c < RawRun<DT, EPT>::CHUNKS; ++c) {
            // Streaming (non-temporal) loads: each run is read once per
            // launch, and buffer positions are rewritten in place right after.
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b + 16 * c));
            const uint4 a = make_uint4(v[0], v[1], v[2], v[3]);
            r.d[4 * c] = a.x; r.d[4 * c + 1] = a.y; r.d[4 * c + 2] = a.z; r.d[4 * c + 3] = a.w;
        }
    }
}

template <int DT, int EPT>
__device__ __forceinline__ void unpack_run(const RawRun<DT, EPT>& r, float (&f)[EPT])
{
    if constexpr (EPT == 1) {
        f[0] = unpack_one<DT>(r.d[0]);
    } else if constexpr (DT == GDN_F32) {
#pragma unroll
        for (int i = 0; i < EPT; ++i)
            f[i] = __uint_as_float(r.d[i]);
    } else {
#pragma unroll
        for (int i = 0; i < EPT / 2; ++i) {
            const float2 v = unpack_pair<DT>(r.d[i]);
            f[2 * i] = v.x;
            f[2 * i + 1] = v.y;
        }
    }
}

// Stores EPT values rounded into DT; NT selects non-temporal stores.
template <int DT, int EPT, bool NT>
__device__ __forceinline__ void store_run(char* b, const float (&f)[EPT])
{
    if constexpr (EPT == 1) {
        if constexpr (DT == GDN_F32)
            *reinterpret_cast<float*>(b) = f[0];
        else
            *reinterpret_cast<uint16_t*>(b) =
                static_cast<uint16_t>(pack2<DT>(f[0], 0.0f) & 0xffffu);
    } else {
        constexpr int ESZ = DT == GDN_F32 ? 4 : 2;
        constexpr int PER = 16 / ESZ;                  // elements per chunk
#pragma unroll
        for (int c = 0; c < EPT / PER; ++c) {
            u32x4 w;
            if constexpr (DT == GDN_F32) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w[i] = __float_as_uint(f[PER * c + i]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w[i] = pack2<DT>(f[PER * c + 2 * i], f[PER * c + 2 * i + 1]);
            }
            u32x4* q = reinterpret_cast<u32x4*>(b + 16 * c);
            if constexpr (NT)
                __builtin_nontemporal_store(w, q);
            else
                *q = w;
        }
    }
}

// Read-only metadata through the constant address space: a block-uniform
// index then compiles to a scalar load.  The arrays are never written during
// a launch (the buffers and outputs may not overlap them).
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* ro(const T* q)
{
    return reinterpret_cast<const __attribute__((address_space(4))) T*>(
        reinterpret_cast<uintptr_t>(q));
}

// SiLU with the hardware exp2 and reciprocal (about 1 ulp each, far inside
// the output tolerance); the limits come out as 0 for s -> -inf and s for
// s -> +inf.
__device__ __forceinline__ float silu(float s)
{
    const float e = __builtin_amdgcn_exp2f(-s * 1.4426950408889634f);
    return s * __builtin_amdgcn_rcpf(1.0f + e);
}

// One block per (sequence, block of CB channels); wave t is token slot t and
// lane r owns channels c0 .. c0 + EPT - 1.  The window of every token of the
// block is staged in LDS, right-aligned: slot s holds window position
// s - lead (lead = 4 - width leading slots are zero), so token t's taps
// always read slots t .. t + 3 against a right-aligned weight vector whose
// leading taps are zero -- no per-width branches, and exact
// (x + 0 * finite == x).  Wave t stages slots t, t + TOK, ...; after the
// block barrier it writes back the history shifts q < width - 2 with
// q = t (mod TOK) and its own token's input, and computes its token's
// outputs.  Slot, position and row are wave-uniform, so every address is a
// scalar base plus a 32-bit lane offset.  Every read of the line happens
// before the barrier, every write after it, and blocks of one sequence own
// disjoint channels: the in-place rewrite needs no other ordering.  A
// speculative block stages the weights of its channels in LDS once for its
// eight waves; a decode block (one wave) loads them directly.
template <int XT, int OT, bool SPEC, bool VEC>
__global__ void __launch_bounds__((Geo<SPEC, VEC>::THREADS)) conv_update_kernel(const ConvParams p)
{
    using G = Geo<SPEC, VEC>;
    constexpr int TOK = G::TOK;
    constexpr int EPT = G::EPT;
    constexpr int CB = G::CB;
    constexpr int NSLOT = MAXW - 1 + TOK;
    constexpr int KPT = (NSLOT + TOK - 1) / TOK;      // slots staged per wave
    constexpr int XSZ = XT == GDN_F32 ? 4 : 2;
    constexpr int OSZ = OT == GDN_F32 ? 4 : 2;
    constexpr bool WLDS = SPEC;                       // weights through LDS
    __shared__ __attribute__((aligned(16))) float E[NSLOT][CB];
    __shared__ __attribute__((aligned(16))) float Wl[WLDS ? CB : 1][MAXW];
    __shared__ __attribute__((aligned(16))) float Bl[WLDS ? CB : 1];

    const int64_t seq = blockIdx.x / p.nblk;
    const int64_t cbase = (blockIdx.x - seq * p.nblk) * static_cast<int64_t>(CB);
    const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / WAVE);
    const int r = static_cast<int>(threadIdx.x) % WAVE;
    const int64_t c0 = cbase + static_cast<int64_t>(r) * EPT;
    const bool live = c0 < p.C;
    const int W = p.W;
    const int lead = MAXW - W;

    // ---- block-uniform metadata, all loads first; one range predicate ----
    const int64_t line = ro(p.lines)[seq];
    int64_t first = seq;
    int L = 1, a = 1;
    if constexpr (SPEC) {
        const int32_t lo = ro(p.cu)[seq], hi = ro(p.cu)[seq + 1];
        a = ro(p.acc)[seq];
        first = lo;
        L = hi - lo;
    }
    const int64_t o = a > 1 ? a - 1 : 0;
    if (!(line >= 0 && line < p.num_lines && first >= 0 && L >= 1 && L <= p.max_q_len &&
          L <= TOK && a >= 0 && o + W - 1 <= p.state_len && W - 2 + L <= p.state_len))
        return;
    int64_t rows[TOK];
    bool rows_ok = true;
    if (p.tix) {
        const auto* tix = ro(p.tix);
#pragma unroll
        for (int i = 0; i < TOK; ++i)
            rows[i] = tix[first + (i < L ? i : L - 1)];
    } else {
#pragma unroll
        for (int i = 0; i < TOK; ++i)
            rows[i] = first + (i < L ? i : L - 1);
    }
#pragma unroll
    for (int i = 0; i < TOK; ++i)
        rows_ok = rows_ok && rows[i] >= 0 && rows[i] < p.n_tok;
    if (!rows_ok)
        return;

    // Lane offsets in bytes (the channel stride is 1 on the vector path).
    const int64_t cstep = VEC ? 1 : p.c_chan;
    const int64_t lane_c = static_cast<int64_t>(r) * EPT * cstep * XSZ;
    const uint32_t lane_x = static_cast<uint32_t>(r * EPT * XSZ);
    const uint32_t lane_o = static_cast<uint32_t>(r * EPT * OSZ);
    const char* const cache_line = static_cast<const char*>(p.cache) +
                                   (line * p.c_line + cbase * cstep) * XSZ;

    // ---- stage the window: issue every load, then fill LDS ----
    RawRun<XT, EPT> raw[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        const int sl = t + k * TOK;
        const int q = sl - lead;                      // window position (uniform)
#pragma unroll
        for (int i = 0; i < RawRun<XT, EPT>::N; ++i)
            raw[k].d[i] = 0;                          // zero in every format
        if (sl < NSLOT && q >= 0 && q < W - 1 + L && live) {
            if (q < W - 1) {
                load_raw<XT, EPT>(cache_line + (o + q) * p.c_pos * XSZ + lane_c, raw[k]);
            } else {
                int64_t row = rows[0];
#pragma unroll
                for (int i = 1; i < TOK; ++i)
                    row = (q - (W - 1) == i) ? rows[i] : row;
                load_raw<XT, EPT>(static_cast<const char*>(p.x) +
                                      (row * p.x_st + cbase) * XSZ + lane_x, raw[k]);
            }
        }
    }
    // weights and bias of the block's channels, right-aligned taps
    float wt[MAXW][EPT], bs[EPT];
    if constexpr (WLDS) {
        for (int ch = static_cast<int>(threadIdx.x); ch < CB; ch += G::THREADS) {
            const int64_t c = cbase + ch;
            float4 w = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            float b = 0.0f;
            if (c < p.C) {
                if (W == MAXW && VEC) {
                    w = reinterpret_cast<const float4*>(p.weight)[c];
                } else {
                    float ww[MAXW];
#pragma unroll
                    for (int j = 0; j < MAXW; ++j)
                        ww[j] = j >= lead ? p.weight[c * W + (j - lead)] : 0.0f;
                    w = make_float4(ww[0], ww[1], ww[2], ww[3]);
                }
                b = p.bias ? p.bias[c] : 0.0f;
            }
            *reinterpret_cast<float4*>(&Wl[ch][0]) = w;
            Bl[ch] = b;
        }
    } else if (live) {
        if (VEC && W == MAXW) {
            const float4* w4 = reinterpret_cast<const float4*>(p.weight + c0 * MAXW);
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const float4 w = w4[e];
                wt[0][e] = w.x; wt[1][e] = w.y; wt[2][e] = w.z; wt[3][e] = w.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPT; ++e)
#pragma unroll
                for (int j = 0; j < MAXW; ++j)
                    wt[j][e] = j >= lead ? p.weight[(c0 + e) * W + (j - lead)] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            bs[e] = p.bias ? p.bias[c0 + e] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        const int sl = t + k * TOK;
        if (sl < NSLOT) {
            float v[EPT];
            unpack_run<XT, EPT>(raw[k], v);
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                E[sl][r * EPT + e] = v[e];
        }
    }
    __syncthreads();
    if (!live)
        return;

    // ---- write-back: history shifts q < W - 2, then this token's input ----
    char* const cache_w = static_cast<char*>(p.cache) + (line * p.c_line + cbase * cstep) * XSZ;
    for (int q = t; q < W - 2; q += TOK) {
        float h[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            h[e] = E[q + 1 + lead][r * EPT + e];
        store_run<XT, EPT, true>(cache_w + q * p.c_pos * XSZ + lane_c, h);
    }
    if (t >= L)
        return;
    if (W - 2 + t >= 0) {
        float u[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            u[e] = E[MAXW - 1 + t][r * EPT + e];
        store_run<XT, EPT, true>(cache_w + (W - 2 + t) * p.c_pos * XSZ + lane_c, u);
    }

    // ---- this token's outputs: taps in ascending order, one FMA each ----
    if constexpr (WLDS) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const float4 w = *reinterpret_cast<const float4*>(&Wl[r * EPT + e][0]);
            wt[0][e] = w.x; wt[1][e] = w.y; wt[2][e] = w.z; wt[3][e] = w.w;
            bs[e] = Bl[r * EPT + e];
        }
    }
    int64_t row = rows[0];
#pragma unroll
    for (int i = 1; i < TOK; ++i)
        row = (t == i) ? rows[i] : row;
    float y[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        float acc = bs[e];
#pragma unroll
        for (int j = 0; j < MAXW; ++j)
            acc = fmaf(wt[j][e], E[t + j][r * EPT + e], acc);
        y[e] = p.act == GDN_CONV_ACT_SILU ? silu(acc) : acc;
    }
    store_run<OT, EPT, false>(static_cast<char*>(p.out) + (row * p.o_st + cbase) * OSZ + lane_o,
                              y);
}

// Stores the raw bits of a run (a copy of loaded input bits), non-temporal
// (vector path only).
template <int DT, int EPT>
__device__ __forceinline__ void store_raw_nt(char* b, const RawRun<DT, EPT>& r)
{
#pragma unroll
    for (int c = 0; c < RawRun<DT, EPT>::CHUNKS; ++c) {
        u32x4 w;
        w[0] = r.d[4 * c]; w[1] = r.d[4 * c + 1]; w[2] = r.d[4 * c + 2]; w[3] = r.d[4 * c + 3];
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(b + 16 * c));
    }
}

// Width-4 vector path: one wave per (entry, 512 channels).  Window slot s
// holds window position s: slots 0..2 the history, slot 3 + t draft input t.
template <int XT, int OT, bool SPEC>
__global__ void __launch_bounds__(WAVE) conv_window_kernel(const ConvParams p)
{
    constexpr int NT = SPEC ? MAXT : 1;
    constexpr int EPT = VEC_EPT;
    constexpr int CB = WAVE * EPT;
    constexpr int XSZ = XT == GDN_F32 ? 4 : 2;
    constexpr int OSZ = OT == GDN_F32 ? 4 : 2;
    constexpr int H = MAXW - 1;                     // history positions
    const int r = static_cast<int>(threadIdx.x);
    const int64_t seq = blockIdx.x / p.nblk;
    const int64_t cbase = (blockIdx.x - seq * p.nblk) * static_cast<int64_t>(CB);
    const int64_t c0 = cbase + static_cast<int64_t>(r) * EPT;

    // ---- wave-uniform metadata, all loads first; one range predicate ----
    const int64_t line = ro(p.lines)[seq];
    int64_t first = seq;
    int L = 1, a = 1;
    if constexpr (SPEC) {
        const int32_t lo = ro(p.cu)[seq], hi = ro(p.cu)[seq + 1];
        a = ro(p.acc)[seq];
        first = lo;
        L = hi - lo;
    }
    const int64_t o = a > 1 ? a - 1 : 0;
    if (!(line >= 0 && line < p.num_lines && first >= 0 && L >= 1 && L <= p.max_q_len &&
          L <= NT && a >= 0 && o + H <= p.state_len && H - 1 + L <= p.state_len))
        return;
    int64_t rows[NT];
    bool rows_ok = true;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t g = first + (i < L ? i : L - 1);
        rows[i] = p.tix ? static_cast<int64_t>(ro(p.tix)[g]) : g;
        rows_ok = rows_ok && rows[i] >= 0 && rows[i] < p.n_tok;
    }
    if (!rows_ok || c0 >= p.C)
        return;

    const uint32_t lane_x = static_cast<uint32_t>(r * EPT * XSZ);
    const uint32_t lane_o = static_cast<uint32_t>(r * EPT * OSZ);
    char* const cline = static_cast<char*>(p.cache) + (line * p.c_line + cbase) * XSZ + lane_x;

    // ---- every load first: history, draft inputs, weights and bias ----
    RawRun<XT, EPT> raw[H + NT];
#pragma unroll
    for (int q = 0; q < H; ++q)
        load_raw<XT, EPT>(cline + (o + q) * p.c_pos * XSZ, raw[q]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < RawRun<XT, EPT>::N; ++i)
            raw[H + t].d[i] = 0;
        if (t < L)
            load_raw<XT, EPT>(static_cast<const char*>(p.x) + (rows[t] * p.x_st + cbase) * XSZ +
                                  lane_x, raw[H + t]);
    }
    float4 w4[EPT];
    float bs[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        w4[e] = reinterpret_cast<const float4*>(p.weight)[c0 + e];
        bs[e] = 0.0f;
    }
    if (p.bias) {
        const float4 b0 = reinterpret_cast<const float4*>(p.bias + c0)[0];
        const float4 b1 = reinterpret_cast<const float4*>(p.bias + c0)[1];
        bs[0] = b0.x; bs[1] = b0.y; bs[2] = b0.z; bs[3] = b0.w;
        bs[4] = b1.x; bs[5] = b1.y; bs[6] = b1.z; bs[7] = b1.w;
    }

    // ---- write-back: position q <- slot q + 1 for q < H - 1 + L, as loaded ----
#pragma unroll
    for (int q = 0; q < H - 1 + NT; ++q)
        if (q < H - 1 + L)
            store_raw_nt<XT, EPT>(cline + q * p.c_pos * XSZ, raw[q + 1]);

    // ---- outputs: taps in ascending order, one FMA each ----
    float e[H + NT][EPT];
#pragma unroll
    for (int sl = 0; sl < H + NT; ++sl)
        unpack_run<XT, EPT>(raw[sl], e[sl]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < L) {
            float y[EPT];
#pragma unroll
            for (int c = 0; c < EPT; ++c) {
                float acc = bs[c];
                acc = fmaf(w4[c].x, e[t][c], acc);
                acc = fmaf(w4[c].y, e[t + 1][c], acc);
                acc = fmaf(w4[c].z, e[t + 2][c], acc);
                acc = fmaf(w4[c].w, e[t + 3][c], acc);
                y[c] = p.act == GDN_CONV_ACT_SILU ? silu(acc) : acc;
            }
            store_run<OT, EPT, false>(
                static_cast<char*>(p.out) + (rows[t] * p.o_st + cbase) * OSZ + lane_o, y);
        }
    }
}

template <int X, int O, bool SPEC>
hipError_t launch_ept(const ConvParams& p, bool vec, hipStream_t s)
{
    ConvParams args = p;
    void* argv[] = {&args};
    if (vec && p.W == MAXW) {
        args.nblk = (p.C + WAVE * VEC_EPT - 1) / (WAVE * VEC_EPT);
        const int64_t grid = static_cast<int64_t>(p.num_seqs) * args.nblk;
        return hipLaunchKernel(reinterpret_cast<const void*>(&conv_window_kernel<X, O, SPEC>),
                               dim3(static_cast<uint32_t>(grid)), dim3(WAVE), argv, 0, s);
    }
    const int64_t grid = static_cast<int64_t>(p.num_seqs) * p.nblk;
    const void* fn = vec ? reinterpret_cast<const void*>(&conv_update_kernel<X, O, SPEC, true>)
                         : reinterpret_cast<const void*>(&conv_update_kernel<X, O, SPEC, false>);
    const int threads = vec ? Geo<SPEC, true>::THREADS : Geo<SPEC, false>::THREADS;
    return hipLaunchKernel(fn, dim3(static_cast<uint32_t>(grid)), dim3(threads), argv, 0, s);
}

template <int X, bool SPEC>
hipError_t launch_out(int out, const ConvParams& p, bool vec, hipStream_t s)
{
    switch (out) {
    case GDN_F32: return launch_ept<X, GDN_F32, SPEC>(p, vec, s);
    case GDN_F16: return launch_ept<X, GDN_F16, SPEC>(p, vec, s);
    default: return launch_ept<X, GDN_BF16, SPEC>(p, vec, s);
    }
}

template <bool SPEC>
hipError_t launch(int xt, int out, const ConvParams& p, bool vec, hipStream_t s)
{
    switch (xt) {
    case GDN_F32: return launch_out<GDN_F32, SPEC>(out, p, vec, s);
    case GDN_F16: return launch_out<GDN_F16, SPEC>(out, p, vec, s);
    default: return launch_out<GDN_BF16, SPEC>(out, p, vec, s);
    }
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// The vector path needs every run to be whole aligned 16-byte chunks:
// channel-contiguous buffer, channel count a multiple of the run length,
// row/position strides multiples of 8 elements, 16-byte aligned bases and
// parameters.
bool vector_path_ok(const gdn_conv_layer* L, const gdn_conv_cache* c, bool spec)
{
    (void)spec;
    return L->channels % VEC_EPT == 0 && c->stride_chan == 1 && c->stride_line % 8 == 0 &&
           c->stride_pos % 8 == 0 && L->x_stride_tok % 8 == 0 &&
           L->out_stride_tok % 8 == 0 && aligned16(c->data) && aligned16(L->x) &&
           aligned16(L->out) && aligned16(L->weight) && (!L->bias || aligned16(L->bias));
}

// Channels one block covers: (256 / token slots) runs of 1 or 8 channels.
int channels_per_block(bool spec, bool vec)
{
    return spec ? (vec ? Geo<true, true>::CB : Geo<true, false>::CB)
                : (vec ? Geo<false, true>::CB : Geo<false, false>::CB);
}

ConvParams make_params(const gdn_conv_layer* L, const gdn_conv_cache* c, bool spec, bool vec)
{
    ConvParams p{};
    p.x = L->x;
    p.x_st = L->x_stride_tok;
    p.out = L->out;
    p.o_st = L->out_stride_tok;
    p.weight = L->weight;
    p.bias = L->bias;
    p.cache = c->data;
    p.c_line = c->stride_line;
    p.c_pos = c->stride_pos;
    p.c_chan = c->stride_chan;
    p.num_lines = c->num_lines;
    p.n_tok = L->n_tok;
    p.state_len = c->state_len;
    p.C = L->channels;
    p.W = L->width;
    p.act = L->activation;
    const int cb = channels_per_block(spec, vec);
    p.nblk = (L->channels + cb - 1) / cb;
    return p;
}

gdn_status launch_status(hipError_t e)
{
    if (e == hipSuccess)
        return GDN_OK;
    return gdn::fail(GDN_ERR_DEVICE, "conv kernel launch failed: %s", hipGetErrorString(e));
}

gdn_status check_grid(int32_t n, const ConvParams& p)
{
    if (static_cast<int64_t>(n) * p.nblk > 0x7fffffffLL)
        return gdn::fail(GDN_ERR_INVALID, "sequences x channels exceeds the grid limit");
    return GDN_OK;
}

}  // namespace

extern "C" gdn_status gdn_conv_spec_update(const gdn_conv_layer* layer,
                                           const gdn_conv_cache* cache,
                                           const int32_t* cu_seqlens, int32_t num_seqs,
                                           int32_t max_q_len, const int32_t* conv_indices,
                                           const int32_t* num_accepted_tokens,
                                           const int32_t* token_indx, hipStream_t stream)
{
    gdn::clear_error();
    gdn_status st;
    if ((st = gdn::check_conv_layer(layer)) != GDN_OK ||
        (st = gdn::check_conv_cache(cache, layer)) != GDN_OK)
        return st;
    if (num_seqs < 0)
        return gdn::fail(GDN_ERR_INVALID, "num_seqs is negative");
    if (max_q_len < 1)
        return gdn::fail(GDN_ERR_INVALID, "max_q_len must be >= 1");
    if (max_q_len > GDN_MAX_DRAFT_TOKENS)
        return gdn::fail(GDN_ERR_UNSUPPORTED, "max_q_len %d exceeds %d draft tokens", max_q_len,
                         GDN_MAX_DRAFT_TOKENS);
    if (layer->width - 2 + max_q_len > cache->state_len)
        return gdn::fail(GDN_ERR_INVALID,
                         "state_len %d < width - 2 + max_q_len = %d: the buffer cannot hold a "
                         "rewound history plus the drafts",
                         cache->state_len, layer->width - 2 + max_q_len);
    if (num_seqs == 0 || layer->n_tok == 0)
        return GDN_OK;
    if (!cu_seqlens || !conv_indices || !num_accepted_tokens)
        return gdn::fail(GDN_ERR_INVALID, "spec metadata pointer is NULL");
    const bool vec = vector_path_ok(layer, cache, true);
    ConvParams p = make_params(layer, cache, true, vec);
    if ((st = check_grid(num_seqs, p)) != GDN_OK)
        return st;
    p.cu = cu_seqlens;
    p.lines = conv_indices;
    p.acc = num_accepted_tokens;
    p.tix = token_indx;
    p.num_seqs = num_seqs;
    p.max_q_len = max_q_len;
    return launch_status(launch<true>(layer->x_dtype, layer->out_dtype, p, vec, stream));
}

extern "C" gdn_status gdn_conv_decode_update(const gdn_conv_layer* layer,
                                             const gdn_conv_cache* cache,
                                             const int32_t* conv_indices, int32_t num_tokens,
                                             const int32_t* token_indx, hipStream_t stream)
{
    gdn::clear_error();
    gdn_status st;
    if ((st = gdn::check_conv_layer(layer)) != GDN_OK ||
        (st = gdn::check_conv_cache(cache, layer)) != GDN_OK)
        return st;
    if (num_tokens < 0)
        return gdn::fail(GDN_ERR_INVALID, "num_tokens is negative");
    if (num_tokens == 0 || layer->n_tok == 0)
        return GDN_OK;
    if (!conv_indices)
        return gdn::fail(GDN_ERR_INVALID, "conv_indices is NULL");
    const bool vec = vector_path_ok(layer, cache, false);
    ConvParams p = make_params(layer, cache, false, vec);
    if ((st = check_grid(num_tokens, p)) != GDN_OK)
        return st;
    p.lines = conv_indices;
    p.tix = token_indx;
    p.num_seqs = num_tokens;
    p.max_q_len = 1;
    return launch_status(launch<false>(layer->x_dtype, layer->out_dtype, p, vec, stream));
}
