// W8A16 GEMV for decode (the M <= 2 path of gemv_w8a16; any M through the tiled
// entry): per-channel INT8 weights dequantized in
// registers against f16 activations, fp32 accumulation, f16 output.
//
// What is computed follows the ChatGLM2-6B W8A16 write-up (TPU-MLIR): section 2
// (weights stored per channel as INT8, computed in F16) and section 4 (load the
// INT8 weight, cast it to F16, apply the scale, multiply with the activation).
// The scale belongs to the output channel, so it is applied once to the finished
// sum instead of to each weight; that differs from scaling first only by fp32
// rounding.
//
// Work split as in the W4A8 kernel, with 1 KB tiles of 2 rows x 512 k (32 chunks
// of 16 INT8 weights per row): each wave streams the tiles of whole row groups, two
// batches in flight; a row's 32 lanes add their partial sums with DPP when the row
// group ends.  When K <= 4096 and M == 1 each lane loads the f16 activations of its
// chunks straight into registers (no LDS, no barrier); otherwise the workgroup
// stages X in LDS in chunk order, zero-padded to whole batches.
//
// Cast.  For a word of four int8 codes, XOR 0x80 per byte gives u = q + 128; a
// byte permute places 0x64 above each u, which as a binary16 is exactly 1024 + u;
// one packed f16 add of -1152 leaves q exactly.  Two 2-way f16 dots with fp32
// accumulation then consume the four weights.
#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

__device__ __forceinline__ void cast_i8x4_to_f16(uint32_t wd, half2_t& lo, half2_t& hi)
{
    const uint32_t u = wd ^ 0x80808080u;
    const uint32_t plo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // 0x64 u1 0x64 u0
    const uint32_t phi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // 0x64 u3 0x64 u2
    const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    lo = __builtin_bit_cast(half2_t, plo) + bias;
    hi = __builtin_bit_cast(half2_t, phi) + bias;
}

__device__ __forceinline__ void dot_chunk_f16(const uint4 w, const uint32_t (&a)[8], float (&acc)[4])
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        half2_t lo, hi;
        cast_i8x4_to_f16(wd[d], lo, hi);
        acc[d] = __builtin_amdgcn_fdot2(lo, __builtin_bit_cast(half2_t, a[2 * d]), acc[d], false);
        acc[d] = __builtin_amdgcn_fdot2(hi, __builtin_bit_cast(half2_t, a[2 * d + 1]), acc[d], false);
    }
}

__device__ __forceinline__ void split8(const uint4 e, const uint4 o, uint32_t (&a)[8])
{
    a[0] = e.x; a[1] = e.y; a[2] = e.z; a[3] = e.w;
    a[4] = o.x; a[5] = o.y; a[6] = o.z; a[7] = o.w;
}

// X (f16) staged in LDS in chunk order: row mm's chunk c (16 f16) is 16-byte pieces
// mm * 2 * chunks + 2c and + 2c + 1; pieces past K read zeros.  Pass `pass` of the
// pieces, kXP per thread, into xp.
template <int MT, int kXP, int kThreads>
__device__ __forceinline__ void load_x_pass(rsrc_t xres, int chunks, int K, int pass, int tid,
                                            uint4 (&xp)[kXP])
{
#pragma unroll
    for (int i = 0; i < kXP; ++i) {
        const int q = pass * kXP * kThreads + i * kThreads + tid;
        const int mm = q / (chunks * 2);
        const int r = q - mm * (chunks * 2);
        const bool in = mm < MT && r * 8 < K;
        xp[i] = load16(xres, in ? (uint32_t)(mm * K + r * 8) * 2u : 0x80000000u);
    }
}

// Writes the staged pieces to LDS; xp holds pass 0 on entry.  One pass (K <= 8192
// at MT = 1 with 4 waves) is a straight line whose stores wait for X alone, not for
// the weight loads issued after it.
template <int MT, int kXP, int kThreads>
__device__ __forceinline__ void store_x(rsrc_t xres, uint4 (&xp)[kXP], uint32_t* lds, int chunks,
                                        int K, int tid)
{
    const int pieces = MT * chunks * 2;
    const int npass = (pieces + kXP * kThreads - 1) / (kXP * kThreads);
    if (npass == 1) {
#pragma unroll
        for (int i = 0; i < kXP; ++i) {
            const int q = i * kThreads + tid;
            if (q < pieces)
                reinterpret_cast<uint4*>(lds)[q] = xp[i];
        }
    } else {
        for (int pass = 0; pass < npass; ++pass) {
            if (pass > 0)
                load_x_pass<MT, kXP, kThreads>(xres, chunks, K, pass, tid, xp);
#pragma unroll
            for (int i = 0; i < kXP; ++i) {
                const int q = pass * kXP * kThreads + i * kThreads + tid;
                if (q < pieces)
                    reinterpret_cast<uint4*>(lds)[q] = xp[i];
            }
        }
    }
}

// RCG > 0: register variant for exactly RCG tiles per row group (MT == 1).
// RCG == 0: LDS variant, U tiles per batch; S > 1 splits K as in the W4A8 kernel, the
// fp32 partial sums of the S slices being added in slice order.
template <int MT, int RCG, int U, int NW, int S = 1>
__global__ __launch_bounds__(64 * NW) void k_gemv_w8a16(W8A16Args p)
{
    constexpr int kThreads = 64 * NW;
    constexpr bool kReg = RCG > 0;
    constexpr int NR = NW / S;  // row runs per workgroup
    static_assert(!kReg || MT == 1, "register variant is for one row of X");
    static_assert(!kReg || S == 1, "split-K is in the LDS variant");
    constexpr int kB = kReg ? RCG : U;
    extern __shared__ uint32_t s_dyn[];  // LDS variant: [MT][padded chunks][8 words]; then scales

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, sub = lane >> 5;
    const int M = p.M, N = p.N, K = p.K, CG = p.cg;
    const int m0 = blockIdx.y * MT;
    const int mt = min(MT, M - m0);
    // k-slice of this wave: tiles [c_lo, c_lo + Tw) of each of its row groups
    const int ks = S > 1 ? wave % S : 0;
    const int rw = S > 1 ? wave / S : wave;
    const int T = (CG + S - 1) / S;
    const int c_lo = ks * T;
    const int Tw = max(0, min(CG, c_lo + T) - c_lo);
    const int nb = kReg ? 1 : (T + U - 1) / U;
    const int chunks = S * nb * kB * 32;  // LDS variant: chunks per X row in LDS (zero padded)

    // Row runs along N split the row groups evenly: run gw owns [rg_of(gw), rg_of(gw + 1)).
    const int W = p.nwaves;
    const int gw0 = blockIdx.x * NR;
    const int rg_blk = rg_of(gw0, p.per, p.rem);
    const int rg_blk_end = rg_of(min(gw0 + NR, W), p.per, p.rem);
    const int nrg_blk = rg_blk_end - rg_blk;
    const int gw = gw0 + rw;
    const int rg0 = gw < W ? rg_of(gw, p.per, p.rem) : rg_blk_end;
    const int rg1 = gw < W ? rg_of(gw + 1, p.per, p.rem) : rg_blk_end;
    const int nrg_w = rg1 - rg0;
    const int nq = nrg_w * nb;  // batches of this wave
    const rsrc_t wres =
        make_rsrc(p.Wq + (size_t)rg_blk * CG * 1024u, (uint32_t)(nrg_blk * CG) * 1024u);
    const uint32_t wbase = (uint32_t)((rg0 - rg_blk) * CG) * 1024u + (uint32_t)lane * 16u;

    uint4 wa[kB], wb[kB];
#define QW_LOAD(WBUF, Q)                                                                        \
    {                                                                                           \
        const int r_ = (Q) / nb, c0_ = ((Q) - r_ * nb) * kB;                                    \
        _Pragma("unroll") for (int u_ = 0; u_ < kB; ++u_)                                       \
        {                                                                                       \
            const bool ok_ = (Q) < nq && c0_ + u_ < Tw;                                         \
            WBUF[u_] = load16_stream(wres, ok_ ? wbase + (uint32_t)(r_ * CG + c_lo + c0_ + u_) * 1024u \
                                        : 0x80000000u);                                         \
        }                                                                                       \
        /* keep the batch's loads ahead of the dots that follow: without this the    */       \
        /* scheduler sinks them below the previous batch's dots, which then waits    */       \
        /* for its whole batch first and only one batch is ever in flight            */       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
    }

    // ---- prologue: scales, activations, then the first weight batch
    uint16_t* s_scale = reinterpret_cast<uint16_t*>(s_dyn + (kReg ? 0 : (size_t)MT * chunks * 8));
    const int rows_blk = min(nrg_blk * 2, N - rg_blk * 2);
    const rsrc_t sres = make_rsrc(p.w_scale + (size_t)rg_blk * 2, (uint32_t)max(rows_blk, 0) * 2u);
    uint16_t sc_reg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        sc_reg[i] = load2(sres, (uint32_t)(tid + i * kThreads) * 2u);
    const rsrc_t xres = make_rsrc(p.X + (size_t)m0 * K, (uint32_t)mt * (uint32_t)K * 2u);

    uint32_t act[kReg ? RCG : 1][8];
    if constexpr (kReg) {
        // chunk 32*c + j of row 0: 16 f16 at k = 16*(32c + j); past K reads zeros
#pragma unroll
        for (int c = 0; c < RCG; ++c) {
            const uint32_t xo = (uint32_t)((c * 32 + j) * 16) * 2u;
            const uint4 e = load16(xres, (c * 32 + j) * 16 < K ? xo : 0x80000000u);
            const uint4 o = load16(xres, (c * 32 + j) * 16 < K ? xo + 16u : 0x80000000u);
            split8(e, o, act[c]);
        }
        issue_barrier();
        QW_LOAD(wa, 0);
    } else {
        // stage X in LDS: 16-byte pieces, 2 per chunk
        constexpr int kXP = 4;
        uint4 xp[kXP];
        load_x_pass<MT, kXP, kThreads>(xres, chunks, K, 0, tid, xp);
        issue_barrier();
        QW_LOAD(wa, 0);
        store_x<MT, kXP, kThreads>(xres, xp, s_dyn, chunks, K, tid);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
        s_scale[tid + i * kThreads] = sc_reg[i];
    __syncthreads();

    const int nw0 = rg0 * 2;
    // split-K partial sums [run][row group][m][row][slice], after the scales
    const int PW = p.per + (p.rem > 0 ? 1 : 0);
    float* s_part = reinterpret_cast<float*>(s_scale + 2 * kThreads);
    auto finish_row_group = [&](float (&acc)[4], int mm, int rgi) {
        const float v = half_wave_sum_from_rows(row_sum16((acc[0] + acc[1]) + (acc[2] + acc[3])));
        const int n = nw0 + rgi * 2 + sub;
        if constexpr (S > 1) {
            if (j == 31)
                s_part[(((rw * PW + rgi) * MT + mm) * 2 + sub) * S + ks] = v;
        } else if (j == 31 && n < N && mm < mt) {
            const float s = __half2float(__ushort_as_half(s_scale[n - rg_blk * 2]));
            p.Y[(size_t)(m0 + mm) * N + n] = __half_as_ushort(__float2half_rn(v * s));
        }
    };

    if constexpr (kReg) {
#define QW_COMPUTE(WBUF, Q)                                                                     \
        {                                                                                       \
            float acc_[4] = {0.0f, 0.0f, 0.0f, 0.0f};                                           \
            _Pragma("unroll") for (int c_ = 0; c_ < RCG; ++c_) dot_chunk_f16(WBUF[c_], act[c_], acc_); \
            finish_row_group(acc_, 0, (Q));                                                     \
        }
        // Pairs of batches with no branch in the loop body, the odd one after it: an
        // exit from the middle of the body would let the compiler see the next batch
        // as possibly pending at the loop head and wait for every load there.
        int q = 0;
        for (; q + 1 < nq; q += 2) {
            QW_LOAD(wb, q + 1);
            QW_COMPUTE(wa, q);
            QW_LOAD(wa, q + 2);
            QW_COMPUTE(wb, q + 1);
        }
        if (q < nq)
            QW_COMPUTE(wa, q);
#undef QW_COMPUTE
    } else {
        float acc[MT][4];
#pragma unroll
        for (int mm = 0; mm < MT; ++mm)
            acc[mm][0] = acc[mm][1] = acc[mm][2] = acc[mm][3] = 0.0f;
#define QW_COMPUTE(WBUF, Q)                                                                     \
        {                                                                                       \
            const int r_ = (Q) / nb, b_ = (Q) - r_ * nb;                                        \
            _Pragma("unroll") for (int mm = 0; mm < MT; ++mm)                                   \
            {                                                                                   \
                uint32_t a_[U][8];                                                              \
                _Pragma("unroll") for (int u_ = 0; u_ < U; ++u_)                                \
                {                                                                               \
                    const uint4* ap_ = reinterpret_cast<const uint4*>(                          \
                        s_dyn + ((size_t)mm * chunks + (c_lo + b_ * U + u_) * 32 + j) * 8);     \
                    split8(ap_[0], ap_[1], a_[u_]);                                             \
                }                                                                               \
                _Pragma("unroll") for (int u_ = 0; u_ < U; ++u_)                                \
                    dot_chunk_f16(WBUF[u_], a_[u_], acc[mm]);                                   \
            }                                                                                   \
            if (b_ == nb - 1) {                                                                 \
                _Pragma("unroll") for (int mm = 0; mm < MT; ++mm)                               \
                {                                                                               \
                    finish_row_group(acc[mm], mm, r_);                                          \
                    acc[mm][0] = acc[mm][1] = acc[mm][2] = acc[mm][3] = 0.0f;                   \
                }                                                                               \
            }                                                                                   \
        }
        // Pairs of batches with no branch in the loop body, the odd one after it: an
        // exit from the middle of the body would let the compiler see the next batch
        // as possibly pending at the loop head and wait for every load there.
        int q = 0;
        for (; q + 1 < nq; q += 2) {
            QW_LOAD(wb, q + 1);
            QW_COMPUTE(wa, q);
            QW_LOAD(wa, q + 2);
            QW_COMPUTE(wb, q + 1);
        }
        if (q < nq)
            QW_COMPUTE(wa, q);
#undef QW_COMPUTE
        if constexpr (S > 1) {
            // every wave reaches this barrier; slice 0's wave of each run adds the
            // partials in slice order and applies the scale
            __syncthreads();
            if (ks == 0 && lane < 2) {
                for (int rgi = 0; rgi < nrg_w; ++rgi) {
                    const int n = nw0 + rgi * 2 + lane;
#pragma unroll
                    for (int mm = 0; mm < MT; ++mm) {
                        const float* pp = s_part + (((rw * PW + rgi) * MT + mm) * 2 + lane) * S;
                        float v = pp[0];
#pragma unroll
                        for (int k = 1; k < S; ++k)
                            v += pp[k];
                        if (n < N && mm < mt) {
                            const float sc = __half2float(__ushort_as_half(s_scale[n - rg_blk * 2]));
                            p.Y[(size_t)(m0 + mm) * N + n] = __half_as_ushort(__float2half_rn(v * sc));
                        }
                    }
                }
            }
        }
    }
#undef QW_LOAD
    (void)act;
}

// Eager variant (see the W4A8 kernel): every tile of the wave, at most TMAX, is
// requested right after X; X is staged in LDS and read one tile ahead of the dots.
template <int MT, int TMAX, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv_w8a16_eager(W8A16Args p)
{
    constexpr int kThreads = 64 * NW;
    extern __shared__ uint32_t s_dyn[];  // [MT][cg*32 chunks][8 words of f16 pairs]; then scales

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, sub = lane >> 5;
    const int M = p.M, N = p.N, K = p.K, CG = p.cg;
    const int m0 = blockIdx.y * MT;
    const int mt = min(MT, M - m0);
    const int chunks = CG * 32;

    const int W = p.nwaves;
    const int gw0 = blockIdx.x * NW;
    const int rg_blk = rg_of(gw0, p.per, p.rem);
    const int rg_blk_end = rg_of(min(gw0 + NW, W), p.per, p.rem);
    const int nrg_blk = rg_blk_end - rg_blk;
    const int gw = gw0 + wave;
    const int rg0 = gw < W ? rg_of(gw, p.per, p.rem) : rg_blk_end;
    const int rg1 = gw < W ? rg_of(gw + 1, p.per, p.rem) : rg_blk_end;
    const int T = (rg1 - rg0) * CG;
    const rsrc_t wres =
        make_rsrc(p.Wq + (size_t)rg_blk * CG * 1024u, (uint32_t)(nrg_blk * CG) * 1024u);
    const uint32_t wbase = (uint32_t)((rg0 - rg_blk) * CG) * 1024u + (uint32_t)lane * 16u;

    uint16_t* s_scale = reinterpret_cast<uint16_t*>(s_dyn + (size_t)MT * chunks * 8);
    const int rows_blk = min(nrg_blk * 2, N - rg_blk * 2);
    const rsrc_t sres = make_rsrc(p.w_scale + (size_t)rg_blk * 2, (uint32_t)max(rows_blk, 0) * 2u);
    uint16_t sc_reg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        sc_reg[i] = load2(sres, (uint32_t)(tid + i * kThreads) * 2u);
    const rsrc_t xres = make_rsrc(p.X + (size_t)m0 * K, (uint32_t)mt * (uint32_t)K * 2u);
    constexpr int kXP = 4;
    uint4 xp[kXP];
    load_x_pass<MT, kXP, kThreads>(xres, chunks, K, 0, tid, xp);
    issue_barrier();
    uint4 w[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
        w[t] = load16_stream(wres, t < T ? wbase + (uint32_t)t * 1024u : 0x80000000u);
    store_x<MT, kXP, kThreads>(xres, xp, s_dyn, chunks, K, tid);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        s_scale[tid + i * kThreads] = sc_reg[i];
    __syncthreads();

    float acc[MT][4];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
        acc[mm][0] = acc[mm][1] = acc[mm][2] = acc[mm][3] = 0.0f;
    uint32_t a_cur[MT][8];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
        const uint4* ap = reinterpret_cast<const uint4*>(s_dyn + ((size_t)mm * chunks + j) * 8);
        split8(ap[0], ap[1], a_cur[mm]);
    }
    int c = 0, rgi = 0;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t < T) {
            const int cn = c + 1 == CG ? 0 : c + 1;
            uint32_t a_nxt[MT][8];
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) {
                const uint4* ap =
                    reinterpret_cast<const uint4*>(s_dyn + ((size_t)mm * chunks + cn * 32 + j) * 8);
                split8(ap[0], ap[1], a_nxt[mm]);
            }
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
                dot_chunk_f16(w[t], a_cur[mm], acc[mm]);
            if (cn == 0) {
                const int n = (rg0 + rgi) * 2 + sub;
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) {
                    const float v = half_wave_sum_from_rows(
                        row_sum16((acc[mm][0] + acc[mm][1]) + (acc[mm][2] + acc[mm][3])));
                    acc[mm][0] = acc[mm][1] = acc[mm][2] = acc[mm][3] = 0.0f;
                    if (j == 31 && n < N && mm < mt) {
                        const float sc = __half2float(__ushort_as_half(s_scale[n - rg_blk * 2]));
                        p.Y[(size_t)(m0 + mm) * N + n] = __half_as_ushort(__float2half_rn(v * sc));
                    }
                }
                ++rgi;
            }
            c = cn;
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    a_cur[mm][e] = a_nxt[mm][e];
        }
    }
}

template <int MT, int TMAX, int NW>
hipError_t launch_eager(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    const dim3 grid(t.blocks, t.m_tiles);
    hipLaunchKernelGGL((k_gemv_w8a16_eager<MT, TMAX, NW>), grid, dim3(64 * NW), t.lds_bytes, st, a);
    return hipGetLastError();
}

template <int MT, int NW>
hipError_t launch_eager_t(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    return t.tmax == 8 ? launch_eager<MT, 8, NW>(a, t, st) : launch_eager<MT, 16, NW>(a, t, st);
}

// All-in-flight variant (M == 1, RCG tiles per row group, at most RPW row groups per
// wave), as in the W4A8 kernel: every weight tile of the wave is requested right after
// the scales and X, X is staged once per workgroup in LDS in chunk order, and each lane
// then holds the f16 activations of its RCG chunks in registers.
template <int RCG, int RPW, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv_w8a16_flight(W8A16Args p)
{
    constexpr int kThreads = 64 * NW;
    constexpr int chunks = RCG * 32;
    constexpr int kXP = (chunks * 2 + kThreads - 1) / kThreads;  // 16-byte X pieces per thread
    extern __shared__ uint32_t s_dyn[];  // [RCG * 32 chunks][8 words] X, then scales

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, sub = lane >> 5;
    const int N = p.N, K = p.K, CG = p.cg;

    const int W = p.nwaves;
    const int gw0 = blockIdx.x * NW;
    const int rg_blk = rg_of(gw0, p.per, p.rem);
    const int rg_blk_end = rg_of(min(gw0 + NW, W), p.per, p.rem);
    const int nrg_blk = rg_blk_end - rg_blk;
    const int gw = gw0 + wave;
    const int rg0 = gw < W ? rg_of(gw, p.per, p.rem) : rg_blk_end;
    const int rg1 = gw < W ? rg_of(gw + 1, p.per, p.rem) : rg_blk_end;
    const int nrg_w = rg1 - rg0;
    const rsrc_t wres =
        make_rsrc(p.Wq + (size_t)rg_blk * CG * 1024u, (uint32_t)(nrg_blk * CG) * 1024u);
    const uint32_t wbase = (uint32_t)((rg0 - rg_blk) * CG) * 1024u + (uint32_t)lane * 16u;

    uint16_t* s_scale = reinterpret_cast<uint16_t*>(s_dyn + (size_t)chunks * 8);
    const int rows_blk = min(nrg_blk * 2, N - rg_blk * 2);
    const rsrc_t sres = make_rsrc(p.w_scale + (size_t)rg_blk * 2, (uint32_t)max(rows_blk, 0) * 2u);
    uint16_t sc_reg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        sc_reg[i] = load2(sres, (uint32_t)(tid + i * kThreads) * 2u);
    const rsrc_t xres = make_rsrc(p.X, (uint32_t)K * 2u);
    uint4 xp[kXP];
#pragma unroll
    for (int i = 0; i < kXP; ++i) {
        const int q = i * kThreads + tid;  // piece q: f16 elements 8q .. 8q+7
        xp[i] = load16(xres, q * 8 < K ? (uint32_t)q * 16u : 0x80000000u);
    }
    issue_barrier();
    uint4 w[RPW][RCG];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int c = 0; c < RCG; ++c)
            w[r][c] = load16_stream(wres, r < nrg_w ? wbase + (uint32_t)(r * CG + c) * 1024u
                                                    : 0x80000000u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kXP; ++i) {
        const int q = i * kThreads + tid;
        if (q < chunks * 2)
            reinterpret_cast<uint4*>(s_dyn)[q] = xp[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
        s_scale[tid + i * kThreads] = sc_reg[i];
    __syncthreads();

    uint32_t act[RCG][8];
#pragma unroll
    for (int c = 0; c < RCG; ++c) {
        const uint4* ap = reinterpret_cast<const uint4*>(s_dyn + (size_t)(c * 32 + j) * 8);
        split8(ap[0], ap[1], act[c]);
    }
    const int nw0 = rg0 * 2;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < RCG; ++c)
            dot_chunk_f16(w[r][c], act[c], acc);
        const float v = half_wave_sum_from_rows(row_sum16((acc[0] + acc[1]) + (acc[2] + acc[3])));
        const int n = nw0 + r * 2 + sub;
        if (j == 31 && r < nrg_w && n < N) {
            const float sc = __half2float(__ushort_as_half(s_scale[n - rg_blk * 2]));
            p.Y[n] = __half_as_ushort(__float2half_rn(v * sc));
        }
    }
}

// Long-K form of the all-in-flight variant (M == 1), as in the W4A8 kernel: one row run
// of up to RPW row groups per workgroup, its S waves each taking a k-slice of 8 tiles;
// fp32 partial sums added in slice order by wave 0.  K up to 4096 * S.
template <int RPW, int S>
__global__ __launch_bounds__(64 * S) void k_gemv_w8a16_flight_split(W8A16Args p)
{
    constexpr int kThreads = 64 * S, RCG = 8;
    constexpr int chunks = S * RCG * 32;
    constexpr int kXP = (chunks * 2 + kThreads - 1) / kThreads;  // 16-byte X pieces per thread
    extern __shared__ uint32_t s_dyn[];  // [S * 8 * 32 chunks][8 words] X; scales; partials

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ks = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, sub = lane >> 5;
    const int N = p.N, K = p.K, CG = p.cg;
    const int c_lo = ks * RCG;
    const int Tw = max(0, min(CG, c_lo + RCG) - c_lo);

    const int W = p.nwaves;
    const int gw = blockIdx.x;
    const int rg0 = rg_of(gw, p.per, p.rem);
    const int rg1 = rg_of(gw + 1, p.per, p.rem);
    const int nrg_w = gw < W ? rg1 - rg0 : 0;
    const rsrc_t wres = make_rsrc(p.Wq + (size_t)rg0 * CG * 1024u, (uint32_t)(nrg_w * CG) * 1024u);
    const uint32_t wbase = (uint32_t)c_lo * 1024u + (uint32_t)lane * 16u;

    uint16_t* s_scale = reinterpret_cast<uint16_t*>(s_dyn + (size_t)chunks * 8);
    float* s_part = reinterpret_cast<float*>(s_dyn + (size_t)chunks * 8 + RPW);  // [RPW][2][S]
    const rsrc_t sres = make_rsrc(p.w_scale + (size_t)rg0 * 2, (uint32_t)max(0, min(nrg_w * 2, N - rg0 * 2)) * 2u);
    const uint16_t sc_reg = load2(sres, (uint32_t)(tid < RPW * 2 ? tid : 0x20000000) * 2u);
    const rsrc_t xres = make_rsrc(p.X, (uint32_t)K * 2u);
    uint4 xp[kXP];
#pragma unroll
    for (int i = 0; i < kXP; ++i) {
        const int q = i * kThreads + tid;
        xp[i] = load16(xres, q * 8 < K ? (uint32_t)q * 16u : 0x80000000u);
    }
    issue_barrier();
    uint4 w[RPW][RCG];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int c = 0; c < RCG; ++c)
            w[r][c] = load16_stream(wres, r < nrg_w && c < Tw ? wbase + (uint32_t)(r * CG + c) * 1024u
                                                             : 0x80000000u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kXP; ++i) {
        const int q = i * kThreads + tid;
        if (q < chunks * 2)
            reinterpret_cast<uint4*>(s_dyn)[q] = xp[i];
    }
    if (tid < RPW * 2)
        s_scale[tid] = sc_reg;
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);

    uint32_t act[RCG][8];
#pragma unroll
    for (int c = 0; c < RCG; ++c) {
        const uint4* ap = reinterpret_cast<const uint4*>(s_dyn + (size_t)((c_lo + c) * 32 + j) * 8);
        split8(ap[0], ap[1], act[c]);
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < RCG; ++c)
            dot_chunk_f16(w[r][c], act[c], acc);
        const float v = half_wave_sum_from_rows(row_sum16((acc[0] + acc[1]) + (acc[2] + acc[3])));
        if (j == 31)
            s_part[(r * 2 + sub) * S + ks] = v;
    }
    __syncthreads();
    if (tid < RPW * 2) {
        const int r = tid >> 1, n = rg0 * 2 + tid;
        float v = s_part[tid * S];
#pragma unroll
        for (int k = 1; k < S; ++k)
            v += s_part[tid * S + k];
        if (r < nrg_w && n < N) {
            const float sc = __half2float(__ushort_as_half(s_scale[tid]));
            p.Y[n] = __half_as_ushort(__float2half_rn(v * sc));
        }
    }
}

// Balanced long-K form: one workgroup per CU (more only past U row groups per CU) owns
// an even run of row groups; its S waves each take a k-slice of T tiles of every row
// group of the run, so each lane's f16 activations of the slice (T chunks of 16, for
// each of the workgroup's MT rows of X) stay in registers for the whole run.  A unit
// is one row group's T tiles of the wave's slice; the run goes through an unrolled
// pipeline with one unit requested ahead, X and the scales requested before any
// weight.  Each weight word is cast once for the MT rows of X.  The per-slice fp32 row
// sums meet in LDS and are added in slice order (deterministic) before the scale and
// the f16 rounding.  Grid: workgroups x ceil(M / MT) in one dimension, the groups of rows
// of one run numbered onto one XCD.  Up to 16 waves with MT == 1
// and slices of at most 4 tiles, else up to 8 (their registers).
constexpr int kBsMaxWaves = 16;

template <int T, int U, int MT>
__global__ __launch_bounds__(T <= 4 && MT == 1 ? 64 * kBsMaxWaves : 512) void k_gemv_w8a16_bsplit(W8A16Args p)
{
    __shared__ float s_part[MT * 2 * U * kBsMaxWaves];  // [row of X][row of the run][slice]
    __shared__ float s_sc[2 * U];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ks = __builtin_amdgcn_readfirstlane(tid >> 6);  // the k-slice of this wave
    const int nthreads = (int)blockDim.x;
    const int S = nthreads >> 6;
    const int j = lane & 31, sub = lane >> 5;
    const int N = p.N, K = p.K, CG = p.cg;
    const int c_lo = ks * T;
    // workgroup (run b, rows m0 ..): with several groups of rows, the groups of one run
    // are logical neighbours on one XCD, so the repeated reads of its weights meet in L2
    const int mtiles = (p.M + MT - 1) / MT;
    const int L = mtiles > 1 ? xcd_block((int)blockIdx.x, (int)gridDim.x) : (int)blockIdx.x;
    const int b = L / mtiles;
    const int m0 = MT * (L - b * mtiles);
    const int mv = min(MT, p.M - m0);
    const int rg0 = rg_of(b, p.per, p.rem);
    const int nb = min(U, rg_of(b + 1, p.per, p.rem) - rg0);
    const int nrows = max(0, min(2 * nb, N - 2 * rg0));
    const rsrc_t wres = make_rsrc(p.Wq + (size_t)rg0 * CG * 1024u, (uint32_t)(nb * CG) * 1024u);
    const rsrc_t sres = make_rsrc(p.w_scale + (size_t)rg0 * 2, (uint32_t)nrows * 2u);
    const rsrc_t xres = make_rsrc(p.X + (size_t)m0 * K, (uint32_t)mv * (uint32_t)K * 2u);

    // lane (j, sub): chunk j (16 k) of tile c of the slice -> X[m0 + m][512 (c_lo + c) + 16 j ..];
    // lanes j and j + 32 need the same chunk: each loads half of it (sub) and the
    // halves are swapped across the two half-waves
    uint4 xh[MT][T];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < T; ++c) {
            const int k = 512 * (c_lo + c) + 16 * j;
            xh[m][c] = load16(xres, m < mv && k < K ? (uint32_t)(m * K + k + 8 * sub) * 2u : 0x80000000u);
        }
    const uint16_t sc_reg = load2(sres, (uint32_t)tid * 2u);
    uint4 w[U][T];
    // the T tiles of unit U_ (row group U_ of the run; zeros past the run and past CG)
#define QW_LOADW(U_)                                                                             \
    _Pragma("unroll") for (int c_ = 0; c_ < T; ++c_)                                             \
        w[U_][c_] = load16_stream(wres, (U_) < nb && c_lo + c_ < CG                              \
                                            ? (uint32_t)((U_) * CG + c_lo + c_) * 1024u +        \
                                                  (uint32_t)lane * 16u                           \
                                            : 0x80000000u);
    issue_barrier();
    QW_LOADW(0);
    __builtin_amdgcn_sched_barrier(0);
    if (tid < 2 * U)
        s_sc[tid] = __half2float(__ushort_as_half(sc_reg));
    uint32_t act[MT][T][8];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < T; ++c) {
            const uint4 mine = xh[m][c];
            uint4 other;
            other.x = (uint32_t)__shfl_xor((int)mine.x, 32, 64);
            other.y = (uint32_t)__shfl_xor((int)mine.y, 32, 64);
            other.z = (uint32_t)__shfl_xor((int)mine.z, 32, 64);
            other.w = (uint32_t)__shfl_xor((int)mine.w, 32, 64);
            if (sub == 0)
                split8(mine, other, act[m][c]);
            else
                split8(other, mine, act[m][c]);
        }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u + 1 < U) {
            QW_LOADW(u + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (u < nb) {
            float acc[MT][4];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    acc[m][d] = 0.0f;
#pragma unroll
            for (int c = 0; c < T; ++c) {
                const uint32_t wd[4] = {w[u][c].x, w[u][c].y, w[u][c].z, w[u][c].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    half2_t lo, hi;
                    cast_i8x4_to_f16(wd[d], lo, hi);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        acc[m][d] = __builtin_amdgcn_fdot2(lo, __builtin_bit_cast(half2_t, act[m][c][2 * d]),
                                                           acc[m][d], false);
                        acc[m][d] = __builtin_amdgcn_fdot2(hi, __builtin_bit_cast(half2_t, act[m][c][2 * d + 1]),
                                                           acc[m][d], false);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float v = half_wave_sum_from_rows(row_sum16((acc[m][0] + acc[m][1]) + (acc[m][2] + acc[m][3])));
                if (j == 31)
                    s_part[((m * U + u) * 2 + sub) * kBsMaxWaves + ks] = v;
            }
        }
    }
#undef QW_LOADW
    __syncthreads();
    for (int e = tid; e < mv * nrows; e += nthreads) {
        const int m = e / nrows, rr = e - m * nrows;
        const float* src = s_part + (m * 2 * U + rr) * kBsMaxWaves;
        float v = src[0];
        for (int k = 1; k < S; ++k)
            v += src[k];
        p.Y[(size_t)(m0 + m) * N + 2 * rg0 + rr] = __half_as_ushort(__float2half_rn(v * s_sc[rr]));
    }
}

template <int T, int U, int MT>
hipError_t launch_bsplit_m(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    if (t.splitk > (T <= 4 && MT == 1 ? kBsMaxWaves : 8))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gemv_w8a16_bsplit<T, U, MT>), dim3(t.blocks * t.m_tiles), dim3(64 * t.splitk), 0,
                       st, a);
    return hipGetLastError();
}

template <int T, int U>
hipError_t launch_bsplit_u(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.mt) {
    case 1: return launch_bsplit_m<T, U, 1>(a, t, st);
    case 2: return launch_bsplit_m<T, U, 2>(a, t, st);
    case 4:
        if constexpr (T <= 5)
            return launch_bsplit_m<T, U, 4>(a, t, st);
        else
            return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int T>
hipError_t launch_bsplit_t(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    const int per = a.per + (a.rem > 0 ? 1 : 0);
    return per <= 8 ? launch_bsplit_u<T, 8>(a, t, st) : launch_bsplit_u<T, 16>(a, t, st);
}

hipError_t launch_bsplit(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.reg_cg) {
    case 1: return launch_bsplit_t<1>(a, t, st);
    case 2: return launch_bsplit_t<2>(a, t, st);
    case 3: return launch_bsplit_t<3>(a, t, st);
    case 4: return launch_bsplit_t<4>(a, t, st);
    case 5: return launch_bsplit_t<5>(a, t, st);
    case 6: return launch_bsplit_t<6>(a, t, st);
    case 7: return launch_bsplit_t<7>(a, t, st);
    case 8: return launch_bsplit_t<8>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

template <int RPW, int S>
hipError_t launch_flight_split(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    hipLaunchKernelGGL((k_gemv_w8a16_flight_split<RPW, S>), dim3(t.blocks), dim3(64 * S),
                       t.lds_bytes, st, a);
    return hipGetLastError();
}

template <int RPW>
hipError_t launch_flight_split_s(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.splitk) {
    case 2: return launch_flight_split<RPW, 2>(a, t, st);
    case 3: return launch_flight_split<RPW, 3>(a, t, st);
    case 4: return launch_flight_split<RPW, 4>(a, t, st);
    case 5: return launch_flight_split<RPW, 5>(a, t, st);
    case 6: return launch_flight_split<RPW, 6>(a, t, st);
    case 7: return launch_flight_split<RPW, 7>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_flight_split_any(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.tmax) {
    case 1: return launch_flight_split_s<1>(a, t, st);
    case 2: return launch_flight_split_s<2>(a, t, st);
    case 4: return launch_flight_split_s<4>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

template <int RCG, int RPW>
hipError_t launch_flight(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    hipLaunchKernelGGL((k_gemv_w8a16_flight<RCG, RPW, 4>), dim3(t.blocks), dim3(256),
                       t.lds_bytes, st, a);
    return hipGetLastError();
}

template <int RCG>
hipError_t launch_flight_r(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.tmax) {
    case 1: return launch_flight<RCG, 1>(a, t, st);
    case 2: return launch_flight<RCG, 2>(a, t, st);
    case 3: return launch_flight<RCG, 3>(a, t, st);
    case 4: return launch_flight<RCG, 4>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_flight_any(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.reg_cg) {
    case 1: return launch_flight_r<1>(a, t, st);
    case 2: return launch_flight_r<2>(a, t, st);
    case 3: return launch_flight_r<3>(a, t, st);
    case 4: return launch_flight_r<4>(a, t, st);
    case 5: return launch_flight_r<5>(a, t, st);
    case 6: return launch_flight_r<6>(a, t, st);
    case 7: return launch_flight_r<7>(a, t, st);
    case 8: return launch_flight_r<8>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

template <int MT, int RCG, int U, int NW, int S = 1>
hipError_t launch4(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    const dim3 grid(t.blocks, t.m_tiles);
    hipLaunchKernelGGL((k_gemv_w8a16<MT, RCG, U, NW, S>), grid, dim3(64 * NW), t.lds_bytes, st, a);
    return hipGetLastError();
}

// split-K: at most 2 rows of X per workgroup, 4 or 8 waves
template <int MT, int NW>
hipError_t launch_split(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    if (t.u == 4)
        return t.splitk == 2 ? launch4<MT, 0, 4, NW, 2>(a, t, st) : launch4<MT, 0, 4, NW, 4>(a, t, st);
    return t.splitk == 2 ? launch4<MT, 0, 8, NW, 2>(a, t, st) : launch4<MT, 0, 8, NW, 4>(a, t, st);
}

template <int NW>
hipError_t launch_reg(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.reg_cg) {
    case 1: return launch4<1, 1, 4, NW>(a, t, st);
    case 2: return launch4<1, 2, 4, NW>(a, t, st);
    case 3: return launch4<1, 3, 4, NW>(a, t, st);
    case 4: return launch4<1, 4, 4, NW>(a, t, st);
    case 5: return launch4<1, 5, 4, NW>(a, t, st);
    case 6: return launch4<1, 6, 4, NW>(a, t, st);
    case 7: return launch4<1, 7, 4, NW>(a, t, st);
    case 8: return launch4<1, 8, 4, NW>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

template <int MT, int NW>
hipError_t launch_lds(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    return t.u == 4 ? launch4<MT, 0, 4, NW>(a, t, st) : launch4<MT, 0, 8, NW>(a, t, st);
}

template <int NW>
hipError_t launch_nw(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    if (t.splitk > 1) {
        if constexpr (NW == 16) {
            return hipErrorInvalidValue;
        } else {
            switch (t.mt) {
            case 1: return launch_split<1, NW>(a, t, st);
            case 2: return launch_split<2, NW>(a, t, st);
            default: return hipErrorInvalidValue;
            }
        }
    }
    if (t.u == 1) {
        switch (t.mt) {
        case 1: return launch_eager_t<1, NW>(a, t, st);
        case 2: return launch_eager_t<2, NW>(a, t, st);
        case 4: return launch_eager_t<4, NW>(a, t, st);
        default: return hipErrorInvalidValue;
        }
    }
    if (t.reg_cg > 0)
        return launch_reg<NW>(a, t, st);
    switch (t.mt) {
    case 1: return launch_lds<1, NW>(a, t, st);
    case 2: return launch_lds<2, NW>(a, t, st);
    case 4: return launch_lds<4, NW>(a, t, st);
    case 8: return launch_lds<8, NW>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv_w8a16(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    if (t.u == 2)
        return launch_flight_any(a, t, st);
    if (t.u == 3)
        return launch_flight_split_any(a, t, st);
    if (t.u == 7)
        return launch_bsplit(a, t, st);
    switch (t.nw) {
    case 4: return launch_nw<4>(a, t, st);
    case 8: return launch_nw<8>(a, t, st);
    case 16: return launch_nw<16>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qw
