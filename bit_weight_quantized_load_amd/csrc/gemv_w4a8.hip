// W4A8 GEMV for decode (the M == 1 path of gemv_w4a8; any M through the tiled entry):
// INT4 weights, INT8 activations quantized in the prologue, int8 dot products into
// int32, output acc * w_scale * a_scale.
//
// What is computed follows "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s":
// section 正确方向 (INT4 widened to int8 lanes in registers, 4-way int8 dot into
// int32) and section 当前实现方式 (row-wise weight scale, per-vector dynamic
// activation scale, output = int32 acc * weight_scale * activation_scale).  The
// page's first follow-up item (fold the activation quantization into the linear
// kernel) is the prologue below.
//
// Work split.  The packed weights are 1 KB tiles of 4 rows x 512 k (16 chunks of
// 32 nibbles per row, see kernels.hpp).  Each wave owns an even share of whole row
// groups (nwaves waves split them), a contiguous run of tiles, and streams it with one 16-byte load per lane
// per tile, two batches in flight.  Lane (sub, j) always meets row 4*rg + sub and
// chunk 16*cg + j, so a row's partial sums live in the 16 lanes of one DPP row and
// are added with four DPP steps when the row group ends.  No row is split across
// waves or workgroups.
//
// Two variants.  When K <= 4096 and M == 1 (kRegCG tiles per row group), a batch is
// one whole row group and each lane keeps the activation codes of its chunks in
// registers, read from LDS once.  Otherwise a batch is U tiles of a row group and
// the codes are read from LDS per batch, all U tiles' words before the dots; LDS is
// zero-padded to whole batches so the batch body has no branches.
//
// Prologue.  Output scales and X row 0 are loaded first and the first weight batch
// right after them (loads complete in order, so anything the prologue waits on must
// be issued before the weights).  The workgroup takes max|X[m,:]| from registers,
// reduces it across waves, and quantizes the same registers into LDS in the order
// the unpack consumes: for each 8 consecutive k, the even-k codes form one 32-bit
// word and the odd-k codes the next.  Chunks past K get zero codes, which also
// cancels whatever the padding weights hold.
//
// Unpack.  A 32-bit word of packed weights holds k..k+7, even k in the low
// nibbles.  (w << 4) & 0xF0F0F0F0 puts the even nibbles, and w & 0xF0F0F0F0 the odd
// nibbles, into the top half of each byte: each byte is then 16*q as an int8, so
// two 4-way dots against the even and odd activation words accumulate 16 * sum(q*x)
// exactly; an arithmetic shift by 4 at the end is exact.  |16 * acc| stays below
// 2^31 for K <= 131072.  Four independent accumulators (one per word of a chunk)
// keep the dot latency off the critical path.
#include "common.hpp"
#include "kernels.hpp"
#include "w4a8_prod.hpp"

namespace qw {

namespace {

// Block `blk` of X row m0 + mm (XV float4 per thread, kThreads threads) into xv.
// Rows past the workgroup's mt rows and elements past K read zeros.
template <int XV, int kThreads>
__device__ __forceinline__ void load_x_block(const W4A8Args& p, int m0, int mt, int mm, int blk,
                                             int tid, float4 (&xv)[XV])
{
    const rsrc_t xr = make_rsrc(p.X + (size_t)(m0 + mm) * p.K, mm < mt ? (uint32_t)p.K * 4u : 0u);
#pragma unroll
    for (int i = 0; i < XV; ++i)
        xv[i] = load16f(xr, (uint32_t)(blk * XV * kThreads + i * kThreads + tid) * 16u);
}

// The activation prologue (the per-vector dynamic quantization of the Jetson Orin
// INT4 write-up, section 当前实现方式), for the MT rows of X of this workgroup: per
// row a = maxabs / 127 and codes clamp(rint(x / a), -127, 127), written to LDS at
// act + mm * chunks * 8 words.  In chunk c (32 consecutive k), word 2d holds the
// codes of k = 32c + 8d + {0, 2, 4, 6} and word 2d + 1 those of k = 32c + 8d + {1, 3,
// 5, 7}, the order in which the INT4 unpack presents the weights; padding chunks are
// zero.  Block 0 of row 0 must already be in xv.  kOne: K fits one block, so X is
// never re-read; the only wait before the codes are written is then the one for X
// itself, not for weight loads issued after it.
template <int MT, int NW, int XV, bool kOne, bool kDebug>
__device__ __forceinline__ void quantize_rows(const W4A8Args& p, float4 (&xv)[XV],
                                              uint32_t* act, float (&s_red)[MT][NW],
                                              float (&s_a)[MT], int chunks, int nblk, int m0,
                                              int mt, int tid)
{
    constexpr int kThreads = 64 * NW;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K4 = p.K >> 2;
    const int cpr = p.K >> 5;  // real chunks per row
    const int nb = kOne ? 1 : nblk;
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
        float mx = 0.0f;
        for (int blk = 0; blk < nb; ++blk) {
            if (mm > 0 || blk > 0)
                load_x_block<XV, kThreads>(p, m0, mt, mm, blk, tid, xv);
#pragma unroll
            for (int i = 0; i < XV; ++i)
                mx = fmaxf(mx, max_abs4(xv[i]));  // past K the loads read zeros
        }
        mx = wave_max_dpp(mx);
        if (lane == 0)
            s_red[mm][wave] = mx;
        __syncthreads();
        mx = s_red[mm][0];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            mx = fmaxf(mx, s_red[mm][w]);
        const float a = mx / 127.0f;
        const float r = 1.0f / a;
        const bool fast = r <= 3.0e38f;  // finite reciprocal (a is not 0 or tiny)
        if (tid == 0)
            s_a[mm] = a;
        uint16_t* act16 = reinterpret_cast<uint16_t*>(act + (size_t)mm * chunks * 8);
        for (int blk = 0; blk < nb; ++blk) {
            if (!kOne)
                load_x_block<XV, kThreads>(p, m0, mt, mm, blk, tid, xv);
#pragma unroll
            for (int i = 0; i < XV; ++i) {
                const int f = blk * XV * kThreads + i * kThreads + tid;  // k = 4f .. 4f+3
                if (f < K4) {
                    uint32_t e[4];  // the codes in byte 2
                    if (quant4_e(xv[i], r, e) || !fast)
                        quant4_e_div(xv[i], a, e);
                    // chunk f/8, 8-group (f/2)%4, half f%2: even codes -> word 2d, odd -> 2d+1
                    const int c = f >> 3, d = (f >> 1) & 3, h = f & 1;
                    const int wi = (c * 8 + 2 * d) * 2 + h;  // halfword index in the even word
                    act16[wi] = (uint16_t)__builtin_amdgcn_perm(e[2], e[0], 0x0C0C0602u);
                    act16[wi + 2] = (uint16_t)__builtin_amdgcn_perm(e[3], e[1], 0x0C0C0602u);
                    if (kDebug && p.dbg_xq != nullptr && blockIdx.x == 0 && mm < mt)
                        *reinterpret_cast<uint32_t*>(p.dbg_xq + (size_t)(m0 + mm) * p.K + 4 * f) =
                            __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0602u) |
                            __builtin_amdgcn_perm(e[3], e[2], 0x06020C0Cu);
                }
            }
        }
        // zero codes for the padding chunks
        for (int w = cpr * 8 + tid; w < chunks * 8; w += kThreads)
            act[(size_t)mm * chunks * 8 + w] = 0u;
    }
    if (kDebug && p.dbg_a != nullptr && blockIdx.x == 0 && tid < mt)
        p.dbg_a[m0 + tid] = s_a[tid];
    // keep the weight unpacking of the caller below this barrier: hoisted above it, it
    // makes every wave wait for its first weight tile before the barrier can complete
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// RCG > 0: register variant for exactly RCG tiles per row group (MT == 1).
// RCG == 0: LDS variant, U tiles per batch; S > 1 splits K: the S waves that share a
// row group each take one of S runs of its tiles, and their int32 partial sums are
// added in LDS once every wave of the workgroup is done.
template <int MT, int RCG, int U, int NW, int S, bool kDebug>
__global__ __launch_bounds__(64 * NW) void k_gemv_w4a8(W4A8Args p)
{
    constexpr int kThreads = 64 * NW;
    constexpr bool kReg = RCG > 0;
    constexpr int NR = NW / S;  // row runs per workgroup
    static_assert(!kReg || MT == 1, "register variant is for one row of X");
    static_assert(!kReg || S == 1, "split-K is in the LDS variant");
    constexpr int kB = kReg ? RCG : U;                                     // tiles per batch
    constexpr int XV = kReg ? (RCG * 128 + kThreads - 1) / kThreads : 16;  // X float4 per thread
    extern __shared__ uint32_t s_dyn[];  // [MT][padded chunks][8 words] codes, then scales
    __shared__ float s_red[MT][NW];
    __shared__ float s_a[MT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index as a wave-uniform (scalar) value: loop bounds and tile tests below
    // are then scalar branches, not per-lane ones
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, sub = lane >> 4;
    const int M = p.M, N = p.N, K = p.K, CG = p.cg;
    const int m0 = blockIdx.y * MT;
    const int mt = min(MT, M - m0);
    const int K4 = K >> 2;
    // k-slice of this wave: tiles [c_lo, c_lo + Tw) of each of its row groups
    const int ks = S > 1 ? wave % S : 0;
    const int rw = S > 1 ? wave / S : wave;
    const int T = (CG + S - 1) / S;
    const int c_lo = ks * T;
    const int Tw = max(0, min(CG, c_lo + T) - c_lo);
    const int nb = kReg ? 1 : (T + U - 1) / U;  // batches per row group
    const int chunks = S * nb * kB * 16;         // chunks per X row in LDS (zero padded)

    // ---- this wave's run of tiles
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
    // batch q = (row group q / nb, tiles (q % nb) * kB ..); tiles past the row group
    // and batches past the wave's run read zeros
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

    // ---- prologue: scales, X row 0, then the first weight batch
    float* s_scale = reinterpret_cast<float*>(s_dyn + (size_t)MT * chunks * 8);
    const int rows_blk = min(nrg_blk * 4, N - rg_blk * 4);
    const rsrc_t sres = make_rsrc(p.w_scale + (size_t)rg_blk * 4, (uint32_t)max(rows_blk, 0) * 4u);
    uint32_t sc_reg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        sc_reg[i] = load4(sres, (uint32_t)(tid + i * kThreads) * 4u);
    const int nblk = (K4 + XV * kThreads - 1) / (XV * kThreads);
    float4 xv[XV];
    load_x_block<XV, kThreads>(p, m0, mt, 0, 0, tid, xv);
    issue_barrier();
    QW_LOAD(wa, 0);
    // unconditional stores (rows past the block read zeros): a guarded store would
    // let the compiler sink the scale load behind the weight loads
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s_scale[tid + i * kThreads] = __uint_as_float(sc_reg[i]);
    if (kReg || nblk == 1)
        quantize_rows<MT, NW, XV, true, kDebug>(p, xv, s_dyn, s_red, s_a, chunks, nblk, m0, mt, tid);
    else
        quantize_rows<MT, NW, XV, false, kDebug>(p, xv, s_dyn, s_red, s_a, chunks, nblk, m0, mt, tid);

    const int nw0 = rg0 * 4;  // first row of this wave
    // split-K partial sums [run][row group][m][row][slice], after the scales
    const int PW = p.per + (p.rem > 0 ? 1 : 0);
    int* s_part = reinterpret_cast<int*>(s_scale + 4 * kThreads);
    auto finish_row_group = [&](int (&acc)[4], int mm, int rgi) {
        const int v = row_sum16(acc[0] + acc[1] + acc[2] + acc[3]) >> 4;
        const int n = nw0 + rgi * 4 + sub;
        if constexpr (S > 1) {
            if (j == 0)
                s_part[(((rw * PW + rgi) * MT + mm) * 4 + sub) * S + ks] = v;
        } else if (j == 0 && n < N && mm < mt) {
            const size_t o = (size_t)(m0 + mm) * N + n;
            if (kDebug && p.dbg_acc != nullptr)
                p.dbg_acc[o] = v;
            p.Y[o] = ((float)v * s_scale[n - rg_blk * 4]) * s_a[mm];
        }
    };

    if constexpr (kReg) {
        // ---- register variant: the lane's codes for its RCG chunks, read once
        uint32_t act[RCG][8];
#pragma unroll
        for (int c = 0; c < RCG; ++c)
            load_act(s_dyn + (size_t)(c * 16 + j) * 8, act[c]);
#define QW_COMPUTE(WBUF, Q)                                                                     \
        {                                                                                       \
            int acc_[4] = {0, 0, 0, 0};                                                         \
            _Pragma("unroll") for (int c_ = 0; c_ < RCG; ++c_) dot_chunk(WBUF[c_], act[c_], acc_); \
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
        // ---- LDS variant: U tiles per batch, codes read from LDS per tile
        int acc[MT][4];
#pragma unroll
        for (int mm = 0; mm < MT; ++mm)
            acc[mm][0] = acc[mm][1] = acc[mm][2] = acc[mm][3] = 0;
#define QW_COMPUTE(WBUF, Q)                                                                     \
        {                                                                                       \
            const int r_ = (Q) / nb, b_ = (Q) - r_ * nb;                                        \
            _Pragma("unroll") for (int mm = 0; mm < MT; ++mm)                                   \
            {                                                                                   \
                uint32_t a_[U][8];                                                              \
                _Pragma("unroll") for (int u_ = 0; u_ < U; ++u_)                                \
                    load_act(s_dyn + ((size_t)mm * chunks + (c_lo + b_ * U + u_) * 16 + j) * 8, a_[u_]); \
                _Pragma("unroll") for (int u_ = 0; u_ < U; ++u_)                                \
                    dot_chunk(WBUF[u_], a_[u_], acc[mm]);                                       \
            }                                                                                   \
            if (b_ == nb - 1) {                                                                 \
                _Pragma("unroll") for (int mm = 0; mm < MT; ++mm)                               \
                {                                                                               \
                    finish_row_group(acc[mm], mm, r_);                                          \
                    acc[mm][0] = acc[mm][1] = acc[mm][2] = acc[mm][3] = 0;                      \
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
            // every wave of the workgroup reaches this barrier (a wave without row
            // groups skips the loop); slice 0's wave of each run adds the partials
            __syncthreads();
            if (ks == 0 && lane < 4) {
                for (int rgi = 0; rgi < nrg_w; ++rgi) {
                    const int n = nw0 + rgi * 4 + lane;
#pragma unroll
                    for (int mm = 0; mm < MT; ++mm) {
                        const int* pp = s_part + (((rw * PW + rgi) * MT + mm) * 4 + lane) * S;
                        int v = 0;
#pragma unroll
                        for (int k = 0; k < S; ++k)
                            v += pp[k];
                        if (n < N && mm < mt) {
                            const size_t o = (size_t)(m0 + mm) * N + n;
                            if (kDebug && p.dbg_acc != nullptr)
                                p.dbg_acc[o] = v;
                            p.Y[o] = ((float)v * s_scale[n - rg_blk * 4]) * s_a[mm];
                        }
                    }
                }
            }
        }
    }
#undef QW_LOAD
}

// Eager variant: every tile of the wave (at most TMAX) is requested before the
// prologue, so the whole matrix is in flight while the activations are quantized;
// the codes are then read from LDS one tile ahead of the dots.
template <int MT, int TMAX, int NW, bool kDebug>
__global__ __launch_bounds__(64 * NW) void k_gemv_w4a8_eager(W4A8Args p)
{
    constexpr int kThreads = 64 * NW;
    extern __shared__ uint32_t s_dyn[];  // [MT][cg*16 chunks][8 words] codes, then scales
    __shared__ float s_red[MT][NW];
    __shared__ float s_a[MT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, sub = lane >> 4;
    const int M = p.M, N = p.N, K = p.K, CG = p.cg;
    const int m0 = blockIdx.y * MT;
    const int mt = min(MT, M - m0);
    const int K4 = K >> 2;
    const int chunks = CG * 16;

    const int W = p.nwaves;
    const int gw0 = blockIdx.x * NW;
    const int rg_blk = rg_of(gw0, p.per, p.rem);
    const int rg_blk_end = rg_of(min(gw0 + NW, W), p.per, p.rem);
    const int nrg_blk = rg_blk_end - rg_blk;
    const int gw = gw0 + wave;
    const int rg0 = gw < W ? rg_of(gw, p.per, p.rem) : rg_blk_end;
    const int rg1 = gw < W ? rg_of(gw + 1, p.per, p.rem) : rg_blk_end;
    const int T = (rg1 - rg0) * CG;  // tiles of this wave, at most TMAX
    const rsrc_t wres =
        make_rsrc(p.Wq + (size_t)rg_blk * CG * 1024u, (uint32_t)(nrg_blk * CG) * 1024u);
    const uint32_t wbase = (uint32_t)((rg0 - rg_blk) * CG) * 1024u + (uint32_t)lane * 16u;

    // ---- scales and X row 0 first, then every weight tile of the wave
    float* s_scale = reinterpret_cast<float*>(s_dyn + (size_t)MT * chunks * 8);
    const int rows_blk = min(nrg_blk * 4, N - rg_blk * 4);
    const rsrc_t sres = make_rsrc(p.w_scale + (size_t)rg_blk * 4, (uint32_t)max(rows_blk, 0) * 4u);
    uint32_t sc_reg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        sc_reg[i] = load4(sres, (uint32_t)(tid + i * kThreads) * 4u);
    constexpr int XV = 4;
    const int nblk = (K4 + XV * kThreads - 1) / (XV * kThreads);
    float4 xv[XV];
    load_x_block<XV, kThreads>(p, m0, mt, 0, 0, tid, xv);
    issue_barrier();
    uint4 w[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
        w[t] = load16_stream(wres, t < T ? wbase + (uint32_t)t * 1024u : 0x80000000u);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s_scale[tid + i * kThreads] = __uint_as_float(sc_reg[i]);
    if (nblk == 1)
        quantize_rows<MT, NW, XV, true, kDebug>(p, xv, s_dyn, s_red, s_a, chunks, nblk, m0, mt, tid);
    else
        quantize_rows<MT, NW, XV, false, kDebug>(p, xv, s_dyn, s_red, s_a, chunks, nblk, m0, mt, tid);

    // ---- tiles in order; the codes of the next tile are read while this one computes
    int acc[MT][4];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
        acc[mm][0] = acc[mm][1] = acc[mm][2] = acc[mm][3] = 0;
    uint32_t a_cur[MT][8];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
        load_act(s_dyn + ((size_t)mm * chunks + j) * 8, a_cur[mm]);
    int c = 0, rgi = 0;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t < T) {
            const int cn = c + 1 == CG ? 0 : c + 1;
            uint32_t a_nxt[MT][8];
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
                load_act(s_dyn + ((size_t)mm * chunks + cn * 16 + j) * 8, a_nxt[mm]);
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
                dot_chunk(w[t], a_cur[mm], acc[mm]);
            if (cn == 0) {
                const int n = (rg0 + rgi) * 4 + sub;
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) {
                    const int v = row_sum16(acc[mm][0] + acc[mm][1] + acc[mm][2] + acc[mm][3]) >> 4;
                    acc[mm][0] = acc[mm][1] = acc[mm][2] = acc[mm][3] = 0;
                    if (j == 0 && n < N && mm < mt) {
                        const size_t o = (size_t)(m0 + mm) * N + n;
                        if (kDebug && p.dbg_acc != nullptr)
                            p.dbg_acc[o] = v;
                        p.Y[o] = ((float)v * s_scale[n - rg_blk * 4]) * s_a[mm];
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

// All-in-flight variant (M == 1, RCG tiles per row group, at most RPW row groups per
// wave): every weight tile of the wave is requested right after the scales and X,
// before the prologue waits for anything, so the whole weight stream of the launch is
// in flight while the activations are quantized, and each wave meets one memory
// latency instead of one per batch.  Straight-line code: tiles of row groups the wave
// does not own read zeros and only their stores are skipped.  The activation codes of
// the lane's RCG chunks are then held in registers, as in the register variant.
template <int RCG, int RPW, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv_w4a8_flight(W4A8Args p)
{
    constexpr int kThreads = 64 * NW;
    constexpr int XV = (RCG * 128 + kThreads - 1) / kThreads;  // X float4 per thread
    extern __shared__ uint32_t s_dyn[];  // [RCG * 16 chunks][8 words] codes, then scales
    __shared__ float s_red[1][NW];
    __shared__ float s_a[1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, sub = lane >> 4;
    const int N = p.N, CG = p.cg;
    constexpr int chunks = RCG * 16;

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

    float* s_scale = reinterpret_cast<float*>(s_dyn + (size_t)chunks * 8);
    const int rows_blk = min(nrg_blk * 4, N - rg_blk * 4);
    const rsrc_t sres = make_rsrc(p.w_scale + (size_t)rg_blk * 4, (uint32_t)max(rows_blk, 0) * 4u);
    uint32_t sc_reg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        sc_reg[i] = load4(sres, (uint32_t)(tid + i * kThreads) * 4u);
    float4 xv[XV];
    load_x_block<XV, kThreads>(p, 0, 1, 0, 0, tid, xv);
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
    for (int i = 0; i < 4; ++i)
        s_scale[tid + i * kThreads] = __uint_as_float(sc_reg[i]);
    quantize_rows<1, NW, XV, true, false>(p, xv, s_dyn, s_red, s_a, chunks, 1, 0, 1, tid);

    uint32_t act[RCG][8];
#pragma unroll
    for (int c = 0; c < RCG; ++c)
        load_act(s_dyn + (size_t)(c * 16 + j) * 8, act[c]);
    const float a = s_a[0];
    const int nw0 = rg0 * 4;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        int acc[4] = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < RCG; ++c)
            dot_chunk(w[r][c], act[c], acc);
        const int v = row_sum16(acc[0] + acc[1] + acc[2] + acc[3]) >> 4;
        const int n = nw0 + r * 4 + sub;
        if (j == 0 && r < nrg_w && n < N)
            p.Y[n] = ((float)v * s_scale[n - rg_blk * 4]) * a;
    }
}

// Long-K form of the all-in-flight variant (M == 1): one row run of up to RPW row groups
// per workgroup, its S waves each taking one k-slice of 8 tiles (the last one shorter).
// Each wave requests all of its tiles right after X, holds its slice's activation codes
// in registers, and leaves one int32 partial per row in LDS; after one barrier wave 0
// adds the S partials and applies the epilogue.  K up to 4096 * S.
template <int RPW, int S>
__global__ __launch_bounds__(64 * S) void k_gemv_w4a8_flight_split(W4A8Args p)
{
    constexpr int NW = S, kThreads = 64 * S, RCG = 8;
    constexpr int XV = 16;  // X float4 per thread: K / 4 <= 16 * kThreads
    extern __shared__ uint32_t s_dyn[];  // [S * 8 * 16 chunks][8 words] codes; scales; partials
    __shared__ float s_red[1][NW];
    __shared__ float s_a[1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ks = __builtin_amdgcn_readfirstlane(tid >> 6);  // this wave's k-slice
    const int j = lane & 15, sub = lane >> 4;
    const int N = p.N, CG = p.cg;
    constexpr int chunks = S * RCG * 16;
    const int c_lo = ks * RCG;
    const int Tw = max(0, min(CG, c_lo + RCG) - c_lo);

    const int W = p.nwaves;  // row runs, one per workgroup
    const int gw = blockIdx.x;
    const int rg0 = rg_of(gw, p.per, p.rem);
    const int rg1 = rg_of(gw + 1, p.per, p.rem);
    const int nrg_w = gw < W ? rg1 - rg0 : 0;
    const rsrc_t wres = make_rsrc(p.Wq + (size_t)rg0 * CG * 1024u, (uint32_t)(nrg_w * CG) * 1024u);
    const uint32_t wbase = (uint32_t)c_lo * 1024u + (uint32_t)lane * 16u;

    float* s_scale = reinterpret_cast<float*>(s_dyn + (size_t)chunks * 8);
    int* s_part = reinterpret_cast<int*>(s_scale + RPW * 4);  // [RPW][4 rows][S]
    const rsrc_t sres = make_rsrc(p.w_scale + (size_t)rg0 * 4, (uint32_t)max(0, min(nrg_w * 4, N - rg0 * 4)) * 4u);
    const uint32_t sc_reg = load4(sres, (uint32_t)(tid < RPW * 4 ? tid : 0x20000000) * 4u);
    float4 xv[XV];
    load_x_block<XV, kThreads>(p, 0, 1, 0, 0, tid, xv);
    issue_barrier();
    uint4 w[RPW][RCG];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int c = 0; c < RCG; ++c)
            w[r][c] = load16_stream(wres, r < nrg_w && c < Tw ? wbase + (uint32_t)(r * CG + c) * 1024u
                                                             : 0x80000000u);
    __builtin_amdgcn_sched_barrier(0);
    if (tid < RPW * 4)
        s_scale[tid] = __uint_as_float(sc_reg);
    quantize_rows<1, NW, XV, true, false>(p, xv, s_dyn, s_red, s_a, chunks, 1, 0, 1, tid);

    uint32_t act[RCG][8];
#pragma unroll
    for (int c = 0; c < RCG; ++c)
        load_act(s_dyn + (size_t)((c_lo + c) * 16 + j) * 8, act[c]);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        int acc[4] = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < RCG; ++c)
            dot_chunk(w[r][c], act[c], acc);
        const int v = row_sum16(acc[0] + acc[1] + acc[2] + acc[3]) >> 4;
        if (j == 0)
            s_part[(r * 4 + sub) * S + ks] = v;
    }
    __syncthreads();
    if (tid < RPW * 4) {
        const int r = tid >> 2, n = rg0 * 4 + tid;
        int v = 0;
#pragma unroll
        for (int k = 0; k < S; ++k)
            v += s_part[tid * S + k];
        if (r < nrg_w && n < N)
            p.Y[n] = ((float)v * s_scale[tid]) * s_a[0];
    }
}

template <int RPW, int S>
hipError_t launch_flight_split(const W4A8Args& a, const GemvTiling& t, hipStream_t st)
{
    hipLaunchKernelGGL((k_gemv_w4a8_flight_split<RPW, S>), dim3(t.blocks), dim3(64 * S),
                       t.lds_bytes, st, a);
    return hipGetLastError();
}

template <int RPW>
hipError_t launch_flight_split_s(const W4A8Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.splitk) {
    case 2: return launch_flight_split<RPW, 2>(a, t, st);
    case 3: return launch_flight_split<RPW, 3>(a, t, st);
    case 4: return launch_flight_split<RPW, 4>(a, t, st);
    case 5: return launch_flight_split<RPW, 5>(a, t, st);
    case 6: return launch_flight_split<RPW, 6>(a, t, st);
    case 7: return launch_flight_split<RPW, 7>(a, t, st);
    case 8: return launch_flight_split<RPW, 8>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_flight_split_any(const W4A8Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.tmax) {
    case 1: return launch_flight_split_s<1>(a, t, st);
    case 2: return launch_flight_split_s<2>(a, t, st);
    case 4: return launch_flight_split_s<4>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

template <int RCG, int RPW, int NW>
hipError_t launch_flight(const W4A8Args& a, const GemvTiling& t, hipStream_t st)
{
    hipLaunchKernelGGL((k_gemv_w4a8_flight<RCG, RPW, NW>), dim3(t.blocks), dim3(64 * NW),
                       t.lds_bytes, st, a);
    return hipGetLastError();
}

// at most 5 row groups per wave with 4 waves per workgroup, 3 with 8
template <int RCG>
hipError_t launch_flight_r(const W4A8Args& a, const GemvTiling& t, hipStream_t st)
{
    if (t.nw == 8) {
        switch (t.tmax) {
        case 1: return launch_flight<RCG, 1, 8>(a, t, st);
        case 2: return launch_flight<RCG, 2, 8>(a, t, st);
        case 3: return launch_flight<RCG, 3, 8>(a, t, st);
        default: return hipErrorInvalidValue;
        }
    }
    switch (t.tmax) {
    case 1: return launch_flight<RCG, 1, 4>(a, t, st);
    case 2: return launch_flight<RCG, 2, 4>(a, t, st);
    case 3: return launch_flight<RCG, 3, 4>(a, t, st);
    case 4: return launch_flight<RCG, 4, 4>(a, t, st);
    case 5: return launch_flight<RCG, 5, 4>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_flight_any(const W4A8Args& a, const GemvTiling& t, hipStream_t st)
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
hipError_t launch4(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    const dim3 grid(t.blocks, t.m_tiles);
    if (debug)
        hipLaunchKernelGGL((k_gemv_w4a8<MT, RCG, U, NW, S, true>), grid, dim3(64 * NW),
                           t.lds_bytes, st, a);
    else
        hipLaunchKernelGGL((k_gemv_w4a8<MT, RCG, U, NW, S, false>), grid, dim3(64 * NW),
                           t.lds_bytes, st, a);
    return hipGetLastError();
}

// split-K: at most 2 rows of X per workgroup, 4 or 8 waves
template <int MT, int NW>
hipError_t launch_split(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    if (t.u == 4)
        return t.splitk == 2 ? launch4<MT, 0, 4, NW, 2>(a, t, debug, st)
                             : launch4<MT, 0, 4, NW, 4>(a, t, debug, st);
    return t.splitk == 2 ? launch4<MT, 0, 8, NW, 2>(a, t, debug, st)
                         : launch4<MT, 0, 8, NW, 4>(a, t, debug, st);
}

template <int MT, int TMAX, int NW>
hipError_t launch_eager(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    const dim3 grid(t.blocks, t.m_tiles);
    if (debug)
        hipLaunchKernelGGL((k_gemv_w4a8_eager<MT, TMAX, NW, true>), grid, dim3(64 * NW),
                           t.lds_bytes, st, a);
    else
        hipLaunchKernelGGL((k_gemv_w4a8_eager<MT, TMAX, NW, false>), grid, dim3(64 * NW),
                           t.lds_bytes, st, a);
    return hipGetLastError();
}

template <int MT, int NW>
hipError_t launch_eager_t(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    return t.tmax == 8 ? launch_eager<MT, 8, NW>(a, t, debug, st)
                       : launch_eager<MT, 16, NW>(a, t, debug, st);
}

template <int NW>
hipError_t launch_reg(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    switch (t.reg_cg) {
    case 1: return launch4<1, 1, 4, NW>(a, t, debug, st);
    case 2: return launch4<1, 2, 4, NW>(a, t, debug, st);
    case 3: return launch4<1, 3, 4, NW>(a, t, debug, st);
    case 4: return launch4<1, 4, 4, NW>(a, t, debug, st);
    case 5: return launch4<1, 5, 4, NW>(a, t, debug, st);
    case 6: return launch4<1, 6, 4, NW>(a, t, debug, st);
    case 7: return launch4<1, 7, 4, NW>(a, t, debug, st);
    case 8: return launch4<1, 8, 4, NW>(a, t, debug, st);
    default: return hipErrorInvalidValue;
    }
}

template <int MT, int NW>
hipError_t launch_lds(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    return t.u == 4 ? launch4<MT, 0, 4, NW>(a, t, debug, st) : launch4<MT, 0, 8, NW>(a, t, debug, st);
}

template <int NW>
hipError_t launch_nw(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    if (t.splitk > 1) {
        if constexpr (NW == 16) {
            return hipErrorInvalidValue;
        } else {
            switch (t.mt) {
            case 1: return launch_split<1, NW>(a, t, debug, st);
            case 2: return launch_split<2, NW>(a, t, debug, st);
            default: return hipErrorInvalidValue;
            }
        }
    }
    if (t.u == 1) {
        switch (t.mt) {
        case 1: return launch_eager_t<1, NW>(a, t, debug, st);
        case 2: return launch_eager_t<2, NW>(a, t, debug, st);
        case 4: return launch_eager_t<4, NW>(a, t, debug, st);
        default: return hipErrorInvalidValue;
        }
    }
    if (t.reg_cg > 0)
        return launch_reg<NW>(a, t, debug, st);
    switch (t.mt) {
    case 1: return launch_lds<1, NW>(a, t, debug, st);
    case 2: return launch_lds<2, NW>(a, t, debug, st);
    case 4: return launch_lds<4, NW>(a, t, debug, st);
    case 8: return launch_lds<8, NW>(a, t, debug, st);
    default: return hipErrorInvalidValue;
    }
}

template <int T, int NW, int P, int S>
hipError_t launch_prod(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    if (debug) {
        if constexpr ((NW == 8 && P == 2 && S == 1) || (NW == 4 && P == 4 && S == 1) ||
                      (NW == 8 && P == 8 && S > 1))
            hipLaunchKernelGGL((k_gemv_w4a8_prod<T, NW, P, S, 0, true>), dim3(t.blocks),
                               dim3(64 * (NW + P)), 0, st, a);
        else
            return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((k_gemv_w4a8_prod<T, NW, P, S, 0, false>), dim3(t.blocks),
                           dim3(64 * (NW + P)), 0, st, a);
    }
    return hipGetLastError();
}

// K <= 4096: every row of codes in registers (T = tiles per row group)
template <int T>
hipError_t launch_prod_w(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    if (t.nw == 8 && t.prod == 2) return launch_prod<T, 8, 2, 1>(a, t, debug, st);
    if (t.nw == 6 && t.prod == 2) return launch_prod<T, 6, 2, 1>(a, t, debug, st);
    if (t.nw == 5 && t.prod == 3) return launch_prod<T, 5, 3, 1>(a, t, debug, st);
    if (t.nw == 4 && t.prod == 4) return launch_prod<T, 4, 4, 1>(a, t, debug, st);
    return hipErrorInvalidValue;
}

// K split over S waves of 5..7 tiles each: 8 consumer and 8 producer waves (with 16 waves
// per CU a wave has 128 registers; 8 tiles per slice would spill)
template <int S>
hipError_t launch_prod_s(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    if (t.nw != 8 || t.prod != 8)
        return hipErrorInvalidValue;
    switch (t.reg_cg) {
    case 5: return launch_prod<5, 8, 8, S>(a, t, debug, st);
    case 6: return launch_prod<6, 8, 8, S>(a, t, debug, st);
    case 7: return launch_prod<7, 8, 8, S>(a, t, debug, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prod_any(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    switch (t.splitk) {
    case 2: return launch_prod_s<2>(a, t, debug, st);
    case 4: return launch_prod_s<4>(a, t, debug, st);
    case 8: return launch_prod_s<8>(a, t, debug, st);
    default: break;
    }
    switch (t.reg_cg) {
    case 1: return launch_prod_w<1>(a, t, debug, st);
    case 2: return launch_prod_w<2>(a, t, debug, st);
    case 3: return launch_prod_w<3>(a, t, debug, st);
    case 4: return launch_prod_w<4>(a, t, debug, st);
    case 5: return launch_prod_w<5>(a, t, debug, st);
    case 6: return launch_prod_w<6>(a, t, debug, st);
    case 7: return launch_prod_w<7>(a, t, debug, st);
    case 8: return launch_prod_w<8>(a, t, debug, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t prod_guard_status_rowwise(unsigned* trips, bool clear)
{
    return read_prod_guard(trips, clear);
}

hipError_t launch_gemv_w4a8(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    if (t.u == 5 || t.u == 6)
        return launch_prod_any(a, t, debug, st);
    if (t.u == 2)
        return debug ? hipErrorInvalidValue : launch_flight_any(a, t, st);
    if (t.u == 3)
        return debug ? hipErrorInvalidValue : launch_flight_split_any(a, t, st);
    switch (t.nw) {
    case 4: return launch_nw<4>(a, t, debug, st);
    case 8: return launch_nw<8>(a, t, debug, st);
    case 16: return launch_nw<16>(a, t, debug, st);
    default: return hipErrorInvalidValue;
    }
}

namespace {

// Activation quantization for the long-K kernel and the tiled GEMM: one workgroup of T
// threads per row of X (512 up to K = 4096: 0.3-0.6 us less than 1024 threads of one
// float4 each; 1024 beyond), which loads the whole row into registers at once (NV float4
// per thread, so a single memory round trip), takes max|x| across the workgroup and
// writes the row-major codes from the same registers.  The scale and the codes are
// computed exactly as by the standalone quantization kernel (four values per step, by
// the reciprocal, with the division taken for any four of which one lies near a
// rounding boundary).  With UNPACK, each 16-byte
// group of codes (16 k) is written in the order the INT4 unpack presents the weights
// (k 0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15): the lane holding k 4j .. 4j + 3
// of a group and its neighbour exchange their words, the even lane keeps the even k of
// both and the odd lane the odd k, and each writes the word at its own position.
template <int T, int NV, bool UNPACK>
__global__ __launch_bounds__(T) void k_quant_act_rows(const float* __restrict__ X, int K, int8_t* __restrict__ Xq,
                                                      float* __restrict__ a_scale)
{
    __shared__ float red[T / 64];
    const int tid = threadIdx.x;
    const int m = blockIdx.x;
    const int K4 = K >> 2;
    const rsrc_t xr = make_rsrc(X + (size_t)m * K, (uint32_t)K * 4u);
    float4 v[NV];
    float mx = 0.0f;
#pragma unroll
    for (int t = 0; t < NV; ++t) {
        const int i = tid + T * t;
        v[t] = load16f(xr, i < K4 ? (uint32_t)i * 16u : 0x80000000u);
        mx = fmaxf(mx, max_abs4(v[t]));
    }
    mx = wave_max(mx);
    if ((tid & 63) == 0)
        red[tid >> 6] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < T / 64; ++w)
        mx = fmaxf(mx, red[w]);
    const float a = mx / 127.0f;
    const float r = 1.0f / a;
    const bool fast = r <= 3.0e38f;
    if (tid == 0)
        a_scale[m] = a;
    uint32_t* out = reinterpret_cast<uint32_t*>(Xq + (size_t)m * K);
#pragma unroll
    for (int t = 0; t < NV; ++t) {
        const int i = tid + T * t;
        // the four codes arrive in byte 2 of e[0 .. 3]; the word takes them in k order
        uint32_t e[4];
        if (quant4_e(v[t], r, e) || !fast)
            quant4_e_div(v[t], a, e);
        uint32_t wd = __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0602u) | __builtin_amdgcn_perm(e[3], e[2], 0x06020C0Cu);
        if constexpr (UNPACK) {
            // the neighbour's word (lanes 2 u and 2 u + 1 swap: quad permutation 1, 0, 3, 2);
            // K is a multiple of 32, so both lanes of a pair are inside the row or both past it
            const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)wd, 0xB1, 0xF, 0xF, false);
            wd = (tid & 1) == 0 ? __builtin_amdgcn_perm(nb, wd, 0x06040200u)   // own k 0, 2; its k 4, 6
                                : __builtin_amdgcn_perm(wd, nb, 0x07050301u);  // its k 1, 3; own k 5, 7
        }
        if (i < K4)
            out[i] = wd;
    }
}

// Balanced long-K W4A8 kernel for 1 to 16 rows of X (grid rows of MT rows): the same
// split as the W8A16 long-K form.  One workgroup per CU (more only past U row groups
// per CU) owns an even run of row groups; its S waves each take a k-slice of T tiles of
// every row group of the run.  The activation codes come from the workspace (row-major
// int8, written by the standalone quantization kernel, with one scale per row); each
// lane loads the 32 codes of its chunk of each tile of its slice for its MT rows once
// and regroups every 8 of them into the even-k and odd-k words the unpack meets.  A
// unit is one row group's T tiles of the wave's slice, one unit requested ahead.  The
// per-slice int32 row sums (16 times the dot, exact) meet in LDS; the epilogue adds
// them (exact in any order) and writes ((sum >> 4) * w_scale) * a_scale.
constexpr int kW4BsMaxWaves = 8;

template <int T, int U, int MT>
__global__ __launch_bounds__(64 * kW4BsMaxWaves) void k_gemv_w4a8_bsplit(W4A8BsplitArgs p)
{
    __shared__ int s_part[MT * 4 * U * kW4BsMaxWaves];  // [row of X][row of the run][slice]
    __shared__ float s_sc[4 * U];
    __shared__ float s_a[MT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ks = __builtin_amdgcn_readfirstlane(tid >> 6);  // the k-slice of this wave
    const int nthreads = (int)blockDim.x;
    const int S = nthreads >> 6;
    const int j = lane & 15, sub = lane >> 4;
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
    const int nrows = max(0, min(4 * nb, N - 4 * rg0));
    const rsrc_t wres = make_rsrc(p.Wq + (size_t)rg0 * CG * 1024u, (uint32_t)(nb * CG) * 1024u);
    const rsrc_t sres = make_rsrc(p.w_scale + (size_t)rg0 * 4, (uint32_t)nrows * 4u);
    const rsrc_t xres = make_rsrc(p.Xq + (size_t)m0 * K, (uint32_t)mv * (uint32_t)K);
    const rsrc_t ares = make_rsrc(p.a_scale + m0, (uint32_t)mv * 4u);

    // lane (j, sub): chunk j (32 k) of tile c of the slice -> codes X[m0 + m][512 (c_lo + c) + 32 j ..]
    uint4 xp[MT][T][2];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < T; ++c) {
            const int k = 512 * (c_lo + c) + 32 * j;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                xp[m][c][h] = load16(xres, m < mv && k < K ? (uint32_t)(m * K + k + 16 * h) : 0x80000000u);
        }
    const uint32_t sc_reg = load4(sres, (uint32_t)tid * 4u);
    const uint32_t a_reg = load4(ares, (uint32_t)(tid < MT ? tid : 0x10000000) * 4u);
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
    if (tid < 4 * U)
        s_sc[tid] = __uint_as_float(sc_reg);
    if (tid < MT)
        s_a[tid] = __uint_as_float(a_reg);
    // codes k .. k + 7 of word d: the even-k codes in one word, the odd-k codes in the next
    uint32_t act[MT][T][8];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < T; ++c) {
            const uint32_t nat[8] = {xp[m][c][0].x, xp[m][c][0].y, xp[m][c][0].z, xp[m][c][0].w,
                                     xp[m][c][1].x, xp[m][c][1].y, xp[m][c][1].z, xp[m][c][1].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                act[m][c][2 * d] = __builtin_amdgcn_perm(nat[2 * d + 1], nat[2 * d], 0x06040200u);
                act[m][c][2 * d + 1] = __builtin_amdgcn_perm(nat[2 * d + 1], nat[2 * d], 0x07050301u);
            }
        }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u + 1 < U) {
            QW_LOADW(u + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (u < nb) {
            int acc[MT][4];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    acc[m][d] = 0;
#pragma unroll
            for (int c = 0; c < T; ++c) {
                const uint32_t wd[4] = {w[u][c].x, w[u][c].y, w[u][c].z, w[u][c].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int lo = (int)((wd[d] << 4) & 0xF0F0F0F0u);
                    const int hi = (int)(wd[d] & 0xF0F0F0F0u);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        acc[m][d] = __builtin_amdgcn_sdot4(lo, (int)act[m][c][2 * d], acc[m][d], false);
                        acc[m][d] = __builtin_amdgcn_sdot4(hi, (int)act[m][c][2 * d + 1], acc[m][d], false);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int v = row_sum16((acc[m][0] + acc[m][1]) + (acc[m][2] + acc[m][3]));
                if (j == 0)
                    s_part[((m * U + u) * 4 + sub) * kW4BsMaxWaves + ks] = v;
            }
        }
    }
#undef QW_LOADW
    __syncthreads();
    for (int e = tid; e < mv * nrows; e += nthreads) {
        const int m = e / nrows, rr = e - m * nrows;
        const int* src = s_part + (m * 4 * U + rr) * kW4BsMaxWaves;
        int v = 0;
        for (int k = 0; k < S; ++k)
            v += src[k];
        p.Y[(size_t)(m0 + m) * N + 4 * rg0 + rr] = ((float)(v >> 4) * s_sc[rr]) * s_a[m];
    }
}

template <int T, int U, int MT>
hipError_t launch_w4_bsplit_m(const W4A8BsplitArgs& a, int blocks, int waves, hipStream_t st)
{
    const int mtiles = (a.M + MT - 1) / MT;
    hipLaunchKernelGGL((k_gemv_w4a8_bsplit<T, U, MT>), dim3(blocks * mtiles), dim3(64 * waves), 0, st, a);
    return hipGetLastError();
}

template <int T, int U>
hipError_t launch_w4_bsplit_u(const W4A8BsplitArgs& a, int blocks, int waves, int mt, hipStream_t st)
{
    switch (mt) {
    case 1: return launch_w4_bsplit_m<T, U, 1>(a, blocks, waves, st);
    case 2: return launch_w4_bsplit_m<T, U, 2>(a, blocks, waves, st);
    case 4:
        if constexpr (T <= 5)
            return launch_w4_bsplit_m<T, U, 4>(a, blocks, waves, st);
        else
            return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int T>
hipError_t launch_w4_bsplit_t(const W4A8BsplitArgs& a, int blocks, int waves, int mt, hipStream_t st)
{
    const int per = a.per + (a.rem > 0 ? 1 : 0);
    return per <= 8 ? launch_w4_bsplit_u<T, 8>(a, blocks, waves, mt, st)
                    : launch_w4_bsplit_u<T, 16>(a, blocks, waves, mt, st);
}

}  // namespace

namespace {

template <int T, bool UNPACK>
hipError_t launch_qar_t(const float* X, int M, int K, int8_t* Xq, float* a, hipStream_t st)
{
    const int nv = (K / 4 + T - 1) / T;  // float4 per thread
    const dim3 grid((unsigned)M), block(T);
    if (nv <= 1)
        hipLaunchKernelGGL((k_quant_act_rows<T, 1, UNPACK>), grid, block, 0, st, X, K, Xq, a);
    else if (nv <= 2)
        hipLaunchKernelGGL((k_quant_act_rows<T, 2, UNPACK>), grid, block, 0, st, X, K, Xq, a);
    else if (nv <= 4)
        hipLaunchKernelGGL((k_quant_act_rows<T, 4, UNPACK>), grid, block, 0, st, X, K, Xq, a);
    else if (nv <= 8)
        hipLaunchKernelGGL((k_quant_act_rows<T, 8, UNPACK>), grid, block, 0, st, X, K, Xq, a);
    else if (nv <= 14)
        hipLaunchKernelGGL((k_quant_act_rows<T, 14, UNPACK>), grid, block, 0, st, X, K, Xq, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <bool UNPACK>
hipError_t launch_qar(const float* X, int M, int K, int8_t* Xq, float* a, hipStream_t st)
{
    return K / 4 <= 2 * 512 ? launch_qar_t<512, UNPACK>(X, M, K, Xq, a, st)
                            : launch_qar_t<1024, UNPACK>(X, M, K, Xq, a, st);
}

}  // namespace

hipError_t launch_quant_act_rows(const float* X, int M, int K, int8_t* Xq, float* a, hipStream_t st,
                                 bool unpack_order)
{
    return unpack_order ? launch_qar<true>(X, M, K, Xq, a, st) : launch_qar<false>(X, M, K, Xq, a, st);
}

hipError_t launch_gemv_w4a8_bsplit(const W4A8BsplitArgs& a, int blocks, int waves, hipStream_t st)
{
    if (waves < 1 || waves > kW4BsMaxWaves || blocks < 1)
        return hipErrorInvalidValue;
    const int T = (a.cg + waves - 1) / waves;
    const int mt = a.M == 1 ? 1 : (a.M >= 3 && T <= 5 ? 4 : 2);
    switch (T) {
    case 1: return launch_w4_bsplit_t<1>(a, blocks, waves, mt, st);
    case 2: return launch_w4_bsplit_t<2>(a, blocks, waves, mt, st);
    case 3: return launch_w4_bsplit_t<3>(a, blocks, waves, mt, st);
    case 4: return launch_w4_bsplit_t<4>(a, blocks, waves, mt, st);
    case 5: return launch_w4_bsplit_t<5>(a, blocks, waves, mt, st);
    case 6: return launch_w4_bsplit_t<6>(a, blocks, waves, mt, st);
    case 7: return launch_w4_bsplit_t<7>(a, blocks, waves, mt, st);
    case 8: return launch_w4_bsplit_t<8>(a, blocks, waves, mt, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qw
