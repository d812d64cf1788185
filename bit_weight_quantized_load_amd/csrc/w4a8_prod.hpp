// Producer-wave W4A8 GEMV kernel (M == 1) and the INT4 dot helpers, shared by the
// row-wise entry point (gemv_w4a8.hip, LG == 0) and the group-wise one (gemv_w4a8g.hip).
//
// What is computed follows "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s":
// sections 正确方向 and 当前实现方式 (INT4 weights widened to int8 lanes, int8 dot into
// int32, output acc * weight_scale * activation_scale, the activation quantized per
// vector before the linear), section 后续优化方向 (the quantization fused into the
// linear kernel; group-wise scales).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

// Set to 1 by a producer wave whose bounded wait for the other producers' maxima ran out
// (never expected: every producer adds its maximum after its own loads only).  One word
// per source file that includes this header, read and cleared from the host through
// read_prod_guard; the kernel still finishes normally when it trips.
__device__ unsigned int g_prod_guard_trips;

inline hipError_t read_prod_guard(unsigned* out, bool clear)
{
    hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_prod_guard_trips), sizeof(unsigned), 0,
                                       hipMemcpyDeviceToHost);
    if (e == hipSuccess && clear) {
        const unsigned zero = 0;
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_prod_guard_trips), &zero, sizeof(unsigned), 0,
                              hipMemcpyHostToDevice);
    }
    return e;
}

// acc[d] += 16 * (q . x) over the 8 weights of word d of a chunk.
__device__ __forceinline__ void dot_chunk(const uint4 w, const uint32_t (&a)[8], int (&acc)[4])
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int lo = (int)((wd[d] << 4) & 0xF0F0F0F0u);
        const int hi = (int)(wd[d] & 0xF0F0F0F0u);
        acc[d] = __builtin_amdgcn_sdot4(lo, (int)a[2 * d], acc[d], false);
        acc[d] = __builtin_amdgcn_sdot4(hi, (int)a[2 * d + 1], acc[d], false);
    }
}

// Sums over one chunk (16 bytes of weights, 32 k) with 4-bit dots, for activation codes
// held as nibble words (the producer-wave layout): a[2d] = the low nibbles of the codes of
// weight word d's eight k, offset by -8 ((xq & 15) ^ 8 read as signed), a[2d + 1] = the
// high nibbles (xq >> 4).  Since xq = 16 (xq >> 4) + ((xq & 15) - 8) + 8, the exact dot is
// q . xq = 16 hi + lo + 8 (q . 1), accumulated here as hi, lo and sq.
__device__ __forceinline__ void dot8_chunk(const uint4 w, const uint32_t (&a)[8], int& hi, int& lo,
                                           int& sq)
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        lo = __builtin_amdgcn_sdot8((int)wd[d], (int)a[2 * d], lo, false);
        hi = __builtin_amdgcn_sdot8((int)wd[d], (int)a[2 * d + 1], hi, false);
        sq = __builtin_amdgcn_sdot8((int)wd[d], 0x11111111, sq, false);
    }
}

__device__ __forceinline__ void load_act(const uint32_t* p, uint32_t (&a)[8])
{
    const uint4 e = reinterpret_cast<const uint4*>(p)[0];
    const uint4 o = reinterpret_cast<const uint4*>(p)[1];
    a[0] = e.x; a[1] = e.y; a[2] = e.z; a[3] = e.w;
    a[4] = o.x; a[5] = o.y; a[6] = o.z; a[7] = o.w;
}

// Sum of an int32 over the LG consecutive lanes of a group inside a 16-lane DPP row (LG =
// 1, 2, 4, 8 or 16); every lane of the group receives the total, exactly.  Quad
// permutations pair lanes (1, 0, 3, 2) then (2, 3, 0, 1); the half-row mirror (lane i
// with 7 - i) joins quads 0 and 1; the row mirror (i with 15 - i) joins the two halves.
template <int LG>
__device__ __forceinline__ int group_sum(int v)
{
    if constexpr (LG >= 2)
        v += __builtin_amdgcn_mov_dpp(v, 0xb1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
    if constexpr (LG >= 4)
        v += __builtin_amdgcn_mov_dpp(v, 0x4e, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
    if constexpr (LG >= 8)
        v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xf, 0xf, false);  // row_half_mirror
    if constexpr (LG >= 16)
        v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xf, 0xf, false);  // row_mirror
    return v;
}

// Producer-wave variant (M == 1, one workgroup per CU): P producer waves quantize X
// while NW consumer waves stream weights.
//
// Why: a CU accepts new vector loads only as fast as data comes back, so a wave that
// has just requested weight tiles stalls on its next load instruction, and any barrier
// after those loads waits for that stall.  When every wave both requests weights and
// takes part in the activation reduction (the register variant), the prologue ends
// only once the first weight batch has been accepted; measured per wave, the codes
// were ready after 1.3-1.9 us and a second workgroup on the same CU waited 4 us, its X
// queued behind the first one's weights.  Here the producers request X (before any
// weight, by the first barrier), reduce the maximum among themselves through an LDS
// atomic and a counter (no barrier, so no wait on the consumers' load stalls), and
// write the codes; the consumers request their first row group and meet the producers
// at the second barrier, then stream the rest with two row groups in flight.
//
// Arithmetic: the producers quantize with quant4_e (one fused multiply-add per value and
// a 16-bit test for the values that need the division) and store each code split into
// nibbles; the consumers' dots are then three 4-bit dots per weight word (dot8_chunk)
// instead of two nibble masks and two 8-bit dots.  On 18944 -> 3584 this took the
// producers' code writing from about 1.5 to 0.9 us and each row group's dots from about
// 0.43 to 0.35 us (per-phase timestamps), 8.3 -> 8.0 us per launch.
//
// Work split: row groups split evenly over the workgroups (p.per / p.rem count row
// groups per workgroup, not per wave).  The NW consumers form NW / S row runs of S
// waves; each run takes an even share of the workgroup's row groups and each of its S
// waves one k-slice of at most T tiles of them (ceil(cg / S) tiles, T >= that), whose
// activation codes it holds in registers.  With S > 1 (long K) the int32 partial sums
// of the slices are added in LDS after a last barrier.  Codes, accumulators and outputs
// are those of the other variants bit for bit.
//
// LG > 0: group-wise INT4 scales (the INT4 write-up's section 后续优化方向 lists
// group-wise scales as future work): one fp32 scale per output row and group of
// 32 * LG consecutive k; each group's int32 dot is scaled once and the groups are
// added in fp32 (the order differs from a sequential sum; the fp32 summation bound
// covers any order).
constexpr int kProdMaxRgS = 16;  // row groups per workgroup when K is split (S > 1)

template <int T, int NW, int P, int S, int LG, bool kDebug>
__global__ __launch_bounds__(64 * (NW + P)) void k_gemv_w4a8_prod(W4A8Args p)
{
    constexpr int XP = (S * T * 128 + 64 * P - 1) / (64 * P);  // X float4 per producer lane
    constexpr int CH = S * T * 16;                             // chunks of codes in LDS
    constexpr int NR = NW / S;                                 // row runs
    // row groups a consumer requests before the codes barrier: two when K is split (its
    // batches are short and the quantization of a long X takes longer)
    constexpr int PRE = S > 1 ? 2 : 1;
    static_assert(NR * S == NW, "consumer waves must form whole row runs");
    // group-wise scales: LG lanes (chunks of 32 k) per group, GT groups per tile; a lane
    // holds the scales of its group in each of its tiles (GN of them)
    constexpr bool kGroup = LG > 0;
    constexpr int GT = kGroup ? 16 / LG : 1;
    constexpr int GN = !kGroup ? 1 : (S == 1 ? 4 * ((T + 3) / 4) : T);
    static_assert(!kGroup || LG == 1 || LG == 2 || LG == 4 || LG == 8 || LG == 16, "group size");
    static_assert(!kGroup || !kDebug, "no debug outputs for group-wise scales");
    __shared__ uint32_t s_act[CH * 8];
    __shared__ float s_a;
    __shared__ unsigned s_max, s_cnt;
    __shared__ int s_part[S > 1 && !kGroup ? kProdMaxRgS * 4 * S : 1];
    __shared__ float s_partf[S > 1 && kGroup ? kProdMaxRgS * 4 * S : 1];
    __shared__ float s_sc[S > 1 ? kProdMaxRgS * 4 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, sub = lane >> 4;
    const int N = p.N, K = p.K, CG = p.cg;
    const int rg_blk = rg_of(blockIdx.x, p.per, p.rem);
    const int nrg_blk = rg_of(blockIdx.x + 1, p.per, p.rem) - rg_blk;
    if (tid == 0) {
        s_max = 0u;
        s_cnt = 0u;
    }
    if (wave >= NW) {
        // ---- producer pr: float4 blocks [pr * XP, (pr + 1) * XP) of X
        const int pr = wave - NW;
        const int K4 = K >> 2;
        const rsrc_t xr = make_rsrc(p.X, (uint32_t)K * 4u);
        float4 xv[XP];
#pragma unroll
        for (int i = 0; i < XP; ++i)
            xv[i] = load16f(xr, (uint32_t)((pr * XP + i) * 64 + lane) * 16u);
        __syncthreads();  // (1) X is requested before any weight tile; counters are zero
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < XP; ++i)
            mx = fmaxf(mx, max_abs4(xv[i]));  // past K the loads read zeros
        mx = wave_max_dpp(mx);
        // non-negative floats order like their bit patterns: an unsigned maximum
        if (lane == 0) {
            __hip_atomic_fetch_max(&s_max, __float_as_uint(mx), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_add(&s_cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        // Every producer adds 1 once, unconditionally, after its own X only, so the
        // count reaches P; the bound is a guard, not a path taken.  If it ever runs out,
        // the codes would come from a partial maximum: the status word records it.
        for (int spin = 0; spin < (1 << 20) &&
                           __hip_atomic_load(&s_cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <
                               (unsigned)P;
             ++spin)
            __builtin_amdgcn_s_sleep(1);
        if (lane == 0 &&
            __hip_atomic_load(&s_cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < (unsigned)P)
            atomicOr(&g_prod_guard_trips, 1u);
        mx = __uint_as_float(__hip_atomic_load(&s_max, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        const float a = mx / 127.0f;
        const float r = 1.0f / a;
        const bool fast = r <= 3.0e38f;  // finite reciprocal (a is not 0 or tiny)
        // Codes of every staged position (past K, X reads zeros and the codes are 0), as
        // the nibble words the consumers' 4-bit dots take: in chunk c, word 2d holds the
        // low nibbles of the codes of k = 32c + 8d .. + 7 (nibble j: k = 32c + 8d + j),
        // each offset by 8, (xq & 15) ^ 8, and word 2d + 1 their high nibbles, xq >> 4.
        // A float4 gives 16 bits of each.
        uint16_t* act16 = reinterpret_cast<uint16_t*>(s_act);
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int f = (pr * XP + i) * 64 + lane;  // k = 4f .. 4f + 3
            if (f < CH * 8) {
                uint32_t e[4];
                if (quant4_e(xv[i], r, e) || !fast)
                    quant4_e_div(xv[i], a, e);
                const uint32_t ev = __builtin_amdgcn_perm(e[2], e[0], 0x0C0C0602u);  // k, k + 2
                const uint32_t od = __builtin_amdgcn_perm(e[3], e[1], 0x0C0C0602u);  // k + 1, k + 3
                const int c = f >> 3, d = (f >> 1) & 3, h = f & 1;
                const int wi = (c * 8 + 2 * d) * 2 + h;
                act16[wi] = (uint16_t)(((ev & 0x0F0Fu) | ((od << 4) & 0xF0F0u)) ^ 0x8888u);
                act16[wi + 2] = (uint16_t)(((ev >> 4) & 0x0F0Fu) | (od & 0xF0F0u));
                if (kDebug && p.dbg_xq != nullptr && blockIdx.x == 0 && f < K4)
                    *reinterpret_cast<uint32_t*>(p.dbg_xq + 4 * f) =
                        (e[0] >> 16 & 0xffu) | (e[1] >> 8 & 0xff00u) | (e[2] & 0xff0000u) |
                        (e[3] << 8 & 0xff000000u);
            }
        }
        if (pr == 0 && lane == 0) {
            s_a = a;
            if (kDebug && p.dbg_a != nullptr && blockIdx.x == 0)
                p.dbg_a[0] = a;
        }
        __syncthreads();  // (2) codes in LDS
    } else {
        // ---- consumer: run rw, k-slice ks (tiles [c_lo, c_lo + Tw)), nq row groups from rg0
        const int rw = S > 1 ? wave / S : wave;
        const int ks = S > 1 ? wave - rw * S : 0;
        const int Ts = (CG + S - 1) / S;
        const int c_lo = ks * Ts;
        const int Tw = max(0, min(CG, c_lo + Ts) - c_lo);
        const int pw = nrg_blk / NR, pr_ = nrg_blk - pw * NR;
        const int rgi0 = rg_of(rw, pw, pr_);  // first row group of the run in the workgroup
        const int rg0 = rg_blk + rgi0;
        const int nq = rg_of(rw + 1, pw, pr_) - rgi0;
        const rsrc_t wres =
            make_rsrc(p.Wq + (size_t)rg_blk * CG * 1024u, (uint32_t)(nrg_blk * CG) * 1024u);
        const uint32_t wbase = (uint32_t)(rgi0 * CG + c_lo) * 1024u + (uint32_t)lane * 16u;
        const rsrc_t sres =
            make_rsrc(p.w_scale + (size_t)rg0 * 4, (uint32_t)max(0, min(nq * 4, N - rg0 * 4)) * 4u);
        // group-wise: scales [row group][row][group of the tile][tile, padded to 4]
        const int cgp = (CG + 3) & ~3;
        const rsrc_t gres = make_rsrc(p.w_scale + (size_t)rg_blk * 4 * GT * cgp,
                                      (uint32_t)(nrg_blk * 4 * GT * cgp) * 4u);
        const uint32_t gbase = (uint32_t)((rgi0 * 4 + sub) * GT + j / (kGroup ? LG : 1)) * (uint32_t)cgp;
        uint4 wa[T], wb[T];
        float sa, sb;
        float ga[GN], gb[GN];
        // row group Q of the run, this wave's slice, with its output scales; tiles past the
        // slice or the run read zeros (straight-line code: see the register variant)
#define QW_PLOAD(WBUF, SC, GS, Q)                                                               \
        {                                                                                       \
            _Pragma("unroll") for (int u_ = 0; u_ < T; ++u_)                                   \
                WBUF[u_] = load16_stream(wres, (Q) < nq && u_ < Tw                              \
                                                   ? wbase + (uint32_t)((Q) * CG + u_) * 1024u \
                                                   : 0x80000000u);                              \
            if constexpr (!kGroup) {                                                            \
                SC = __uint_as_float(load4(sres, (uint32_t)((Q) * 4 + sub) * 4u));              \
            } else if constexpr (S == 1) {                                                      \
                _Pragma("unroll") for (int i_ = 0; i_ < GN / 4; ++i_)                          \
                {                                                                               \
                    const float4 v_ = load16f(gres, (Q) < nq ? (gbase + (uint32_t)((Q) * 4 * GT * cgp + 4 * i_)) * 4u \
                                                             : 0x80000000u);                    \
                    GS[4 * i_] = v_.x; GS[4 * i_ + 1] = v_.y; GS[4 * i_ + 2] = v_.z; GS[4 * i_ + 3] = v_.w; \
                }                                                                               \
            } else {                                                                            \
                _Pragma("unroll") for (int u_ = 0; u_ < T; ++u_)                               \
                    GS[u_] = __uint_as_float(load4(gres, (Q) < nq && u_ < Tw                    \
                        ? (gbase + (uint32_t)((Q) * 4 * GT * cgp + c_lo + u_)) * 4u : 0x80000000u)); \
            }                                                                                   \
            __builtin_amdgcn_sched_barrier(0);                                                  \
        }
        __syncthreads();  // (1)
        QW_PLOAD(wa, sa, ga, 0);
        if constexpr (PRE == 2)
            QW_PLOAD(wb, sb, gb, 1);
        __syncthreads();  // (2)
        uint32_t act[T][8];
#pragma unroll
        for (int c = 0; c < T; ++c)
            load_act(s_act + (size_t)((c_lo + c) * 16 + j) * 8, act[c]);
        const float a = s_a;
        // S == 1: the row is complete, write it; S > 1: leave the slice's partial sum.
        // Group-wise: per tile, the group's exact int32 dot (summed over its LG lanes)
        // times the group scale, added in fp32 by the group's first lane in tile order;
        // the 16 lanes' sums then meet in a DPP tree, and the activation scale comes last.
#define QW_PCOMPUTE(WBUF, SC, GS, Q)                                                            \
        if constexpr (kGroup) {                                                                 \
            float f_ = 0.0f;                                                                    \
            _Pragma("unroll") for (int c_ = 0; c_ < T; ++c_)                                   \
            {                                                                                   \
                int h_ = 0, l_ = 0, q_ = 0;                                                     \
                dot8_chunk(WBUF[c_], act[c_], h_, l_, q_);                                      \
                const int g_ = group_sum<LG>(16 * h_ + l_ + 8 * q_);                            \
                const float p_ = (float)g_ * GS[c_];                                            \
                f_ += (j % LG) == 0 ? p_ : 0.0f;                                                \
            }                                                                                   \
            f_ = row_sum16(f_);                                                                 \
            if constexpr (S > 1) {                                                              \
                if (j == 0)                                                                     \
                    s_partf[((rgi0 + (Q)) * 4 + sub) * S + ks] = f_;                            \
            } else {                                                                            \
                const int n_ = (rg0 + (Q)) * 4 + sub;                                           \
                if (j == 0 && n_ < N)                                                           \
                    p.Y[n_] = f_ * a;                                                           \
            }                                                                                   \
        } else {                                                                                \
            int h_ = 0, l_ = 0, q_ = 0;                                                         \
            _Pragma("unroll") for (int c_ = 0; c_ < T; ++c_) dot8_chunk(WBUF[c_], act[c_], h_, l_, q_); \
            const int v_ = row_sum16(16 * h_ + l_ + 8 * q_);                                    \
            if constexpr (S > 1) {                                                              \
                if (j == 0) {                                                                   \
                    s_part[((rgi0 + (Q)) * 4 + sub) * S + ks] = v_;                             \
                    if (ks == 0)                                                                \
                        s_sc[(rgi0 + (Q)) * 4 + sub] = SC;                                      \
                }                                                                               \
            } else {                                                                            \
                const int n_ = (rg0 + (Q)) * 4 + sub;                                           \
                if (j == 0 && n_ < N) {                                                         \
                    if (kDebug && p.dbg_acc != nullptr)                                         \
                        p.dbg_acc[n_] = v_;                                                     \
                    p.Y[n_] = ((float)v_ * SC) * a;                                             \
                }                                                                               \
            }                                                                                   \
        }
        int q = 0;
        for (; q + 1 < nq; q += 2) {
            if constexpr (PRE == 1)
                QW_PLOAD(wb, sb, gb, q + 1);
            QW_PCOMPUTE(wa, sa, ga, q);
            QW_PLOAD(wa, sa, ga, q + 2);
            QW_PCOMPUTE(wb, sb, gb, q + 1);
            if constexpr (PRE == 2)
                QW_PLOAD(wb, sb, gb, q + 3);
        }
        if (q < nq) {
            QW_PCOMPUTE(wa, sa, ga, q);
        }
#undef QW_PLOAD
#undef QW_PCOMPUTE
    }
    if constexpr (S > 1) {
        // every wave of the workgroup, producers included, reaches this barrier once
        __syncthreads();
        const int rows = min(nrg_blk * 4, N - rg_blk * 4);
        const float a = s_a;
        for (int i = tid; i < rows; i += 64 * (NW + P)) {
            const int n = rg_blk * 4 + i;
            if constexpr (kGroup) {
                float v = 0.0f;
#pragma unroll
                for (int k = 0; k < S; ++k)
                    v += s_partf[i * S + k];
                p.Y[n] = v * a;
            } else {
                int v = 0;
#pragma unroll
                for (int k = 0; k < S; ++k)
                    v += s_part[i * S + k];
                if (kDebug && p.dbg_acc != nullptr)
                    p.dbg_acc[n] = v;
                p.Y[n] = ((float)v * s_sc[i]) * a;
            }
        }
    }
}

}  // namespace

}  // namespace qw
