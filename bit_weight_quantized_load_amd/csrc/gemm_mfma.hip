// Skinny GEMM on the matrix cores: the same linears as the GEMV kernels (W4A8:
// "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s", sections
// 当前实现方式 and 正确方向; W8A16: ChatGLM2-6B W8A16 write-up (TPU-MLIR), section 4),
// computed with v_mfma_i32_16x16x64_i8 (W4A8) and v_mfma_f32_16x16x32_f16 (W8A16).
//
// Operands.  For a 16x16xKL MFMA, lane l supplies row l % 16 of A and column l % 16 of
// B, each at the KL/4 consecutive k of block l / 16, and receives D[4 (l / 16) + i][l % 16]
// for i = 0..3.  A is the weight (16 output rows n), B is X transposed (16 rows m), so
// D holds Y transposed: D[n][m].
//
// Work split.  A workgroup of NW waves owns NW * NBW * 16 consecutive output rows and
// MB blocks of 16 rows of X; each wave owns NBW blocks of 16 output rows and walks K
// in 512-k steps (one weight tile per row group).  Weights stay in the tile layout of
// the GEMV (kernels.hpp): per step a wave issues one 1 KB wave load per row group it
// owns, straight into registers, two steps ahead of the one it multiplies (three
// register buffers), and passes them through its own LDS region to regroup them in
// operand order (a wave's own LDS writes are seen by its later reads, so no barrier).
// The X operands of a 512-k step are shared by the workgroup through a double-buffered
// LDS slice: step c+1's slice is loaded while step c multiplies, one barrier per step.
// Loads are issued X first, then weights, so waiting for X never waits for the weights
// two steps ahead.  Workgroups that share a slice of weights (different blocks of X)
// are placed on one XCD so that its L2 serves the repeats.
//
// The balanced kernels (K up to 4096; the defaults up to 16 rows of X, and for W4A8 up
// to 64 rows where measured faster) split the work differently: one workgroup per CU,
// each with an even share of the row groups cut into units that its waves take in
// contiguous runs (see their comments).
//
// W4A8: X is quantized once per call into the workspace by k_quant_act_mfma (the same
// per-row scale and codes as quant_act_i8) in B-operand order.  An INT4 operand of 16 k
// is 8 bytes of nibbles presented as 16 * q (nibble moved to the high half of its
// byte; even k from the low nibbles, odd k from the high ones), and the X codes are
// stored in the same k order; the int32 result is exactly 16 * acc, so acc >> 4 is
// exact and the output equals the GEMV's bit for bit.
//
// W8A16: X (f16) is staged from its row-major input; the INT8 weights are cast to f16
// exactly in registers (the byte-permute cast of the GEMV) and the per-channel scale
// multiplies the fp32 sum once.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// The 512-k steps of a kernel: three weight register buffers (step c in w[c % 3]) and
// two X register buffers (step c in x[c % 2]) rotate, so six steps make one loop trip
// with no branch inside; the last zero to five steps follow the loop.  Expects QW_STEP,
// the buffers w0, w1, w2, xa, xb and the step count CG.
#define QW_STEPS_SIX()                                                                           \
    {                                                                                            \
        int c_ = 0;                                                                              \
        for (; c_ + 6 <= CG; c_ += 6) {                                                          \
            QW_STEP(w0, w2, xa, xb, c_);                                                         \
            QW_STEP(w1, w0, xb, xa, c_ + 1);                                                     \
            QW_STEP(w2, w1, xa, xb, c_ + 2);                                                     \
            QW_STEP(w0, w2, xb, xa, c_ + 3);                                                     \
            QW_STEP(w1, w0, xa, xb, c_ + 4);                                                     \
            QW_STEP(w2, w1, xb, xa, c_ + 5);                                                     \
        }                                                                                        \
        if (c_ < CG)                                                                             \
            QW_STEP(w0, w2, xa, xb, c_);                                                         \
        if (c_ + 1 < CG)                                                                         \
            QW_STEP(w1, w0, xb, xa, c_ + 1);                                                     \
        if (c_ + 2 < CG)                                                                         \
            QW_STEP(w2, w1, xa, xb, c_ + 2);                                                     \
        if (c_ + 3 < CG)                                                                         \
            QW_STEP(w0, w2, xb, xa, c_ + 3);                                                     \
        if (c_ + 4 < CG)                                                                         \
            QW_STEP(w1, w0, xa, xb, c_ + 4);                                                     \
    }

// ---------------------------------------------------------------- W4A8 --------

// Position p of the 16 codes of one B operand holds k = 16 g + kPerm[p] of its step:
// the order in which the INT4 unpack presents the weights.  The code of k = 4 e + i is
// byte 2 of c[e][i] (the four-value quantizer's form).
__device__ __forceinline__ uint4 pack_perm16(const uint32_t (&c)[4][4])
{
    uint4 o;
    o.x = __builtin_amdgcn_perm(c[0][2], c[0][0], 0x0C0C0602u) | __builtin_amdgcn_perm(c[1][2], c[1][0], 0x06020C0Cu);
    o.y = __builtin_amdgcn_perm(c[0][3], c[0][1], 0x0C0C0602u) | __builtin_amdgcn_perm(c[1][3], c[1][1], 0x06020C0Cu);
    o.z = __builtin_amdgcn_perm(c[2][2], c[2][0], 0x0C0C0602u) | __builtin_amdgcn_perm(c[3][2], c[3][0], 0x06020C0Cu);
    o.w = __builtin_amdgcn_perm(c[2][3], c[2][1], 0x0C0C0602u) | __builtin_amdgcn_perm(c[3][3], c[3][1], 0x06020C0Cu);
    return o;
}

// One workgroup per row of X (grid-strided over ceil(M / 16) * 16 rows; rows past M
// are written as zeros).  a = maxabs / 127 and the codes exactly as k_quant_act, laid
// out as B operands: row m, step st (64 k), lane block g -> 16 bytes at
// ((m / 16) * KS + st) * 1024 + (16 g + m % 16) * 16.  A thread owns NS slots of 16
// consecutive k (slot sl = tid + NT t) and keeps their values in registers between
// the maximum and the quantization, so X is read once.  NT = 256 threads, or 1024 for
// rows of more than 1024 slots (K > 16384), which keeps NS <= 4.
template <int NS, int NT>
__global__ __launch_bounds__(NT) void k_quant_act_mfma(const float* __restrict__ X, int M,
                                                       int K, int Mp, int KS,
                                                       uint8_t* __restrict__ Xp,
                                                       float* __restrict__ a_scale)
{
    constexpr int kBlock = NT;
    __shared__ float red[NT / 64];
    const int slots = KS * 4;  // 16-code slots per row
    for (int m = blockIdx.x; m < Mp; m += gridDim.x) {
        const bool live = m < M;
        // rows past M read zeros, and so do k past K
        const rsrc_t xr = make_rsrc(X + (size_t)(live ? m : 0) * K, live ? (uint32_t)K * 4u : 0u);
        float4 v[NS][4];
        float mx = 0.0f;
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            const int sl = (int)threadIdx.x + kBlock * t;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[t][e] = load16f(xr, sl < slots ? (uint32_t)(16 * sl + 4 * e) * 4u : 0x80000000u);
                mx = fmaxf(mx, max_abs4(v[t][e]));
            }
        }
        if constexpr (NT == 256) {
            mx = block_max(mx, red);
        } else {
            mx = wave_max(mx);
            if ((threadIdx.x & 63) == 0)
                red[threadIdx.x >> 6] = mx;
            __syncthreads();
            mx = red[0];
#pragma unroll
            for (int w = 1; w < NT / 64; ++w)
                mx = fmaxf(mx, red[w]);
            __syncthreads();  // red is reused by the next row of the grid-stride loop
        }
        const float a = mx / 127.0f;
        const float r = 1.0f / a;
        const bool fast = r <= 3.0e38f;
        if (live && threadIdx.x == 0)
            a_scale[m] = a;
        uint8_t* base = Xp + (size_t)(m >> 4) * KS * 1024u + (size_t)(m & 15) * 16u;
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            const int sl = (int)threadIdx.x + kBlock * t;
            if (sl < slots) {
                uint32_t c[4][4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (quant4_e(v[t][e], r, c[e]) || !fast)
                        quant4_e_div(v[t][e], a, c[e]);
                const int st = sl >> 2, g = sl & 3;
                *reinterpret_cast<uint4*>(base + (size_t)st * 1024u + (size_t)g * 256u) =
                    pack_perm16(c);
            }
        }
    }
}

// Padded LDS image of one INT4 tile (4 rows x 16 chunks): row sub at sub * 272, chunk
// j at j * 16, so the 16 lanes reading 16 different rows of a 16-row block hit
// different banks.
constexpr int kW4TilePitch = 1088, kW4RowPitch = 272;

template <int NW, int MB, int NBW>
__global__ __launch_bounds__(64 * NW) void k_gemm_w4a8(MfmaW4A8Args p)
{
    constexpr int kThreads = 64 * NW;
    constexpr int kXStep = MB * 8 * 1024;                // X codes of one 512-k step
    constexpr int kXLoads = kXStep / (kThreads * 16);    // 16-byte loads per thread
    static_assert(kXLoads * kThreads * 16 == kXStep, "X slice must split evenly");
    constexpr int kWT = 4 * NBW;                         // row groups (tiles per step) per wave
    extern __shared__ uint8_t s_mem[];  // X [2][kXStep], then per wave kWT padded tiles

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int CG = p.cg, KS = p.ks, MG = p.mgroups;
    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int mg = blk % MG, nb = blk / MG;
    const int mb0 = mg * MB;
    const int rgw = (nb * NW + wave) * kWT;  // first row group (4 rows) of this wave
    const int nrg_w = max(0, min(kWT, p.nrg - rgw));
    const rsrc_t wres =
        make_rsrc(p.Wq + (size_t)min(rgw, p.nrg) * CG * 1024u, (uint32_t)(nrg_w * CG) * 1024u);
    // this workgroup's blocks of X codes (at most MB * KS KB)
    const int mbw = max(0, min(MB, p.mbtot - mb0));
    const rsrc_t xres = make_rsrc(p.Xp + (size_t)min(mb0, p.mbtot) * KS * 1024u,
                                  (uint32_t)mbw * (uint32_t)KS * 1024u);
    uint8_t* s_x = s_mem;
    uint8_t* s_w = s_mem + 2 * kXStep + wave * kWT * kW4TilePitch;
#define QW_KT(C) (C)

    uint4 w0[kWT], w1[kWT], w2[kWT], xa[kXLoads], xb[kXLoads];
    // weights of step c (zeros past K); X codes of step c (zeros past K and past M)
#define QW_LOADW(WB, C)                                                                          \
    _Pragma("unroll") for (int i_ = 0; i_ < kWT; ++i_)                                           \
        WB[i_] = load16_stream(wres, (C) < CG ? (uint32_t)(i_ * CG + QW_KT(C)) * 1024u + (uint32_t)lane * 16u \
                                              : 0x80000000u);
#define QW_LOADX(XB, C)                                                                          \
    _Pragma("unroll") for (int v_ = 0; v_ < kXLoads; ++v_)                                       \
    {                                                                                            \
        const int pc_ = v_ * kThreads + tid; /* [mbl][s][lane] */                                \
        const int mbl_ = pc_ >> 9, s_ = (pc_ >> 6) & 7, sl_ = pc_ & 63;                          \
        const bool ok_ = (C) < CG && mbl_ < mbw && 8 * QW_KT(C) + s_ < KS;                       \
        XB[v_] = load16(xres, ok_ ? ((uint32_t)mbl_ * (uint32_t)KS + (uint32_t)(8 * QW_KT(C) + s_)) * 1024u + \
                                         (uint32_t)sl_ * 16u                                     \
                                   : 0x80000000u);                                               \
    }
#define QW_STOREX(XB, BUF)                                                                       \
    _Pragma("unroll") for (int v_ = 0; v_ < kXLoads; ++v_)                                       \
        *reinterpret_cast<uint4*>(s_x + (BUF) * kXStep + (size_t)(v_ * kThreads + tid) * 16) = XB[v_];

    v4i acc[NBW][MB];
#pragma unroll
    for (int b = 0; b < NBW; ++b)
#pragma unroll
        for (int i = 0; i < MB; ++i)
            acc[b][i] = v4i{0, 0, 0, 0};

    const int sub = lane >> 4, j = lane & 15;
    // A operand of block b, step s for lane (g, r): row r of the block = tile 4 b + r / 4,
    // tile row r % 4; 16 k = chunk 2 s + g / 2, half g % 2
    const int a_off = (r >> 2) * kW4TilePitch + (r & 3) * kW4RowPitch + (g >> 1) * 16 + (g & 1) * 8;

    // One 512-k step C.  X of step C+2 (into XL, whose step C was stored last step) and
    // the weights of step C+2 (into WN) are requested first; the weights of step C (WC)
    // are regrouped through LDS and multiplied with the X slice in buffer C % 2; then X
    // of step C+1 (XS) is stored and the workgroup syncs.  Waiting for XS waits only for
    // loads issued before it, i.e. up to the weights of step C: the weights of steps C+1
    // and C+2 stay in flight.
#define QW_STEP(WC, WN, XL, XS, C)                                                               \
    {                                                                                            \
        QW_LOADX(XL, (C) + 2);                                                                   \
        QW_LOADW(WN, (C) + 2);                                                                   \
        __builtin_amdgcn_sched_barrier(0);                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < kWT; ++i_)                                       \
            *reinterpret_cast<uint4*>(s_w + i_ * kW4TilePitch + sub * kW4RowPitch + j * 16) = WC[i_]; \
        const uint8_t* xb_ = s_x + ((C) & 1) * kXStep;                                           \
        _Pragma("unroll") for (int s_ = 0; s_ < 8; ++s_)                                         \
        {                                                                                        \
            v4i bo_[MB];                                                                         \
            _Pragma("unroll") for (int mbl_ = 0; mbl_ < MB; ++mbl_)                              \
            {                                                                                    \
                const uint4 b4_ = *reinterpret_cast<const uint4*>(xb_ + ((mbl_ * 8 + s_) * 64 + lane) * 16); \
                bo_[mbl_] = v4i{(int)b4_.x, (int)b4_.y, (int)b4_.z, (int)b4_.w};                  \
            }                                                                                    \
            _Pragma("unroll") for (int b_ = 0; b_ < NBW; ++b_)                                   \
            {                                                                                    \
                const uint2 w_ = *reinterpret_cast<const uint2*>(s_w + b_ * 4 * kW4TilePitch + a_off + s_ * 32); \
                const v4i a_ = {(int)((w_.x << 4) & 0xF0F0F0F0u), (int)(w_.x & 0xF0F0F0F0u),     \
                                (int)((w_.y << 4) & 0xF0F0F0F0u), (int)(w_.y & 0xF0F0F0F0u)};    \
                _Pragma("unroll") for (int mbl_ = 0; mbl_ < MB; ++mbl_)                          \
                    acc[b_][mbl_] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_, bo_[mbl_], acc[b_][mbl_], 0, 0, 0); \
            }                                                                                    \
        }                                                                                        \
        QW_STOREX(XS, ((C) + 1) & 1);                                                            \
        __syncthreads();                                                                         \
    }

    QW_LOADX(xa, 0);
    QW_LOADX(xb, 1);
    QW_LOADW(w0, 0);
    QW_LOADW(w1, 1);
    __builtin_amdgcn_sched_barrier(0);
    QW_STOREX(xa, 0);
    __syncthreads();
    QW_STEPS_SIX();
#undef QW_STEP
#undef QW_STOREX
#undef QW_LOADX
#undef QW_LOADW
#undef QW_KT

    // lane (g, r) holds D[n = 4 g + i][m = r] of each 16 x 16 block
    const rsrc_t sres = make_rsrc(p.w_scale, (uint32_t)p.N * 4u);
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        const int n0 = 4 * rgw + 16 * b + 4 * g;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sc[i] = __uint_as_float(load4(sres, (uint32_t)(n0 + i) * 4u));
#pragma unroll
        for (int mbl = 0; mbl < MB; ++mbl) {
            const int m = (mb0 + mbl) * 16 + r;
            if (m < p.M) {
                const float am = p.a_scale[m];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n0 + i < p.N)
                        p.Y[(size_t)m * p.N + n0 + i] = ((float)(acc[b][mbl][i] >> 4) * sc[i]) * am;
            }
        }
    }
}

// Largest X code slice a balanced workgroup keeps in LDS: K up to 4096.
constexpr int kXAllMaxBytes = 64 * 1024;

// The same linear with the work balanced over the CUs, for K up to 4096.  Workgroup
// (b, mb) takes block mb of 16 rows of X (blockIdx.y) and a contiguous run of row groups
// (per or per + 1 of them; one workgroup per CU and block of X), i.e. nb output blocks
// of 16 rows (the last one partial: rows past the run read zeros) and T = nb * CG
// (512-k step, block) units in step-major order, so that consecutive units share
// their X operands.  Wave w takes units [w T / NW, (w + 1) T / NW), at most U of them,
// in a fully unrolled software pipeline: the weights of unit u + 1 are requested just
// before unit u is multiplied.  (Requesting many units ahead was measured slower: a
// wave stalls in its requests while the CU's queue is full, and the units left when
// the stream ends are multiplied one after another.)  Every wave first requests its
// share of the block's X codes and of the scales, and only after an issue barrier its
// first unit of weights, so that no X load queues behind another wave's weights.  The
// X codes go to LDS; each unit's four tiles are regrouped through the wave's LDS tile
// area into A operands and multiplied against them, and the unit's int32 sums are
// added into the workgroup's LDS totals (integer adds: exact in any order).  After one
// more barrier the workgroup writes its outputs, consecutive threads on consecutive n.
//
// FR > 0 (fused quantization of up to FR rows of X, 8 waves): instead of reading codes
// that a separate pre-pass launch wrote, the workgroup requests the rows of X itself
// (fp32, before its first weights), takes each row's maximum (a wave reduction, one
// value per wave in LDS, the maximum of those), and writes the codes straight into the LDS operand layout
// with quant4_e, the same codes and scales as quant_act_i8.  Rows past M in the block
// of 16 are left unwritten: they only reach outputs that are never stored.
constexpr int kBalMaxBlocks = 40;      // output blocks per workgroup (LDS totals)
constexpr int kBalSumPitch = 17;       // int32 per row of m in the LDS totals
constexpr int kFqRows = 4;             // most rows of X the fused prologue takes

template <int NW, int U, int FR>
__global__ __launch_bounds__(64 * NW) void k_gemm_w4a8_bal(MfmaW4A8Args p)
{
    constexpr int kThreads = 64 * NW;
    constexpr int kXP = kXAllMaxBytes / 16 / kThreads;  // 16-byte X pieces per thread
    constexpr bool FQ = FR > 0;
    constexpr int kFV = 4096 / 4 / kThreads;            // FQ: float4 per thread per row (K <= 4096)
    static_assert(!FQ || (NW == 8 && FR <= kFqRows), "the fused prologue: 8 waves, up to kFqRows rows");
    constexpr int kScales = 4 * 4 * kBalMaxBlocks;       // row scales of the workgroup
    constexpr int kSP = (kScales + kThreads - 1) / kThreads;
    // LDS: X [CG steps][8 KB], per wave 4 padded tiles, the int32 totals
    // [nbmax][16 m][17], the row scales and the 16 activation scales
    extern __shared__ uint8_t s_mem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int CG = p.cg, KS = p.ks;
    const int b = blockIdx.x, mb = blockIdx.y;
    const int rg0 = min(b * p.per + min(b, p.rem), p.nrg);
    const int nrg_b = max(0, min(p.per + (b < p.rem ? 1 : 0), p.nrg - rg0));
    const int nb = max(1, (nrg_b + 3) >> 2);
    const int T = nb * CG;
    const int u0 = (wave * T) / NW, u1 = ((wave + 1) * T) / NW;
    const int n0 = 4 * rg0;
    const int nrows = max(0, min(4 * nrg_b, p.N - n0));
    const int mv = min(p.M - 16 * mb, 16);  // live rows of this block of X
    const rsrc_t wres = make_rsrc(p.Wq + (size_t)rg0 * CG * 1024u, (uint32_t)(nrg_b * CG) * 1024u);
    const rsrc_t xres = make_rsrc(p.Xp + (size_t)mb * KS * 1024u, (uint32_t)KS * 1024u);
    const rsrc_t sres = make_rsrc(p.w_scale + n0, (uint32_t)nrows * 4u);
    const rsrc_t ares = make_rsrc(p.a_scale + 16 * mb, (uint32_t)mv * 4u);
    const int xbytes = CG * 8 * 1024;  // whole 512-k steps; past K the loads read zeros
    uint8_t* s_x = s_mem;
    uint8_t* s_w = s_mem + xbytes + wave * 4 * kW4TilePitch;
    int* s_sum = reinterpret_cast<int*>(s_mem + xbytes + NW * 4 * kW4TilePitch);
    float* s_sc = reinterpret_cast<float*>(s_sum + p.nbmax * 16 * kBalSumPitch);
    float* s_a = s_sc + 4 * 4 * p.nbmax;
    float* s_wmax = s_a + 16;  // FQ: [wave][row] maxima

    // (step, block) of the wave's unit u, step-major: c = (u0 + u) / nb
    const int c0 = u0 / nb, blk0 = u0 - c0 * nb;
    uint4 wb[U][4];
    // the four tiles of unit u (zeros past the wave's run and past the workgroup's rows)
#define QW_LOADU(U_)                                                                             \
    {                                                                                            \
        const int q_ = blk0 + (U_);                                                              \
        const int c_ = c0 + q_ / nb, blk_ = q_ % nb;                                             \
        const bool live_ = u0 + (U_) < u1;                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                         \
            wb[U_][i_] = load16_stream(wres, live_ ? (uint32_t)((4 * blk_ + i_) * CG + c_) * 1024u + \
                                                         (uint32_t)lane * 16u                    \
                                                   : 0x80000000u);                               \
    }

    uint4 xr[FQ ? 1 : kXP];
    float4 xf[FQ ? FR : 1][FQ ? kFV : 1];  // FQ: float4 v of row m: k = 4 (v T + tid)
    const int K4 = p.K >> 2;
    if constexpr (FQ) {
        const rsrc_t xfr = make_rsrc(p.X + (size_t)16 * mb * p.K, (uint32_t)(mv * p.K) * 4u);
#pragma unroll
        for (int m = 0; m < FR; ++m)
#pragma unroll
            for (int v = 0; v < kFV; ++v) {
                const int f = v * kThreads + tid;
                xf[m][v] = load16f(xfr, m < mv && f < K4 ? (uint32_t)(m * p.K + 4 * f) * 4u : 0x80000000u);
            }
    } else {
#pragma unroll
        for (int v = 0; v < kXP; ++v) {
            const int pc = v * kThreads + tid;
            xr[v] = load16(xres, pc * 16 < xbytes ? (uint32_t)pc * 16u : 0x80000000u);
        }
    }
    uint32_t sr[kSP];
#pragma unroll
    for (int v = 0; v < kSP; ++v)
        sr[v] = load4(sres, (uint32_t)(v * kThreads + tid) * 4u);
    const uint32_t ar = FQ ? 0u : load4(ares, (uint32_t)(tid & 15) * 4u);
    issue_barrier();
    QW_LOADU(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FQ) {
        // each row's maximum |x|: per wave, then over the waves
#pragma unroll
        for (int m = 0; m < FR; ++m) {
            float mx = 0.0f;
#pragma unroll
            for (int v = 0; v < kFV; ++v)
                mx = fmaxf(mx, max_abs4(xf[m][v]));
            mx = wave_max_dpp(mx);
            if (lane == 0)
                s_wmax[wave * FR + m] = mx;
        }
        __syncthreads();
        // codes of 64-k step st, lane group g (16 k), row m at st 1024 + g 256 + m 16:
        // bytes 0-3 the even k of its first 8, 4-7 their odd k, 8-15 the same for the
        // next 8; a float4 (k = 4f .. 4f + 3, quarter h of the 16) gives two 16-bit pairs
#pragma unroll
        for (int m = 0; m < FR; ++m) {
            if (m < mv) {
                float mxm = s_wmax[m];
#pragma unroll
                for (int w = 1; w < NW; ++w)
                    mxm = fmaxf(mxm, s_wmax[w * FR + m]);
                const float a = mxm / 127.0f;
                const float r = 1.0f / a;
                const bool fast = r <= 3.0e38f;
                if (tid == 0)
                    s_a[m] = a;
#pragma unroll
                for (int v = 0; v < kFV; ++v) {
                    const int f = v * kThreads + tid;
                    if (f < CG * 128) {  // whole 512-k steps; past K, X read zeros
                        uint32_t e[4];
                        if (quant4_e(xf[m][v], r, e) || !fast)
                            quant4_e_div(xf[m][v], a, e);
                        const int st = f >> 4, g4 = (f >> 2) & 3, h = f & 3;
                        uint8_t* d = s_x + (size_t)st * 1024 + g4 * 256 + m * 16 + (h & 1) * 2 + (h >> 1) * 8;
                        *reinterpret_cast<uint16_t*>(d) = (uint16_t)__builtin_amdgcn_perm(e[2], e[0], 0x0C0C0602u);
                        *reinterpret_cast<uint16_t*>(d + 4) = (uint16_t)__builtin_amdgcn_perm(e[3], e[1], 0x0C0C0602u);
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int v = 0; v < kXP; ++v) {
            const int pc = v * kThreads + tid;
            if (pc * 16 < xbytes)
                *reinterpret_cast<uint4*>(s_x + (size_t)pc * 16) = xr[v];
        }
    }
#pragma unroll
    for (int v = 0; v < kSP; ++v)
        if (v * kThreads + tid < 4 * 4 * p.nbmax)
            s_sc[v * kThreads + tid] = __uint_as_float(sr[v]);
    if (!FQ && tid < 16)
        s_a[tid] = __uint_as_float(ar);
    for (int e = tid; e < nb * 16 * kBalSumPitch; e += kThreads)
        s_sum[e] = 0;
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);

    const int sub = lane >> 4, j = lane & 15;
    // A operand of step s for lane (g, r): row r of the block = tile r / 4, tile row
    // r % 4; 16 k = chunk 2 s + g / 2, half g % 2
    const int a_off = (r >> 2) * kW4TilePitch + (r & 3) * kW4RowPitch + (g >> 1) * 16 + (g & 1) * 8;
    v4i bo[8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u + 1 < U)
            QW_LOADU(u + 1);
        __builtin_amdgcn_sched_barrier(0);
        const int q = blk0 + u;
        const int c = c0 + q / nb, blk = q % nb;
        if (u0 + u < u1) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint4*>(s_w + i * kW4TilePitch + sub * kW4RowPitch + j * 16) = wb[u][i];
            if (u == 0 || blk == 0) {
                // B operands of step c (the first unit, or a new step)
                const uint8_t* xb = s_x + (size_t)c * 8 * 1024;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const uint4 b4 = *reinterpret_cast<const uint4*>(xb + (s * 64 + lane) * 16);
                    bo[s] = v4i{(int)b4.x, (int)b4.y, (int)b4.z, (int)b4.w};
                }
            }
            v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint2 w = *reinterpret_cast<const uint2*>(s_w + a_off + s * 32);
                const v4i a = {(int)((w.x << 4) & 0xF0F0F0F0u), (int)(w.x & 0xF0F0F0F0u),
                               (int)((w.y << 4) & 0xF0F0F0F0u), (int)(w.y & 0xF0F0F0F0u)};
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bo[s], acc, 0, 0, 0);
            }
            // lane (g, r) holds D[n = 4 g + i][m = r] of block blk
            int* dst = s_sum + (blk * 16 + r) * kBalSumPitch + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __hip_atomic_fetch_add(dst + i, acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
#undef QW_LOADU
    __syncthreads();

    // outputs (m, nn), independent across threads
    for (int e = tid; e < mv * nrows; e += kThreads) {
        const int m = e / nrows, nn = e - m * nrows;
        const int v = s_sum[((nn >> 4) * 16 + m) * kBalSumPitch + (nn & 15)];
        p.Y[(size_t)(16 * mb + m) * p.N + n0 + nn] = ((float)(v >> 4) * s_sc[nn]) * s_a[m];
    }
}

constexpr int kBalsMaxRows = 1024;   // rows of X of the kernel over many blocks

// The balanced W4A8 kernel over many blocks of X with one wave per 512-k step (K up
// to 4096, 1 to 1024 rows of X).  Workgroup b owns an even run of row groups, nb <= U
// output blocks of 16 rows; wave w takes step w of every one of them (unit u = block u
// at step w), so that the X operands it needs for one block of 16 rows of X are the
// 8 KB of step w, loaded straight into registers.  Block 0 of X goes through the
// one-unit-ahead pipeline as the weights stream in, and each unit's regrouped A
// operands stay in registers (16 VGPRs a unit); blocks 1 .. MBT-1 are then multiplied
// against them, the next block's operands requested one block ahead; with PAIR, two
// blocks at a time, each unpacked A operand feeding both (the block loop is bound by the
// nibble unpack on the vector ALU, 6 instructions per multiply), their operands
// requested at the start of the pair.  The CG partial sums of an output meet in one of
// two (PAIR: four) LDS total buffers (integer adds, exact in any order); after one
// barrier per block (pair) the workgroup writes the outputs and zeroes each entry it
// reads.
template <int U, bool PAIR>
__global__ __launch_bounds__(512) void k_gemm_w4a8_bals(MfmaW4A8Args p)
{
    // LDS: per wave 4 padded tiles, two int32 total buffers [nbmax][16 m][17], the row
    // scales and two sets of 16 activation scales
    extern __shared__ uint8_t s_mem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // = the 512-k step
    const int nthreads = (int)blockDim.x;
    const int g = lane >> 4, r = lane & 15;
    const int CG = p.cg, KS = p.ks, MBT = p.mbtot;
    const int b = blockIdx.x;
    const int rg0 = min(b * p.per + min(b, p.rem), p.nrg);
    const int nrg_b = max(0, min(p.per + (b < p.rem ? 1 : 0), p.nrg - rg0));
    const int nb = min(U, (nrg_b + 3) >> 2);
    const int n0 = 4 * rg0;
    const int nrows = max(0, min(4 * nrg_b, p.N - n0));
    const int bsum = p.nbmax * 16 * kBalSumPitch;
    const rsrc_t wres = make_rsrc(p.Wq + (size_t)rg0 * CG * 1024u, (uint32_t)(nrg_b * CG) * 1024u);
    const rsrc_t sres = make_rsrc(p.w_scale + n0, (uint32_t)nrows * 4u);
    const rsrc_t ares = make_rsrc(p.a_scale, (uint32_t)p.M * 4u);
    uint8_t* s_w = s_mem + wave * 4 * kW4TilePitch;
    int* s_sum = reinterpret_cast<int*>(s_mem + 8 * 4 * kW4TilePitch);
    constexpr int kBufs = PAIR ? 4 : 2;  // int32 total buffers (and sets of a-scales)
    float* s_sc = reinterpret_cast<float*>(s_sum + kBufs * bsum);
    float* s_a = s_sc + 4 * 4 * p.nbmax;  // [kBufs][16]

    // X operands of block MB_ at step w: substep s -> 16 bytes at (MB_ KS + 8 w + s) KB
    // + 16 lane (zeros past K)
#define QW_LOADB(BO, MB_)                                                                        \
    {                                                                                            \
        const rsrc_t xres_ = make_rsrc(p.Xp + (size_t)(MB_) * KS * 1024u, (uint32_t)KS * 1024u); \
        _Pragma("unroll") for (int s_ = 0; s_ < 8; ++s_)                                         \
            BO[s_] = load16(xres_, (uint32_t)(8 * wave + s_) * 1024u + (uint32_t)lane * 16u);    \
    }
    // the four tiles of unit U_: block U_ at step w (zeros past the run)
#define QW_LOADU(U_)                                                                             \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                             \
        wb[U_][i_] = load16_stream(wres, (U_) < nb ? (uint32_t)((4 * (U_) + i_) * CG + wave) * 1024u + \
                                                         (uint32_t)lane * 16u                    \
                                                   : 0x80000000u);
    // one unit's eight multiplies against bo, its sums into total buffer SB.  The shift
    // and mask of the nibble unpack are scalars the compiler cannot see through (an
    // opaque zero added per block of X): hoisted out of the loop over blocks, the
    // unpacked operands of every unit would not fit the registers
#define QW_UNIT_MFMA(U_, SB)                                                                     \
    {                                                                                            \
        v4i acc_ = v4i{0, 0, 0, 0};                                                              \
        _Pragma("unroll") for (int s_ = 0; s_ < 8; ++s_)                                         \
        {                                                                                        \
            const uint2 w_ = ua[U_][s_];                                                         \
            const v4i a_ = {(int)((w_.x << ush) & umask), (int)(w_.x & umask),                   \
                            (int)((w_.y << ush) & umask), (int)(w_.y & umask)};                  \
            const v4i b_ = {(int)bo[s_].x, (int)bo[s_].y, (int)bo[s_].z, (int)bo[s_].w};         \
            acc_ = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_, b_, acc_, 0, 0, 0);                 \
        }                                                                                        \
        int* dst_ = (SB) + ((U_) * 16 + r) * kBalSumPitch + 4 * g;                               \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                         \
            __hip_atomic_fetch_add(dst_ + i_, acc_[i_], __ATOMIC_RELAXED,                        \
                                   __HIP_MEMORY_SCOPE_WORKGROUP);                                \
    }
    // outputs of block MB_ (total buffer and scales (MB_) % 2), each entry zeroed once
    // read; thread t takes output row n0 + t % 64 (+ 64) and rows of X t / 64, t / 64 +
    // nthreads / 64, ... (a workgroup's run is at most 16 U <= 128 rows)
#define QW_OUT_BLOCK(MB_)                                                                        \
    {                                                                                            \
        int* sb_ = s_sum + ((MB_) & (kBufs - 1)) * bsum;                                         \
        const float* sa_ = s_a + ((MB_) & (kBufs - 1)) * 16;                                     \
        const int mv_ = min(p.M - 16 * (MB_), 16);                                               \
        float* y_ = p.Y + (size_t)(16 * (MB_)) * p.N + n0;                                       \
        _Pragma("unroll") for (int h_ = 0; h_ < (U > 4 ? 2 : 1); ++h_)                           \
        {                                                                                        \
            const int nn_ = lane + 64 * h_;                                                      \
            if (nn_ < nrows) {                                                                   \
                const float sc_ = s_sc[nn_];                                                     \
                for (int m_ = wave; m_ < mv_; m_ += nthreads >> 6) {                             \
                    int* cell_ = sb_ + ((nn_ >> 4) * 16 + m_) * kBalSumPitch + (nn_ & 15);       \
                    const int v_ = *cell_;                                                       \
                    *cell_ = 0;                                                                  \
                    y_[(size_t)m_ * p.N + nn_] = ((float)(v_ >> 4) * sc_) * sa_[m_];             \
                }                                                                                \
            }                                                                                    \
        }                                                                                        \
    }

    uint4 bo[8], bn[8];
    QW_LOADB(bo, 0);
    const uint32_t sr0 = load4(sres, (uint32_t)tid * 4u);
    const uint32_t sr1 = load4(sres, (uint32_t)(tid + nthreads) * 4u);
    const uint32_t ar = load4(ares, (uint32_t)(tid & 15) * 4u);
    uint4 wb[U][4];
    issue_barrier();
    QW_LOADU(0);
    __builtin_amdgcn_sched_barrier(0);
    if (tid < 4 * 4 * p.nbmax)
        s_sc[tid] = __uint_as_float(sr0);
    if (tid + nthreads < 4 * 4 * p.nbmax)
        s_sc[tid + nthreads] = __uint_as_float(sr1);
    if (tid < 16)
        s_a[tid] = __uint_as_float(ar);
    for (int e = tid; e < kBufs * bsum; e += nthreads)
        s_sum[e] = 0;
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);

    const int sub = lane >> 4, j = lane & 15;
    // A operand of substep s for lane (g, r): row r of the block = tile r / 4, tile row
    // r % 4; 16 k = chunk 2 s + g / 2, half g % 2
    const int a_off = (r >> 2) * kW4TilePitch + (r & 3) * kW4RowPitch + (g >> 1) * 16 + (g & 1) * 8;
    uint2 ua[U][8];  // regrouped A operands of every unit of the wave
    uint32_t ush = 4u, umask = 0xF0F0F0F0u;
    // block 0 of X as the weights stream in
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u + 1 < U) {
            QW_LOADU(u + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (u < nb) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint4*>(s_w + i * kW4TilePitch + sub * kW4RowPitch + j * 16) = wb[u][i];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                ua[u][s] = *reinterpret_cast<const uint2*>(s_w + a_off + s * 32);
            QW_UNIT_MFMA(u, s_sum);
        }
    }
    if (!PAIR && MBT > 1)
        QW_LOADB(bn, 1);
    float an = 0.0f;
    if (!PAIR && MBT > 1)
        an = __uint_as_float(load4(ares, (uint32_t)(16 + (tid & 15)) * 4u));
    __syncthreads();
    QW_OUT_BLOCK(0);
    if (PAIR) {
        // blocks 1 .. MBT-1 two at a time: each unpacked A operand feeds two multiplies
        for (int mb = 1; mb < MBT; mb += 2) {
            uint32_t z;
            asm volatile("s_mov_b32 %0, 0" : "=s"(z));
            ush = 4u + z;
            umask = 0xF0F0F0F0u + z;
            const bool two = mb + 1 < MBT;
            QW_LOADB(bo, mb);
            if (two) {
                QW_LOADB(bn, mb + 1);
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    bn[s] = uint4{0u, 0u, 0u, 0u};
            }
            if (tid < 16) {
                s_a[(mb & 3) * 16 + tid] = __uint_as_float(load4(ares, (uint32_t)(16 * mb + tid) * 4u));
                s_a[((mb + 1) & 3) * 16 + tid] =
                    __uint_as_float(load4(ares, (uint32_t)(16 * (mb + 1) + tid) * 4u));
            }
            int* sb0 = s_sum + (mb & 3) * bsum;
            int* sb1 = s_sum + ((mb + 1) & 3) * bsum;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u < nb) {
                    v4i acc0 = v4i{0, 0, 0, 0}, acc1 = v4i{0, 0, 0, 0};
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        const uint2 w_ = ua[u][s];
                        const v4i a_ = {(int)((w_.x << ush) & umask), (int)(w_.x & umask),
                                        (int)((w_.y << ush) & umask), (int)(w_.y & umask)};
                        const v4i b0 = {(int)bo[s].x, (int)bo[s].y, (int)bo[s].z, (int)bo[s].w};
                        const v4i b1 = {(int)bn[s].x, (int)bn[s].y, (int)bn[s].z, (int)bn[s].w};
                        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_, b0, acc0, 0, 0, 0);
                        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_, b1, acc1, 0, 0, 0);
                    }
                    int* d0 = sb0 + (u * 16 + r) * kBalSumPitch + 4 * g;
                    int* d1 = sb1 + (u * 16 + r) * kBalSumPitch + 4 * g;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        __hip_atomic_fetch_add(d0 + i, acc0[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                        if (two)
                            __hip_atomic_fetch_add(d1 + i, acc1[i], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP);
                    }
                }
            }
            __syncthreads();
            QW_OUT_BLOCK(mb);
            if (two)
                QW_OUT_BLOCK(mb + 1);
        }
    } else {
        // blocks 1 .. MBT-1 against the A operands held in registers
        for (int mb = 1; mb < MBT; ++mb) {
            uint32_t z;
            asm volatile("s_mov_b32 %0, 0" : "=s"(z));
            ush = 4u + z;
            umask = 0xF0F0F0F0u + z;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                bo[s] = bn[s];
            if (tid < 16)
                s_a[(mb & 1) * 16 + tid] = an;
            if (mb + 1 < MBT) {
                QW_LOADB(bn, mb + 1);
                an = __uint_as_float(load4(ares, (uint32_t)(16 * (mb + 1) + (tid & 15)) * 4u));
            }
            int* sb = s_sum + (mb & 1) * bsum;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (u < nb)
                    QW_UNIT_MFMA(u, sb);
            __syncthreads();
            QW_OUT_BLOCK(mb);
        }
    }
#undef QW_LOADB
#undef QW_LOADU
#undef QW_UNIT_MFMA
#undef QW_OUT_BLOCK
}

// ---------------------------------------------------------------- W8A16 -------

// Padded LDS image of one INT8 tile (2 rows x 32 chunks): row sub at sub * 528, chunk
// j at j * 16.
constexpr int kW8TilePitch = 1056, kW8RowPitch = 528;
// X slice of one 512-k step in LDS: 16 MB rows of 1 KB, rows padded to 1040 bytes.
constexpr int kXRowPitch = 1040;

// int8 x 4 -> f16 x 4, exact (see the GEMV kernel): bytes ^ 0x80 under a 0x64 byte
// read as 1024 + q + 128, minus 1152.
__device__ __forceinline__ void cast4(uint32_t wd, half2_t& lo, half2_t& hi)
{
    const uint32_t u = wd ^ 0x80808080u;
    const uint32_t l = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t h = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    const half2_t off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    lo = __builtin_bit_cast(half2_t, l) + off;
    hi = __builtin_bit_cast(half2_t, h) + off;
}

template <int NW, int MB, int NBW>
__global__ __launch_bounds__(64 * NW) void k_gemm_w8a16(MfmaW8A16Args p)
{
    constexpr int kThreads = 64 * NW;
    constexpr int kXStep = MB * 16 * kXRowPitch;           // LDS bytes of one X slice
    constexpr int kXPieces = MB * 16 * 64;                 // 16-byte pieces of one slice
    constexpr int kXLoads = (kXPieces + kThreads - 1) / kThreads;
    constexpr int kWT = 8 * NBW;                           // row groups (2 rows) per wave
    extern __shared__ uint8_t s_mem[];  // X [2][kXStep], then per wave kWT padded tiles

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int M = p.M, K = p.K, CG = p.cg, MG = p.mgroups;
    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int mg = blk % MG, nb = blk / MG;
    const int m0 = mg * MB * 16;
    const int rgw = (nb * NW + wave) * kWT;  // first row group (2 rows) of this wave
    const int nrg_w = max(0, min(kWT, p.nrg - rgw));
    const rsrc_t wres =
        make_rsrc(p.Wq + (size_t)min(rgw, p.nrg) * CG * 1024u, (uint32_t)(nrg_w * CG) * 1024u);
    const int rows_x = max(0, min(MB * 16, M - m0));
    const rsrc_t xres = make_rsrc(p.X + (size_t)min(m0, M) * K, (uint32_t)rows_x * (uint32_t)K * 2u);
    uint8_t* s_x = s_mem;
    uint8_t* s_w = s_mem + 2 * kXStep + wave * kWT * kW8TilePitch;
#define QW_KT(C) (C)

    uint4 w0[kWT], w1[kWT], w2[kWT], xa[kXLoads], xb[kXLoads];
#define QW_LOADW(WB, C)                                                                          \
    _Pragma("unroll") for (int i_ = 0; i_ < kWT; ++i_)                                           \
        WB[i_] = load16_stream(wres, (C) < CG ? (uint32_t)(i_ * CG + QW_KT(C)) * 1024u + (uint32_t)lane * 16u \
                                              : 0x80000000u);
    // piece pc of the slice of step C: row pc / 64, k = 512 QW_KT(C) + 8 (pc % 64)
#define QW_LOADX(XB, C)                                                                          \
    _Pragma("unroll") for (int v_ = 0; v_ < kXLoads; ++v_)                                       \
    {                                                                                            \
        const int pc_ = v_ * kThreads + tid;                                                     \
        const int row_ = pc_ >> 6, k_ = 512 * QW_KT(C) + 8 * (pc_ & 63);                         \
        const bool ok_ = (C) < CG && pc_ < kXPieces && k_ < K;                                   \
        XB[v_] = load16(xres, ok_ ? (uint32_t)(row_ * K + k_) * 2u : 0x80000000u);               \
    }
#define QW_STOREX(XB, BUF)                                                                       \
    _Pragma("unroll") for (int v_ = 0; v_ < kXLoads; ++v_)                                       \
    {                                                                                            \
        const int pc_ = v_ * kThreads + tid;                                                     \
        if (pc_ < kXPieces)                                                                      \
            *reinterpret_cast<uint4*>(s_x + (BUF) * kXStep + (pc_ >> 6) * kXRowPitch + (pc_ & 63) * 16) = XB[v_]; \
    }

    v4f acc[NBW][MB];
#pragma unroll
    for (int b = 0; b < NBW; ++b)
#pragma unroll
        for (int i = 0; i < MB; ++i)
            acc[b][i] = v4f{0.f, 0.f, 0.f, 0.f};

    const int sub = lane >> 5, j = lane & 31;
    // A operand of block b, step s (32 k) for lane (g, r): row r of the block = tile
    // 8 b + r / 2, tile row r % 2; k = 32 s + 8 g .. + 7 = chunk 2 s + g / 2, half g % 2
    const int a_off = (r >> 1) * kW8TilePitch + (r & 1) * kW8RowPitch + (g >> 1) * 16 + (g & 1) * 8;

    // One 512-k step, ordered as in the W4A8 kernel.  The 16 MFMA steps go in groups
    // of four, so that the compiler does not hold every operand of the step at once.
#define QW_STEP(WC, WN, XL, XS, C)                                                               \
    {                                                                                            \
        QW_LOADX(XL, (C) + 2);                                                                   \
        QW_LOADW(WN, (C) + 2);                                                                   \
        __builtin_amdgcn_sched_barrier(0);                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < kWT; ++i_)                                       \
            *reinterpret_cast<uint4*>(s_w + i_ * kW8TilePitch + sub * kW8RowPitch + j * 16) = WC[i_]; \
        const uint8_t* xb_ = s_x + ((C) & 1) * kXStep;                                           \
        _Pragma("unroll") for (int s_ = 0; s_ < 16; ++s_)                                        \
        {                                                                                        \
            v8h bo_[MB];                                                                         \
            _Pragma("unroll") for (int mbl_ = 0; mbl_ < MB; ++mbl_)                              \
                bo_[mbl_] = __builtin_bit_cast(v8h, *reinterpret_cast<const uint4*>(             \
                    xb_ + (mbl_ * 16 + r) * kXRowPitch + s_ * 64 + g * 16));                     \
            _Pragma("unroll") for (int b_ = 0; b_ < NBW; ++b_)                                   \
            {                                                                                    \
                const uint2 w_ = *reinterpret_cast<const uint2*>(s_w + b_ * 8 * kW8TilePitch + a_off + s_ * 32); \
                half2_t h0_, h1_, h2_, h3_;                                                      \
                cast4(w_.x, h0_, h1_);                                                           \
                cast4(w_.y, h2_, h3_);                                                           \
                const v8h a_ = {h0_[0], h0_[1], h1_[0], h1_[1], h2_[0], h2_[1], h3_[0], h3_[1]}; \
                _Pragma("unroll") for (int mbl_ = 0; mbl_ < MB; ++mbl_)                          \
                    acc[b_][mbl_] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_, bo_[mbl_], acc[b_][mbl_], 0, 0, 0); \
            }                                                                                    \
            if ((s_ & 3) == 3)                                                                   \
                __builtin_amdgcn_sched_barrier(0);                                               \
        }                                                                                        \
        QW_STOREX(XS, ((C) + 1) & 1);                                                            \
        __syncthreads();                                                                         \
    }

    QW_LOADX(xa, 0);
    QW_LOADX(xb, 1);
    QW_LOADW(w0, 0);
    QW_LOADW(w1, 1);
    __builtin_amdgcn_sched_barrier(0);
    QW_STOREX(xa, 0);
    __syncthreads();
    QW_STEPS_SIX();
#undef QW_STEP
#undef QW_STOREX
#undef QW_LOADX
#undef QW_LOADW
#undef QW_KT

    const rsrc_t sres = make_rsrc(p.w_scale, (uint32_t)p.N * 2u);
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        const int n0 = 2 * rgw + 16 * b + 4 * g;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sc[i] = __half2float(__ushort_as_half(load2(sres, (uint32_t)(n0 + i) * 2u)));
#pragma unroll
        for (int mbl = 0; mbl < MB; ++mbl) {
            const int m = m0 + mbl * 16 + r;
            if (m < M) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n0 + i < p.N)
                        p.Y[(size_t)m * p.N + n0 + i] =
                            __half_as_ushort(__float2half_rn(acc[b][mbl][i] * sc[i]));
            }
        }
    }
}

// The W8A16 linear for one block of 16 rows of X (M <= 16, K up to 4096), balanced
// over the CUs like the W4A8 kernel above, but with one wave per 512-k step: wave w of
// a workgroup of CG waves takes step w of every output block of the workgroup's run of
// row groups, so that its X operands (16 rows x 512 k of f16, 16 KB) stay in its
// registers for all its units; a unit is one block of 16 rows (eight INT8 tiles, 8 KB).
// The same one-unit-ahead pipeline and issue order as there; the tiles are regrouped
// through the wave's LDS tile area and cast exactly to f16.  Each wave stores its fp32
// partial sums per block in LDS, and the epilogue adds the CG partials of an output in
// step order (deterministic), scales once and rounds to f16.
constexpr int kW8BalMaxBlocks = 8;   // output blocks per workgroup
constexpr size_t kLdsBytes = 160 * 1024;  // LDS of one CU
constexpr int kW8BalMaxSteps = 8;    // waves per workgroup (K <= 4096)

template <int U, int MB2>
__global__ __launch_bounds__(64 * kW8BalMaxSteps) void k_gemm_w8a16_bal(MfmaW8A16Args p)
{
    // LDS: per wave 8 padded tiles (4 with MB2 == 2: a unit is regrouped in two halves),
    // then the fp32 partials [MB2][CG][nbmax][16 m][17] and the row scales
    extern __shared__ uint8_t s_mem[];
    constexpr int kStageTiles = MB2 == 2 ? 4 : 8;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // = the 512-k step
    const int nthreads = (int)blockDim.x;
    const int g = lane >> 4, r = lane & 15;
    const int CG = p.cg, K = p.K;
    const int m0 = 16 * MB2 * (int)blockIdx.y;  // first row of X of this workgroup
    const int M = min(p.M - m0, 16 * MB2);
    const int b = blockIdx.x;
    const int rg0 = min(b * p.per + min(b, p.rem), p.nrg);
    const int nrg_b = max(0, min(p.per + (b < p.rem ? 1 : 0), p.nrg - rg0));
    const int nb = min(U, (nrg_b + 7) >> 3);
    const int n0 = 2 * rg0;
    const int nrows = max(0, min(2 * nrg_b, p.N - n0));
    const int bpart = CG * p.nbmax * 16 * 17;  // floats of the partials of one block of X
    const rsrc_t wres = make_rsrc(p.Wq + (size_t)rg0 * CG * 1024u, (uint32_t)(nrg_b * CG) * 1024u);
    const rsrc_t xres = make_rsrc(p.X + (size_t)m0 * K, (uint32_t)M * (uint32_t)K * 2u);
    const rsrc_t sres = make_rsrc(p.w_scale + n0, (uint32_t)nrows * 2u);
    uint8_t* s_w = s_mem + wave * kStageTiles * kW8TilePitch;
    float* s_part = reinterpret_cast<float*>(s_mem + kW8BalMaxSteps * kStageTiles * kW8TilePitch);
    float* s_sc = s_part + MB2 * bpart;

    // X operands of step w for block bl of X: substep s (32 k), lane (g, r) ->
    // X[m0 + 16 bl + r][512 w + 32 s + 8 g .. + 7]
    uint4 xb[MB2][16];
#pragma unroll
    for (int bl = 0; bl < MB2; ++bl)
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int k = 512 * wave + 32 * s + 8 * g, m = 16 * bl + r;
            xb[bl][s] = load16(xres, m < M && k < K ? (uint32_t)(m * K + k) * 2u : 0x80000000u);
        }
    // the workgroup's row scales (at most 16 nbmax <= 128 rows, two per thread)
    const uint32_t sr0 = load2(sres, (uint32_t)tid * 2u);
    const uint32_t sr1 = load2(sres, (uint32_t)(tid + nthreads) * 2u);
    uint4 wb[U][8];
    // the eight tiles of unit u: block u of the run at step w (zeros past the run)
#define QW_LOADU8(U_)                                                                            \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_)                                             \
        wb[U_][i_] = load16_stream(wres, (U_) < nb ? (uint32_t)((8 * (U_) + i_) * CG + wave) * 1024u + \
                                                         (uint32_t)lane * 16u                    \
                                                   : 0x80000000u);
    issue_barrier();
    QW_LOADU8(0);
    __builtin_amdgcn_sched_barrier(0);
    if (tid < 16 * p.nbmax)
        s_sc[tid] = __half2float(__ushort_as_half((uint16_t)sr0));
    if (tid + nthreads < 16 * p.nbmax)
        s_sc[tid + nthreads] = __half2float(__ushort_as_half((uint16_t)sr1));

    const int sub = lane >> 5, j = lane & 31;
    // A operand of substep s for lane (g, r): row r of the block = tile r / 2, tile row
    // r % 2; k = 32 s + 8 g .. + 7 = chunk 2 s + g / 2, half g % 2 (with a half-unit
    // staging area, tile (r % 8) / 2 of half r / 8)
    const int a_off = ((MB2 == 2 ? (r & 7) : r) >> 1) * kW8TilePitch + (r & 1) * kW8RowPitch +
                      (g >> 1) * 16 + (g & 1) * 8;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u + 1 < U) {
            QW_LOADU8(u + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (u < nb) {
            v4f acc[MB2];
#pragma unroll
            for (int bl = 0; bl < MB2; ++bl)
                acc[bl] = v4f{0.f, 0.f, 0.f, 0.f};
            if constexpr (MB2 == 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<uint4*>(s_w + i * kW8TilePitch + sub * kW8RowPitch + j * 16) = wb[u][i];
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const uint2 w = *reinterpret_cast<const uint2*>(s_w + a_off + s * 32);
                    half2_t h0, h1, h2, h3;
                    cast4(w.x, h0, h1);
                    cast4(w.y, h2, h3);
                    const v8h a = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
                    acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(v8h, xb[0][s]),
                                                                    acc[0], 0, 0, 0);
                }
            } else {
                // regroup in two halves (tiles 0-3: rows 0-7, tiles 4-7: rows 8-15); a
                // lane reads its row's operands in its half, the wave's own LDS writes
                // and reads in program order
                uint2 wa[16];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *reinterpret_cast<uint4*>(s_w + i * kW8TilePitch + sub * kW8RowPitch + j * 16) =
                            wb[u][4 * h + i];
                    if ((r >> 3) == h) {
#pragma unroll
                        for (int s = 0; s < 16; ++s)
                            wa[s] = *reinterpret_cast<const uint2*>(s_w + a_off + s * 32);
                    }
                }
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    half2_t h0, h1, h2, h3;
                    cast4(wa[s].x, h0, h1);
                    cast4(wa[s].y, h2, h3);
                    const v8h a = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
#pragma unroll
                    for (int bl = 0; bl < MB2; ++bl)
                        acc[bl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(v8h, xb[bl][s]),
                                                                         acc[bl], 0, 0, 0);
                }
            }
            // lane (g, r) holds D[n = 4 g + i][m = r] of block u
#pragma unroll
            for (int bl = 0; bl < MB2; ++bl) {
                float* dst = s_part + bl * bpart + ((wave * p.nbmax + u) * 16 + r) * 17 + 4 * g;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[i] = acc[bl][i];
            }
        }
    }
#undef QW_LOADU8
    __syncthreads();

    // outputs (m, nn), independent across threads: the CG partials in step order,
    // times the row scale, rounded to f16
    const int nout = M * nrows;
    for (int e = tid; e < nout; e += nthreads) {
        const int m = e / nrows, nn = e - m * nrows;
        const float* src = s_part + (m >> 4) * bpart + ((nn >> 4) * 16 + (m & 15)) * 17 + (nn & 15);
        float pv[kW8BalMaxSteps];
#pragma unroll
        for (int c = 0; c < kW8BalMaxSteps; ++c)
            pv[c] = c < CG ? src[c * p.nbmax * 16 * 17] : 0.0f;
        float v = pv[0];
#pragma unroll
        for (int c = 1; c < kW8BalMaxSteps; ++c)
            if (c < CG)
                v += pv[c];
        p.Y[(size_t)(m0 + m) * p.N + n0 + nn] = __half_as_ushort(__float2half_rn(v * s_sc[nn]));
    }
}

template <int NW, int MB, int NBW>
size_t lds_w4() { return (size_t)2 * MB * 8 * 1024 + (size_t)NW * 4 * NBW * kW4TilePitch; }

template <int NW, int MB, int NBW>
size_t lds_w8() { return (size_t)2 * MB * 16 * kXRowPitch + (size_t)NW * 8 * NBW * kW8TilePitch; }

// Dynamic LDS above 64 KB has to be allowed per kernel (gfx950 has 160 KB per CU).
hipError_t allow_lds(const void* kernel, size_t bytes)
{
    return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int NW, int MB, int NBW>
hipError_t go_w4(const MfmaW4A8Args& p, hipStream_t st)
{
    // once per kernel, before its first launch
    static const hipError_t e =
        allow_lds(reinterpret_cast<const void*>(k_gemm_w4a8<NW, MB, NBW>), lds_w4<NW, MB, NBW>());
    if (e != hipSuccess)
        return e;
    const int64_t nblocks = ((int64_t)p.nrg + NW * 4 * NBW - 1) / (NW * 4 * NBW);
    if (nblocks * p.mgroups > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_gemm_w4a8<NW, MB, NBW>), dim3((unsigned)(nblocks * p.mgroups)),
                       dim3(64 * NW), (lds_w4<NW, MB, NBW>()), st, p);
    return hipGetLastError();
}

template <int NW, int U, int FR>
hipError_t go_w4_bal_u(const MfmaW4A8Args& p, int nwg, size_t lds, hipStream_t st)
{
    // once per kernel, before its first launch
    static const hipError_t e = allow_lds(reinterpret_cast<const void*>(k_gemm_w4a8_bal<NW, U, FR>),
                                          (size_t)kXAllMaxBytes + (size_t)NW * 4 * kW4TilePitch +
                                              (size_t)kBalMaxBlocks * (16 * kBalSumPitch + 16) * 4 + 64 + 4 * NW * kFqRows);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((k_gemm_w4a8_bal<NW, U, FR>), dim3((unsigned)nwg, (unsigned)p.mbtot),
                       dim3(64 * NW), lds, st, p);
    return hipGetLastError();
}

// Units per wave the balanced kernel is built for.
constexpr int kBalMaxUnits = 16;

template <int NW, int FR = 0>
hipError_t go_w4_bal(MfmaW4A8Args p, int cus, hipStream_t st)
{
    if ((size_t)p.cg * 8 * 1024 > (size_t)kXAllMaxBytes || p.mbtot > 65535)
        return hipErrorInvalidValue;
    if (FR > 0 && (p.M > FR || p.K > 4096 || p.X == nullptr))
        return hipErrorInvalidValue;
    // one workgroup per CU with at least four row groups each; more workgroups when a
    // wave would take more than kBalMaxUnits units or the totals more than
    // kBalMaxBlocks blocks
    const int bmax = std::min(kBalMaxBlocks, kBalMaxUnits * NW / p.cg);
    int nwg = std::max(1, std::min(cus, p.nrg / 4));
    nwg = std::max(nwg, (p.nrg + 4 * bmax - 1) / (4 * bmax));
    p.per = p.nrg / nwg;
    p.rem = p.nrg % nwg;
    p.nbmax = (p.per + (p.rem > 0 ? 1 : 0) + 3) / 4;
    p.mgroups = p.mbtot;
    const int umax = (p.nbmax * p.cg + NW - 1) / NW;
    const size_t lds = (size_t)p.cg * 8 * 1024 + (size_t)NW * 4 * kW4TilePitch +
                       (size_t)p.nbmax * (16 * kBalSumPitch + 16) * 4 + 64 + 4 * NW * FR;
    if (umax <= 4)
        return go_w4_bal_u<NW, 4, FR>(p, nwg, lds, st);
    if (umax <= 8)
        return go_w4_bal_u<NW, 8, FR>(p, nwg, lds, st);
    return go_w4_bal_u<NW, 16, FR>(p, nwg, lds, st);
}

template <int U, bool PAIR>
hipError_t go_w4_bals_u(const MfmaW4A8Args& p, int nwg, size_t lds, hipStream_t st)
{
    static const hipError_t e = allow_lds(reinterpret_cast<const void*>(k_gemm_w4a8_bals<U, PAIR>),
                                          (size_t)96 * 1024);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((k_gemm_w4a8_bals<U, PAIR>), dim3((unsigned)nwg), dim3(64 * p.cg), lds, st, p);
    return hipGetLastError();
}

hipError_t go_w4_bals(MfmaW4A8Args p, int cus, hipStream_t st)
{
    // blocks after the first two at a time from three blocks of X on (measured on
    // 4096 -> 27392: 88.8 against 104.6 us at 512 rows, 33.9 against 37.6 at 128;
    // with two blocks the pair would be half empty: 18.9 against 18.0 us at 17 rows)
    const bool pair = p.mbtot >= 3;
    if (p.cg > 8 || p.M > kBalsMaxRows)
        return hipErrorInvalidValue;
    // one workgroup per CU, at least four row groups and at most 8 output blocks each
    int nwg = std::max(1, std::min(cus, p.nrg / 4));
    nwg = std::max(nwg, (p.nrg + 31) / 32);
    p.per = p.nrg / nwg;
    p.rem = p.nrg % nwg;
    p.nbmax = (p.per + (p.rem > 0 ? 1 : 0) + 3) / 4;
    p.mgroups = 1;
    // the LDS it needs, padded so that one workgroup fills a CU
    const size_t need = (size_t)8 * 4 * kW4TilePitch + (size_t)4 * p.nbmax * 16 * kBalSumPitch * 4 +
                        (size_t)(16 * p.nbmax + 64) * 4;
    const size_t lds = std::max(need, (size_t)82 * 1024);
    if (pair)
        return p.nbmax <= 4 ? go_w4_bals_u<4, true>(p, nwg, lds, st) : go_w4_bals_u<8, true>(p, nwg, lds, st);
    return p.nbmax <= 4 ? go_w4_bals_u<4, false>(p, nwg, lds, st) : go_w4_bals_u<8, false>(p, nwg, lds, st);
}

template <int NW, int MB, int NBW>
hipError_t go_w8(const MfmaW8A16Args& p, hipStream_t st)
{
    static const hipError_t e =
        allow_lds(reinterpret_cast<const void*>(k_gemm_w8a16<NW, MB, NBW>), lds_w8<NW, MB, NBW>());
    if (e != hipSuccess)
        return e;
    const int64_t nblocks = ((int64_t)p.nrg + NW * 8 * NBW - 1) / (NW * 8 * NBW);
    if (nblocks * p.mgroups > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_gemm_w8a16<NW, MB, NBW>), dim3((unsigned)(nblocks * p.mgroups)),
                       dim3(64 * NW), (lds_w8<NW, MB, NBW>()), st, p);
    return hipGetLastError();
}

template <int U, int MB2>
hipError_t go_w8_bal_u(const MfmaW8A16Args& p, int nwg, size_t lds, hipStream_t st)
{
    static const hipError_t e = allow_lds(reinterpret_cast<const void*>(k_gemm_w8a16_bal<U, MB2>), kLdsBytes);
    if (e != hipSuccess)
        return e;
    const int mrows = ((p.M + 15) / 16 + MB2 - 1) / MB2;  // workgroup rows along M
    hipLaunchKernelGGL((k_gemm_w8a16_bal<U, MB2>), dim3((unsigned)nwg, (unsigned)mrows), dim3(64 * p.cg),
                       lds, st, p);
    return hipGetLastError();
}

// mb2: blocks of 16 rows of X per workgroup (1: M <= 16; 2: any M, workgroup rows of 32)
hipError_t go_w8_bal(MfmaW8A16Args p, int cus, int mb2, hipStream_t st)
{
    if (p.cg > kW8BalMaxSteps || (mb2 == 1 && p.M > 16) || p.M > 1024)
        return hipErrorInvalidValue;
    // one workgroup per CU and row of X blocks with at least one block (8 row groups of
    // 2 rows) each, at most kW8BalMaxBlocks blocks
    // 2 rows of X blocks: blocks per workgroup as many as the partials leave room for
    // in LDS (7 at 8 steps)
    const size_t fixed = (size_t)kW8BalMaxSteps * (mb2 == 2 ? 4 : 8) * kW8TilePitch;
    const int bmax = std::min<int>(kW8BalMaxBlocks,
                                   (int)((kLdsBytes - fixed) / ((size_t)mb2 * p.cg * 16 * 17 * 4 + 16 * 4)));
    int nwg = std::max(1, std::min(cus, p.nrg / 8));
    nwg = std::max(nwg, (p.nrg + 8 * bmax - 1) / (8 * bmax));
    p.per = p.nrg / nwg;
    p.rem = p.nrg % nwg;
    p.nbmax = (p.per + (p.rem > 0 ? 1 : 0) + 7) / 8;
    p.mgroups = 1;
    const size_t lds = fixed + (size_t)mb2 * p.cg * p.nbmax * 16 * 17 * 4 + (size_t)16 * p.nbmax * 4;
    if (mb2 == 2)
        return p.nbmax <= 4 ? go_w8_bal_u<4, 2>(p, nwg, lds, st) : go_w8_bal_u<8, 2>(p, nwg, lds, st);
    if (p.nbmax <= 4)
        return go_w8_bal_u<4, 1>(p, nwg, lds, st);
    return go_w8_bal_u<8, 1>(p, nwg, lds, st);
}

}  // namespace

bool mfma_shape_ok(int bits, int nw, int mb, int nbw)
{
    if (nw != 4 && nw != 8)
        return false;
    if (nbw != 1 && nbw != 2)
        return false;
    if (bits == 4)
        return ((mb == 1 || mb == 2 || mb == 4) && !(nw == 4 && mb == 4 && nbw == 2) &&
                !(nw == 8 && mb == 1 && nbw == 2)) ||
               (mb == 0 && (nbw == 1 || nw == 8));
    // W8A16 X slices are 16 KB per block of 16 rows; eight waves of two blocks of
    // rows would not fit the registers.  mb 0: the balanced kernel (one wave per 512-k
    // step), nw 8, with nbw 1 (up to 16 rows) or 2 (two blocks of X per workgroup)
    return ((mb == 1 || mb == 2) && !(nw == 8 && nbw == 2)) || (mb == 0 && nw == 8);
}

void mfma_default_shape(int bits, int64_t M, int64_t K, int* nw, int* mb, int* nbw)
{
    // measured on MI355X: W4A8 with K <= 4096 and up to 16 rows on the balanced kernel,
    // 17 to 1024 rows on the one with one wave per step and the weights held in
    // registers (on 4096 -> 27392: 25.4 against 25.8 us for the streaming kernel at 64
    // rows, 39.0 against 44.2 at 128, 114.5 against 138.0 at 512); else the streaming
    // kernel with 8 waves and 2 or 4 blocks of X.  W8A16 with K <= 4096: the balanced
    // kernel up to 16 rows, its two-block form for 17 to 64 (25.3 against 31.0 us for
    // the streaming kernel at 17 rows, 28.6 against 32.3 at 32, 41.9 against 49.6 at 64
    // on 3584 -> 18944); else 8 waves with 1 or 2 blocks.  K > 4096 (the long-K GEMV
    // kernels take up to 16 rows): each workgroup walks all of K, so more, smaller
    // workgroups win up to 128 rows: 4 waves with one block of X (18944 -> 3584 at 32
    // rows: W4A8 39.0 against 54.6 us with 8 waves and 2 blocks, W8A16 59.9 against
    // 106.0; at 128 rows W4A8 50.4 against 78.3), W8A16 from 65 to 128 rows with 2 blocks
    // (77.3 against 105.8); beyond, the 8-wave shapes (512 rows: W4A8 90.8 us with 4
    // blocks against 147.2 with 4 waves of one).
    const int64_t mbtot = (M + 15) / 16;
    if (K > 4096 && M <= 128) {
        *nw = 4;
        *nbw = 1;
        *mb = bits == 8 && M > 64 ? 2 : 1;
        return;
    }
    const bool k_fits = (K + 511) / 512 * 8192 <= kXAllMaxBytes;
    *nw = 8;
    *nbw = 1;
    if (bits == 4) {
        if (mbtot == 1 && k_fits) {
            *mb = 0;
        } else if (k_fits && M <= kBalsMaxRows) {
            *mb = 0;
            *nbw = 2;
        } else {
            *mb = mbtot >= 4 ? 4 : (mbtot >= 2 ? 2 : 1);
        }
    } else if (mbtot <= 4 && (K + 511) / 512 <= 8) {
        *mb = 0;
        *nbw = mbtot == 1 ? 1 : 2;
    } else {
        *mb = mbtot >= 2 ? 2 : 1;
    }
}

size_t mfma_w4a8_workspace_bytes(int64_t M, int64_t K)
{
    const size_t mbtot = (size_t)((M + 15) / 16), ks = (size_t)((K + 63) / 64);
    const size_t xp = (mbtot * ks * 1024u + 255u) & ~(size_t)255u;
    return xp + (((size_t)M * 4u + 255u) & ~(size_t)255u);
}

hipError_t launch_gemm_w4a8(const float* X, int M, int N, int K, const uint8_t* Wq,
                            const float* w_scale, float* Y, void* workspace, int nw, int mb,
                            int nbw, int cus, hipStream_t st)
{
    const TileLayout L = tile_layout(4, N, K);
    const int mbtot = (M + 15) / 16, ks = (K + 63) / 64;
    uint8_t* xp = static_cast<uint8_t*>(workspace);
    const size_t xp_bytes = ((size_t)mbtot * ks * 1024u + 255u) & ~(size_t)255u;
    float* a = reinterpret_cast<float*>(xp + xp_bytes);
    MfmaW4A8Args p;
    p.X = X;
    p.Xp = xp;
    p.a_scale = a;
    p.Wq = Wq;
    p.w_scale = w_scale;
    p.Y = Y;
    p.M = M;
    p.N = N;
    p.K = K;
    p.cg = L.cg;
    p.nrg = L.nrg;
    p.ks = ks;
    p.mbtot = mbtot;
    // up to 4 rows on the 8-wave balanced kernel: it quantizes X itself, no pre-pass
    // launch (4096 -> 27392: 11.8 / 12.3 / 12.7 us at 2 / 3 / 4 rows against 14.5-14.8
    // with the pre-pass, which took 4.3 us of them; 8 rows in the prologue measured
    // slower than the pre-pass)
    if (mb == 0 && nbw != 2 && nw == 8 && M <= kFqRows && K <= 4096)
        return M <= 2 ? go_w4_bal<8, 2>(p, cus, st) : go_w4_bal<8, 4>(p, cus, st);
    const int qgrid = mbtot * 16 < 65536 ? mbtot * 16 : 65536;
    const int ns = (ks * 4 + kBlock - 1) / kBlock;  // 16-code slots per thread of 256
    const int ns_wide = (ks * 4 + 1023) / 1024;      // ... of 1024 (at most 4: K <= 65536)
    if (ns <= 1)
        hipLaunchKernelGGL((k_quant_act_mfma<1, kBlock>), dim3(qgrid), dim3(kBlock), 0, st, X, M, K,
                           mbtot * 16, ks, xp, a);
    else if (ns <= 2)
        hipLaunchKernelGGL((k_quant_act_mfma<2, kBlock>), dim3(qgrid), dim3(kBlock), 0, st, X, M, K,
                           mbtot * 16, ks, xp, a);
    else if (ns <= 4)
        hipLaunchKernelGGL((k_quant_act_mfma<4, kBlock>), dim3(qgrid), dim3(kBlock), 0, st, X, M, K,
                           mbtot * 16, ks, xp, a);
    else if (ns_wide <= 2)
        hipLaunchKernelGGL((k_quant_act_mfma<2, 1024>), dim3(qgrid), dim3(1024), 0, st, X, M, K,
                           mbtot * 16, ks, xp, a);
    else if (ns_wide <= 4)
        hipLaunchKernelGGL((k_quant_act_mfma<4, 1024>), dim3(qgrid), dim3(1024), 0, st, X, M, K,
                           mbtot * 16, ks, xp, a);
    else
        return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (mb == 0) {  // balanced: one workgroup per CU, X codes of one block resident in LDS
        if (nbw == 2)  // one wave per 512-k step, weights held in registers across the blocks
            return nw == 8 ? go_w4_bals(p, cus, st) : hipErrorInvalidValue;
        if (nw == 8)
            return go_w4_bal<8>(p, cus, st);
        if (nw == 4)
            return go_w4_bal<4>(p, cus, st);
        return hipErrorInvalidValue;
    }
    p.mgroups = (mbtot + mb - 1) / mb;
#define QW_GO(NW_, MB_, NBW_)                                                                    \
    if (nw == NW_ && mb == MB_ && nbw == NBW_)                                                   \
        return go_w4<NW_, MB_, NBW_>(p, st);
    QW_GO(4, 1, 1) QW_GO(4, 2, 1) QW_GO(4, 4, 1) QW_GO(4, 1, 2) QW_GO(4, 2, 2)
    QW_GO(8, 1, 1) QW_GO(8, 2, 1) QW_GO(8, 4, 1) QW_GO(8, 2, 2) QW_GO(8, 4, 2)
#undef QW_GO
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_w8a16(const uint16_t* X, int M, int N, int K, const uint8_t* Wq,
                             const uint16_t* w_scale, uint16_t* Y, int nw, int mb, int nbw,
                             int cus, hipStream_t st)
{
    const TileLayout L = tile_layout(8, N, K);
    const int mbtot = (M + 15) / 16;
    MfmaW8A16Args p;
    p.X = X;
    p.Wq = Wq;
    p.w_scale = w_scale;
    p.Y = Y;
    p.M = M;
    p.N = N;
    p.K = K;
    p.cg = L.cg;
    p.nrg = L.nrg;
    if (mb == 0)  // balanced: nbw 1 one block of X per workgroup, nbw 2 two
        return nw == 8 ? go_w8_bal(p, cus, nbw, st) : hipErrorInvalidValue;
    p.mgroups = (mbtot + mb - 1) / mb;
#define QW_GO(NW_, MB_, NBW_)                                                                    \
    if (nw == NW_ && mb == MB_ && nbw == NBW_)                                                   \
        return go_w8<NW_, MB_, NBW_>(p, st);
    QW_GO(4, 1, 1) QW_GO(4, 2, 1) QW_GO(4, 1, 2) QW_GO(4, 2, 2)
    QW_GO(8, 1, 1) QW_GO(8, 2, 1)
#undef QW_GO
    return hipErrorInvalidValue;
}

}  // namespace qw
