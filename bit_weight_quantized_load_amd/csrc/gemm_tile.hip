// Tiled matrix-core GEMM for the weight-quantized linear with many rows of X (the top of
// the skinny-GEMM sweep), where the problem is a dense contraction: 2 M N K operations
// against N K weight bytes.
//
// W8A16 (ChatGLM2-6B W8A16 write-up, section 4: load the INT8 weights, cast them to F16,
// multiply by the per-channel scale, multiply with the F16 activation):
//   Y[m][n] = f16(s16[n] * sum_k q[n][k] x[m][k]), the sum in fp32 on
//   v_mfma_f32_32x32x16_f16; the per-channel scale factors out of the sum and is applied
//   once to it.
// W4A8 ("Jetson Orin AGX 上的 INT4 量化推理实践", sections 当前实现方式 and 正确方向:
// INT4 weights, dynamic INT8 activations, int8 dot products into int32, output
// acc * weight scale * activation scale):
//   Y[m][n] = ((float)acc * w_scale[n]) * a_scale[m], acc = sum_k q[n][k] xq[m][k] in
//   int32 on v_mfma_i32_32x32x32_i8, with xq and a_scale computed by a pre-pass into
//   the workspace (the codes of quant_act_i8).  An INT4 weight enters the multiply as
//   16 q (its nibble moved to the top of an int8 lane), so the sum is exactly 16 acc and
//   acc = sum >> 4; the outputs equal every other W4A8 path's bit for bit.
//
// Work split.  A workgroup owns an output tile of BN rows of W (n) by BM rows of X (m)
// and walks K in stages (64 k for W8A16, 128 k for W4A8: 128 bytes of operand per row).
// Its NWN x NWM waves each own WN x WM of the tile, (WN / 32) x (WM / 32) blocks of
// 32 x 32 accumulators.  Each stage, the workgroup's threads load the stage's weights
// (16-byte loads from the tile layout, in which a row's k are contiguous) and its rows
// of X, widen the weights (INT8 -> f16 by the exact byte-permute cast: bytes q ^ 0x80
// under a 0x64 byte read as 1024 + q + 128, minus 1152; INT4 -> int8 lanes of 16 q)
// and store both in LDS, so each weight is widened once per workgroup and multiplied
// against all BM rows of X.  LDS holds two stages; the global loads run two stages
// ahead (two register sets), so a stage's memory latency overlaps two stages of
// multiplies.  Loads past K, N or M read zeros (buffer loads out of range), which
// keeps the loop free of branches around the loads.
//
// LDS layout: rows of 128 bytes (eight 16-byte chunks), chunk c of row r at position
// c ^ ((r / 2) % 8).  The LDS serves 16 lanes of a 16-byte access per cycle across 64
// banks (256 bytes, two rows): an operand read (rows r..r+15 at one chunk) and a staging
// write (two rows, or four rows at four chunks) each land on 16 distinct 16-byte slots
// of that width.  (With chunk c at c ^ (r % 8), rows r and r + 8 met in one bank: the
// bank-conflict counter read 1.36 conflict cycles per LDS-active cycle.)
//
// W4A8 operand order: a 16-byte group of 16 k holds them in the order the INT4 unpack
// produces (k 0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15); the X codes are
// permuted the same way when staged, and the int32 dot over the group is unchanged.
//
// Epilogue: the multiplies take X as the A operand and the weights as B, so each
// accumulator register holds one row of Y across 32 consecutive output columns and the
// stores of a half-wave are contiguous (with the operands the other way round each
// store scattered over 32 rows, and HBM write traffic was 2-3x the output).
//
// Grid: one workgroup per tile, numbered so that the tiles of X that share a block of
// weights are neighbours on one XCD (dispatched together, the repeated weight reads
// meet in that XCD's L2).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kRowB = 128;  // LDS bytes per row of a stage

// int8 x 4 -> f16 x 4, exact.
__device__ __forceinline__ uint2 cast4_f16(uint32_t wd)
{
    const uint32_t u = wd ^ 0x80808080u;
    const uint32_t l = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t h = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    const half2_t off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const half2_t lo = __builtin_bit_cast(half2_t, l) + off;
    const half2_t hi = __builtin_bit_cast(half2_t, h) + off;
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// 16 int8 codes in k order -> the INT4 unpack order (even k of each 8, then odd k).
__device__ __forceinline__ uint4 perm16(uint4 x)
{
    // bytes of (hi:lo) = (x.y:x.x): selector byte i picks byte i (0..3 of x.x, 4..7 of x.y)
    return make_uint4(__builtin_amdgcn_perm(x.y, x.x, 0x06040200u),
                      __builtin_amdgcn_perm(x.y, x.x, 0x07050301u),
                      __builtin_amdgcn_perm(x.w, x.z, 0x06040200u),
                      __builtin_amdgcn_perm(x.w, x.z, 0x07050301u));
}

__device__ __forceinline__ int swz(int r, int c) { return r * kRowB + 16 * (c ^ ((r >> 1) & 7)); }

// Narrow weight rows: 64 bytes, eight 8-byte units, unit u of row r at position
// u ^ ((r / 4) % 8).  An operand read (8 bytes per lane, rows r..r+31 at one unit) puts
// the eight rows that share a quarter of the 64 banks (rows r + 4t) on eight distinct
// positions.
__device__ __forceinline__ int swz_n(int r, int u) { return r * 64 + 8 * (u ^ ((r >> 2) & 7)); }

// 8 bytes of narrow weights (one MFMA operand per lane) -> the wide operand: 8 f16
// (INT8) or 16 int8 lanes of 16 q in the unpack order (INT4).
template <int BITS>
__device__ __forceinline__ uint4 widen8(uint2 w)
{
    if constexpr (BITS == 8) {
        const uint2 a = cast4_f16(w.x), b = cast4_f16(w.y);
        return make_uint4(a.x, a.y, b.x, b.y);
    } else {
        return make_uint4((w.x << 4) & 0xF0F0F0F0u, w.x & 0xF0F0F0F0u, (w.y << 4) & 0xF0F0F0F0u,
                          w.y & 0xF0F0F0F0u);
    }
}

// Buffer resource from values that are uniform but may have been computed in vector
// registers (a clamp becomes v_med3): taken through readfirstlane so that the resource
// stays in scalar registers and each buffer load is a single instruction.
__device__ __forceinline__ rsrc_t make_rsrc_u(const void* base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                     __builtin_amdgcn_readfirstlane(bytes));
}

// NARROW: the weights stay in LDS as stored in memory (INT8 or packed INT4, 64 bytes
// per row per stage in both cases: 64 k of INT8, 128 k of INT4) and each wave widens
// the operands it reads; otherwise they are widened once when staged (128 bytes per
// row).  Narrow weights halve the weight bytes written to and read from LDS, the
// bound of the many-row case, at the price of widening each operand in every wave
// that reads it.
template <int BITS, int WN, int WM, int NWN, int NWM, bool NARROW = false>
struct TileCfg {
    static constexpr int NWN_ = NWN, NWM_ = NWM;
    static constexpr bool NARROW_ = NARROW;
    static constexpr int T = 64 * NWN * NWM;
    static constexpr int BN = WN * NWN, BM = WM * NWM;
    static constexpr int BK = BITS == 8 ? 64 : 128;  // k per stage
    static constexpr int IN = WN / 32, JM = WM / 32;
    static constexpr int PW = BN * 4 / T;  // 16-byte weight loads per thread (64 B per row)
    static constexpr int PX = BM * 8 / T;  // 16-byte X loads per thread (128 B per row)
    static constexpr int WREG = BN * (NARROW ? 64 : kRowB);
    static constexpr int STAGE = WREG + BM * kRowB;
    static_assert(PW >= 1 && PX >= 1 && BN * 4 % T == 0 && BM * 8 % T == 0, "whole loads");
};

template <int PW, int PX>
struct TileRegs {
    uint4 w[PW], x[PX];
};

// Stage s of the workgroup's weights and rows of X into r; a stage past the last reads
// zeros (offsets out of range).  The buffer resources are passed by value: they are
// uniform, and the loads stay single scalar-addressed buffer loads.
template <class C, int BITS>
__device__ __forceinline__ void tile_gload(rsrc_t wr, rsrc_t xr, int s, int stages, int CG, int xrow,
                                           int tid, TileRegs<C::PW, C::PX>& r)
{
    constexpr int R = BITS == 8 ? 2 : 4;  // rows per tile of the weight layout
    const bool live = s < stages;
    const int k0 = s * C::BK;
#pragma unroll
    for (int q = 0; q < C::PW; ++q) {
        const int i = tid + C::T * q, row = i >> 2, j = i & 3;
        const uint32_t off = (uint32_t)(((row / R) * CG + (k0 >> 9)) * 1024 + (row % R) * (1024 / R) +
                                        (k0 & 511) * BITS / 8 + 16 * j);
        r.w[q] = load16_stream(wr, live ? off : 0x80000000u);
    }
#pragma unroll
    for (int q = 0; q < C::PX; ++q) {
        const int i = tid + C::T * q, row = i >> 3, c = i & 7;
        const uint32_t off = (uint32_t)row * (uint32_t)xrow + (uint32_t)(k0 * (BITS == 8 ? 2 : 1) + 16 * c);
        r.x[q] = load16(xr, live ? off : 0x80000000u);
    }
}

// Widens piece q (q < PW: 16 bytes of weights; else 16 bytes of X) of register set r
// and stores it in LDS buffer wl.
template <class C, int BITS>
__device__ __forceinline__ void tile_lstore_piece(uint8_t* wl, int tid, const TileRegs<C::PW, C::PX>& r,
                                                  int q)
{
    if (q < C::PW && C::NARROW_) {
        // 16 bytes = units 2j and 2j + 1 of the row, stored as they are
        const int i = tid + C::T * q, row = i >> 2, j = i & 3;
        *reinterpret_cast<uint2*>(wl + swz_n(row, 2 * j)) = make_uint2(r.w[q].x, r.w[q].y);
        *reinterpret_cast<uint2*>(wl + swz_n(row, 2 * j + 1)) = make_uint2(r.w[q].z, r.w[q].w);
    } else if (q < C::PW) {
        const int i = tid + C::T * q, row = i >> 2, j = i & 3;
        uint4 lo, hi;
        if constexpr (BITS == 8) {
            const uint2 a = cast4_f16(r.w[q].x), b = cast4_f16(r.w[q].y);
            const uint2 c = cast4_f16(r.w[q].z), d = cast4_f16(r.w[q].w);
            lo = make_uint4(a.x, a.y, b.x, b.y);
            hi = make_uint4(c.x, c.y, d.x, d.y);
        } else {
            // 32 nibbles (k 32j .. 32j + 31) -> 32 int8 lanes of 16 q, unpack order
            const uint32_t wd[4] = {r.w[q].x, r.w[q].y, r.w[q].z, r.w[q].w};
            lo = make_uint4((wd[0] << 4) & 0xF0F0F0F0u, wd[0] & 0xF0F0F0F0u,
                            (wd[1] << 4) & 0xF0F0F0F0u, wd[1] & 0xF0F0F0F0u);
            hi = make_uint4((wd[2] << 4) & 0xF0F0F0F0u, wd[2] & 0xF0F0F0F0u,
                            (wd[3] << 4) & 0xF0F0F0F0u, wd[3] & 0xF0F0F0F0u);
        }
        *reinterpret_cast<uint4*>(wl + swz(row, 2 * j)) = lo;
        *reinterpret_cast<uint4*>(wl + swz(row, 2 * j + 1)) = hi;
    } else {
        const int qx = q - C::PW;
        const int i = tid + C::T * qx, row = i >> 3, c = i & 7;
        *reinterpret_cast<uint4*>(wl + C::WREG + swz(row, c)) = BITS == 8 ? r.x[qx] : perm16(r.x[qx]);
    }
}

template <class C, int BITS>
__device__ __forceinline__ void tile_lstore(uint8_t* wl, int tid, const TileRegs<C::PW, C::PX>& r)
{
#pragma unroll
    for (int q = 0; q < C::PW + C::PX; ++q)
        tile_lstore_piece<C, BITS>(wl, tid, r, q);
}

// The multiplies of one stage from LDS buffer wl; the staging of the next stage into
// buffer nl (from register set r) is spread over the four 16/32-k steps, after each
// step's multiplies are issued: the MFMAs run asynchronously, so the cast and the LDS
// stores issue while they execute instead of after them.
template <class C, int BITS, class A>
__device__ __forceinline__ void tile_compute(const uint8_t* wl, uint8_t* nl, int tid, int wn, int wm,
                                             int rl, int half, const TileRegs<C::PW, C::PX>& r,
                                             A (&acc)[C::IN][C::JM])
{
    const uint8_t* xl = wl + C::WREG;
    constexpr int WN = C::BN / C::NWN_, WM = C::BM / C::NWM_;
    constexpr int NP = C::PW + C::PX;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int c = 2 * kk + half;
        uint4 a[C::IN], b[C::JM];
#pragma unroll
        for (int i = 0; i < C::IN; ++i) {
            if constexpr (C::NARROW_)
                a[i] = widen8<BITS>(*reinterpret_cast<const uint2*>(wl + swz_n(wn * WN + 32 * i + rl, c)));
            else
                a[i] = *reinterpret_cast<const uint4*>(wl + swz(wn * WN + 32 * i + rl, c));
        }
#pragma unroll
        for (int j = 0; j < C::JM; ++j)
            b[j] = *reinterpret_cast<const uint4*>(xl + swz(wm * WM + 32 * j + rl, c));
#pragma unroll
        for (int i = 0; i < C::IN; ++i)
#pragma unroll
            for (int j = 0; j < C::JM; ++j) {
                // X is the A operand and the weights the B operand, so the result is Y
                // itself (rows m, columns n) and a store instruction covers 32
                // consecutive n of one row
                if constexpr (BITS == 8)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(v8h, b[j]), __builtin_bit_cast(v8h, a[i]), acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        __builtin_bit_cast(v4i, b[j]), __builtin_bit_cast(v4i, a[i]), acc[i][j], 0, 0, 0);
            }
#pragma unroll
        for (int q = kk * NP / 4; q < (kk + 1) * NP / 4; ++q)
            tile_lstore_piece<C, BITS>(nl, tid, r, q);
    }
}

template <int BITS, int WN, int WM, int NWN, int NWM, int DEPTH, bool NARROW>
__global__ __launch_bounds__(64 * NWN * NWM, 1) void k_gemm_tile(TileGemmArgs p)
{
    using C = TileCfg<BITS, WN, WM, NWN, NWM, NARROW>;
    constexpr int BN = C::BN, BM = C::BM, BK = C::BK, IN = C::IN, JM = C::JM;
    constexpr int STAGE = C::STAGE;
    constexpr int R = BITS == 8 ? 2 : 4;  // rows per tile of the weight layout
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % NWN, wm = wave / NWN;
    const int L = xcd_block(blockIdx.x, gridDim.x);
    const int nb = L / p.mblocks, mb = L - nb * p.mblocks;
    const int n0 = nb * BN, m0 = mb * BM;
    const int M = p.M, N = p.N, K = p.K, CG = p.cg;
    const int stages = (K + BK - 1) / BK;
    const int xrow = BITS == 8 ? K * 2 : K;  // bytes per row of X

    const int rg0 = n0 / R;
    const rsrc_t wr = make_rsrc_u(p.Wq + (size_t)rg0 * CG * 1024u,
                                (uint32_t)max(0, min(BN / R, p.nrg - rg0)) * (uint32_t)CG * 1024u);
    const rsrc_t xr = make_rsrc_u(static_cast<const uint8_t*>(p.X) + (size_t)m0 * xrow,
                                (uint32_t)max(0, min(BM, M - m0)) * (uint32_t)xrow);
    using Regs = TileRegs<C::PW, C::PX>;

    typedef typename std::conditional<BITS == 8, v16f, v16i>::type acc_t;
    acc_t acc[IN][JM];
#pragma unroll
    for (int i = 0; i < IN; ++i)
#pragma unroll
        for (int j = 0; j < JM; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0;

    const int rl = lane & 31, half = lane >> 5;
    // DEPTH register sets: at stage t, set t % DEPTH (stored to LDS during stage t - 1)
    // takes the loads of stage t + DEPTH, and set (t + 1) % DEPTH, loaded DEPTH - 1 stages
    // earlier, is staged into the other LDS buffer while stage t is multiplied.  The loop
    // is unrolled DEPTH times so that buffers and register sets are static; stages past
    // the last read zeros and add nothing.
    Regs r[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        tile_gload<C, BITS>(wr, xr, d, stages, CG, xrow, tid, r[d]);
    tile_lstore<C, BITS>(lds, tid, r[0]);
    for (int s = 0; s < stages; s += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            __syncthreads();  // stage s + d in buffer d % 2; every wave is done with the other
            tile_gload<C, BITS>(wr, xr, s + d + DEPTH, stages, CG, xrow, tid, r[d]);
            __builtin_amdgcn_sched_barrier(0);
            tile_compute<C, BITS>(lds + (d & 1) * STAGE, lds + ((d + 1) & 1) * STAGE, tid, wn, wm, rl,
                                  half, r[(d + 1) % DEPTH], acc);
        }
    }

    // Epilogue: lane (rl, half) of block (i, j) holds rows m = 8 g + 4 half + e of X's
    // block j (g, e = 0..3: register 4 g + e) and column n = rl of W's block i; the 32
    // lanes of a half-wave store 32 consecutive n of one row.
    const rsrc_t sr = make_rsrc_u(p.w_scale, (uint32_t)N * (BITS == 8 ? 2u : 4u));
    const rsrc_t ar = make_rsrc_u(p.a_scale, BITS == 4 ? (uint32_t)M * 4u : 0u);
#pragma unroll
    for (int i = 0; i < IN; ++i) {
        const int n = n0 + wn * WN + 32 * i + rl;
        const float sc = BITS == 8 ? __half2float(__ushort_as_half(load2(sr, (uint32_t)n * 2u)))
                                   : __uint_as_float(load4(sr, (uint32_t)n * 4u));
        if (n >= N)
            continue;
#pragma unroll
        for (int j = 0; j < JM; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int mb0 = m0 + wm * WM + 32 * j + 8 * g + 4 * half;
                float av[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (BITS == 4) {
                    const float4 a4 = load16f(ar, (uint32_t)mb0 * 4u);
                    av[0] = a4.x;
                    av[1] = a4.y;
                    av[2] = a4.z;
                    av[3] = a4.w;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = mb0 + e;
                    if (m >= M)
                        continue;
                    if constexpr (BITS == 8)
                        static_cast<uint16_t*>(p.Y)[(size_t)m * N + n] =
                            __half_as_ushort(__float2half_rn(sc * acc[i][j][4 * g + e]));
                    else
                        static_cast<float*>(p.Y)[(size_t)m * N + n] =
                            ((float)(acc[i][j][4 * g + e] >> 4) * sc) * av[e];
                }
            }
        }
    }
}

template <int BITS, int WN, int WM, int NWN, int NWM, int DEPTH = 2, bool NARROW = false>
hipError_t go_tile(TileGemmArgs p, hipStream_t st)
{
    using C = TileCfg<BITS, WN, WM, NWN, NWM, NARROW>;
    const size_t lds = (size_t)2 * C::STAGE;
    const void* kern = reinterpret_cast<const void*>(k_gemm_tile<BITS, WN, WM, NWN, NWM, DEPTH, NARROW>);
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    const int64_t nbn = ((int64_t)p.N + C::BN - 1) / C::BN, nbm = ((int64_t)p.M + C::BM - 1) / C::BM;
    if (nbn * nbm > 0x7fffffff)
        return hipErrorInvalidValue;
    p.mblocks = (int)nbm;
    hipLaunchKernelGGL((k_gemm_tile<BITS, WN, WM, NWN, NWM, DEPTH, NARROW>), dim3((unsigned)(nbn * nbm)), dim3(C::T),
                       lds, st, p);
    return hipGetLastError();
}

template <int BITS>
hipError_t go_variant(const TileGemmArgs& p, int variant, hipStream_t st)
{
    switch (variant) {
    case 0: return go_tile<BITS, 64, 64, 2, 2>(p, st);   // 128 n x 128 m, 4 waves
    case 1: return go_tile<BITS, 64, 128, 2, 2>(p, st);  // 128 n x 256 m, 4 waves
    case 2: return go_tile<BITS, 64, 32, 2, 2>(p, st);   // 128 n x 64 m, 4 waves
    case 3: return go_tile<BITS, 32, 32, 2, 2>(p, st);   // 64 n x 64 m, 4 waves
    case 4: return go_tile<BITS, 64, 64, 4, 2>(p, st);   // 256 n x 128 m, 8 waves
    case 5: return go_tile<BITS, 128, 128, 2, 2>(p, st); // 256 n x 256 m, 4 waves
    case 6: return go_tile<BITS, 64, 128, 4, 2>(p, st);  // 256 n x 256 m, 8 waves
    case 7: return go_tile<BITS, 64, 32, 2, 2, 4>(p, st); // variant 2, four stages in flight
    case 8: return go_tile<BITS, 32, 32, 2, 2, 4>(p, st); // variant 3, four stages in flight
    case 9: return go_tile<BITS, 64, 64, 2, 2, 4>(p, st); // variant 0, four stages in flight
    case 10: return go_tile<BITS, 128, 64, 2, 4, 2, true>(p, st);  // 256 x 256, narrow weights
    case 11: return go_tile<BITS, 64, 128, 4, 2, 2, true>(p, st);  // variant 6, narrow weights
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int tile_rows_m(int variant)
{
    switch (variant) {
    case 0: return 128;
    case 1: return 256;
    case 2: return 64;
    case 3: return 64;
    case 4: return 128;
    case 5: return 256;
    case 6: return 256;
    case 7: return 64;
    case 8: return 64;
    case 9: return 128;
    case 10: return 256;
    case 11: return 256;
    default: return 0;
    }
}

int tile_rows_n(int variant)
{
    switch (variant) {
    case 4: case 5: case 6: case 10: case 11: return 256;
    case 3: case 8: return 64;
    default: return 128;
    }
}

hipError_t launch_gemm_w8a16_tile(const uint16_t* X, int M, int N, int K, const uint8_t* Wq,
                                  const uint16_t* w_scale, uint16_t* Y, int variant, hipStream_t st)
{
    const TileLayout L = tile_layout(8, N, K);
    TileGemmArgs p;
    p.X = X;
    p.Wq = Wq;
    p.w_scale = w_scale;
    p.Y = Y;
    p.a_scale = nullptr;
    p.M = M;
    p.N = N;
    p.K = K;
    p.cg = L.cg;
    p.nrg = L.nrg;
    p.mblocks = 0;
    return go_variant<8>(p, variant, st);
}

hipError_t launch_gemm_w4a8_tile(const int8_t* Xq, const float* a_scale, int M, int N, int K,
                                 const uint8_t* Wq, const float* w_scale, float* Y, int variant,
                                 hipStream_t st)
{
    const TileLayout L = tile_layout(4, N, K);
    TileGemmArgs p;
    p.X = Xq;
    p.Wq = Wq;
    p.w_scale = w_scale;
    p.Y = Y;
    p.a_scale = a_scale;
    p.M = M;
    p.N = N;
    p.K = K;
    p.cg = L.cg;
    p.nrg = L.nrg;
    p.mblocks = 0;
    return go_variant<4>(p, variant, st);
}

}  // namespace qw
