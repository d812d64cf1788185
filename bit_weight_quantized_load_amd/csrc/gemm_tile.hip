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
//   the workspace (the codes of quant_act_i8, each 16-byte group in the INT4 unpack
//   order).  An INT4 weight enters the multiply as 16 q (its nibble moved to the top of
//   an int8 lane), so the sum is exactly 16 acc and acc = sum >> 4; the outputs equal
//   every other W4A8 path's bit for bit.
//
// Work split.  A workgroup owns an output tile of BN rows of W (n) by BM rows of X (m)
// and walks K in stages (64 k for W8A16, 128 k for W4A8: 64 bytes of weights and 128
// bytes of X per row).  Its NWN x NWM waves each own WN x WM of the tile, (WN / 32) x
// (WM / 32) blocks of 32 x 32 accumulators; with KS > 1 there are KS such groups of
// waves, each taking part of every stage's k.  Each weight byte is read from memory once
// per grid row of X tiles and multiplied against BM rows of X from LDS.
//
// Multiplies: X is the A operand and the weights the B operand, so each accumulator
// register holds one row of Y across 32 consecutive output columns and the stores of a
// half-wave are contiguous (with the operands the other way round each store scattered
// over 32 rows, and HBM write traffic was 2-3x the output).  The INT8 -> f16 cast is the
// exact byte-permute one (bytes q ^ 0x80 under a 0x64 byte read as 1024 + q + 128, minus
// 1152); the INT4 widening moves each nibble to the top of an int8 lane.
//
// Grid: one workgroup per tile, numbered so that the tiles of X that share a block of
// weights are neighbours on one XCD (dispatched together, the repeated weight reads
// meet in that XCD's L2).
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

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


// 8 bytes of weights as stored (one MFMA operand per lane) -> the operand: 8 f16 (INT8)
// or 16 int8 lanes of 16 q in the unpack order (INT4).
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

// Epilogue: lane (rl, half) of block (i, j) holds rows m = 8 g + 4 half + e of X's block
// j (g, e = 0..3: register 4 g + e) and column n = rl of W's block i; the 32 lanes of a
// half-wave store 32 consecutive n of one row.
template <int BITS, int IN, int JM, int WN, int WM, class A>
__device__ __forceinline__ void tile_epilogue(const TileGemmArgs& p, const A (&acc)[IN][JM], int n0, int m0,
                                              int wn, int wm, int rl, int half)
{
    const int M = p.M, N = p.N;
    const rsrc_t sr = make_rsrc_u(p.w_scale, (uint32_t)N * (BITS == 8 ? 2u : 4u));
    const rsrc_t ar = make_rsrc_u(p.a_scale, BITS == 4 ? (uint32_t)M * 4u : 0u);
    if constexpr (BITS == 8 && IN % 2 == 0) {
        if ((N & 1) == 0) {
            // f16 outputs two columns per lane: lanes 2t and 2t + 1 trade one scaled value,
            // so that lane 2t holds columns 2t, 2t + 1 of block i and lane 2t + 1 those of
            // block i + 1, and a half-wave stores 128 contiguous bytes of a row (one
            // block's 64 would leave the rest of each 128-byte line to another store)
            const bool odd = (rl & 1) != 0;
#pragma unroll
            for (int i = 0; i < IN; i += 2) {
                const int na = n0 + wn * WN + 32 * i + rl;  // this lane's column in block i
                const int nb = na + 32;                     // and in block i + 1
                const float sa = __half2float(__ushort_as_half(load2(sr, (uint32_t)na * 2u)));
                const float sb = __half2float(__ushort_as_half(load2(sr, (uint32_t)nb * 2u)));
                const int nc = odd ? nb - 1 : na;  // first column of the lane's pair (even)
#pragma unroll
                for (int j = 0; j < JM; ++j) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int m = m0 + wm * WM + 32 * j + 8 * (v >> 2) + 4 * half + (v & 3);
                        const float va = sa * acc[i][j][v], vb = sb * acc[i + 1][j][v];
                        const float got = __int_as_float(
                            __builtin_amdgcn_mov_dpp(__float_as_int(odd ? va : vb), 0xB1, 0xF, 0xF, false));
                        const float lo = odd ? got : va, hi = odd ? vb : got;
                        if (m < M && nc < N)  // N even: nc + 1 < N as well
                            *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.Y) + (size_t)m * N + nc) =
                                (uint32_t)__half_as_ushort(__float2half_rn(lo)) |
                                ((uint32_t)__half_as_ushort(__float2half_rn(hi)) << 16);
                    }
                }
            }
            return;
        }
    }
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

// W4A8 epilogue through LDS: the fp32 outputs of one 32 x 32 block go to a 4 KB LDS
// scratch of the wave row by row, and come back as 16 bytes (4 columns) of one row per
// lane, so that each store instruction writes 8 rows x 128 contiguous bytes with 16 bytes
// per lane (storing straight from the accumulators, 4 bytes per lane, took 13.5 of 62
// us at 512 rows on 4096 -> 27392; 16-byte stores of whole 128-byte row runs, 5 us).
// Row r of the block sits at (r / 8) KB + (r % 4) * 256 + ((r / 4) % 2) * 128: the 64
// lanes of a write (rows r and r + 4 of one column range) and the 16 lanes of an LDS read
// cycle (rows r and r + 4) each cover the 64 banks once.  Needs N % 4 == 0 (aligned
// 16-byte runs); scr is private to the wave.
template <int IN, int JM, int WN, int WM, class A>
__device__ __forceinline__ void tile_epilogue_w4_lds(const TileGemmArgs& p, const A (&acc)[IN][JM], int n0, int m0,
                                                     int wn, int wm, int rl, int half, uint8_t* scr)
{
    const int M = p.M, N = p.N, lane = rl + 32 * half;
    const rsrc_t sr = make_rsrc_u(p.w_scale, (uint32_t)N * 4u);
    const rsrc_t ar = make_rsrc_u(p.a_scale, (uint32_t)M * 4u);
    const int a8 = lane >> 3, c4 = lane & 7;
    const int rr = ((a8 & 1) << 2) + (a8 >> 1);  // row (mod 8) this lane reads back
#pragma unroll
    for (int i = 0; i < IN; ++i) {
        const float sc = __uint_as_float(load4(sr, (uint32_t)(n0 + wn * WN + 32 * i + rl) * 4u));
        const int n = n0 + wn * WN + 32 * i + 4 * c4;  // first of the 4 columns this lane stores
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const int mb = m0 + wm * WM + 32 * j;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 a4 = load16f(ar, (uint32_t)(mb + 8 * g + 4 * half) * 4u);
                const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<float*>(scr + g * 1024 + e * 256 + half * 128 + rl * 4) =
                        ((float)(acc[i][j][4 * g + e] >> 4) * sc) * av[e];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 8 * q + rr;
                const float4 v = *reinterpret_cast<const float4*>(scr + q * 1024 + (r & 3) * 256 +
                                                                  ((r >> 2) & 1) * 128 + c4 * 16);
                const int m = mb + r;
                if (m < M && n < N)  // N % 4 == 0: the 4 columns are inside together
                    *reinterpret_cast<float4*>(static_cast<float*>(p.Y) + (size_t)m * N + n) = v;
            }
        }
    }
}

// W8A16 epilogue through LDS, the same way: blocks i and i + 1 (64 columns of f16, 128
// bytes per row) go to the wave's 4 KB scratch, two adjacent columns per lane (lanes 2t
// and 2t + 1 trade one scaled value first), and come back as 16 bytes (8 columns) per
// lane, 8 rows x 128 contiguous bytes per store instruction.  Needs N % 8 == 0.
template <int IN, int JM, int WN, int WM, class A>
__device__ __forceinline__ void tile_epilogue_w8_lds(const TileGemmArgs& p, const A (&acc)[IN][JM], int n0, int m0,
                                                     int wn, int wm, int rl, int half, uint8_t* scr)
{
    static_assert(IN % 2 == 0, "blocks in pairs");
    const int M = p.M, N = p.N, lane = rl + 32 * half;
    const rsrc_t sr = make_rsrc_u(p.w_scale, (uint32_t)N * 2u);
    const bool odd = (rl & 1) != 0;
    const int a8 = lane >> 3, c4 = lane & 7;
    const int rr = ((a8 & 1) << 2) + (a8 >> 1);  // row (mod 8) this lane reads back
#pragma unroll
    for (int i = 0; i < IN; i += 2) {
        const int na = n0 + wn * WN + 32 * i + rl;  // this lane's column in block i
        const float sa = __half2float(__ushort_as_half(load2(sr, (uint32_t)na * 2u)));
        const float sb = __half2float(__ushort_as_half(load2(sr, (uint32_t)(na + 32) * 2u)));
        // lane 2t holds columns 2t, 2t + 1 of block i, lane 2t + 1 those of block i + 1
        const int cb = odd ? 64 + 2 * (rl - 1) : 2 * rl;  // byte offset of the pair in the row
        const int n = n0 + wn * WN + 32 * i + 8 * c4;     // first of the 8 columns this lane stores
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const int mb = m0 + wm * WM + 32 * j;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float va = sa * acc[i][j][v], vb = sb * acc[i + 1][j][v];
                const float got = __int_as_float(
                    __builtin_amdgcn_mov_dpp(__float_as_int(odd ? va : vb), 0xB1, 0xF, 0xF, false));
                const float lo = odd ? got : va, hi = odd ? vb : got;
                const int g = v >> 2, e = v & 3;
                *reinterpret_cast<uint32_t*>(scr + g * 1024 + e * 256 + half * 128 + cb) =
                    (uint32_t)__half_as_ushort(__float2half_rn(lo)) |
                    ((uint32_t)__half_as_ushort(__float2half_rn(hi)) << 16);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 8 * q + rr;
                const uint4 o = *reinterpret_cast<const uint4*>(scr + q * 1024 + (r & 3) * 256 +
                                                                ((r >> 2) & 1) * 128 + c4 * 16);
                const int m = mb + r;
                if (m < M && n < N)  // N % 8 == 0: the 8 columns are inside together
                    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.Y) + (size_t)m * N + n) = o;
            }
        }
    }
}

// Staging.  The stage's weights and rows of X go from memory straight into LDS (buffer
// loads with the LDS destination: no registers, no VALU, no LDS store instructions),
// NBUF stages in flight.  The weights stay in LDS as stored in memory (16 CW bytes per
// row per stage, INT8 or packed INT4) and each wave widens the operands it reads; for
// W4A8 the activation codes arrive already in the unpack order.
//
// A load instruction of one wave writes 1 KB of LDS, lane l's 16 bytes at l * 16, so the
// swizzle is applied on the memory side: the lane that fills LDS slot s loads the chunk
// that belongs there.  The LDS serves 16 lanes of a 16-byte access per cycle across 64
// banks (256 bytes); the swizzles (swz_wc, swz_xc) put the 16 rows of an operand read on
// 16 distinct 16-byte slots of that width.  (With X chunk c of a 128-byte row at
// c ^ (r % 8), rows r and r + 8 met in one bank: the bank-conflict counter read 1.36
// conflict cycles per LDS-active cycle.)
//
// k assignment within a stage: lane half h reads weight chunks h CW / 2 .. h CW / 2 +
// CW / 2 - 1 of its row (one 16-byte read each, two multiplies' operands); at step kk it
// multiplies chunk h CW / 2 + kk / 2, half kk % 2, against X chunk h CW + kk.  Both
// operands of every multiply then hold the same k (W8A16: k 8 (h CW + kk) .. + 7; W4A8:
// 16 (h CW + kk) .. + 15), and each k of the stage is taken once.
//
// Pipeline, stage t in buffer t % NBUF: wait until this wave's loads of stage t have
// landed (at most (NBUF - 2) stages of loads still in flight), barrier (every wave's
// loads of stage t are in LDS, and every wave is done with buffer (t - 1) % NBUF), multiply
// stage t while issuing the loads of stage t + NBUF - 1 into buffer (t - 1) % NBUF in parts
// between its steps (all of them before the next barrier's wait).  Loads of
// stages past the last are issued out of range (zeros) so that the count in flight is the
// same at every stage.  Loads past K, N or M read zeros (buffer loads out of range), which
// keeps the loop free of branches around the loads.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// CW: 16-byte chunks of weights per row per stage (4: 64 k of INT8 or 128 k of INT4, with
// 128 bytes of X per row; 8: twice that).  Deeper stages halve the barriers and the
// per-stage start for the same k, at twice the LDS per stage.
//
// KS > 1 splits each stage's k over KS groups of NWN x NWM waves (group g takes the
// multiplies of steps kk = CW g / KS .. CW (g + 1) / KS - 1 of every stage, on its own
// accumulators), so that a small tile still has several waves per SIMD to overlap one
// wave's LDS latency and operand widening with another's multiplies.  The groups' sums
// meet in LDS at the end (int32: exact; fp32: added in group order).
template <int BITS, int WN, int WM, int NWN, int NWM, int NBUF, int KS, int CW>
struct DmaCfg {
    static constexpr int NWN_ = NWN, NWM_ = NWM, KS_ = KS, CW_ = CW;
    static constexpr int NWG = NWN * NWM;  // waves of one k-group
    static constexpr int NWAVES = NWG * KS, T = 64 * NWAVES;
    static constexpr int BN = WN * NWN, BM = WM * NWM;
    static constexpr int WRB = 16 * CW, XRB = 32 * CW;  // LDS bytes per row of W and of X
    static constexpr int BK = (BITS == 8 ? 16 : 32) * CW;  // k per stage
    static constexpr int SPT = 512 / BK;                   // stages per 512-k tile of the weight layout
    static constexpr int IN = WN / 32, JM = WM / 32;
    // waves that issue the stage loads: all of them where the stage divides evenly
    static constexpr int LW = (BN * CW % T == 0 && BM * 2 * CW % T == 0) ? NWAVES
                            : (BN * CW % (T / 2) == 0 && BM * 2 * CW % (T / 2) == 0) ? NWAVES / 2 : NWG;
    static constexpr int PW = BN * CW / (64 * LW);      // 16-byte weight loads per loading thread
    static constexpr int PX = BM * 2 * CW / (64 * LW);  // 16-byte X loads per loading thread
    static constexpr int WREG = BN * WRB;
    static constexpr int STAGE = WREG + BM * XRB;
    static constexpr int VM = (NBUF - 2) * (PW + PX);  // loads left in flight at a barrier
    // the k-group sums meet in the stage buffers: 4 KB blocks (one 32 x 32 accumulator of
    // one wave), BPB of them per buffer
    static constexpr int BPB = STAGE / 4096;
    static_assert(CW == 4 || CW == 8, "stage depth");
    static_assert(PW >= 1 && PX >= 1 && BN * CW % (64 * LW) == 0 && BM * 2 * CW % (64 * LW) == 0, "whole loads");
    static_assert(NBUF >= 2 && NBUF <= 8 && VM <= 63, "wait count");
    static_assert(NBUF * STAGE + 16 * 1024 <= 160 * 1024, "LDS");
    static_assert(KS == 1 || KS == 2 || KS == 4, "k split");
    static_assert(KS == 1 || (BPB >= 1 && (NWG * IN * JM + BPB - 1) / BPB <= NBUF), "room for one group's sums");
    static_assert(KS > 1 || (NWAVES + NBUF - 1) / NBUF * 4096 <= STAGE, "room for the epilogue scratch");
};

// Chunk c of weight row r and of X row r in LDS.  Weight rows of 64 bytes: c ^ ((r / 4) % 4);
// of 128 bytes: c ^ ((r / 2) % 8).  X rows of 128 bytes: c ^ ((r / 2) % 8); of 256 bytes:
// c ^ (r % 16).  Sixteen consecutive rows at one chunk then fill the 64 banks once.
template <int CW>
__device__ __forceinline__ int swz_wc(int r, int c)
{
    return CW == 4 ? r * 64 + 16 * (c ^ ((r >> 2) & 3)) : r * 128 + 16 * (c ^ ((r >> 1) & 7));
}
template <int CW>
__device__ __forceinline__ int swz_xc(int r, int c)
{
    return CW == 4 ? r * 128 + 16 * (c ^ ((r >> 1) & 7)) : r * 256 + 16 * (c ^ (r & 15));
}

// The bits of an accumulator element, taken by value (a bit cast applied to an element
// of a vector-typed value in place reads element 0 with this compiler).
template <class T>
__device__ __forceinline__ uint32_t u32_of(T x)
{
    return __builtin_bit_cast(uint32_t, x);
}

// This wave's loads of stage t with slot index LO .. HI - 1 (slots 0 .. PW - 1: its weight
// loads, PW .. PW + PX - 1: its loads of X).
template <class C, int BITS, int LO = 0, int HI = C::PW + C::PX>
__device__ __forceinline__ void dma_stage(uint8_t* buf, rsrc_t wr, rsrc_t xr, const uint32_t (&vw)[C::PW],
                                          const uint32_t (&vx)[C::PX], int t, int stages, int wave)
{
    if (C::LW < C::NWAVES && wave >= C::LW)
        return;
    const bool live = t < stages;
    const uint32_t kw = (uint32_t)(t / C::SPT) * 1024u + (uint32_t)(t % C::SPT) * (uint32_t)C::WRB;
    const uint32_t kx = (uint32_t)t * (uint32_t)C::XRB;
#pragma unroll
    for (int q = 0; q < C::PW; ++q)
        if (q >= LO && q < HI)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(buf + 1024 * (wave + C::LW * q)), 16,
                                                     live ? vw[q] + kw : 0x80000000u, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < C::PX; ++q)
        if (C::PW + q >= LO && C::PW + q < HI)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(buf + C::WREG + 1024 * (wave + C::LW * q)),
                                                     16, live ? vx[q] + kx : 0x80000000u, 0, 0, 0);
}

// The loads of one stage, issued in NS parts while the multiplies of the stage before run:
// part 0 before its first step, part p after the multiplies of step p - 1.  Issued all at
// once after the barrier, the loads of 8 waves queue up in the load path and a wave that
// cannot issue its next load does not issue its multiplies either (spread: 1-3% faster on
// 256-row tiles).
template <class C>
struct StageLoads {
    uint8_t* buf;
    rsrc_t wr, xr;
    const uint32_t (&vw)[C::PW];
    const uint32_t (&vx)[C::PX];
    int t, stages, wave;
};

template <class C, int BITS, int NS, int PART>
__device__ __forceinline__ void dma_stage_part(const StageLoads<C>& ld)
{
    constexpr int NL = C::PW + C::PX, LO = NL * PART / NS, HI = NL * (PART + 1) / NS;
    if constexpr (PART < NS && LO < HI) {
        __builtin_amdgcn_sched_barrier(0);
        dma_stage<C, BITS, LO, HI>(ld.buf, ld.wr, ld.xr, ld.vw, ld.vx, ld.t, ld.stages, ld.wave);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// part st + 1, after the multiplies of step st (st is a constant once the step loop is
// unrolled)
template <class C, int BITS, int NS, int... P>
__device__ __forceinline__ void dma_parts_after(int st, const StageLoads<C>& ld, std::integer_sequence<int, P...>)
{
    ((st == P ? dma_stage_part<C, BITS, NS, P + 1>(ld) : (void)0), ...);
}

template <int BITS, class A>
__device__ __forceinline__ void mfma_tile(A& acc, uint4 x, uint4 w)
{
    if constexpr (BITS == 8)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, x), __builtin_bit_cast(v8h, w), acc, 0, 0, 0);
    else
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, x), __builtin_bit_cast(v4i, w), acc, 0, 0, 0);
}

// The multiplies of NS steps of one stage from LDS buffer buf, from step kk0 (even unless
// NS == 1): at step kk, lane half h multiplies weight chunk h CW / 2 + kk / 2 (its half
// kk % 2) against X chunk h CW + kk.  The operands of step kk + 1 are read before the
// multiplies of step kk are issued, so their LDS latency overlaps those multiplies.
template <class C, int BITS, int NS, class A>
__device__ __forceinline__ void dma_steps(const uint8_t* buf, int wn, int wm, int rl, int h, int kk0,
                                          A (&acc)[C::IN][C::JM], const StageLoads<C>& ld)
{
    constexpr int WN = C::BN / C::NWN_, WM = C::BM / C::NWM_, CW = C::CW_;
    const uint8_t* xl = buf + C::WREG;
    const int wc0 = h * CW / 2 + (kk0 >> 1), xc0 = h * CW + kk0;
    uint4 w[2][C::IN], b[2][C::JM];
#pragma unroll
    for (int i = 0; i < C::IN; ++i)
        w[0][i] = *reinterpret_cast<const uint4*>(buf + swz_wc<CW>(wn * WN + 32 * i + rl, wc0));
#pragma unroll
    for (int j = 0; j < C::JM; ++j)
        b[0][j] = *reinterpret_cast<const uint4*>(xl + swz_xc<CW>(wm * WM + 32 * j + rl, xc0));
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        if (st + 1 < NS) {
            if (((st + 1) & 1) == 0) {
#pragma unroll
                for (int i = 0; i < C::IN; ++i)
                    w[((st + 1) >> 1) & 1][i] = *reinterpret_cast<const uint4*>(
                        buf + swz_wc<CW>(wn * WN + 32 * i + rl, wc0 + (st + 1) / 2));
            }
#pragma unroll
            for (int j = 0; j < C::JM; ++j)
                b[(st + 1) & 1][j] = *reinterpret_cast<const uint4*>(xl + swz_xc<CW>(wm * WM + 32 * j + rl, xc0 + st + 1));
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this step's multiplies
        const bool hi_half = NS == 1 ? (kk0 & 1) != 0 : (st & 1) != 0;
#pragma unroll
        for (int i = 0; i < C::IN; ++i) {
            const uint4 wv = w[(st >> 1) & 1][i];
            const uint4 a = widen8<BITS>(hi_half ? make_uint2(wv.z, wv.w) : make_uint2(wv.x, wv.y));
#pragma unroll
            for (int j = 0; j < C::JM; ++j)
                mfma_tile<BITS>(acc[i][j], b[st & 1][j], a);
        }
        dma_parts_after<C, BITS, NS>(st, ld, std::make_integer_sequence<int, NS>{});
    }
}

// The multiplies of k-group kg of one stage from LDS buffer buf.
template <class C, int BITS, class A>
__device__ __forceinline__ void dma_compute(const uint8_t* buf, int wn, int wm, int kg, int rl, int h,
                                            A (&acc)[C::IN][C::JM], const StageLoads<C>& ld)
{
    constexpr int PER = C::CW_ / C::KS_;  // steps per k-group
    static_assert(PER == 1 || PER % 2 == 0, "a k-group starts at an even step");
    dma_steps<C, BITS, PER>(buf, wn, wm, rl, h, C::KS_ == 1 ? 0 : kg * PER, acc, ld);
}

// Wait for this wave's loads of the current stage, then the workgroup barrier.  The
// compiler barriers keep LDS accesses on their side of it (the barrier instruction
// itself is not a memory operation to the compiler).
template <int VM>
__device__ __forceinline__ void dma_barrier()
{
    // s_waitcnt vmcnt(VM) lgkmcnt(0): vmcnt in bits 3:0 and 15:14, expcnt 6:4 left at 7
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int BITS, int WN, int WM, int NWN, int NWM, int NBUF, int KS, int CW>
__global__ __launch_bounds__(64 * NWN * NWM * KS) void k_gemm_dma(TileGemmArgs p)
{
    using C = DmaCfg<BITS, WN, WM, NWN, NWM, NBUF, KS, CW>;
    constexpr int BN = C::BN, BM = C::BM, BK = C::BK, IN = C::IN, JM = C::JM;
    constexpr int R = BITS == 8 ? 2 : 4;  // rows per tile of the weight layout
    // one array per buffer: the compiler then knows which buffer a DMA writes and which
    // one an LDS read reads, and does not wait for the later stages' loads before reads
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[NBUF > 2 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[NBUF > 3 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds4[NBUF > 4 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds5[NBUF > 5 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds6[NBUF > 6 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds7[NBUF > 7 ? C::STAGE : 16];
    auto bufs = [&](int b) -> uint8_t* {
        return b == 0 ? lds0 : b == 1 ? lds1 : b == 2 ? lds2 : b == 3 ? lds3 : b == 4 ? lds4 : b == 5 ? lds5
             : b == 6 ? lds6 : lds7;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wg = wave % C::NWG, kg = wave / C::NWG;  // position in the tile, k-group
    const int wn = wg % NWN, wm = wg / NWN;
    const int L = xcd_block(blockIdx.x, gridDim.x);
    const int nb = L / p.mblocks, mb = L - nb * p.mblocks;
    const int n0 = nb * BN, m0 = mb * BM;
    const int M = p.M, K = p.K, CG = p.cg;
    const int stages = (K + BK - 1) / BK;
    const int xrow = BITS == 8 ? K * 2 : K;  // bytes per row of X

    const int rg0 = n0 / R;
    const rsrc_t wr = make_rsrc_u(p.Wq + (size_t)rg0 * CG * 1024u,
                                (uint32_t)max(0, min(BN / R, p.nrg - rg0)) * (uint32_t)CG * 1024u);
    const rsrc_t xr = make_rsrc_u(static_cast<const uint8_t*>(p.X) + (size_t)m0 * xrow,
                                (uint32_t)max(0, min(BM, M - m0)) * (uint32_t)xrow);

    // per-lane load offsets at stage 0: LDS slot i of a region holds the chunk that the
    // swizzle puts there
    uint32_t vw[C::PW], vx[C::PX];
#pragma unroll
    for (int q = 0; q < C::PW; ++q) {
        const int i = tid + 64 * C::LW * q, r = i / CW;
        const int c = (swz_wc<CW>(r, i % CW) - r * C::WRB) / 16;  // the chunk that lands in slot i
        vw[q] = (uint32_t)(((r / R) * CG) * 1024 + (r % R) * (1024 / R) + 16 * c);
    }
#pragma unroll
    for (int q = 0; q < C::PX; ++q) {
        const int i = tid + 64 * C::LW * q, r = i / (2 * CW);
        const int c = (swz_xc<CW>(r, i % (2 * CW)) - r * C::XRB) / 16;
        vx[q] = (uint32_t)r * (uint32_t)xrow + 16u * (uint32_t)c;
    }

    typedef typename std::conditional<BITS == 8, v16f, v16i>::type acc_t;
    acc_t acc[IN][JM];
#pragma unroll
    for (int i = 0; i < IN; ++i)
#pragma unroll
        for (int j = 0; j < JM; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0;

    const int rl = lane & 31, h = lane >> 5;
#pragma unroll
    for (int d = 0; d < NBUF - 1; ++d)
        dma_stage<C, BITS>(bufs(d), wr, xr, vw, vx, d, stages, wave);
    for (int s = 0; s < stages; s += NBUF) {
#pragma unroll
        for (int d = 0; d < NBUF; ++d) {
            dma_barrier<C::VM>();
            const StageLoads<C> ld{bufs((d + NBUF - 1) % NBUF), wr, xr, vw, vx, s + d + NBUF - 1, stages, wave};
            dma_stage_part<C, BITS, C::CW_ / KS, 0>(ld);
            dma_compute<C, BITS>(bufs(d), wn, wm, kg, rl, h, acc, ld);
        }
    }
    // the loads of the stages past the last (zeros) may still be in flight
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));

    if constexpr (KS > 1) {
        // k-groups KS - 1 .. 1 hand their sums to group 0 through LDS (the stage
        // buffers, free once every wave is past its last multiply), one group at a time;
        // block (wave wg, i, j) sits in buffer blk / BPB at 4 KB x (blk % BPB), register
        // v of lane l at (v / 4) * 1 KB + 16 l + 4 (v % 4)
#pragma unroll
        for (int g = KS - 1; g >= 1; --g) {
            dma_barrier<0>();
#pragma unroll
            for (int i = 0; i < IN; ++i)
#pragma unroll
                for (int j = 0; j < JM; ++j) {
                    const int blk = (wg * IN + i) * JM + j;
                    uint8_t* red = bufs(blk / C::BPB) + 4096 * (blk % C::BPB) + 16 * lane;
                    if (kg == g) {
#pragma unroll
                        for (int v = 0; v < 16; v += 4)
                            *reinterpret_cast<uint4*>(red + 256 * v) =
                                make_uint4(u32_of(acc[i][j][v]), u32_of(acc[i][j][v + 1]), u32_of(acc[i][j][v + 2]),
                                           u32_of(acc[i][j][v + 3]));
                    }
                }
            dma_barrier<0>();
#pragma unroll
            for (int i = 0; i < IN; ++i)
#pragma unroll
                for (int j = 0; j < JM; ++j) {
                    const int blk = (wg * IN + i) * JM + j;
                    const uint8_t* red = bufs(blk / C::BPB) + 4096 * (blk % C::BPB) + 16 * lane;
                    if (kg == 0) {
#pragma unroll
                        for (int v = 0; v < 16; v += 4) {
                            const uint4 o = *reinterpret_cast<const uint4*>(red + 256 * v);
                            const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                if constexpr (BITS == 8)
                                    acc[i][j][v + e] += __builtin_bit_cast(float, ov[e]);
                                else
                                    acc[i][j][v + e] += (int)ov[e];
                            }
                        }
                    }
                }
        }
        if (kg != 0)
            return;
    }

    if constexpr (BITS == 4 || IN % 2 == 0) {
        if ((p.N & (BITS == 4 ? 3 : 7)) == 0) {
            // a 4 KB scratch per wave: after the k-group hand-off, the wave's own first
            // hand-off block (read back by this wave only); otherwise a slice of the stage
            // buffers, once every wave is past its last multiply
            uint8_t* scr;
            if constexpr (KS > 1) {
                const int blk = wg * IN * JM;
                scr = bufs(blk / C::BPB) + 4096 * (blk % C::BPB);
            } else {
                dma_barrier<0>();
                scr = bufs(wave % NBUF) + 4096 * (wave / NBUF);
            }
            if constexpr (BITS == 4)
                tile_epilogue_w4_lds<IN, JM, BN / NWN, BM / NWM>(p, acc, n0, m0, wn, wm, rl, h, scr);
            else
                tile_epilogue_w8_lds<IN, JM, BN / NWN, BM / NWM>(p, acc, n0, m0, wn, wm, rl, h, scr);
            return;
        }
    }
    tile_epilogue<BITS, IN, JM, BN / NWN, BM / NWM>(p, acc, n0, m0, wn, wm, rl, h);
}

template <int BITS, int WN, int WM, int NWN, int NWM, int NBUF, int KS = 1, int CW = 4>
hipError_t go_dma(TileGemmArgs p, hipStream_t st)
{
    using C = DmaCfg<BITS, WN, WM, NWN, NWM, NBUF, KS, CW>;
    const int64_t nbn = ((int64_t)p.N + C::BN - 1) / C::BN, nbm = ((int64_t)p.M + C::BM - 1) / C::BM;
    if (nbn * nbm > 0x7fffffff)
        return hipErrorInvalidValue;
    p.mblocks = (int)nbm;
    hipLaunchKernelGGL((k_gemm_dma<BITS, WN, WM, NWN, NWM, NBUF, KS, CW>), dim3((unsigned)(nbn * nbm)), dim3(C::T), 0,
                       st, p);
    return hipGetLastError();
}

// Launch variants: tile (BN x BM), waves, stages in flight, k split, stage depth.  The LDS
// footprint decides how many workgroups share a CU (variants 0, 1, 7: one; 2 to 5 and 8:
// two; 6: three).
template <int BITS>
hipError_t go_variant(const TileGemmArgs& p, int variant, hipStream_t st)
{
    switch (variant) {
    case 0: return go_dma<BITS, 64, 128, 4, 2, 3>(p, st);    // 256 n x 256 m, 8 waves
    case 1: return go_dma<BITS, 64, 64, 4, 2, 4>(p, st);     // 256 n x 128 m, 8 waves
    case 2: return go_dma<BITS, 64, 64, 2, 2, 3>(p, st);     // 128 n x 128 m, 4 waves
    case 3: return go_dma<BITS, 64, 64, 2, 2, 3, 2>(p, st);  // 128 n x 128 m, 2 k-groups of 4 waves
    case 4: return go_dma<BITS, 64, 32, 2, 2, 4>(p, st);     // 128 n x 64 m, 4 waves
    case 5: return go_dma<BITS, 64, 32, 2, 2, 4, 2>(p, st);  // 128 n x 64 m, 2 k-groups of 4 waves
    case 6: return go_dma<BITS, 32, 32, 2, 2, 4>(p, st);     // 64 n x 64 m, 4 waves
    case 7: return go_dma<BITS, 64, 32, 2, 2, 4, 2, 8>(p, st);  // variant 5 with stages twice as deep
    case 8: return go_dma<BITS, 32, 32, 4, 1, 4, 1, 8>(p, st);  // 128 n x 32 m, 4 waves, deep stages
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int tile_rows_m(int variant)
{
    switch (variant) {
    case 0: return 256;
    case 1: case 2: case 3: return 128;
    case 4: case 5: case 6: case 7: return 64;
    case 8: return 32;
    default: return 0;
    }
}

int tile_rows_n(int variant)
{
    switch (variant) {
    case 0: case 1: return 256;
    case 2: case 3: case 4: case 5: case 7: case 8: return 128;
    case 6: return 64;
    default: return 0;
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
