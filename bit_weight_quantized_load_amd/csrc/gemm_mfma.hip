// Skinny GEMM for M >= 16 on the matrix cores: the same linears as the GEMV kernels
// (W4A8: "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s", sections
// 当前实现方式 and 正确方向; W8A16: ChatGLM2-6B W8A16 write-up (TPU-MLIR), section 4),
// computed with v_mfma_i32_16x16x64_i8 (W4A8) and v_mfma_f32_16x16x32_f16 (W8A16).
//
// Operands.  For a 16x16xKL MFMA, lane l supplies row l % 16 of A and column l % 16 of
// B, each at the KL consecutive k of block l / 16, and receives D[4 (l / 16) + i][l % 16]
// for i = 0..3.  A is the weight (16 output rows n), B is X transposed (16 rows m), so
// D holds Y transposed: D[n][m].
//
// Weights stay in the tile layout of the GEMV (kernels.hpp).  A workgroup owns 64
// consecutive rows (four waves of 16 rows = 4 INT4 or 8 INT8 row groups) and a run of
// row blocks of X; per 512-k tile each wave copies its tiles (one 1 KB wave load each)
// into its own LDS region, padded so that the 16 lanes reading 16 different rows hit
// different banks, and reads them back in operand order.
//
// W4A8: X is quantized once per call into the workspace by k_quant_act_mfma (the same
// per-row scale and codes as quant_act_i8) in B-operand order, so the workgroup stages
// it into LDS with plain 16-byte copies.  An INT4 operand of 16 k is 8 bytes of nibbles
// presented as 16 * q (nibble moved to the high half of its byte; even k from the low
// nibbles, odd k from the high ones), and the X codes are stored in the same k order;
// the int32 result is exactly 16 * acc, so acc >> 4 is exact and the output equals the
// GEMV's bit for bit.
//
// W8A16: X (f16) is staged in LDS in 128-k slices straight from the input; the INT8
// weights are cast to f16 exactly in registers (the byte-permute cast of the GEMV) and
// the per-channel scale multiplies the fp32 sum once.
#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreadsG = 64 * kWaves;

// ---------------------------------------------------------------- W4A8 --------

// Position p of the 16 codes of one B operand holds k = 16 g + kPerm[p] of its step:
// the order in which the INT4 unpack presents the weights.
__device__ __forceinline__ uint4 pack_perm16(const int (&q)[16])
{
    uint4 o;
    o.x = pack_i8x4(q[0], q[2], q[4], q[6]);
    o.y = pack_i8x4(q[1], q[3], q[5], q[7]);
    o.z = pack_i8x4(q[8], q[10], q[12], q[14]);
    o.w = pack_i8x4(q[9], q[11], q[13], q[15]);
    return o;
}

// One workgroup per row of X (grid-strided over ceil(M / 16) * 16 rows; rows past M
// are written as zeros).  a = maxabs / 127 and the codes exactly as k_quant_act, laid
// out as B operands: row m, step st (64 k), lane block g -> 16 bytes at
// ((m / 16) * KS + st) * 1024 + (16 g + m % 16) * 16.
__global__ __launch_bounds__(kBlock) void k_quant_act_mfma(const float* __restrict__ X, int M,
                                                           int K, int Mp, int KS,
                                                           uint8_t* __restrict__ Xp,
                                                           float* __restrict__ a_scale)
{
    __shared__ float red[4];
    const int K4 = K >> 2;
    const int slots = KS * 4;  // 16-code slots per row
    for (int m = blockIdx.x; m < Mp; m += gridDim.x) {
        const bool live = m < M;
        const float4* row = reinterpret_cast<const float4*>(X + (size_t)(live ? m : 0) * K);
        float mx = 0.0f;
        if (live)
            for (int i = threadIdx.x; i < K4; i += kBlock)
                mx = fmaxf(mx, max_abs4(row[i]));
        mx = block_max(mx, red);
        const float a = mx / 127.0f;
        const float r = 1.0f / a;
        const bool fast = r <= 3.0e38f;
        if (live && threadIdx.x == 0)
            a_scale[m] = a;
        uint8_t* base = Xp + (size_t)(m >> 4) * KS * 1024u + (size_t)(m & 15) * 16u;
        for (int sl = threadIdx.x; sl < slots; sl += kBlock) {
            int q[16];
            const int k0 = 16 * sl;
            if (live && k0 < K) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float4 x = row[(k0 >> 2) + v];
                    const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        q[4 * v + e] = fast ? quant_code_fast(xs[e], a, r, 127.f)
                                            : quant_code(xs[e], a, 127.f);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    q[e] = 0;
            }
            const int st = sl >> 2, g = sl & 3;
            *reinterpret_cast<uint4*>(base + (size_t)st * 1024u + (size_t)g * 256u) = pack_perm16(q);
        }
    }
}

// Padded LDS image of one wave's four INT4 tiles: tile i at i * 1088, tile row sub at
// sub * 272, 16-byte chunk j at j * 16.
constexpr int kW4TilePitch = 1088, kW4RowPitch = 272, kW4WaveBytes = 4 * kW4TilePitch;

template <int MB>
__global__ __launch_bounds__(kThreadsG) void k_gemm_w4a8(MfmaW4A8Args p)
{
    extern __shared__ uint8_t s_mem[];  // [waves][4 tiles padded] then X [MB][8 steps][1 KB]
    uint8_t* s_w = s_mem;
    uint8_t* s_x = s_mem + kWaves * kW4WaveBytes;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int CG = p.cg, KS = p.ks, MG = p.mgroups;
    const int mg = blockIdx.x % MG, nb = blockIdx.x / MG;
    const int mb0 = mg * MB;
    const int rgw = nb * 16 + wave * 4;  // first row group of this wave
    const int nrg_w = max(0, min(4, p.nrg - rgw));
    const rsrc_t wres = make_rsrc(p.Wq + (size_t)rgw * CG * 1024u, (uint32_t)(nrg_w * CG) * 1024u);
    const rsrc_t xres = make_rsrc(p.Xp, (uint32_t)p.mbtot * (uint32_t)KS * 1024u);

    uint4 wr[4], xr[2 * MB];
    auto load_tiles = [&](int c) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            wr[i] = load16_stream(wres, (uint32_t)(i * CG + c) * 1024u + (uint32_t)lane * 16u);
#pragma unroll
        for (int v = 0; v < 2 * MB; ++v) {
            const int piece = v * kThreadsG + tid;  // [mbl][s][lane slot]
            const int mbl = piece >> 9, s = (piece >> 6) & 7, sl = piece & 63;
            const bool ok = mb0 + mbl < p.mbtot && 8 * c + s < KS;
            xr[v] = load16(xres, ok ? ((uint32_t)(mb0 + mbl) * (uint32_t)KS + (uint32_t)(8 * c + s)) * 1024u +
                                          (uint32_t)sl * 16u
                                    : 0x80000000u);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    v4i acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
        acc[i] = v4i{0, 0, 0, 0};

    uint8_t* my_w = s_w + wave * kW4WaveBytes;
    const int sub = lane >> 4, j = lane & 15;
    // A operand of step s for lane (g, r): row r = tile r / 4, tile row r % 4; chunk
    // 2 s + g / 2, half g % 2
    const int a_off = (r >> 2) * kW4TilePitch + (r & 3) * kW4RowPitch + (g >> 1) * 16 + (g & 1) * 8;

    load_tiles(0);
    for (int c = 0; c < CG; ++c) {
        __syncthreads();  // every wave is done with the previous tile's X
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(my_w + i * kW4TilePitch + sub * kW4RowPitch + j * 16) = wr[i];
#pragma unroll
        for (int v = 0; v < 2 * MB; ++v)
            *reinterpret_cast<uint4*>(s_x + (size_t)(v * kThreadsG + tid) * 16) = xr[v];
        __syncthreads();
        if (c + 1 < CG)
            load_tiles(c + 1);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint2 w = *reinterpret_cast<const uint2*>(my_w + a_off + s * 32);
            v4i a;
            a[0] = (int)((w.x << 4) & 0xF0F0F0F0u);
            a[1] = (int)(w.x & 0xF0F0F0F0u);
            a[2] = (int)((w.y << 4) & 0xF0F0F0F0u);
            a[3] = (int)(w.y & 0xF0F0F0F0u);
#pragma unroll
            for (int mbl = 0; mbl < MB; ++mbl) {
                const uint4 b4 = *reinterpret_cast<const uint4*>(s_x + ((mbl * 8 + s) * 64 + lane) * 16);
                const v4i b = {(int)b4.x, (int)b4.y, (int)b4.z, (int)b4.w};
                acc[mbl] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[mbl], 0, 0, 0);
            }
        }
    }

    // lane (g, r) holds D[n = 4 g + i][m = r] of each 16 x 16 block
    const int n0 = 4 * rgw + 4 * g;
    const rsrc_t sres = make_rsrc(p.w_scale, (uint32_t)p.N * 4u);
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
                    p.Y[(size_t)m * p.N + n0 + i] = ((float)(acc[mbl][i] >> 4) * sc[i]) * am;
        }
    }
}

// ---------------------------------------------------------------- W8A16 -------

// Padded LDS image of one wave's eight INT8 tiles (2 rows x 32 chunks each): tile i at
// i * 1056, tile row sub at sub * 528, chunk j at j * 16.
constexpr int kW8TilePitch = 1056, kW8RowPitch = 528, kW8WaveBytes = 8 * kW8TilePitch;
// X slice in LDS: 128 k (256 bytes) per row, rows padded to 272 bytes.
constexpr int kXSliceK = 128, kXRowPitch = 272;

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

template <int MB>
__global__ __launch_bounds__(kThreadsG) void k_gemm_w8a16(MfmaW8A16Args p)
{
    extern __shared__ uint8_t s_mem[];  // [waves][8 tiles padded] then X [16 MB rows][272 B]
    uint8_t* s_w = s_mem;
    uint8_t* s_x = s_mem + kWaves * kW8WaveBytes;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int M = p.M, K = p.K, CG = p.cg, MG = p.mgroups;
    const int mg = blockIdx.x % MG, nb = blockIdx.x / MG;
    const int m0 = mg * MB * 16;
    const int rgw = nb * 32 + wave * 8;  // first row group (2 rows) of this wave
    const int nrg_w = max(0, min(8, p.nrg - rgw));
    const rsrc_t wres = make_rsrc(p.Wq + (size_t)rgw * CG * 1024u, (uint32_t)(nrg_w * CG) * 1024u);
    const int rows_x = max(0, min(MB * 16, M - m0));
    const rsrc_t xres = make_rsrc(p.X + (size_t)m0 * K, (uint32_t)rows_x * (uint32_t)K * 2u);

    // X slice: 16 MB rows x 128 k = MB * 256 pieces of 16 bytes, one per thread and pass
    constexpr int kXPieces = MB * 16 * (kXSliceK / 8);
    constexpr int kXPass = (kXPieces + kThreadsG - 1) / kThreadsG;

    uint4 wr[8], xr[kXPass];
    auto load_w = [&](int c) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            wr[i] = load16_stream(wres, (uint32_t)(i * CG + c) * 1024u + (uint32_t)lane * 16u);
    };
    auto load_x = [&](int kk) {  // slice starting at k = kk
#pragma unroll
        for (int v = 0; v < kXPass; ++v) {
            const int piece = v * kThreadsG + tid;
            const int row = piece >> 4, q = piece & 15;
            const bool ok = piece < kXPieces && kk + 8 * q < K;
            xr[v] = load16(xres, ok ? (uint32_t)(row * K + kk + 8 * q) * 2u : 0x80000000u);
        }
    };
    auto store_x = [&]() {
#pragma unroll
        for (int v = 0; v < kXPass; ++v) {
            const int piece = v * kThreadsG + tid;
            if (piece < kXPieces)
                *reinterpret_cast<uint4*>(s_x + (piece >> 4) * kXRowPitch + (piece & 15) * 16) = xr[v];
        }
    };

    v4f acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
        acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

    uint8_t* my_w = s_w + wave * kW8WaveBytes;
    const int sub = lane >> 5, j = lane & 31;
    // A operand of step s (32 k) for lane (g, r): row r = tile r / 2, tile row r % 2;
    // k = 32 s + 8 g .. + 7 = chunk 2 s + g / 2, half g % 2
    const int a_off = (r >> 1) * kW8TilePitch + (r & 1) * kW8RowPitch + (g >> 1) * 16 + (g & 1) * 8;

    load_w(0);
    load_x(0);
    __builtin_amdgcn_sched_barrier(0);
    for (int c = 0; c < CG; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint4*>(my_w + i * kW8TilePitch + sub * kW8RowPitch + j * 16) = wr[i];
        if (c + 1 < CG)
            load_w(c + 1);
        __builtin_amdgcn_sched_barrier(0);
        for (int h = 0; h < 512 / kXSliceK; ++h) {
            __syncthreads();  // every wave is done with the previous slice
            store_x();
            __syncthreads();
            const int kn = 512 * c + kXSliceK * (h + 1);
            if (kn < 512 * CG)
                load_x(kn);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < kXSliceK / 32; ++s) {
                const int st = h * (kXSliceK / 32) + s;  // 32-k step within the tile
                const uint2 w = *reinterpret_cast<const uint2*>(my_w + a_off + st * 32);
                half2_t h0, h1, h2, h3;
                cast4(w.x, h0, h1);
                cast4(w.y, h2, h3);
                const v8h a = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
#pragma unroll
                for (int mbl = 0; mbl < MB; ++mbl) {
                    const uint4 b4 = *reinterpret_cast<const uint4*>(
                        s_x + (mbl * 16 + r) * kXRowPitch + (32 * s + 8 * g) * 2);
                    const v8h b = __builtin_bit_cast(v8h, b4);
                    acc[mbl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[mbl], 0, 0, 0);
                }
            }
        }
    }

    const int n0 = 2 * rgw + 4 * g;
    const rsrc_t sres = make_rsrc(p.w_scale, (uint32_t)p.N * 2u);
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
                    p.Y[(size_t)m * p.N + n0 + i] = __half_as_ushort(__float2half_rn(acc[mbl][i] * sc[i]));
        }
    }
}

}  // namespace

size_t mfma_w4a8_workspace_bytes(int64_t M, int64_t K)
{
    const size_t mbtot = (size_t)((M + 15) / 16), ks = (size_t)((K + 63) / 64);
    const size_t xp = (mbtot * ks * 1024u + 255u) & ~(size_t)255u;
    return xp + (((size_t)M * 4u + 255u) & ~(size_t)255u);
}

hipError_t launch_gemm_w4a8(const float* X, int M, int N, int K, const uint8_t* Wq,
                            const float* w_scale, float* Y, void* workspace, hipStream_t st)
{
    const TileLayout L = tile_layout(4, N, K);
    const int mbtot = (M + 15) / 16, ks = (K + 63) / 64;
    uint8_t* xp = static_cast<uint8_t*>(workspace);
    const size_t xp_bytes = ((size_t)mbtot * ks * 1024u + 255u) & ~(size_t)255u;
    float* a = reinterpret_cast<float*>(xp + xp_bytes);
    const int qgrid = mbtot * 16 < 65536 ? mbtot * 16 : 65536;
    hipLaunchKernelGGL(k_quant_act_mfma, dim3(qgrid), dim3(kBlock), 0, st, X, M, K, mbtot * 16, ks,
                       xp, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    MfmaW4A8Args p;
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
    const int MB = mbtot >= 4 ? 4 : (mbtot >= 2 ? 2 : 1);
    p.mgroups = (mbtot + MB - 1) / MB;
    const int64_t nblocks = (L.nrg + 15) / 16;
    if (nblocks * p.mgroups > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(nblocks * p.mgroups));
    const size_t lds = (size_t)kWaves * kW4WaveBytes + (size_t)MB * 8 * 1024;
    switch (MB) {
    case 1: hipLaunchKernelGGL(k_gemm_w4a8<1>, grid, dim3(kThreadsG), lds, st, p); break;
    case 2: hipLaunchKernelGGL(k_gemm_w4a8<2>, grid, dim3(kThreadsG), lds, st, p); break;
    default: hipLaunchKernelGGL(k_gemm_w4a8<4>, grid, dim3(kThreadsG), lds, st, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_w8a16(const uint16_t* X, int M, int N, int K, const uint8_t* Wq,
                             const uint16_t* w_scale, uint16_t* Y, hipStream_t st)
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
    const int MB = mbtot >= 4 ? 4 : (mbtot >= 2 ? 2 : 1);
    p.mgroups = (mbtot + MB - 1) / MB;
    const int64_t nblocks = (L.nrg + 31) / 32;
    if (nblocks * p.mgroups > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(nblocks * p.mgroups));
    const size_t lds = (size_t)kWaves * kW8WaveBytes + (size_t)MB * 16 * kXRowPitch;
    switch (MB) {
    case 1: hipLaunchKernelGGL(k_gemm_w8a16<1>, grid, dim3(kThreadsG), lds, st, p); break;
    case 2: hipLaunchKernelGGL(k_gemm_w8a16<2>, grid, dim3(kThreadsG), lds, st, p); break;
    default: hipLaunchKernelGGL(k_gemm_w8a16<4>, grid, dim3(kThreadsG), lds, st, p); break;
    }
    return hipGetLastError();
}

}  // namespace qw
