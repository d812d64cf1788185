// The two ablations that "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s"
// times beside its INT4-weight / INT8-activation path (section 速度结果), as GEMVs at
// M == 1 on the same footing as the other kernels here (whole-wave 1 KB loads, every
// tile of a wave requested before its first multiply):
//
//  * FP16 GEMV: no quantization; weights and activations in f16, fp32 accumulation,
//    f16 output.
//  * Weight-only INT4 with float activations (sections 最初的问题 and 问题原因): the
//    row-wise INT4 weights of quantize_pack_w4, each nibble sign-extended, converted to
//    float and multiplied-added with the fp32 activation; the row scale multiplies the
//    finished sum.  Per weight this is a bit-field extract, a conversion and a
//    multiply-add, against 5 integer instructions per 8 weights on the W4A8 path: the
//    page's explanation of why unpacking to float gives the bandwidth saving back.
#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

// FP16 GEMV.  W16 is row-major f16 [N][K], read as 1 KB tiles of one row x 512 k:
// lane j holds halves 8j .. 8j+7 of each tile of its rows, and the matching halves of X
// in registers.  Each wave owns RPW consecutive rows (an even share: rows of wave g are
// [rg_of(g), rg_of(g + 1))), all of their tiles requested up front.  A row's 64 lanes
// meet in DPP row sums and four lane reads, added in a fixed order.
template <int RCG, int RPW, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv_f16(const uint16_t* __restrict__ X,
                                                      const uint16_t* __restrict__ W,
                                                      uint16_t* __restrict__ Y, int N, int K,
                                                      int nwaves, int per, int rem)
{
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * NW + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (gw >= nwaves)
        return;  // no barrier in this kernel
    const int r0 = rg_of(gw, per, rem);
    const int nr = rg_of(gw + 1, per, rem) - r0;
    const rsrc_t xr = make_rsrc(X, (uint32_t)K * 2u);
    uint4 xv[RCG];
#pragma unroll
    for (int c = 0; c < RCG; ++c) {
        const int k = 512 * c + 8 * lane;
        xv[c] = load16(xr, k < K ? (uint32_t)k * 2u : 0x80000000u);
    }
    const rsrc_t wr = make_rsrc(W + (size_t)r0 * K, (uint32_t)nr * (uint32_t)K * 2u);
    uint4 w[RPW][RCG];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int c = 0; c < RCG; ++c) {
            const int k = 512 * c + 8 * lane;
            w[r][c] = load16_stream(wr, r < nr && k < K ? (uint32_t)(r * K + k) * 2u : 0x80000000u);
        }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < RCG; ++c) {
            const uint32_t ww[4] = {w[r][c].x, w[r][c].y, w[r][c].z, w[r][c].w};
            const uint32_t xx[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
#pragma unroll
            for (int d = 0; d < 4; ++d)
                acc[d] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, ww[d]),
                                                __builtin_bit_cast(half2_t, xx[d]), acc[d], false);
        }
        const float v = row_sum16((acc[0] + acc[1]) + (acc[2] + acc[3]));
        const float t0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        const float t1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
        const float t2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
        const float t3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
        if (lane == 0 && r < nr)
            Y[r0 + r] = __half_as_ushort(__float2half_rn((t0 + t1) + (t2 + t3)));
    }
}

// Weight-only INT4 with float activations.  Tile layout of quantize_pack_w4: lane
// (sub, j) meets row 4 rg + sub and chunk j (k = 512c + 32j .. + 31) of every tile.  The
// workgroup stages X (fp32, zero-padded to whole tiles) in LDS, 32 values every 36
// floats so that the 16 lanes of a row, whose slices start 32 values apart, read
// distinct banks; for each tile a lane reads its 32 activations once and uses them for
// all RPW row groups of the wave.  Per 32-bit word of nibbles (k = 8d .. 8d+7 of the
// chunk, nibble i = k 8d+i): extract with sign extension, convert to float, fused
// multiply-add in fp32.
template <int RCG, int RPW, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv_w4f(const float* __restrict__ X,
                                                      const uint8_t* __restrict__ Wq,
                                                      const float* __restrict__ s,
                                                      float* __restrict__ Y, int N, int K,
                                                      int cg, int nwaves, int per, int rem)
{
    constexpr int kThreads = 64 * NW;
    constexpr int XL = (RCG * 128 + kThreads - 1) / kThreads;  // X float4 per thread
    __shared__ float s_x[RCG * 576];  // slice of 32 k at 36 * (k / 32)
    const int tid = threadIdx.x, lane = tid & 63;
    const int j = lane & 15, sub = lane >> 4;
    const int gw = blockIdx.x * NW + __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg0 = gw < nwaves ? rg_of(gw, per, rem) : 0;
    const int nrg = gw < nwaves ? rg_of(gw + 1, per, rem) - rg0 : 0;
    // X first, then the weight tiles and row scales of the wave
    const rsrc_t xr = make_rsrc(X, (uint32_t)K * 4u);
    float4 xv[XL];
#pragma unroll
    for (int i = 0; i < XL; ++i)
        xv[i] = load16f(xr, (uint32_t)(i * kThreads + tid) * 16u);  // past K: zeros
    issue_barrier();
    const rsrc_t wr = make_rsrc(Wq + (size_t)rg0 * cg * 1024u, (uint32_t)(nrg * cg) * 1024u);
    uint4 w[RPW][RCG];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int c = 0; c < RCG; ++c)
            w[r][c] = load16_stream(wr, r < nrg ? (uint32_t)((r * cg + c) * 1024 + lane * 16) : 0x80000000u);
    const rsrc_t sr = make_rsrc(s + (size_t)rg0 * 4, (uint32_t)max(0, min(nrg * 4, N - rg0 * 4)) * 4u);
    float sc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
        sc[r] = __uint_as_float(load4(sr, (uint32_t)(r * 4 + sub) * 4u));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        const int f = i * kThreads + tid;
        if (f < RCG * 128)
            *reinterpret_cast<float4*>(s_x + 36 * (f >> 3) + 4 * (f & 7)) = xv[i];
    }
    __syncthreads();
    float acc[RPW][4];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
        acc[r][0] = acc[r][1] = acc[r][2] = acc[r][3] = 0.0f;
#pragma unroll
    for (int c = 0; c < RCG; ++c) {
        float x[32];
        const float4* xp = reinterpret_cast<const float4*>(s_x + 36 * (16 * c + j));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 v = xp[i];
            x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const uint32_t ww[4] = {w[r][c].x, w[r][c].y, w[r][c].z, w[r][c].w};
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int q = __builtin_amdgcn_sbfe((int)ww[d], 4 * i, 4);
                    acc[r][d] = __builtin_fmaf((float)q, x[8 * d + i], acc[r][d]);
                }
        }
        // one tile's activations live at a time (hoisting every tile's reads ahead of
        // the arithmetic took all registers and left one wave per SIMD)
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const float v = row_sum16((acc[r][0] + acc[r][1]) + (acc[r][2] + acc[r][3]));
        const int n = (rg0 + r) * 4 + sub;
        if (j == 0 && r < nrg && n < N)
            Y[n] = v * sc[r];
    }
}

template <int RCG, int RPW>
hipError_t launch_f16_r(const uint16_t* X, const uint16_t* W, uint16_t* Y, int N, int K,
                        int nwaves, hipStream_t st)
{
    const int blocks = (nwaves + 3) / 4;
    hipLaunchKernelGGL((k_gemv_f16<RCG, RPW, 4>), dim3(blocks), dim3(256), 0, st, X, W, Y, N, K,
                       nwaves, N / nwaves, N % nwaves);
    return hipGetLastError();
}

template <int RCG>
hipError_t launch_f16_c(const uint16_t* X, const uint16_t* W, uint16_t* Y, int N, int K, int rpw,
                        hipStream_t st)
{
    const int nwaves = (N + rpw - 1) / rpw;
    switch (rpw) {
    case 1: return launch_f16_r<RCG, 1>(X, W, Y, N, K, nwaves, st);
    case 2: return launch_f16_r<RCG, 2>(X, W, Y, N, K, nwaves, st);
    case 4: return launch_f16_r<RCG, 4>(X, W, Y, N, K, nwaves, st);
    default: return hipErrorInvalidValue;
    }
}

template <int RCG, int RPW>
hipError_t launch_w4f_r(const float* X, const uint8_t* Wq, const float* s, float* Y, int N, int K,
                        int nwaves, hipStream_t st)
{
    const TileLayout L = tile_layout(4, N, K);
    const int blocks = (nwaves + 3) / 4;
    hipLaunchKernelGGL((k_gemv_w4f<RCG, RPW, 4>), dim3(blocks), dim3(256), 0, st, X, Wq, s, Y, N,
                       K, L.cg, nwaves, L.nrg / nwaves, L.nrg % nwaves);
    return hipGetLastError();
}

template <int RCG>
hipError_t launch_w4f_c(const float* X, const uint8_t* Wq, const float* s, float* Y, int N, int K,
                        int rpw, hipStream_t st)
{
    const int nrg = (N + 3) / 4;
    const int nwaves = (nrg + rpw - 1) / rpw;
    switch (rpw) {
    case 1: return launch_w4f_r<RCG, 1>(X, Wq, s, Y, N, K, nwaves, st);
    case 2: return launch_w4f_r<RCG, 2>(X, Wq, s, Y, N, K, nwaves, st);
    case 4: return launch_w4f_r<RCG, 4>(X, Wq, s, Y, N, K, nwaves, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv_f16(const uint16_t* X, const uint16_t* W, uint16_t* Y, int N, int K,
                           int rpw, hipStream_t st)
{
    switch ((K + 511) / 512) {
    case 1: return launch_f16_c<1>(X, W, Y, N, K, rpw, st);
    case 2: return launch_f16_c<2>(X, W, Y, N, K, rpw, st);
    case 3: return launch_f16_c<3>(X, W, Y, N, K, rpw, st);
    case 4: return launch_f16_c<4>(X, W, Y, N, K, rpw, st);
    case 5: return launch_f16_c<5>(X, W, Y, N, K, rpw, st);
    case 6: return launch_f16_c<6>(X, W, Y, N, K, rpw, st);
    case 7: return launch_f16_c<7>(X, W, Y, N, K, rpw, st);
    case 8: return launch_f16_c<8>(X, W, Y, N, K, rpw, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_w4f32(const float* X, const uint8_t* Wq, const float* s, float* Y, int N,
                             int K, int rpw, hipStream_t st)
{
    switch ((K + 511) / 512) {
    case 1: return launch_w4f_c<1>(X, Wq, s, Y, N, K, rpw, st);
    case 2: return launch_w4f_c<2>(X, Wq, s, Y, N, K, rpw, st);
    case 3: return launch_w4f_c<3>(X, Wq, s, Y, N, K, rpw, st);
    case 4: return launch_w4f_c<4>(X, Wq, s, Y, N, K, rpw, st);
    case 5: return launch_w4f_c<5>(X, Wq, s, Y, N, K, rpw, st);
    case 6: return launch_w4f_c<6>(X, Wq, s, Y, N, K, rpw, st);
    case 7: return launch_w4f_c<7>(X, Wq, s, Y, N, K, rpw, st);
    case 8: return launch_w4f_c<8>(X, Wq, s, Y, N, K, rpw, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qw
