// W8A16 GEMV for decode (M < 16): per-channel INT8 weights dequantized in
// registers against f16 activations, fp32 accumulation, f16 output.
//
// What is computed follows the ChatGLM2-6B W8A16 write-up (TPU-MLIR): section 2
// (weights stored per channel as INT8, computed in F16) and section 4 (load the
// INT8 weight, cast it to F16, apply the scale, multiply with the activation).
// The scale belongs to the output channel, so it is applied once to the finished
// sum instead of to each weight; that differs from scaling first only by fp32
// rounding.
//
// Work split as in the W4A8 kernel: a chunk is 16 bytes = 16 INT8 weights; 16
// lanes cover 16*CPL chunks of a row (one K slice); a wave handles four rows at a
// time; a workgroup is four waves.  Each lane loads the f16 activations of its
// chunks into registers once and keeps them for every row it visits.
//
// Cast.  For a word of four int8 codes, XOR 0x80 per byte gives u = q + 128; a
// byte permute places 0x64 above each u, which as a binary16 is exactly 1024 + u;
// one packed f16 add of -1152 leaves q exactly.  Two 2-way f16 dots with fp32
// accumulation then consume the four weights.
//
// Split K.  Each workgroup stores its fp32 partial sums to part_ws[slice]; the last
// workgroup of a row block (by counter) adds the slices in slice order, so the
// result does not depend on scheduling, and zeroes the partials and the counter.
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

template <int MT, int CPL, int GB, bool kSplit>
__global__ __launch_bounds__(kBlock) void k_gemv_w8a16(W8A16Args p)
{
    constexpr int kSlice = 16 * CPL;
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, sub = lane >> 4;
    const int M = p.M, N = p.N, K = p.K;
    const int m0 = blockIdx.z * MT;
    const int chunks_per_row = K >> 4;
    const int c0 = blockIdx.y * kSlice;
    const int cs = min(kSlice, chunks_per_row - c0);
    const int rows_per_block = 4 * p.rows_per_wave;
    const int nb0 = blockIdx.x * rows_per_block;

    // the lane's activations: 16 f16 per chunk = 8 words, kept in registers
    uint4 act[MT][CPL][2];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int cl = j + 16 * i;
            if (cl < cs && m0 + mm < M) {
                const uint4* xp = reinterpret_cast<const uint4*>(p.X + (size_t)(m0 + mm) * K +
                                                                 (size_t)(c0 + cl) * 16);
                act[mm][i][0] = xp[0];
                act[mm][i][1] = xp[1];
            } else {
                act[mm][i][0] = make_uint4(0, 0, 0, 0);
                act[mm][i][1] = make_uint4(0, 0, 0, 0);
            }
        }

    const size_t row_bytes = (size_t)K;
    const int nw0 = nb0 + wave * p.rows_per_wave;
    const int groups = p.rows_per_wave >> 2;
    const size_t MN = (size_t)M * N;
    for (int g0 = 0; g0 < groups; g0 += GB) {
        uint4 w[GB][CPL];
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            const int n = nw0 + 4 * (g0 + g) + sub;
            const uint8_t* wp = p.Wq + (size_t)n * row_bytes + (size_t)c0 * 16;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int cl = j + 16 * i;
                if (n < N && cl < cs)
                    w[g][i] = *reinterpret_cast<const uint4*>(wp + (size_t)cl * 16);
                else
                    w[g][i] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            float acc[MT];
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
                acc[mm] = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const uint32_t wd[4] = {w[g][i].x, w[g][i].y, w[g][i].z, w[g][i].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    half2_t lo, hi;
                    cast_i8x4_to_f16(wd[d], lo, hi);
#pragma unroll
                    for (int mm = 0; mm < MT; ++mm) {
                        const uint32_t* av = reinterpret_cast<const uint32_t*>(&act[mm][i][0]);
                        acc[mm] = __builtin_amdgcn_fdot2(lo, __builtin_bit_cast(half2_t, av[2 * d]),
                                                         acc[mm], false);
                        acc[mm] = __builtin_amdgcn_fdot2(
                            hi, __builtin_bit_cast(half2_t, av[2 * d + 1]), acc[mm], false);
                    }
                }
            }
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
                acc[mm] = row_sum16(acc[mm]);
            const int n = nw0 + 4 * (g0 + g) + sub;
            if (j == 0 && n < N) {
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) {
                    if (m0 + mm < M) {
                        const size_t o = (size_t)(m0 + mm) * N + n;
                        if (kSplit) {
                            p.part_ws[(size_t)blockIdx.y * MN + o] = acc[mm];
                        } else {
                            const float s = __half2float(__ushort_as_half(p.w_scale[n]));
                            p.Y[o] = __half_as_ushort(__float2half_rn(acc[mm] * s));
                        }
                    }
                }
            }
        }
    }

    if (kSplit) {
        __threadfence();
        __syncthreads();
        const unsigned cidx = blockIdx.z * gridDim.x + blockIdx.x;
        if (tid == 0) {
            const unsigned prev = atomicAdd(&p.counters[cidx], 1u);
            s_last = (prev == gridDim.y - 1) ? 1 : 0;
        }
        __syncthreads();
        if (s_last) {
            __threadfence();
            for (int idx = tid; idx < MT * rows_per_block; idx += kBlock) {
                const int mm = idx / rows_per_block;
                const int n = nb0 + (idx - mm * rows_per_block);
                if (m0 + mm < M && n < N) {
                    const size_t o = (size_t)(m0 + mm) * N + n;
                    float sum = 0.0f;
                    for (int z = 0; z < (int)gridDim.y; ++z) {
                        sum += p.part_ws[(size_t)z * MN + o];
                        p.part_ws[(size_t)z * MN + o] = 0.0f;
                    }
                    const float s = __half2float(__ushort_as_half(p.w_scale[n]));
                    p.Y[o] = __half_as_ushort(__float2half_rn(sum * s));
                }
            }
            if (tid == 0)
                atomicExch(&p.counters[cidx], 0u);
        }
    }
}

template <int MT, int CPL, int GB>
hipError_t launch3(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    if constexpr (MT * CPL > 8 || GB * CPL > 16) {
        return hipErrorInvalidValue;
    } else {
        const dim3 grid(t.row_blocks, t.slices, t.m_tiles);
        if (t.slices > 1)
            hipLaunchKernelGGL((k_gemv_w8a16<MT, CPL, GB, true>), grid, dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL((k_gemv_w8a16<MT, CPL, GB, false>), grid, dim3(kBlock), 0, st, a);
        return hipGetLastError();
    }
}

template <int MT, int CPL>
hipError_t launch2(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.gb) {
    case 1: return launch3<MT, CPL, 1>(a, t, st);
    case 2: return launch3<MT, CPL, 2>(a, t, st);
    case 4: return launch3<MT, CPL, 4>(a, t, st);
    case 8: return launch3<MT, CPL, 8>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

template <int MT>
hipError_t launch1(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.cpl) {
    case 1: return launch2<MT, 1>(a, t, st);
    case 2: return launch2<MT, 2>(a, t, st);
    case 4: return launch2<MT, 4>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv_w8a16(const W8A16Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.mt) {
    case 1: return launch1<1>(a, t, st);
    case 2: return launch1<2>(a, t, st);
    case 4: return launch1<4>(a, t, st);
    case 8: return launch1<8>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qw
