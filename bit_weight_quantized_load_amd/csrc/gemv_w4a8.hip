// W4A8 GEMV for decode (M < 16): INT4 weights, INT8 activations quantized in the
// prologue, int8 dot products into int32, output acc * w_scale * a_scale.
//
// What is computed follows "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s":
// section 正确方向 (INT4 widened to int8 lanes in registers, 4-way int8 dot into
// int32) and section 当前实现方式 (row-wise weight scale, per-vector dynamic
// activation scale, output = int32 acc * weight_scale * activation_scale).  The
// page's first follow-up item (fold the activation quantization into the linear
// kernel) is realised by the prologue below.
//
// Work split.  A chunk is 16 bytes = 32 INT4 weights of one row.  Sixteen lanes
// (one DPP row) cover 16*CPL consecutive chunks of a row: one K slice.  A wave
// handles four rows at a time (one per DPP row) and rows_per_wave rows in all; a
// 256-thread workgroup is four waves, so it owns a tile of 4*rows_per_wave rows by
// one K slice.  grid = (row blocks, K slices, M tiles).
//
// Prologue.  Every workgroup takes max|X[m,:]| over the whole row (the scale needs
// it), then quantizes only its own K slice into LDS, in the order the unpack below
// consumes it: for each 8 consecutive k, the even-k codes form one 32-bit word and
// the odd-k codes the next.  Each lane then copies the codes of its chunks into
// registers, where they stay for every row it visits.
//
// Unpack.  A 32-bit word of packed weights holds k..k+7, even k in the low
// nibbles.  (w << 4) & 0xF0F0F0F0 puts the even nibbles, and w & 0xF0F0F0F0 the odd
// nibbles, into the top half of each byte: each byte is then 16*q as an int8, so
// two 4-way dots against the even and odd activation words accumulate 16 * sum(q*x)
// exactly; an arithmetic shift by 4 at the end is exact.  |16 * acc| stays below
// 2^31 for K <= 131072.  That is three bit operations and two dots per 8 weights.
//
// Split K.  With more than one K slice each workgroup adds its int32 partial sums
// to acc_ws with atomics (exact, so the order does not matter), then counts itself
// done on its row block; the last one applies the epilogue and clears acc_ws and
// the counter, leaving the workspace zeroed for the next call.
#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

template <int MT, int CPL, int GB, bool kSplit, bool kDebug>
__global__ __launch_bounds__(kBlock) void k_gemv_w4a8(W4A8Args p)
{
    constexpr int kSlice = 16 * CPL;  // chunks per K slice
    __shared__ uint4 s_act[MT][kSlice][2];
    __shared__ float s_red[MT][4];
    __shared__ float s_a[MT];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, sub = lane >> 4;
    const int M = p.M, N = p.N, K = p.K;
    const int m0 = blockIdx.z * MT;
    const int chunks_per_row = K >> 5;
    const int c0 = blockIdx.y * kSlice;
    const int cs = min(kSlice, chunks_per_row - c0);
    const int rows_per_block = 4 * p.rows_per_wave;
    const int nb0 = blockIdx.x * rows_per_block;

    // ---- prologue 1: activation scale a[m] = max|X[m,:]| / 127 over the whole row
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
        float mx = 0.0f;
        if (m0 + mm < M) {
            const float4* xr = reinterpret_cast<const float4*>(p.X + (size_t)(m0 + mm) * K);
            for (int i = tid; i < (K >> 2); i += kBlock)
                mx = fmaxf(mx, max_abs4(xr[i]));
        }
        mx = wave_max(mx);
        if (lane == 0)
            s_red[mm][wave] = mx;
    }
    __syncthreads();
    if (tid < MT) {
        const float mx = fmaxf(fmaxf(s_red[tid][0], s_red[tid][1]), fmaxf(s_red[tid][2], s_red[tid][3]));
        s_a[tid] = mx / 127.0f;
    }
    __syncthreads();

    // ---- prologue 2: INT8 codes of this K slice into LDS (even/odd k split)
    for (int u = tid; u < MT * cs * 4; u += kBlock) {
        const int mm = u / (cs * 4);
        const int r = u - mm * (cs * 4);
        const int cl = r >> 2, d = r & 3;
        uint32_t ev = 0, od = 0;
        if (m0 + mm < M) {
            const float a = s_a[mm];
            const int k = (c0 + cl) * 32 + d * 8;
            const float4* xp = reinterpret_cast<const float4*>(p.X + (size_t)(m0 + mm) * K + k);
            const float4 v0 = xp[0], v1 = xp[1];
            const int q0 = quant_code(v0.x, a, 127.f), q1 = quant_code(v0.y, a, 127.f);
            const int q2 = quant_code(v0.z, a, 127.f), q3 = quant_code(v0.w, a, 127.f);
            const int q4 = quant_code(v1.x, a, 127.f), q5 = quant_code(v1.y, a, 127.f);
            const int q6 = quant_code(v1.z, a, 127.f), q7 = quant_code(v1.w, a, 127.f);
            ev = pack_i8x4(q0, q2, q4, q6);
            od = pack_i8x4(q1, q3, q5, q7);
            if (kDebug && p.dbg_xq != nullptr && blockIdx.x == 0) {
                uint32_t* dq = reinterpret_cast<uint32_t*>(p.dbg_xq + (size_t)(m0 + mm) * K + k);
                dq[0] = pack_i8x4(q0, q1, q2, q3);
                dq[1] = pack_i8x4(q4, q5, q6, q7);
            }
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(&s_act[mm][cl][0]);
        dst[2 * d] = ev;
        dst[2 * d + 1] = od;
    }
    if (kDebug && p.dbg_a != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && tid < MT &&
        m0 + tid < M)
        p.dbg_a[m0 + tid] = s_a[tid];
    __syncthreads();

    // ---- the lane's activation words, resident in registers for every row
    uint4 act[MT][CPL][2];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int cl = j + 16 * i;
            if (cl < cs) {
                act[mm][i][0] = s_act[mm][cl][0];
                act[mm][i][1] = s_act[mm][cl][1];
            } else {
                act[mm][i][0] = make_uint4(0, 0, 0, 0);
                act[mm][i][1] = make_uint4(0, 0, 0, 0);
            }
        }

    // ---- main loop: stream the packed weights of this wave's rows
    const size_t row_bytes = (size_t)(K >> 1);
    const int nw0 = nb0 + wave * p.rows_per_wave;
    const int groups = p.rows_per_wave >> 2;
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
            int acc[MT];
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
                acc[mm] = 0;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const uint32_t wd[4] = {w[g][i].x, w[g][i].y, w[g][i].z, w[g][i].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int lo = (int)((wd[d] << 4) & 0xF0F0F0F0u);
                    const int hi = (int)(wd[d] & 0xF0F0F0F0u);
#pragma unroll
                    for (int mm = 0; mm < MT; ++mm) {
                        const uint32_t* av = reinterpret_cast<const uint32_t*>(&act[mm][i][0]);
                        acc[mm] = __builtin_amdgcn_sdot4(lo, (int)av[2 * d], acc[mm], false);
                        acc[mm] = __builtin_amdgcn_sdot4(hi, (int)av[2 * d + 1], acc[mm], false);
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
                        const int v = acc[mm] >> 4;
                        const size_t o = (size_t)(m0 + mm) * N + n;
                        if (kSplit) {
                            atomicAdd(&p.acc_ws[o], v);
                        } else {
                            if (kDebug && p.dbg_acc != nullptr)
                                p.dbg_acc[o] = v;
                            p.Y[o] = ((float)v * p.w_scale[n]) * s_a[mm];
                        }
                    }
                }
            }
        }
    }

    // ---- split-K completion: the last workgroup of a row block finishes it
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
                    const int v = atomicExch(&p.acc_ws[o], 0);
                    if (kDebug && p.dbg_acc != nullptr)
                        p.dbg_acc[o] = v;
                    p.Y[o] = ((float)v * p.w_scale[n]) * s_a[mm];
                }
            }
            if (tid == 0)
                atomicExch(&p.counters[cidx], 0u);
        }
    }
}

template <int MT, int CPL, int GB>
hipError_t launch3(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    if constexpr (MT * CPL > 8 || GB * CPL > 16) {
        return hipErrorInvalidValue;
    } else {
        const dim3 grid(t.row_blocks, t.slices, t.m_tiles);
        const bool split = t.slices > 1;
        if (split && debug)
            hipLaunchKernelGGL((k_gemv_w4a8<MT, CPL, GB, true, true>), grid, dim3(kBlock), 0, st, a);
        else if (split)
            hipLaunchKernelGGL((k_gemv_w4a8<MT, CPL, GB, true, false>), grid, dim3(kBlock), 0, st, a);
        else if (debug)
            hipLaunchKernelGGL((k_gemv_w4a8<MT, CPL, GB, false, true>), grid, dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL((k_gemv_w4a8<MT, CPL, GB, false, false>), grid, dim3(kBlock), 0, st, a);
        return hipGetLastError();
    }
}

template <int MT, int CPL>
hipError_t launch2(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    switch (t.gb) {
    case 1: return launch3<MT, CPL, 1>(a, t, debug, st);
    case 2: return launch3<MT, CPL, 2>(a, t, debug, st);
    case 4: return launch3<MT, CPL, 4>(a, t, debug, st);
    case 8: return launch3<MT, CPL, 8>(a, t, debug, st);
    default: return hipErrorInvalidValue;
    }
}

template <int MT>
hipError_t launch1(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    switch (t.cpl) {
    case 1: return launch2<MT, 1>(a, t, debug, st);
    case 2: return launch2<MT, 2>(a, t, debug, st);
    case 4: return launch2<MT, 4>(a, t, debug, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv_w4a8(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st)
{
    switch (t.mt) {
    case 1: return launch1<1>(a, t, debug, st);
    case 2: return launch1<2>(a, t, debug, st);
    case 4: return launch1<4>(a, t, debug, st);
    case 8: return launch1<8>(a, t, debug, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qw
