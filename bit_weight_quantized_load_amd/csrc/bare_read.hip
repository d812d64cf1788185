// A plain streaming read of device memory: the bandwidth reference for the GEMV kernels.
// The weight-quantized decode linear is bound by the time to stream its weights from HBM
// ("Jetson Orin AGX 上的 INT4 量化推理实践", section 为什么这个结果有意义: decode is
// memory-bound and dominated by GEMV), so the fastest a GEMV of B weight bytes can run is
// the time a kernel that only reads B bytes takes.  This kernel reads every byte once with
// 16-byte loads (the non-temporal hint of the weight stream) and folds them into one
// 32-bit word per workgroup, so the loads cannot be dropped; it computes nothing else.
//
// Work split: `blocks` workgroups of `waves` waves read batches of U loads per lane, all U
// requested before any is used; batch i of workgroup b is the (i blocks + b)-th run of
// U x (threads) 16-byte words, so that the grid sweeps the buffer as one moving window
// (2-4% faster than an even contiguous share per workgroup: 34 MB in 7.05 against 7.20
// us, 68 MB in 11.54 against 11.92, 112 MB in 17.7 against 18.5).  Past the end, buffer
// loads return zeros.
#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

template <int U>
__global__ __launch_bounds__(1024) void k_stream_read(const uint8_t* __restrict__ src, int words,
                                                      uint32_t* __restrict__ sink)
{
    const int b = blockIdx.x;
    const int T = (int)blockDim.x;
    const rsrc_t r = make_rsrc(src, (uint32_t)words * 16u);
    const int step = (int)gridDim.x * U * T;  // words per sweep of the grid
    uint32_t acc = 0;
    for (int base = b * U * T; base < words; base += step) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = load16_stream(r, (uint32_t)(base + u * T + (int)threadIdx.x) * 16u);
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // one word per workgroup: the XOR over its lanes' words
    for (int off = 32; off > 0; off >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    __shared__ uint32_t red[16];
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int w = 0; w < T / 64; ++w)
            x ^= red[w];
        sink[b] = x;
    }
}

}  // namespace

hipError_t launch_stream_read(const uint8_t* src, size_t words, int waves, int blocks, int u,
                              uint32_t* sink, hipStream_t st)
{
    const int w = (int)words;
    const dim3 g(blocks), t(64 * waves);
    switch (u) {
    case 1: hipLaunchKernelGGL(k_stream_read<1>, g, t, 0, st, src, w, sink); break;
    case 2: hipLaunchKernelGGL(k_stream_read<2>, g, t, 0, st, src, w, sink); break;
    case 4: hipLaunchKernelGGL(k_stream_read<4>, g, t, 0, st, src, w, sink); break;
    case 8: hipLaunchKernelGGL(k_stream_read<8>, g, t, 0, st, src, w, sink); break;
    case 16: hipLaunchKernelGGL(k_stream_read<16>, g, t, 0, st, src, w, sink); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qw
