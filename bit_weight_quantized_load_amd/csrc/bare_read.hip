// A plain streaming read of device memory: the bandwidth reference for the GEMV kernels.
// The weight-quantized decode linear is bound by the time to stream its weights from HBM
// ("Jetson Orin AGX 上的 INT4 量化推理实践", section 为什么这个结果有意义: decode is
// memory-bound and dominated by GEMV), so the fastest a GEMV of B weight bytes can run is
// the time a kernel that only reads B bytes takes.  This kernel reads every byte once with
// 16-byte loads (the non-temporal hint of the weight stream) and folds them into one
// 32-bit word per workgroup, so the loads cannot be dropped; it computes nothing else.
//
// Work split: `blocks` workgroups of `waves` waves; workgroup b owns an even share of the
// 16-byte words (the first `rem` get one more), read as batches of U loads per lane, all U
// requested before any is used.  Past the end, buffer loads return zeros.
#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

template <int U>
__global__ __launch_bounds__(1024) void k_stream_read(const uint8_t* __restrict__ src, int per,
                                                      int rem, uint32_t* __restrict__ sink)
{
    const int b = blockIdx.x;
    const int w0 = rg_of(b, per, rem);              // first 16-byte word of the workgroup
    const int nw = rg_of(b + 1, per, rem) - w0;     // words of the workgroup
    const rsrc_t r = make_rsrc(src + (size_t)w0 * 16u, (uint32_t)nw * 16u);
    const int T = (int)blockDim.x;
    uint32_t acc = 0;
    for (int base = 0; base < nw; base += U * T) {
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
    const int per = (int)(words / (size_t)blocks), rem = (int)(words % (size_t)blocks);
    const dim3 g(blocks), t(64 * waves);
    switch (u) {
    case 1: hipLaunchKernelGGL(k_stream_read<1>, g, t, 0, st, src, per, rem, sink); break;
    case 2: hipLaunchKernelGGL(k_stream_read<2>, g, t, 0, st, src, per, rem, sink); break;
    case 4: hipLaunchKernelGGL(k_stream_read<4>, g, t, 0, st, src, per, rem, sink); break;
    case 8: hipLaunchKernelGGL(k_stream_read<8>, g, t, 0, st, src, per, rem, sink); break;
    case 16: hipLaunchKernelGGL(k_stream_read<16>, g, t, 0, st, src, per, rem, sink); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qw
