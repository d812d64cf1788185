// Load-time weight packers, the standalone activation quantizer and small helpers.
//
// Row-wise INT4 weights with one scale per row and dynamic INT8 activations follow
// "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s", section 当前实现方式.
// Per-channel INT8 weights with an f16 scale follow the ChatGLM2-6B W8A16 write-up
// (TPU-MLIR), sections 2 and 3.
#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

constexpr int kMaxGrid = 65536;

// One workgroup per row (grid-strided): max-abs reduction, then codes.  Eight
// consecutive k per thread give one 32-bit word of nibbles, even k in the low one.
__global__ __launch_bounds__(kBlock) void k_pack_w4(const float* __restrict__ W, int N, int K,
                                                    uint8_t* __restrict__ Wq,
                                                    float* __restrict__ scale, int* flag)
{
    __shared__ float red[4];
    const int K4 = K >> 2, K8 = K >> 3;
    for (int n = blockIdx.x; n < N; n += gridDim.x) {
        const float4* row = reinterpret_cast<const float4*>(W + (size_t)n * K);
        float mx = 0.0f;
        int bad = 0;
        for (int i = threadIdx.x; i < K4; i += kBlock) {
            float4 v = row[i];
            bad |= !finite4(v);
            mx = fmaxf(mx, max_abs4(v));
        }
        bad = __syncthreads_or(bad);
        mx = block_max(mx, red);
        if (bad) {
            if (threadIdx.x == 0) {
                atomicOr(flag, 1);
                scale[n] = 0.0f;
            }
            continue;
        }
        const float s = mx / 7.0f;
        if (threadIdx.x == 0)
            scale[n] = s;
        uint32_t* out = reinterpret_cast<uint32_t*>(Wq + (size_t)n * (K >> 1));
        for (int u = threadIdx.x; u < K8; u += kBlock) {
            float4 a = row[2 * u], b = row[2 * u + 1];
            int q[8] = {quant_code(a.x, s, 7.f), quant_code(a.y, s, 7.f), quant_code(a.z, s, 7.f),
                        quant_code(a.w, s, 7.f), quant_code(b.x, s, 7.f), quant_code(b.y, s, 7.f),
                        quant_code(b.z, s, 7.f), quant_code(b.w, s, 7.f)};
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                word |= (uint32_t)(q[i] & 0xf) << (4 * i);
            out[u] = word;
        }
    }
}

// Per-channel INT8: s32 = maxabs/127, rounded to the stored f16 scale, and codes
// taken against that stored scale.
__global__ __launch_bounds__(kBlock) void k_pack_w8(const float* __restrict__ W, int N, int K,
                                                    int8_t* __restrict__ Wq,
                                                    uint16_t* __restrict__ scale, int* flag)
{
    __shared__ float red[4];
    const int K4 = K >> 2;
    for (int n = blockIdx.x; n < N; n += gridDim.x) {
        const float4* row = reinterpret_cast<const float4*>(W + (size_t)n * K);
        float mx = 0.0f;
        int bad = 0;
        for (int i = threadIdx.x; i < K4; i += kBlock) {
            float4 v = row[i];
            bad |= !finite4(v);
            mx = fmaxf(mx, max_abs4(v));
        }
        bad = __syncthreads_or(bad);
        mx = block_max(mx, red);
        const float s32 = mx / 127.0f;
        const __half h = __float2half_rn(s32);
        const float sf = __half2float(h);
        if (bad || isinf(sf)) {
            if (threadIdx.x == 0) {
                atomicOr(flag, 1);
                scale[n] = 0;
            }
            continue;
        }
        if (threadIdx.x == 0)
            scale[n] = __half_as_ushort(h);
        uint32_t* out = reinterpret_cast<uint32_t*>(Wq + (size_t)n * K);
        for (int i = threadIdx.x; i < K4; i += kBlock) {
            float4 v = row[i];
            out[i] = pack_i8x4(quant_code(v.x, sf, 127.f), quant_code(v.y, sf, 127.f),
                               quant_code(v.z, sf, 127.f), quant_code(v.w, sf, 127.f));
        }
    }
}

// Standalone dynamic activation quantization: one workgroup per row of X.
__global__ __launch_bounds__(kBlock) void k_quant_act(const float* __restrict__ X, int M, int K,
                                                      int8_t* __restrict__ Xq,
                                                      float* __restrict__ a_scale)
{
    __shared__ float red[4];
    const int K4 = K >> 2;
    for (int m = blockIdx.x; m < M; m += gridDim.x) {
        const float4* row = reinterpret_cast<const float4*>(X + (size_t)m * K);
        float mx = 0.0f;
        for (int i = threadIdx.x; i < K4; i += kBlock)
            mx = fmaxf(mx, max_abs4(row[i]));
        mx = block_max(mx, red);
        const float a = mx / 127.0f;
        if (threadIdx.x == 0)
            a_scale[m] = a;
        uint32_t* out = reinterpret_cast<uint32_t*>(Xq + (size_t)m * K);
        for (int i = threadIdx.x; i < K4; i += kBlock) {
            float4 v = row[i];
            out[i] = pack_i8x4(quant_code(v.x, a, 127.f), quant_code(v.y, a, 127.f),
                               quant_code(v.z, a, 127.f), quant_code(v.w, a, 127.f));
        }
    }
}

// Packed INT4 -> int8 codes, one thread per packed byte (sign-extended nibbles).
__global__ __launch_bounds__(kBlock) void k_codes_w4(const uint8_t* __restrict__ Wq, size_t nbytes,
                                                     int8_t* __restrict__ codes)
{
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < nbytes;
         i += (size_t)gridDim.x * kBlock) {
        const int b = Wq[i];
        const int lo = b & 0xf, hi = b >> 4;
        codes[2 * i] = (int8_t)(lo >= 8 ? lo - 16 : lo);
        codes[2 * i + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
    }
}

__global__ __launch_bounds__(kBlock) void k_copy_bytes(const int8_t* __restrict__ src, size_t n,
                                                       int8_t* __restrict__ dst)
{
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (size_t)gridDim.x * kBlock)
        dst[i] = src[i];
}

__global__ __launch_bounds__(kBlock) void k_fill_zero(uint32_t* __restrict__ p, size_t words)
{
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < words;
         i += (size_t)gridDim.x * kBlock)
        p[i] = 0u;
}

inline int grid_for(size_t items)
{
    size_t g = (items + kBlock - 1) / kBlock;
    if (g < 1)
        g = 1;
    return (int)(g > (size_t)kMaxGrid ? kMaxGrid : g);
}

}  // namespace

hipError_t launch_pack_w4(const float* W, int N, int K, uint8_t* Wq, float* s, int* flag,
                          hipStream_t st)
{
    hipLaunchKernelGGL(k_pack_w4, dim3(N < kMaxGrid ? N : kMaxGrid), dim3(kBlock), 0, st, W, N, K,
                       Wq, s, flag);
    return hipGetLastError();
}

hipError_t launch_pack_w8(const float* W, int N, int K, int8_t* Wq, uint16_t* s, int* flag,
                          hipStream_t st)
{
    hipLaunchKernelGGL(k_pack_w8, dim3(N < kMaxGrid ? N : kMaxGrid), dim3(kBlock), 0, st, W, N, K,
                       Wq, s, flag);
    return hipGetLastError();
}

hipError_t launch_quant_act(const float* X, int M, int K, int8_t* Xq, float* a, hipStream_t st)
{
    hipLaunchKernelGGL(k_quant_act, dim3(M < kMaxGrid ? M : kMaxGrid), dim3(kBlock), 0, st, X, M,
                       K, Xq, a);
    return hipGetLastError();
}

hipError_t launch_codes_w4(const uint8_t* Wq, int N, int K, int8_t* codes, hipStream_t st)
{
    const size_t nbytes = (size_t)N * (size_t)(K / 2);
    hipLaunchKernelGGL(k_codes_w4, dim3(grid_for(nbytes)), dim3(kBlock), 0, st, Wq, nbytes, codes);
    return hipGetLastError();
}

hipError_t launch_codes_w8(const int8_t* Wq, int N, int K, int8_t* codes, hipStream_t st)
{
    const size_t n = (size_t)N * (size_t)K;
    hipLaunchKernelGGL(k_copy_bytes, dim3(grid_for(n)), dim3(kBlock), 0, st, Wq, n, codes);
    return hipGetLastError();
}

hipError_t launch_fill_zero(uint32_t* p, size_t words, hipStream_t st)
{
    if (words == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(words)), dim3(kBlock), 0, st, p, words);
    return hipGetLastError();
}

}  // namespace qw
