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

// Byte offset of 32-bit word `wi` (0..3) of chunk `c` of row `n` in the tile layout
// (kernels.hpp) with R rows per tile and L = 64 / R chunks per tile row:
// tile (n / R, c / L), slot (n % R) * L + c % L.
__device__ __forceinline__ size_t tile_word_offset(int n, int c, int wi, int cg, int R)
{
    const int L = 64 / R;
    return ((size_t)(n / R) * cg + (c / L)) * 1024u + (size_t)(((n % R) * L + (c % L)) * 16 + wi * 4);
}

// One workgroup per row (grid-strided): max-abs reduction, then codes.  Eight
// consecutive k per thread give one 32-bit word of nibbles, even k in the low one;
// the word goes to its place in the tile layout.
__global__ __launch_bounds__(kBlock) void k_pack_w4(const float* __restrict__ W, int N, int K,
                                                    uint8_t* __restrict__ Wq,
                                                    float* __restrict__ scale, int* flag)
{
    __shared__ float red[4];
    const int K4 = K >> 2, K8 = K >> 3;
    const int cg = (K + 511) >> 9;
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
        for (int u = threadIdx.x; u < K8; u += kBlock) {
            float4 a = row[2 * u], b = row[2 * u + 1];
            int q[8] = {quant_code(a.x, s, 7.f), quant_code(a.y, s, 7.f), quant_code(a.z, s, 7.f),
                        quant_code(a.w, s, 7.f), quant_code(b.x, s, 7.f), quant_code(b.y, s, 7.f),
                        quant_code(b.z, s, 7.f), quant_code(b.w, s, 7.f)};
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                word |= (uint32_t)(q[i] & 0xf) << (4 * i);
            *reinterpret_cast<uint32_t*>(Wq + tile_word_offset(n, u >> 2, u & 3, cg, 4)) = word;
        }
    }
}

// Group-wise INT4 (the INT4 write-up, section 后续优化方向, lists group-wise scales as
// future work): the row-wise rule applied to each group of g consecutive k (g = 32 ..
// 512, K a multiple of g), one fp32 scale per output row and group.  One workgroup per
// row; the g / 8 threads of a group (each holding 8 consecutive k, one word of nibbles)
// take the group's maximum with cross-lane exchanges (a group never straddles a wave).
// Scales go to the device layout of w4g_scale_index (kernels.hpp).  A row with a
// non-finite weight raises the flag and keeps the zero scales the buffer was cleared to.
__global__ __launch_bounds__(kBlock) void k_pack_w4g(const float* __restrict__ W, int N, int K,
                                                     int g, uint8_t* __restrict__ Wq,
                                                     float* __restrict__ scale, int* flag)
{
    const int K4 = K >> 2, K8 = K >> 3;
    const int cg = (K + 511) >> 9;
    const int tpg = g >> 3;  // threads per group
    for (int n = blockIdx.x; n < N; n += gridDim.x) {
        const float4* row = reinterpret_cast<const float4*>(W + (size_t)n * K);
        int bad = 0;
        for (int i = threadIdx.x; i < K4; i += kBlock)
            bad |= !finite4(row[i]);
        bad = __syncthreads_or(bad);
        if (bad) {
            if (threadIdx.x == 0)
                atomicOr(flag, 1);
            continue;
        }
        for (int u = threadIdx.x; u < K8; u += kBlock) {
            const float4 a = row[2 * u], b = row[2 * u + 1];
            float mx = fmaxf(max_abs4(a), max_abs4(b));
            for (int off = 1; off < tpg; off <<= 1)
                mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            const float s = mx / 7.0f;
            if ((u & (tpg - 1)) == 0)
                scale[w4g_scale_index(n, 8 * u, g, cg)] = s;
            const int q[8] = {quant_code(a.x, s, 7.f), quant_code(a.y, s, 7.f), quant_code(a.z, s, 7.f),
                              quant_code(a.w, s, 7.f), quant_code(b.x, s, 7.f), quant_code(b.y, s, 7.f),
                              quant_code(b.z, s, 7.f), quant_code(b.w, s, 7.f)};
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                word |= (uint32_t)(q[i] & 0xf) << (4 * i);
            *reinterpret_cast<uint32_t*>(Wq + tile_word_offset(n, u >> 2, u & 3, cg, 4)) = word;
        }
    }
}

// Device layout of group scales -> canonical [N][K / g].
__global__ __launch_bounds__(kBlock) void k_w4g_scales(const float* __restrict__ scale, int N,
                                                       int K, int g, float* __restrict__ out)
{
    const int G = K / g, cg = (K + 511) >> 9;
    const size_t total = (size_t)N * G;
    for (size_t i = blockIdx.x * (size_t)kBlock + threadIdx.x; i < total;
         i += (size_t)gridDim.x * kBlock) {
        const int n = (int)(i / G), t = (int)(i % G);
        out[i] = scale[w4g_scale_index(n, t * g, g, cg)];
    }
}

// Per-channel INT8: s32 = maxabs/127, rounded to the stored f16 scale, and codes
// taken against that stored scale.
__global__ __launch_bounds__(kBlock) void k_pack_w8(const float* __restrict__ W, int N, int K,
                                                    uint8_t* __restrict__ Wq,
                                                    uint16_t* __restrict__ scale, int* flag)
{
    __shared__ float red[4];
    const int K4 = K >> 2;
    const int cg = (K + 511) >> 9;
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
        for (int i = threadIdx.x; i < K4; i += kBlock) {
            float4 v = row[i];
            *reinterpret_cast<uint32_t*>(Wq + tile_word_offset(n, i >> 2, i & 3, cg, 2)) =
                pack_i8x4(quant_code(v.x, sf, 127.f), quant_code(v.y, sf, 127.f),
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
        const float r = 1.0f / a;
        const bool fast = r <= 3.0e38f;
        if (threadIdx.x == 0)
            a_scale[m] = a;
        uint32_t* out = reinterpret_cast<uint32_t*>(Xq + (size_t)m * K);
        for (int i = threadIdx.x; i < K4; i += kBlock) {
            // four codes per step in byte 2 of e[0 .. 3], by the reciprocal unless one of
            // the four lies near a rounding boundary
            const float4 v = row[i];
            uint32_t e[4];
            if (quant4_e(v, r, e) || !fast)
                quant4_e_div(v, a, e);
            out[i] = __builtin_amdgcn_perm(e[1], e[0], 0x0C0C0602u) | __builtin_amdgcn_perm(e[3], e[2], 0x06020C0Cu);
        }
    }
}

// Tile-layout INT4 -> int8 codes [N][K]: one thread per 32-bit word (8 codes).
__global__ __launch_bounds__(kBlock) void k_codes_w4(const uint8_t* __restrict__ Wq, int N, int K,
                                                     int8_t* __restrict__ codes)
{
    const int words = K >> 3, cg = (K + 511) >> 9;
    const size_t total = (size_t)N * words;
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < total;
         i += (size_t)gridDim.x * kBlock) {
        const int n = (int)(i / words), u = (int)(i % words);
        const uint32_t w = *reinterpret_cast<const uint32_t*>(Wq + tile_word_offset(n, u >> 2, u & 3, cg, 4));
        int8_t* out = codes + (size_t)n * K + 8 * u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int v = (w >> (4 * e)) & 0xf;
            out[e] = (int8_t)(v >= 8 ? v - 16 : v);
        }
    }
}

// Tile-layout INT8 -> int8 codes [N][K]: one thread per 32-bit word (4 codes).
__global__ __launch_bounds__(kBlock) void k_codes_w8(const uint8_t* __restrict__ Wq, int N, int K,
                                                     int8_t* __restrict__ codes)
{
    const int words = K >> 2, cg = (K + 511) >> 9;
    const size_t total = (size_t)N * words;
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < total;
         i += (size_t)gridDim.x * kBlock) {
        const int n = (int)(i / words), u = (int)(i % words);
        *reinterpret_cast<uint32_t*>(codes + (size_t)n * K + 4 * u) =
            *reinterpret_cast<const uint32_t*>(Wq + tile_word_offset(n, u >> 2, u & 3, cg, 2));
    }
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

// Padding (rows past N in the last row group, chunks past K in the last chunk
// group) exists only for ragged shapes; it is cleared before packing so the packed
// buffer is fully defined.
static hipError_t clear_padding(int bits, int N, int K, uint8_t* Wq, hipStream_t st)
{
    const TileLayout t = tile_layout(bits, N, K);
    if (N % t.rows == 0 && K % 512 == 0)
        return hipSuccess;
    return launch_fill_zero(reinterpret_cast<uint32_t*>(Wq), packed_bytes(bits, N, K) / 4, st);
}

hipError_t launch_pack_w4(const float* W, int N, int K, uint8_t* Wq, float* s, int* flag,
                          hipStream_t st)
{
    hipError_t e = clear_padding(4, N, K, Wq, st);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_pack_w4, dim3(N < kMaxGrid ? N : kMaxGrid), dim3(kBlock), 0, st, W, N, K,
                       Wq, s, flag);
    return hipGetLastError();
}

hipError_t launch_pack_w4g(const float* W, int N, int K, int g, uint8_t* Wq, float* s,
                           int* flag, hipStream_t st)
{
    hipError_t e = clear_padding(4, N, K, Wq, st);
    if (e == hipSuccess)
        e = launch_fill_zero(reinterpret_cast<uint32_t*>(s), w4g_scale_floats(N, K, g), st);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_pack_w4g, dim3(N < kMaxGrid ? N : kMaxGrid), dim3(kBlock), 0, st, W, N, K,
                       g, Wq, s, flag);
    return hipGetLastError();
}

hipError_t launch_w4g_scales(const float* s, int N, int K, int g, float* out, hipStream_t st)
{
    const size_t total = (size_t)N * (size_t)(K / g);
    hipLaunchKernelGGL(k_w4g_scales, dim3(grid_for(total)), dim3(kBlock), 0, st, s, N, K, g, out);
    return hipGetLastError();
}

hipError_t launch_pack_w8(const float* W, int N, int K, uint8_t* Wq, uint16_t* s, int* flag,
                          hipStream_t st)
{
    hipError_t e = clear_padding(8, N, K, Wq, st);
    if (e != hipSuccess)
        return e;
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
    const size_t words = (size_t)N * (size_t)(K / 8);
    hipLaunchKernelGGL(k_codes_w4, dim3(grid_for(words)), dim3(kBlock), 0, st, Wq, N, K, codes);
    return hipGetLastError();
}

hipError_t launch_codes_w8(const uint8_t* Wq, int N, int K, int8_t* codes, hipStream_t st)
{
    const size_t words = (size_t)N * (size_t)(K / 4);
    hipLaunchKernelGGL(k_codes_w8, dim3(grid_for(words)), dim3(kBlock), 0, st, Wq, N, K, codes);
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
