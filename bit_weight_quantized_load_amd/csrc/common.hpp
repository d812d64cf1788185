// Device helpers shared by the kernels of the weight-quantized decode linear (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace qw {

constexpr int kBlock = 256;  // threads per workgroup: four wave64s

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Sum over the 16 lanes of a DPP row; every lane of the row receives the total.
// Rotations by 8, 4, 2 and 1 within the row add all 16 partial values.
__device__ __forceinline__ int row_sum16(int v)
{
    v += __builtin_amdgcn_mov_dpp(v, 0x128, 0xf, 0xf, false);  // row_ror:8
    v += __builtin_amdgcn_mov_dpp(v, 0x124, 0xf, 0xf, false);  // row_ror:4
    v += __builtin_amdgcn_mov_dpp(v, 0x122, 0xf, 0xf, false);  // row_ror:2
    v += __builtin_amdgcn_mov_dpp(v, 0x121, 0xf, 0xf, false);  // row_ror:1
    return v;
}

__device__ __forceinline__ float row_sum16(float v)
{
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xf, 0xf, false));
    return v;
}

// Maximum over the 64 lanes of a wave (not on the hot loop).
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Maximum over a 256-thread workgroup.  `red` is 4 floats of LDS; every thread
// must call this, and every thread gets the result.
__device__ __forceinline__ float block_max(float v, float* red)
{
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float max_abs4(float4 v)
{
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ bool finite4(float4 v)
{
    return isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w);
}

// Symmetric code of one value: clamp(rint(x / scale), -qmax, qmax), 0 when the
// scale is 0.  The division is the correctly rounded fp32 division (the library is
// built without fast-math) and rintf rounds half to even.  Every quantizer in the
// library goes through this one function, so the fused GEMV prologue and the
// standalone activation quantizer produce the same codes bit for bit.
__device__ __forceinline__ int quant_code(float x, float scale, float qmax)
{
    if (scale == 0.0f)
        return 0;
    float r = rintf(x / scale);
    r = fminf(fmaxf(r, -qmax), qmax);
    return (int)r;
}

__device__ __forceinline__ uint32_t pack_i8x4(int b0, int b1, int b2, int b3)
{
    return (uint32_t)(b0 & 0xff) | ((uint32_t)(b1 & 0xff) << 8) | ((uint32_t)(b2 & 0xff) << 16) |
           ((uint32_t)(b3 & 0xff) << 24);
}

}  // namespace qw
