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

// Logical block of hardware block b out of G.  Workgroup b runs on XCD b % 8; this
// numbers each XCD's blocks contiguously, so logical neighbours share an L2 (and, being
// dispatched in order, run at about the same time).
__device__ __forceinline__ int xcd_block(int b, int G)
{
    const int per = (G + 7) / 8, r = G % 8;
    const int x = b % 8, i = b / 8;
    if (r == 0 || x < r)
        return x * per + i;
    return r * per + (x - r) * (per - 1) + i;
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

// Maximum of non-negative values over the 64 lanes of a wave with DPP: rotations
// within each 16-lane row, then row 0 -> 1 and row 2 -> 3 (row_bcast:15), then
// row 1 -> rows 2, 3 (row_bcast:31); lane 63 ends with the maximum.  Rows outside a
// broadcast's row mask keep the `old` operand, 0, which is harmless for a maximum
// of non-negative values.
__device__ __forceinline__ float wave_max_dpp(float v)
{
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over the two 16-lane rows of each half wave (rows 0+1 and 2+3), after
// row_sum16: the totals land in rows 1 and 3 (lanes 16..31 and 48..63).
__device__ __forceinline__ float half_wave_sum_from_rows(float v)
{
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
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

// Buffer resource over [base, base + bytes): raw (unstrided) buffer loads through
// it return zeros past the end instead of faulting, so the kernels load without
// per-lane guards (a guarded load becomes a branch that serialises the loads).
// The descriptor's last word is the gfx9 default data format.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ uint4 load16(rsrc_t r, uint32_t offset)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0));
}

// Weight stream: 16 bytes with the non-temporal hint.  Each weight byte is read once
// per launch, so the hint keeps X and the scales, which every workgroup reads, from
// being pushed out of L2 by the stream.
__device__ __forceinline__ uint4 load16_stream(rsrc_t r, uint32_t offset)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 2));
}

__device__ __forceinline__ float4 load16f(rsrc_t r, uint32_t offset)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0));
}

__device__ __forceinline__ uint32_t load4(rsrc_t r, uint32_t offset)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, offset, 0, 0);
}

__device__ __forceinline__ uint16_t load2(rsrc_t r, uint32_t offset)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, offset, 0, 0);
}

// Issue-order barrier: every wave of the workgroup has issued its loads above this
// point before any wave issues a load below it.  A CU serves vector loads in order,
// so the small loads every wave waits on first (X) are not queued behind the weight
// streams of the workgroup's other waves.  No memory ordering is implied.
__device__ __forceinline__ void issue_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// Four INT8 activation codes, equal to quant_code's, by one fused multiply-add per
// value instead of a division.  For a reciprocal r = fl(1/s) of s = fl(m/127),
// m = max |x|, every |x r| is below 127.0001, so u = fl(x r + 384) (one fused rounding)
// lies in (256, 512), where fp32 values are spaced 2^-15 apart.
// e = (bits(u) << 1) + 0x8002 - (128 << 16) then holds in bits 16..23 the integer part of u minus 384, plus one when the fraction is at
// least a half (the +0x8000 carry): rint(x r) modulo 256, the code's byte.  Bits 0..15
// hold the fraction in units of 2^-16, offset so that the three spacings around a half
// map to 0, 2 and 4.  When none of the four values lands there, each exact x r is more
// than 3 * 2^-16 from a half-integer; x / s is within 2^-17 of x r and fl(x / s) within
// 2^-18 of x / s, so rint(fl(x / s)), the definition, is the code found.  Returns true
// when some value needs the division (quant4_e_div, then taken for all four); callers
// pass r only when it is finite (s >= 2^-126), else take the division.
__device__ __forceinline__ bool quant4_e(const float4 x, float r, uint32_t (&e)[4])
{
    const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        e[i] = (__float_as_uint(__builtin_fmaf(xs[i], r, 384.0f)) << 1) + (0x8002u - 0x800000u);
    // smallest offset fraction of the four: two 16-bit minima
    uint32_t m;
    asm("v_min3_u16 %0, %1, %2, %3" : "=v"(m) : "v"(e[0]), "v"(e[1]), "v"(e[2]));
    asm("v_min_u16 %0, %1, %2" : "=v"(m) : "v"(m), "v"(e[3]));
    return (uint16_t)m <= (uint16_t)4;
}

// The division path in quant4_e's format: byte 2 of e[i] = rint(fl(x / s)).  s is 0 only
// when the vector is all zeros, and 0 / 0 (NaN) takes the code 0.  |x / s| < 127.5, so no
// clamp is needed.
__device__ __forceinline__ void quant4_e_div(const float4 x, float s, uint32_t (&e)[4])
{
    const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float q = rintf(xs[i] / s);
        e[i] = q == q ? ((uint32_t)(int)q & 0xffu) << 16 : 0u;
    }
}

__device__ __forceinline__ uint32_t pack_i8x4(int b0, int b1, int b2, int b3)
{
    return (uint32_t)(b0 & 0xff) | ((uint32_t)(b1 & 0xff) << 8) | ((uint32_t)(b2 & 0xff) << 16) |
           ((uint32_t)(b3 & 0xff) << 24);
}

}  // namespace qw
