// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qw {

// Tiling of the GEMV kernels (M < 16).  A "chunk" is 16 bytes of packed weights
// (32 INT4 weights or 16 INT8 weights).  16 lanes cover one row of 16*cpl chunks
// (one K slice); a wave covers 4 rows at a time and `rows_per_wave` rows in all;
// a workgroup is 4 waves.  The grid is (row blocks, K slices, M tiles).
struct GemvTiling {
    int mt;             // rows of X per workgroup (1, 2, 4, 8)
    int cpl;            // chunks per lane per row (1, 2, 4)
    int gb;             // row groups of 4 rows whose loads are issued together
    int rows_per_wave;  // multiple of 4*gb
    int slices;         // K slices = ceil(chunks_per_row / (16*cpl))
    int row_blocks;     // ceil(N / (4*rows_per_wave))
    int m_tiles;        // ceil(M / mt)
};

struct W4A8Args {
    const float* X;
    const uint8_t* Wq;
    const float* w_scale;
    float* Y;
    int M, N, K;
    int rows_per_wave;
    int32_t* acc_ws;     // [M][N] int32, zero on entry and exit (split-K only)
    uint32_t* counters;  // [m_tiles][row_blocks], zero on entry and exit (split-K only)
    int32_t* dbg_acc;    // optional [M][N]
    int8_t* dbg_xq;      // optional [M][K]
    float* dbg_a;        // optional [M]
};

struct W8A16Args {
    const uint16_t* X;
    const uint8_t* Wq;
    const uint16_t* w_scale;
    uint16_t* Y;
    int M, N, K;
    int rows_per_wave;
    float* part_ws;      // [slices][M][N] fp32 partial sums (split-K only)
    uint32_t* counters;  // [m_tiles][row_blocks], zero on entry and exit (split-K only)
};

hipError_t launch_pack_w4(const float* W, int N, int K, uint8_t* Wq, float* s, int* flag,
                          hipStream_t st);
hipError_t launch_pack_w8(const float* W, int N, int K, int8_t* Wq, uint16_t* s, int* flag,
                          hipStream_t st);
hipError_t launch_quant_act(const float* X, int M, int K, int8_t* Xq, float* a, hipStream_t st);
hipError_t launch_codes_w4(const uint8_t* Wq, int N, int K, int8_t* codes, hipStream_t st);
hipError_t launch_codes_w8(const int8_t* Wq, int N, int K, int8_t* codes, hipStream_t st);
hipError_t launch_fill_zero(uint32_t* p, size_t words, hipStream_t st);

hipError_t launch_gemv_w4a8(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st);
hipError_t launch_gemv_w8a16(const W8A16Args& a, const GemvTiling& t, hipStream_t st);

}  // namespace qw
