// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qw {

// Packed weight layout shared by the packers, the GEMV kernels and the code decoders.
// A chunk is 16 bytes of one row: 32 INT4 weights (canonical nibble order, even k in
// the low nibble) or 16 INT8 weights.  A tile is 1 KB covering 512 consecutive k of
// R rows: R = 4 rows x 16 chunks for INT4, R = 2 rows x 32 chunks for INT8.  Inside
// a tile, 16-byte slot (n % R) * L + (c % L) holds row n's chunk c, L = 64 / R being
// the lanes per row.  Tiles are stored row group (R rows) by row group, and within a
// row group in k order, so one wave64 load of 16 bytes per lane reads one whole
// tile (1 KB contiguous), lane (sub, j) = (lane / L, lane % L) always meets row
// R*rg + sub and chunk L*cg + j, and a row group's tiles are contiguous.  Rows past
// N and chunks past K are zero padding.
struct TileLayout {
    int rows;   // R: rows per tile (4 for INT4, 2 for INT8)
    int lanes;  // L: lanes per row = chunks per tile row (16 or 32)
    int cg;     // tiles per row group = ceil(K / 512)
    int nrg;    // row groups = ceil(N / R)
};

inline TileLayout tile_layout(int bits, int64_t N, int64_t K)
{
    TileLayout t;
    t.rows = bits == 4 ? 4 : 2;
    t.lanes = 64 / t.rows;
    t.cg = (int)((K + 511) / 512);
    t.nrg = (int)((N + t.rows - 1) / t.rows);
    return t;
}

inline size_t packed_bytes(int bits, int64_t N, int64_t K)
{
    TileLayout t = tile_layout(bits, N, K);
    return (size_t)t.nrg * (size_t)t.cg * 1024u;
}

// Group-wise INT4 scales (one fp32 scale per output row and group of g consecutive k,
// g = 32, 64, 128, 256 or 512, K a multiple of g).  Device layout: for each row group, each
// of its 4 rows, each of the 512 / g groups of a tile, the scales of that group in tile
// order, padded to a multiple of 4 tiles (cgp = ceil(cg / 4) * 4): index
//   ((((n / 4) * 4 + n % 4) * (512 / g) + (k % 512) / g) * cgp + k / 512
// for the group holding k.  A GEMV lane (row n % 4, chunk group j) then reads the scales
// of all its tiles as consecutive floats.  Padding entries are zero.
__host__ __device__ __forceinline__ size_t w4g_scale_index(int n, int k, int g, int cg)
{
    const int cgp = (cg + 3) & ~3;
    return ((((size_t)(n >> 2) * 4 + (n & 3)) * (size_t)(512 / g) + (size_t)((k & 511) / g)) *
            (size_t)cgp) + (size_t)(k >> 9);
}

inline size_t w4g_scale_floats(int64_t N, int64_t K, int64_t g)
{
    const int64_t cg = (K + 511) / 512, cgp = (cg + 3) / 4 * 4, nrg = (N + 3) / 4;
    return (size_t)(nrg * 4 * (512 / g) * cgp);
}

// First row group of row run g out of W when nrg = per * W + rem row groups are split
// evenly (the first rem runs take one more); g = W gives nrg.  Multiply-add only: the
// quotient and remainder come from the host, so no division runs on the device.
__host__ __device__ __forceinline__ int rg_of(int g, int per, int rem)
{
    return g * per + (g < rem ? g : rem);
}

// K up to kRegCG * 512 keeps a lane's activations for a whole row in registers.
constexpr int kRegCG = 8;

// Launch shape of the GEMV kernels.
struct GemvTiling {
    int mt;           // rows of X per workgroup (1, 2, 4, 8)
    int m_tiles;      // ceil(M / mt)
    int reg_cg;       // > 0: activations in registers, K <= 512 * reg_cg, mt == 1
                      //   0: activations read from LDS tile by tile
    int tmax;         // > 0: eager variant, every tile of a wave (at most tmax) loaded up front
    int u;            // LDS variant: tiles per load batch (4 or 8), two batches in flight
    int nw;           // waves per workgroup (4, 8 or 16)
    int splitk;       // LDS variant: waves sharing each row group, each taking a k-slice
                      //   (1, 2 or 4; above 1 only with 4 or 8 waves and mt <= 2)
    int nwaves;       // row runs along N; they split the row groups evenly
                      //   (producer variant: consumer waves of all workgroups)
    int blocks;       // workgroups along N = ceil(nwaves / (nw / splitk))
    int lds_bytes;    // dynamic LDS
    int prod;         // > 0: producer variant (u == 5 or 6, M == 1) with `prod` producer
                      //   waves and nw consumer waves per workgroup; the row groups
                      //   are split over the workgroups (W4A8Args per / rem); splitk
                      //   consumer waves share each row group's tiles, at most reg_cg
                      //   tiles each
};

struct W4A8Args {
    const float* X;
    const uint8_t* Wq;
    const float* w_scale;
    float* Y;
    int M, N, K;
    int cg, nrg, nwaves;
    int per, rem;      // row groups per row run: nrg = per * nwaves + rem (see rg_of);
                       //   per workgroup in the producer variant: nrg = per * blocks + rem
    int32_t* dbg_acc;  // optional [M][N]
    int8_t* dbg_xq;    // optional [M][K]
    float* dbg_a;      // optional [M]
};

// Balanced long-K W4A8 kernel: activation codes and scales precomputed (workspace).
struct W4A8BsplitArgs {
    const int8_t* Xq;       // [M][K] row-major int8 codes
    const float* a_scale;   // [M]
    const uint8_t* Wq;
    const float* w_scale;
    float* Y;
    int M, N, K;
    int cg, nrg;
    int per, rem;           // row groups per workgroup: nrg = per * blocks + rem (see rg_of)
};

struct W8A16Args {
    const uint16_t* X;
    const uint8_t* Wq;
    const uint16_t* w_scale;
    uint16_t* Y;
    int M, N, K;
    int cg, nrg, nwaves;
    int per, rem;      // row groups per row run: nrg = per * nwaves + rem (see rg_of)
};

// Rows of X from which gemv_w4a8 / gemv_w8a16 run on the matrix cores instead of the
// GEMV kernels (measured on MI355X at K = 4096, N = 27392: the W4A8 GEMM is faster from
// two rows, the W8A16 one from three).
constexpr int kMfmaMinM4 = 2;
constexpr int kMfmaMinM8 = 3;

struct MfmaW4A8Args {
    const float* X;         // [M][K] fp32: read only by the balanced kernel's fused prologue
    const uint8_t* Xp;      // X codes in MFMA operand order (workspace)
    const float* a_scale;   // [M] (workspace)
    const uint8_t* Wq;
    const float* w_scale;
    float* Y;
    int M, N, K;
    int cg, nrg;
    int ks;       // 64-k steps = ceil(K / 64)
    int mbtot;    // 16-row blocks of X = ceil(M / 16)
    int mgroups;  // workgroups along M
    // balanced variant: row groups per workgroup (the first rem get one more) and the
    // most 16-row output blocks a workgroup holds
    int per, rem, nbmax;
};

struct MfmaW8A16Args {
    const uint16_t* X;
    const uint8_t* Wq;
    const uint16_t* w_scale;
    uint16_t* Y;
    int M, N, K;
    int cg, nrg;
    int mgroups;
    int per, rem, nbmax;  // balanced variant (as in MfmaW4A8Args)
};

// Tiled matrix-core GEMM (gemm_tile.hip): one workgroup per output tile of BN rows of W
// by BM rows of X, K walked in double-buffered stages through LDS.
struct TileGemmArgs {
    const void* X;          // W8A16: f16 [M][K]; W4A8: int8 codes [M][K] (workspace)
    const uint8_t* Wq;
    const void* w_scale;    // W8A16: f16 [N]; W4A8: fp32 [N]
    void* Y;                // W8A16: f16 [M][N]; W4A8: fp32 [M][N]
    const float* a_scale;   // W4A8: [M] (workspace)
    int M, N, K;
    int cg, nrg;
    int mblocks;            // tiles along M (set by the launcher)
};
// Rows of X per tile of launch variant `variant` (0 when the variant does not exist).
int tile_rows_m(int variant);
// Rows of W per tile of launch variant `variant`.
int tile_rows_n(int variant);
hipError_t launch_gemm_w8a16_tile(const uint16_t* X, int M, int N, int K, const uint8_t* Wq,
                                  const uint16_t* w_scale, uint16_t* Y, int variant, hipStream_t st);
// Xq: row-major int8 codes [M][K] and a_scale [M] (launch_quant_act_rows)
hipError_t launch_gemm_w4a8_tile(const int8_t* Xq, const float* a_scale, int M, int N, int K,
                                 const uint8_t* Wq, const float* w_scale, float* Y, int variant,
                                 hipStream_t st);

size_t mfma_w4a8_workspace_bytes(int64_t M, int64_t K);
// Launch shape of the matrix-core kernels: nw waves per workgroup (4 or 8), mb blocks
// of 16 rows of X per workgroup, nbw blocks of 16 output rows per wave.
bool mfma_shape_ok(int bits, int nw, int mb, int nbw);
void mfma_default_shape(int bits, int64_t M, int64_t K, int* nw, int* mb, int* nbw);
hipError_t launch_gemm_w4a8(const float* X, int M, int N, int K, const uint8_t* Wq,
                            const float* w_scale, float* Y, void* workspace, int nw, int mb,
                            int nbw, int cus, hipStream_t st);
hipError_t launch_gemm_w8a16(const uint16_t* X, int M, int N, int K, const uint8_t* Wq,
                             const uint16_t* w_scale, uint16_t* Y, int nw, int mb, int nbw,
                             int cus, hipStream_t st);

hipError_t launch_pack_w4(const float* W, int N, int K, uint8_t* Wq, float* s, int* flag,
                          hipStream_t st);
hipError_t launch_pack_w8(const float* W, int N, int K, uint8_t* Wq, uint16_t* s, int* flag,
                          hipStream_t st);
hipError_t launch_quant_act(const float* X, int M, int K, int8_t* Xq, float* a, hipStream_t st);
hipError_t launch_codes_w4(const uint8_t* Wq, int N, int K, int8_t* codes, hipStream_t st);
hipError_t launch_pack_w4g(const float* W, int N, int K, int g, uint8_t* Wq, float* s,
                           int* flag, hipStream_t st);
hipError_t launch_w4g_scales(const float* s, int N, int K, int g, float* out, hipStream_t st);
hipError_t launch_codes_w8(const uint8_t* Wq, int N, int K, int8_t* codes, hipStream_t st);
hipError_t launch_fill_zero(uint32_t* p, size_t words, hipStream_t st);

hipError_t launch_gemv_w4a8(const W4A8Args& a, const GemvTiling& t, bool debug, hipStream_t st);
hipError_t launch_gemv_w8a16(const W8A16Args& a, const GemvTiling& t, hipStream_t st);
// blocks workgroups of `waves` (1..8) waves, one k-slice of ceil(cg / waves) <= 8 tiles
// each; 1, 2 or 4 rows of X per workgroup (chosen from M and the slice length)
hipError_t launch_gemv_w4a8_bsplit(const W4A8BsplitArgs& a, int blocks, int waves, hipStream_t st);
// row-major int8 codes and one scale per row of X, as launch_quant_act; one 1024-thread
// workgroup per row holding the row in registers (K <= 57344)
// With unpack_order, each 16-byte group of codes holds its 16 k in the INT4 unpack order
// (k 0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15), as the tiled GEMM takes them.
hipError_t launch_quant_act_rows(const float* X, int M, int K, int8_t* Xq, float* a, hipStream_t st,
                                 bool unpack_order = false);
// The INT4 page's ablations (M == 1, K <= 4096): FP16 GEMV on row-major f16 weights, and
// weight-only INT4 (quantize_pack_w4 layout) with fp32 activations unpacked to float;
// rpw rows (FP16) or row groups (INT4) per wave, 1, 2 or 4.
// IndexSoftmax (integer softmax over int32 logits): b-bit table (n = 2^b - 1 entries past
// 0), thr[k] = ceil(c_int * (2k - 1) / (2n)) for k = 1..n (thr[0] unused), lut[k] the
// UINT8 exponent table (lut[n] = 0).  1 <= L <= 16384.
struct IndexSoftmaxArgs {
    int32_t c_int;
    int b;
    float scale;  // n / c_int, for the index estimate
    // exact index by multiplication: idx = mulhi(2 n D' + c_int, magic) >> shift, valid when
    // c_int < 2^24 and c_int (2n + 1) < 2^31 (magic = 0 otherwise: the threshold path)
    uint32_t magic;
    int shift;
    uint32_t thr[64];
    uint32_t lut[64];
};
hipError_t launch_index_softmax(const int32_t* A, int64_t rows, int64_t L,
                                const IndexSoftmaxArgs& t, uint8_t* P, hipStream_t st);

hipError_t launch_gemv_f16(const uint16_t* X, const uint16_t* W, uint16_t* Y, int N, int K,
                           int rpw, hipStream_t st);
hipError_t launch_gemv_w4f32(const float* X, const uint8_t* Wq, const float* s, float* Y, int N,
                             int K, int rpw, hipStream_t st);
// Group-wise W4A8 GEMV (M == 1, producer-wave tilings u == 5 or 6): w_scale holds the
// group scales in the layout of w4g_scale_index; group = 32 .. 512.
hipError_t launch_gemv_w4a8g(const W4A8Args& a, const GemvTiling& t, int group, hipStream_t st);
// Plain streaming read of `words` 16-byte words (bandwidth reference): `blocks`
// workgroups of `waves` waves, u loads in flight per lane; one XOR word per workgroup.
hipError_t launch_stream_read(const uint8_t* src, size_t words, int waves, int blocks, int u,
                              uint32_t* sink, hipStream_t st);
// Status words of the producer-wave kernels (row-wise and group-wise builds): nonzero when
// a producer's bounded wait ran out since the last clear; synchronous.
hipError_t prod_guard_status_rowwise(unsigned* trips, bool clear);
hipError_t prod_guard_status_groupwise(unsigned* trips, bool clear);

}  // namespace qw
