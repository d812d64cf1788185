// C ABI of the weight-quantized decode linear: host-side validation, tiling choice
// and dispatch.  Declarations and the contract of every entry point are in
// include/qwgemv.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qwgemv.h"
#include "kernels.hpp"

namespace {

using qw::GemvTiling;

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxK = 131072;  // keeps 16 * 7 * 127 * K below 2^31
constexpr int64_t kMaxM = 65535;
constexpr int64_t kMaxN = (int64_t)1 << 28;

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return QW_OK;
    g_last_hip_error = (int)e;
    return QW_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || M > kMaxM || N > kMaxN || K > kMaxK || (K % 32) != 0)
        return QW_ERR_SHAPE;
    return QW_OK;
}

constexpr int kMaxLds = 60 * 1024;  // dynamic LDS budget per workgroup

// Default launch shape of qw_stream_read: one workgroup per CU of kStreamReadWaves waves,
// kStreamReadLoads 16-byte loads in flight per lane.
constexpr int kStreamReadWaves = 8;
constexpr int kStreamReadLoads = 4;

#include "gemv_shapes.hpp"

// Scratch of gemv_w4a8_noalloc: the activation codes and scales that gemv_w4a8 keeps in a
// caller's workspace from two rows of X, here in a fixed device array instead, for
// callers that cannot allocate.  Each GPU holds its own copy until the process ends.
// Host code uses the address hipGetSymbolAddress gives on each device, never the
// array's name (which on the host is only a stand-in).
constexpr size_t kScratchBytes = (size_t)8 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch[64] = {nullptr};

// The device address of `scratch` on the current device, looked up on the first call
// per device (with that device current) and kept.
int scratch_address(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_status(e);
    if (dev < 0 || dev >= 64)
        return hip_status(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_status(e);
        if (p == nullptr)
            return hip_status(hipErrorInvalidSymbol);
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return QW_OK;
}

// Launch variant of the tiled matrix-core GEMM for M rows of X and N rows of W, or -1
// where the balanced matrix-core kernels stay.  From 33 rows each candidate's time is
// modelled as the tiles on the busiest CU times the tile's work over the variant's
// efficiency, and the least is taken among the variants with at least 96 tiles.  The
// efficiencies are fitted to sweeps of every variant at M = 9 .. 512 on 4096 -> 27392,
// 3584 -> 18944, 4096 -> 9000 and 18944 -> 3584: the choice is within 0.5% of the best
// variant on average and 8% at worst.  W8A16 at 12 to 32 rows takes the 128 x 32 tiles
// where there are at least 128 of them (N >= 16257): 16.5-18.4 against 17.1-22.2 us for
// the balanced kernel on 3584 -> 18944, 22.5-23.0 against 23.0-28.9 on 4096 -> 27392;
// with fewer tiles the balanced kernel, which spreads any N over every CU, is faster
// (4096 -> 9000 at 16 rows: 12.8 against 16.0 us).  W4A8 takes them from 20 rows on the
// same condition (24 and 32 rows on 4096 -> 27392: 16.5 and 16.7 against 18.5 and 18.8
// us; at 16 rows its balanced kernel with the cheaper pre-pass is still ahead, 15.5
// against 16.2).  Measured choices on 4096 -> 27392: W8A16 16 rows
// 128 x 32 (22.5 us), 64 rows 128 x 64 in two k-groups with deep stages (27.4), 128
// rows 128 x 128 in two k-groups (39.3), 256 rows 256 x 128 (62), 512 rows 256 x 256
// (101-107); W4A8 64 rows 128 x 64 (20.3), 128 rows 128 x 128 (26.1), 256 rows 256 x
// 128 (36), 512 rows 256 x 256 (59-61, the activation pre-pass included).
constexpr int64_t kTileMinTiles = 96;

int tile_variant(int bits, int64_t M, int64_t N)
{
    struct Cand {
        int v;
        double eff8, eff4;  // W8A16, W4A8
    };
    static const Cand cand[] = {{0, 1.0, 1.0}, {1, 0.8, 0.8}, {2, 0.4, 0.5}, {3, 0.5, 0.5},
                                {4, 0.3, 0.3}, {5, 0.3, 0.3}, {7, 0.4, 0.4}, {8, 0.35, 0.35},
                                {6, 0.3, 0.3}};
    if (M < 33) {
        if (M >= (bits == 8 ? 12 : 20) && (N + 127) / 128 >= 128)
            return 8;
        return -1;
    }
    const int64_t cus = std::max<int64_t>(1, device_cus());
    double best = 0.0;
    int pick = -1;
    for (const Cand& c : cand) {
        const int64_t bm = qw::tile_rows_m(c.v), bn = qw::tile_rows_n(c.v);
        if (bm <= 0 || bn <= 0)
            continue;
        const int64_t tiles = ((N + bn - 1) / bn) * ((M + bm - 1) / bm);
        if (tiles < kTileMinTiles)
            continue;
        const double cost = (double)((tiles + cus - 1) / cus) * (double)(bn * bm) / (bits == 8 ? c.eff8 : c.eff4);
        if (pick < 0 || cost < best * 0.999) {
            best = cost;
            pick = c.v;
        }
    }
    return pick;
}

// One device int per GPU for the packers' non-finite flag.  A packer call holds the
// lock from clearing the flag to reading it back, so packers called at the same time
// from several host threads run one after another and each reads its own result.
std::mutex g_flag_mu;
int* g_flag[64] = {nullptr};

// Runs pack(flag) between clearing and reading back the device flag, under the lock.
template <class F>
int run_packer(hipStream_t st, F pack)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_status(e);
    if (dev < 0 || dev >= 64)
        return hip_status(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lk(g_flag_mu);
    if (g_flag[dev] == nullptr) {
        void* p = nullptr;
        e = hipMalloc(&p, 256);
        if (e != hipSuccess)
            return hip_status(e);
        g_flag[dev] = static_cast<int*>(p);
    }
    int* flag = g_flag[dev];
    e = qw::launch_fill_zero(reinterpret_cast<uint32_t*>(flag), 1, st);
    if (e == hipSuccess)
        e = pack(flag);
    int host = 0;
    if (e == hipSuccess)
        e = hipMemcpyAsync(&host, flag, sizeof(int), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess)
        e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return hip_status(e);
    return host ? QW_ERR_NONFINITE : QW_OK;
}

int run_w4a8(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
             int64_t K, float* Y, int32_t* acc, int8_t* xq, float* a_scale, void* workspace,
             const GemvTiling& t, bool debug, void* stream)
{
    if (!X || !Wq || !w_scale || !Y)
        return QW_ERR_NULL;
    int st = check_gemv_shape(4, M, N, K);
    if (st != QW_OK)
        return st;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y) ||
        !aligned16(workspace) || !aligned16(acc) || !aligned16(xq) || !aligned16(a_scale))
        return QW_ERR_ALIGN;
    if (t.lds_bytes > kMaxLds)
        return QW_ERR_TILING;
    const qw::TileLayout L = qw::tile_layout(4, N, K);
    qw::W4A8Args a;
    a.X = X;
    a.Wq = static_cast<const uint8_t*>(Wq);
    a.w_scale = w_scale;
    a.Y = Y;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.cg = L.cg;
    a.nrg = L.nrg;
    a.nwaves = t.nwaves;
    // row groups per row run, or per workgroup in the producer variant
    const int runs = t.prod > 0 ? t.blocks : t.nwaves;
    a.per = L.nrg / runs;
    a.rem = L.nrg % runs;
    a.dbg_acc = acc;
    a.dbg_xq = xq;
    a.dbg_a = a_scale;
    return hip_status(qw::launch_gemv_w4a8(a, t, debug, static_cast<hipStream_t>(stream)));
}

int run_w8a16(const uint16_t* X, const void* Wq, const uint16_t* w_scale, int64_t M, int64_t N,
              int64_t K, uint16_t* Y, void* workspace, const GemvTiling& t, void* stream)
{
    if (!X || !Wq || !w_scale || !Y)
        return QW_ERR_NULL;
    int st = check_gemv_shape(8, M, N, K);
    if (st != QW_OK)
        return st;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y) ||
        !aligned16(workspace))
        return QW_ERR_ALIGN;
    if (t.lds_bytes > kMaxLds)
        return QW_ERR_TILING;
    const qw::TileLayout L = qw::tile_layout(8, N, K);
    qw::W8A16Args a;
    a.X = X;
    a.Wq = static_cast<const uint8_t*>(Wq);
    a.w_scale = w_scale;
    a.Y = Y;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.cg = L.cg;
    a.nrg = L.nrg;
    a.nwaves = t.nwaves;
    a.per = L.nrg / t.nwaves;
    a.rem = L.nrg % t.nwaves;
    return hip_status(qw::launch_gemv_w8a16(a, t, static_cast<hipStream_t>(stream)));
}

int run_gemm_w4a8(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
                  int64_t K, float* Y, void* workspace, size_t ws_bytes, int nw, int mb, int nbw,
                  void* stream)
{
    if (!X || !Wq || !w_scale || !Y)
        return QW_ERR_NULL;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y) ||
        !aligned16(workspace))
        return QW_ERR_ALIGN;
    if (!workspace || ws_bytes < qw::mfma_w4a8_workspace_bytes(M, K))
        return QW_ERR_WORKSPACE;
    return hip_status(qw::launch_gemm_w4a8(X, (int)M, (int)N, (int)K,
                                           static_cast<const uint8_t*>(Wq), w_scale, Y, workspace,
                                           nw, mb, nbw, device_cus(), static_cast<hipStream_t>(stream)));
}

int run_gemm_w8a16(const uint16_t* X, const void* Wq, const uint16_t* w_scale, int64_t M,
                   int64_t N, int64_t K, uint16_t* Y, void* workspace, int nw, int mb, int nbw,
                   void* stream)
{
    if (!X || !Wq || !w_scale || !Y)
        return QW_ERR_NULL;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y) ||
        !aligned16(workspace))
        return QW_ERR_ALIGN;
    return hip_status(qw::launch_gemm_w8a16(X, (int)M, (int)N, (int)K,
                                            static_cast<const uint8_t*>(Wq), w_scale, Y, nw, mb,
                                            nbw, device_cus(), static_cast<hipStream_t>(stream)));
}

// ---- group-wise INT4 scales

bool group_ok(int64_t K, int64_t group)
{
    return (group == 32 || group == 64 || group == 128 || group == 256 || group == 512) &&
           K % group == 0;
}

// Launch shapes the group-wise kernels exist for: the producer variant with 8 + 2 or 4 + 4
// waves (K <= 4096), or with the K split over 2, 4 or 8 waves of at most 6 tiles.
bool tiling_ok_g(int64_t M, int u, int nw, int nwaves, int splitk, const qw::TileLayout& L)
{
    if (u == 5)
        return ((nw == 8 && splitk == 2) || (nw == 4 && splitk == 4)) &&
               tiling_ok(4, M, u, nw, nwaves, splitk, L);
    if (u == 6)
        return (L.cg + splitk - 1) / splitk <= 6 && tiling_ok(4, M, u, nw, nwaves, splitk, L);
    return false;
}

// Built-in launch shape of the group-wise GEMV: the row-wise choice of the producer
// variant; false when none fits.
bool default_tiling_g(int64_t N, int64_t K, GemvTiling* t)
{
    const qw::TileLayout L = qw::tile_layout(4, N, K);
    const int cus = device_cus();
    if (L.cg <= qw::kRegCG) {
        const int64_t nrg = L.nrg;
        const int nw = nrg >= 2048 ? 8 : 4, P = nrg >= 2048 ? 2 : 4;
        const int blocks =
            nrg >= 2048 ? cus : (int)std::min<int64_t>(cus, std::max<int64_t>(1, nrg / 2));
        if (!tiling_ok_g(1, 5, nw, blocks * nw, P, L))
            return false;
        *t = make_tiling(4, 1, N, K, 5, nw, blocks * nw, P);
        return true;
    }
    for (int S = 2; S <= 8; S *= 2)
        if (tiling_ok_g(1, 6, 8, cus * 8, S, L)) {
            *t = make_tiling(4, 1, N, K, 6, 8, cus * 8, S);
            return true;
        }
    return false;
}

int run_w4a8g(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
              int64_t K, int64_t group, float* Y, const GemvTiling& t, void* stream)
{
    const qw::TileLayout L = qw::tile_layout(4, N, K);
    qw::W4A8Args a;
    a.X = X;
    a.Wq = static_cast<const uint8_t*>(Wq);
    a.w_scale = w_scale;
    a.Y = Y;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.cg = L.cg;
    a.nrg = L.nrg;
    a.nwaves = t.nwaves;
    a.per = L.nrg / t.blocks;  // row groups per workgroup
    a.rem = L.nrg % t.blocks;
    a.dbg_acc = nullptr;
    a.dbg_xq = nullptr;
    a.dbg_a = nullptr;
    return hip_status(qw::launch_gemv_w4a8g(a, t, (int)group, static_cast<hipStream_t>(stream)));
}

int check_w4a8g(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
                int64_t K, int64_t group, const float* Y)
{
    if (!X || !Wq || !w_scale || !Y)
        return QW_ERR_NULL;
    int st = check_gemv_shape(4, M, N, K);
    if (st != QW_OK)
        return st;
    if (M != 1 || !group_ok(K, group))
        return QW_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y))
        return QW_ERR_ALIGN;
    return QW_OK;
}

}  // namespace

// Balanced long-K W4A8 path: the activations quantized into the workspace (row-major
// codes, then one scale per row; one workgroup per row), then the balanced kernel
// with `waves` k-slices per workgroup and `blocks` workgroups.
bool w4_bsplit_ok(int64_t M, int64_t N, int64_t K, int waves, int blocks)
{
    const qw::TileLayout L = qw::tile_layout(4, N, K);
    if (waves < 1 || waves > 8 || (L.cg + waves - 1) / waves > 8 || blocks < 1 || blocks > L.nrg)
        return false;
    const int64_t per = ((int64_t)L.nrg + blocks - 1) / blocks;
    const int64_t mtiles = M == 1 ? 1 : (M + 1) / 2;  // at least 2 rows of X per workgroup
    return per <= 16 && per * L.cg * 1024 < ((int64_t)1 << 31) && M * K < ((int64_t)1 << 31) &&
           (int64_t)blocks * mtiles * 64 * waves < ((int64_t)1 << 31);
}

int run_w4_bsplit(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
                  int64_t K, float* Y, void* workspace, size_t ws_bytes, int waves, int blocks,
                  void* stream)
{
    if (!X || !Wq || !w_scale || !Y)
        return QW_ERR_NULL;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y) ||
        !aligned16(workspace))
        return QW_ERR_ALIGN;
    if (!workspace || ws_bytes < qw::mfma_w4a8_workspace_bytes(M, K))
        return QW_ERR_WORKSPACE;
    const qw::TileLayout L = qw::tile_layout(4, N, K);
    const size_t codes = ((size_t)M * (size_t)K + 255u) & ~(size_t)255u;
    int8_t* xq = static_cast<int8_t*>(workspace);
    float* a = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + codes);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = qw::launch_quant_act_rows(X, (int)M, (int)K, xq, a, st);
    if (e != hipSuccess)
        return hip_status(e);
    qw::W4A8BsplitArgs p;
    p.Xq = xq;
    p.a_scale = a;
    p.Wq = static_cast<const uint8_t*>(Wq);
    p.w_scale = w_scale;
    p.Y = Y;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.cg = L.cg;
    p.nrg = L.nrg;
    p.per = L.nrg / blocks;
    p.rem = L.nrg % blocks;
    return hip_status(qw::launch_gemv_w4a8_bsplit(p, blocks, waves, st));
}

// Tiled matrix-core W4A8 path: the activations quantized into the workspace (row-major
// codes, then one scale per row at the next multiple of 256 bytes; one workgroup per
// row), then the tile kernel at the given launch variant.
int run_w4_tile(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
                int64_t K, float* Y, void* workspace, int variant, void* stream)
{
    const size_t codes = ((size_t)M * (size_t)K + 255u) & ~(size_t)255u;
    int8_t* xq = static_cast<int8_t*>(workspace);
    float* a = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + codes);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = qw::launch_quant_act_rows(X, (int)M, (int)K, xq, a, st, true);
    if (e != hipSuccess)
        return hip_status(e);
    return hip_status(qw::launch_gemm_w4a8_tile(xq, a, (int)M, (int)N, (int)K,
                                                static_cast<const uint8_t*>(Wq), w_scale, Y, variant, st));
}

void w4_bsplit_default(int64_t N, int64_t K, int* waves, int* blocks)
{
    const qw::TileLayout L = qw::tile_layout(4, N, K);
    *waves = (int)std::min<int64_t>(8, (L.cg + 3) / 4);
    *blocks = (int)std::max<int64_t>(std::min<int64_t>(device_cus(), L.nrg), (L.nrg + 15) / 16);
}

extern "C" {

size_t qw_w4_packed_bytes(int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0 || N > kMaxN || K > kMaxK || (K % 32) != 0)
        return 0;
    return qw::packed_bytes(4, N, K);
}

size_t qw_w8_packed_bytes(int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0 || N > kMaxN || K > kMaxK || (K % 32) != 0)
        return 0;
    return qw::packed_bytes(8, N, K);
}

size_t qw_workspace_bytes(int op, int64_t M, int64_t N, int64_t K)
{
    (void)N;
    // Only the W4A8 matrix-core path needs one: the activation codes and scales,
    // quantized once per call in the matrix cores' operand order.  op 2 is that path
    // at any M (qw_gemm_w4a8_mfma).
    if (M <= 0 || M > kMaxM || K <= 0 || K > kMaxK)
        return 0;
    if ((op == 0 && M >= qw::kMfmaMinM4) || op == 2)
        return qw::mfma_w4a8_workspace_bytes(M, K);
    return 0;
}

int qw_workspace_clear(void* workspace, size_t ws_bytes, void* stream)
{
    if (ws_bytes == 0)
        return QW_OK;
    if (!workspace)
        return QW_ERR_NULL;
    if (!aligned16(workspace) || (ws_bytes % 4) != 0)
        return QW_ERR_ALIGN;
    return hip_status(qw::launch_fill_zero(static_cast<uint32_t*>(workspace), ws_bytes / 4,
                                           static_cast<hipStream_t>(stream)));
}

int quantize_pack_w4(const float* W, int64_t N, int64_t K, void* Wq, float* w_scale,
                     void* stream)
{
    if (!W || !Wq || !w_scale)
        return QW_ERR_NULL;
    int st = check_shape(1, N, K);
    if (st != QW_OK)
        return st;
    if (!aligned16(W) || !aligned16(Wq) || !aligned16(w_scale))
        return QW_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run_packer(s, [&](int* flag) {
        return qw::launch_pack_w4(W, (int)N, (int)K, static_cast<uint8_t*>(Wq), w_scale, flag, s);
    });
}

int quantize_pack_w8(const float* W, int64_t N, int64_t K, void* Wq, uint16_t* w_scale_f16,
                     void* stream)
{
    if (!W || !Wq || !w_scale_f16)
        return QW_ERR_NULL;
    int st = check_shape(1, N, K);
    if (st != QW_OK)
        return st;
    if (!aligned16(W) || !aligned16(Wq) || !aligned16(w_scale_f16))
        return QW_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run_packer(s, [&](int* flag) {
        return qw::launch_pack_w8(W, (int)N, (int)K, static_cast<uint8_t*>(Wq), w_scale_f16, flag,
                                  s);
    });
}

size_t qw_w4g_scale_bytes(int64_t N, int64_t K, int64_t group)
{
    if (check_shape(1, N, K) != QW_OK || !group_ok(K, group))
        return 0;
    return qw::w4g_scale_floats(N, K, group) * sizeof(float);
}

int quantize_pack_w4g(const float* W, int64_t N, int64_t K, int64_t group, void* Wq,
                      float* w_scale, void* stream)
{
    if (!W || !Wq || !w_scale)
        return QW_ERR_NULL;
    int st = check_shape(1, N, K);
    if (st != QW_OK)
        return st;
    if (!group_ok(K, group))
        return QW_ERR_SHAPE;
    if (!aligned16(W) || !aligned16(Wq) || !aligned16(w_scale))
        return QW_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run_packer(s, [&](int* flag) {
        return qw::launch_pack_w4g(W, (int)N, (int)K, (int)group, static_cast<uint8_t*>(Wq),
                                   w_scale, flag, s);
    });
}

int qw_w4g_scales(const float* w_scale, int64_t N, int64_t K, int64_t group, float* out,
                  void* stream)
{
    if (!w_scale || !out)
        return QW_ERR_NULL;
    int st = check_shape(1, N, K);
    if (st != QW_OK)
        return st;
    if (!group_ok(K, group))
        return QW_ERR_SHAPE;
    return hip_status(qw::launch_w4g_scales(w_scale, (int)N, (int)K, (int)group, out,
                                            static_cast<hipStream_t>(stream)));
}

int gemv_w4a8g(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
               int64_t K, int64_t group, float* Y, void* workspace, size_t ws_bytes, void* stream)
{
    (void)workspace;
    (void)ws_bytes;
    int st = check_w4a8g(X, Wq, w_scale, M, N, K, group, Y);
    if (st != QW_OK)
        return st;
    GemvTiling t;
    if (!default_tiling_g(N, K, &t))
        return QW_ERR_SHAPE;
    return run_w4a8g(X, Wq, w_scale, M, N, K, group, Y, t, stream);
}

int qw_gemv_w4a8g_tiled(const float* X, const void* Wq, const float* w_scale, int64_t M,
                        int64_t N, int64_t K, int64_t group, float* Y, int u, int nw, int nwaves,
                        int splitk, void* stream)
{
    int st = check_w4a8g(X, Wq, w_scale, M, N, K, group, Y);
    if (st != QW_OK)
        return st;
    if (!tiling_ok_g(M, u, nw, nwaves, splitk, qw::tile_layout(4, N, K)))
        return QW_ERR_TILING;
    return run_w4a8g(X, Wq, w_scale, M, N, K, group, Y, make_tiling(4, M, N, K, u, nw, nwaves, splitk),
                     stream);
}

int check_ablation(const void* X, const void* W, int64_t M, int64_t N, int64_t K, const void* Y,
                   int rows_per_wave)
{
    if (!X || !W || !Y)
        return QW_ERR_NULL;
    int st = check_shape(M, N, K);
    if (st != QW_OK)
        return st;
    if (M != 1 || K > 4096 || N > ((int64_t)1 << 26))
        return QW_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(W) || !aligned16(Y))
        return QW_ERR_ALIGN;
    if (rows_per_wave != 0 && rows_per_wave != 1 && rows_per_wave != 2 && rows_per_wave != 4)
        return QW_ERR_TILING;
    return QW_OK;
}

int qw_gemv_f16(const uint16_t* X16, const uint16_t* W16, int64_t M, int64_t N, int64_t K,
                uint16_t* Y16, int rows_per_wave, void* stream)
{
    int st = check_ablation(X16, W16, M, N, K, Y16, rows_per_wave);
    if (st != QW_OK)
        return st;
    return hip_status(qw::launch_gemv_f16(X16, W16, Y16, (int)N, (int)K,
                                          rows_per_wave ? rows_per_wave : 2,
                                          static_cast<hipStream_t>(stream)));
}

int qw_gemv_w4f32(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
                  int64_t K, float* Y, int rows_per_wave, void* stream)
{
    int st = check_ablation(X, Wq, M, N, K, Y, rows_per_wave);
    if (st != QW_OK)
        return st;
    if (!w_scale)
        return QW_ERR_NULL;
    if (!aligned16(w_scale))
        return QW_ERR_ALIGN;
    // one row group per wave by default: with more, the compiler keeps several row
    // groups' converted weights live and the kernel runs at one wave per SIMD
    return hip_status(qw::launch_gemv_w4f32(X, static_cast<const uint8_t*>(Wq), w_scale, Y,
                                            (int)N, (int)K, rows_per_wave ? rows_per_wave : 1,
                                            static_cast<hipStream_t>(stream)));
}

int32_t qw_index_cint(double c, int64_t d, double s_q, double s_k)
{
    if (!(c > 0.0) || d < 1 || !(s_q > 0.0) || !(s_k > 0.0))
        return -1;
    const double v = c * std::sqrt((double)d) / (s_q * s_k);
    if (!(v < 2147483647.0))
        return -1;
    return (int32_t)std::llround(v);
}

int qw_index_magic(int32_t c_int, int b, uint32_t* magic, int* shift)
{
    // idx = round(D' n / c_int) half up = floor(x / d), x = 2 n D' + c_int, d = 2 c_int.
    // With s = floor(log2 d) and m = ceil(2^(32 + s) / d), m d = 2^(32 + s) + e, 0 <= e < d
    // < 2^(s + 1), so for x < 2^31 the excess x e / 2^(32 + s) of x m / 2^(32 + s) over x / d
    // stays below 1 / d and floor(mulhi(x, m) / 2^s) = floor(x / d); d a power of two takes
    // m = 2^31 with s - 1.  x < 2^31 for every D' <= c_int when c_int (2n + 1) < 2^31, and
    // the kernel forms 2 n D' with a 24-bit multiply (c_int < 2^24).
    if (!magic || !shift || b < 4 || b > 6 || c_int < 1)
        return 0;
    const int n = (1 << b) - 1;
    if (!(c_int < (1 << 24) && (int64_t)c_int * (2 * n + 1) < ((int64_t)1 << 31)))
        return 0;
    const uint64_t d = 2 * (uint64_t)c_int;
    int sh = 0;
    while ((d >> (sh + 1)) != 0)
        ++sh;
    const unsigned __int128 num = (unsigned __int128)1 << (32 + sh);
    const uint64_t m = (uint64_t)((num + d - 1) / d);
    if (m >= ((uint64_t)1 << 32)) {
        *magic = 1u << 31;
        *shift = sh - 1;
    } else {
        *magic = (uint32_t)m;
        *shift = sh;
    }
    return 1;
}

int index_softmax(const int32_t* A, int64_t rows, int64_t L, int32_t c_int, int b, double c,
                  uint8_t* P, void* stream)
{
    if (!A || !P)
        return QW_ERR_NULL;
    if (rows < 1 || rows > 2147483647 || L < 1 || L > 16384 || c_int < 1 || b < 4 || b > 6 ||
        !(c > 0.0) || !(c < 1e6))
        return QW_ERR_SHAPE;
    if (!aligned16(A) || !aligned16(P))
        return QW_ERR_ALIGN;
    // the exponent table of the IntAttention summary (section 基准/方法设计):
    // LUT[i] = round(255 exp(-c i / n)), the last entry 0; and the index thresholds
    qw::IndexSoftmaxArgs t;
    t.c_int = c_int;
    t.b = b;
    const int n = (1 << b) - 1;
    t.scale = (float)((double)n / (double)c_int);
    for (int i = 0; i < 64; ++i) {
        t.lut[i] = 0;
        t.thr[i] = 0;
    }
    for (int i = 0; i < n; ++i)
        t.lut[i] = (uint32_t)std::lround(255.0 * std::exp(-c * (double)i / (double)n));
    for (int k = 1; k <= n; ++k)
        t.thr[k] = (uint32_t)(((int64_t)c_int * (2 * k - 1) + 2 * n - 1) / (2 * n));
    if (!qw_index_magic(c_int, b, &t.magic, &t.shift)) {
        t.magic = 0;
        t.shift = 0;
    }
    return hip_status(qw::launch_index_softmax(A, rows, L, t, P, static_cast<hipStream_t>(stream)));
}

int quant_act_i8(const float* X, int64_t M, int64_t K, int8_t* Xq, float* a_scale, void* stream)
{
    if (!X || !Xq || !a_scale)
        return QW_ERR_NULL;
    int st = check_shape(M, 1, K);
    if (st != QW_OK)
        return st;
    if (!aligned16(X) || !aligned16(Xq) || !aligned16(a_scale))
        return QW_ERR_ALIGN;
    return hip_status(
        qw::launch_quant_act(X, (int)M, (int)K, Xq, a_scale, static_cast<hipStream_t>(stream)));
}

int gemv_w4a8(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
              int64_t K, float* Y, void* workspace, size_t ws_bytes, void* stream)
{
    if (check_gemv_shape(4, M, N, K) != QW_OK)
        return (!X || !Wq || !w_scale || !Y) ? QW_ERR_NULL : QW_ERR_SHAPE;
    if (M >= qw::kMfmaMinM4 && long_k_rows(4, M, N, K)) {
        // long K, 2 to 8 (16) rows: the matrix-core kernels walk all of K in each
        // workgroup (37 to 46 us at 18944 -> 3584 whatever M), the long-K kernel splits it
        int waves, blocks;
        w4_bsplit_default(N, K, &waves, &blocks);
        if (w4_bsplit_ok(M, N, K, waves, blocks))
            return run_w4_bsplit(X, Wq, w_scale, M, N, K, Y, workspace, ws_bytes, waves, blocks, stream);
    }
    if (M >= qw::kMfmaMinM4) {
        const int v = tile_variant(4, M, N);
        if (v >= 0) {
            if (!X || !Wq || !w_scale || !Y)
                return QW_ERR_NULL;
            if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y) ||
                !aligned16(workspace))
                return QW_ERR_ALIGN;
            if (!workspace || ws_bytes < qw::mfma_w4a8_workspace_bytes(M, K))
                return QW_ERR_WORKSPACE;
            return run_w4_tile(X, Wq, w_scale, M, N, K, Y, workspace, v, stream);
        }
        int nw, mb, nbw;
        qw::mfma_default_shape(4, M, K, &nw, &mb, &nbw);
        return run_gemm_w4a8(X, Wq, w_scale, M, N, K, Y, workspace, ws_bytes, nw, mb, nbw, stream);
    }
    return run_w4a8(X, Wq, w_scale, M, N, K, Y, nullptr, nullptr, nullptr, workspace,
                    default_tiling(4, M, N, K), false, stream);
}

int gemv_w4a8_noalloc(const float* X, const void* Wq, const float* w_scale, int64_t M,
                      int64_t N, int64_t K, float* Y, void* stream)
{
    if (!X || !Wq || !w_scale || !Y)
        return QW_ERR_NULL;
    if (check_gemv_shape(4, M, N, K) != QW_OK)
        return QW_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y))
        return QW_ERR_ALIGN;
    const size_t need = qw_workspace_bytes(0, M, N, K);
    if (need > kScratchBytes)
        return QW_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const int st = scratch_address(&ws);
        if (st != QW_OK)
            return st;
    }
    return gemv_w4a8(X, Wq, w_scale, M, N, K, Y, ws, need, stream);
}

int qw_gemv_w4a8_debug(const float* X, const void* Wq, const float* w_scale, int64_t M,
                       int64_t N, int64_t K, float* Y, int32_t* acc, int8_t* xq, float* a_scale,
                       void* workspace, size_t ws_bytes, void* stream)
{
    (void)ws_bytes;
    if (check_gemv_shape(4, M, N, K) != QW_OK)
        return (!X || !Wq || !w_scale || !Y) ? QW_ERR_NULL : QW_ERR_SHAPE;
    // the debug outputs come from the built-in variant where it has a debug build (the
    // producer, register and LDS variants), else from the register or LDS variant (every
    // variant gives the same bits)
    GemvTiling t = default_tiling(4, M, N, K);
    if (t.u == 5 && !((t.nw == 8 && t.prod == 2) || (t.nw == 4 && t.prod == 4))) {
        // producer shapes built with debug outputs: 8 + 2 waves (one workgroup per CU) or
        // 4 + 4 (at most one workgroup per two row groups); the same bits as any shape
        const qw::TileLayout L = qw::tile_layout(4, N, K);
        const int cus = device_cus();
        t = L.nrg >= 2048 ? make_tiling(4, M, N, K, 5, 8, cus * 8, 2)
                          : make_tiling(4, M, N, K, 5, 4,
                                        (int)std::min<int64_t>(cus, std::max<int64_t>(1, L.nrg / 2)) * 4, 4);
    }
    if (t.u == 2 || t.u == 3) {
        const qw::TileLayout L = qw::tile_layout(4, N, K);
        t = L.cg <= qw::kRegCG && M == 1 ? make_tiling(4, M, N, K, 0, 4, L.nrg < 1600 ? L.nrg : 1600)
                                         : make_tiling(4, M, N, K, 8, 4, L.nrg < 4096 ? L.nrg : 4096);
    }
    return run_w4a8(X, Wq, w_scale, M, N, K, Y, acc, xq, a_scale, workspace, t, true, stream);
}

int qw_gemv_w4a8_tiled(const float* X, const void* Wq, const float* w_scale, int64_t M,
                       int64_t N, int64_t K, float* Y, int u, int nw, int nwaves, int splitk,
                       void* stream)
{
    if (check_gemv_shape(4, M, N, K) != QW_OK)
        return (!X || !Wq || !w_scale || !Y) ? QW_ERR_NULL : QW_ERR_SHAPE;
    if (!tiling_ok(4, M, u, nw, nwaves, splitk, qw::tile_layout(4, N, K)))
        return QW_ERR_TILING;
    const GemvTiling t = make_tiling(4, M, N, K, u, nw, nwaves, splitk);
    if (!fits_lds(t))
        return QW_ERR_TILING;
    return run_w4a8(X, Wq, w_scale, M, N, K, Y, nullptr, nullptr, nullptr, nullptr, t, false,
                    stream);
}

int gemv_w8a16(const uint16_t* X_f16, const void* Wq, const uint16_t* w_scale_f16, int64_t M,
               int64_t N, int64_t K, uint16_t* Y_f16, void* workspace, size_t ws_bytes,
               void* stream)
{
    (void)ws_bytes;
    if (check_gemv_shape(8, M, N, K) != QW_OK)
        return (!X_f16 || !Wq || !w_scale_f16 || !Y_f16) ? QW_ERR_NULL : QW_ERR_SHAPE;
    if (M >= qw::kMfmaMinM8 && !long_k_rows(8, M, N, K)) {
        const int v = tile_variant(8, M, N);
        if (v >= 0)
            return qw_gemm_w8a16_tile(X_f16, Wq, w_scale_f16, M, N, K, Y_f16, v, stream);
        int nw, mb, nbw;
        qw::mfma_default_shape(8, M, K, &nw, &mb, &nbw);
        return run_gemm_w8a16(X_f16, Wq, w_scale_f16, M, N, K, Y_f16, workspace, nw, mb, nbw,
                              stream);
    }
    return run_w8a16(X_f16, Wq, w_scale_f16, M, N, K, Y_f16, workspace,
                     default_tiling(8, M, N, K), stream);
}

int qw_gemv_w8a16_tiled(const uint16_t* X_f16, const void* Wq, const uint16_t* w_scale_f16,
                        int64_t M, int64_t N, int64_t K, uint16_t* Y_f16, int u, int nw,
                        int nwaves, int splitk, void* stream)
{
    if (check_gemv_shape(8, M, N, K) != QW_OK)
        return (!X_f16 || !Wq || !w_scale_f16 || !Y_f16) ? QW_ERR_NULL : QW_ERR_SHAPE;
    if (!tiling_ok(8, M, u, nw, nwaves, splitk, qw::tile_layout(8, N, K)))
        return QW_ERR_TILING;
    const GemvTiling t = make_tiling(8, M, N, K, u, nw, nwaves, splitk);
    if (!fits_lds(t))
        return QW_ERR_TILING;
    return run_w8a16(X_f16, Wq, w_scale_f16, M, N, K, Y_f16, nullptr, t, stream);
}

int qw_gemm_w4a8_mfma(const float* X, const void* Wq, const float* w_scale, int64_t M,
                      int64_t N, int64_t K, float* Y, void* workspace, size_t ws_bytes, int nw,
                      int mb, int nbw, void* stream)
{
    if (check_gemv_shape(4, M, N, K) != QW_OK)
        return (!X || !Wq || !w_scale || !Y) ? QW_ERR_NULL : QW_ERR_SHAPE;
    if (!qw::mfma_shape_ok(4, nw, mb, nbw))
        return QW_ERR_TILING;
    if (mb == 0 && (K + 511) / 512 * 8192 > 65536)  // X resident in LDS: K up to 4096
        return QW_ERR_TILING;
    return run_gemm_w4a8(X, Wq, w_scale, M, N, K, Y, workspace, ws_bytes, nw, mb, nbw, stream);
}

int qw_gemv_w4a8_long_k(const float* X, const void* Wq, const float* w_scale, int64_t M,
                        int64_t N, int64_t K, float* Y, void* workspace, size_t ws_bytes,
                        int waves, int workgroups, void* stream)
{
    if (check_gemv_shape(4, M, N, K) != QW_OK)
        return (!X || !Wq || !w_scale || !Y) ? QW_ERR_NULL : QW_ERR_SHAPE;
    if (!w4_bsplit_ok(M, N, K, waves, workgroups))
        return QW_ERR_TILING;
    return run_w4_bsplit(X, Wq, w_scale, M, N, K, Y, workspace, ws_bytes, waves, workgroups, stream);
}

int qw_gemm_w8a16_mfma(const uint16_t* X_f16, const void* Wq, const uint16_t* w_scale_f16,
                       int64_t M, int64_t N, int64_t K, uint16_t* Y_f16, int nw, int mb, int nbw,
                       void* stream)
{
    if (check_gemv_shape(8, M, N, K) != QW_OK)
        return (!X_f16 || !Wq || !w_scale_f16 || !Y_f16) ? QW_ERR_NULL : QW_ERR_SHAPE;
    if (!qw::mfma_shape_ok(8, nw, mb, nbw))
        return QW_ERR_TILING;
    // balanced: K up to 4096; nbw 1 up to 16 rows of X, nbw 2 up to 1024
    if (mb == 0 && ((K + 511) / 512 > 8 || M > (nbw == 1 ? 16 : 1024)))
        return QW_ERR_TILING;
    return run_gemm_w8a16(X_f16, Wq, w_scale_f16, M, N, K, Y_f16, nullptr, nw, mb, nbw, stream);
}

int qw_gemm_w8a16_tile(const uint16_t* X_f16, const void* Wq, const uint16_t* w_scale_f16,
                       int64_t M, int64_t N, int64_t K, uint16_t* Y_f16, int variant, void* stream)
{
    if (!X_f16 || !Wq || !w_scale_f16 || !Y_f16)
        return QW_ERR_NULL;
    if (check_gemv_shape(8, M, N, K) != QW_OK)
        return QW_ERR_SHAPE;
    if (!aligned16(X_f16) || !aligned16(Wq) || !aligned16(w_scale_f16) || !aligned16(Y_f16))
        return QW_ERR_ALIGN;
    if (qw::tile_rows_m(variant) == 0)
        return QW_ERR_TILING;
    return hip_status(qw::launch_gemm_w8a16_tile(X_f16, (int)M, (int)N, (int)K,
                                                 static_cast<const uint8_t*>(Wq), w_scale_f16, Y_f16,
                                                 variant, static_cast<hipStream_t>(stream)));
}

int qw_tile_variant(int bits, int64_t M, int64_t N)
{
    if ((bits != 4 && bits != 8) || M < 1 || N < 1)
        return -1;
    return tile_variant(bits, M, N);
}

int qw_gemm_w4a8_tile(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
                      int64_t K, float* Y, void* workspace, size_t ws_bytes, int variant,
                      void* stream)
{
    if (!X || !Wq || !w_scale || !Y)
        return QW_ERR_NULL;
    if (check_gemv_shape(4, M, N, K) != QW_OK)
        return QW_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y) ||
        !aligned16(workspace))
        return QW_ERR_ALIGN;
    if (!workspace || ws_bytes < qw::mfma_w4a8_workspace_bytes(M, K))
        return QW_ERR_WORKSPACE;
    if (qw::tile_rows_m(variant) == 0)
        return QW_ERR_TILING;
    return run_w4_tile(X, Wq, w_scale, M, N, K, Y, workspace, variant, stream);
}

int qw_w4_codes(const void* Wq, int64_t N, int64_t K, int8_t* codes, void* stream)
{
    if (!Wq || !codes)
        return QW_ERR_NULL;
    int st = check_shape(1, N, K);
    if (st != QW_OK)
        return st;
    if (!aligned16(Wq) || !aligned16(codes))
        return QW_ERR_ALIGN;
    return hip_status(qw::launch_codes_w4(static_cast<const uint8_t*>(Wq), (int)N, (int)K, codes,
                                          static_cast<hipStream_t>(stream)));
}

int qw_w8_codes(const void* Wq, int64_t N, int64_t K, int8_t* codes, void* stream)
{
    if (!Wq || !codes)
        return QW_ERR_NULL;
    int st = check_shape(1, N, K);
    if (st != QW_OK)
        return st;
    if (!aligned16(Wq) || !aligned16(codes))
        return QW_ERR_ALIGN;
    return hip_status(qw::launch_codes_w8(static_cast<const uint8_t*>(Wq), (int)N, (int)K, codes,
                                          static_cast<hipStream_t>(stream)));
}

const char* qw_status_str(int status)
{
    switch (status) {
    case QW_OK: return "ok";
    case QW_ERR_NULL: return "a required pointer is NULL";
    case QW_ERR_SHAPE: return "M, N or K out of range, or K not a multiple of 32";
    case QW_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case QW_ERR_WORKSPACE: return "workspace missing or smaller than qw_workspace_bytes()";
    case QW_ERR_NONFINITE: return "non-finite weight, or a scale that overflows f16";
    case QW_ERR_HIP: return "HIP runtime error (see qw_last_hip_error)";
    case QW_ERR_TILING: return "invalid tiling arguments";
    default: return "unknown status";
    }
}

int qw_last_hip_error(void) { return g_last_hip_error; }

int qw_stream_read(const void* src, size_t bytes, uint32_t* sink, int waves, int blocks,
                   int loads_in_flight, void* stream)
{
    if (!src || !sink)
        return QW_ERR_NULL;
    if (bytes == 0 || (bytes % 16) != 0)
        return QW_ERR_SHAPE;
    if (!aligned16(src) || ((uintptr_t)sink & 3u) != 0)
        return QW_ERR_ALIGN;
    if (waves == 0)
        waves = kStreamReadWaves;
    if (blocks == 0)
        blocks = device_cus();
    if (loads_in_flight == 0)
        loads_in_flight = kStreamReadLoads;
    const size_t words = bytes / 16;
    const int u = loads_in_flight;
    if (!(waves == 1 || waves == 2 || waves == 4 || waves == 8 || waves == 16) || blocks < 1 ||
        blocks > 65535 || !(u == 1 || u == 2 || u == 4 || u == 8 || u == 16))
        return QW_ERR_TILING;
    // the whole buffer addressed by one buffer resource, below 2^31 bytes
    if (bytes >= ((size_t)1 << 31))
        return QW_ERR_SHAPE;
    return hip_status(qw::launch_stream_read(static_cast<const uint8_t*>(src), words, waves, blocks,
                                             u, sink, static_cast<hipStream_t>(stream)));
}

int qw_device_status(uint32_t* status, int clear)
{
    if (!status)
        return QW_ERR_NULL;
    unsigned a = 0, b = 0;
    hipError_t e = qw::prod_guard_status_rowwise(&a, clear != 0);
    if (e == hipSuccess)
        e = qw::prod_guard_status_groupwise(&b, clear != 0);
    if (e != hipSuccess)
        return hip_status(e);
    *status = (a || b) ? QW_STATUS_PRODUCER_WAIT : 0u;
    return QW_OK;
}

}  // extern "C"
