// C ABI of the weight-quantized decode linear: host-side validation, tiling choice
// and dispatch.  Declarations and the contract of every entry point are in
// include/qwgemv.h.
#include <hip/hip_runtime.h>

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
constexpr size_t kAlign = 256;     // workspace sub-buffer alignment

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return QW_OK;
    g_last_hip_error = (int)e;
    return QW_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_shape(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || M > kMaxM || N > kMaxN || K > kMaxK || (K % 32) != 0)
        return QW_ERR_SHAPE;
    return QW_OK;
}

int mt_for(int64_t M)
{
    if (M >= 8)
        return 8;
    if (M >= 3)
        return M >= 5 ? 8 : 4;
    return (int)M;
}

// Chunks (16 bytes of packed weights) per row: 32 INT4 or 16 INT8 weights each.
int64_t chunks_per_row(int op, int64_t K) { return op == 0 ? K / 32 : K / 16; }

bool tiling_ok(int mt, int cpl, int gb, int rows_per_wave)
{
    if (cpl != 1 && cpl != 2 && cpl != 4)
        return false;
    if (gb != 1 && gb != 2 && gb != 4 && gb != 8)
        return false;
    if (mt * cpl > 8 || gb * cpl > 16)
        return false;
    if (rows_per_wave <= 0 || rows_per_wave % (4 * gb) != 0 || rows_per_wave > 4096)
        return false;
    return true;
}

GemvTiling make_tiling(int op, int64_t M, int64_t N, int64_t K, int cpl, int gb,
                       int rows_per_wave)
{
    GemvTiling t;
    t.mt = mt_for(M);
    t.cpl = cpl;
    t.gb = gb;
    t.rows_per_wave = rows_per_wave;
    const int64_t slice = 16 * (int64_t)cpl;
    t.slices = (int)((chunks_per_row(op, K) + slice - 1) / slice);
    t.row_blocks = (int)((N + 4 * rows_per_wave - 1) / (4 * rows_per_wave));
    t.m_tiles = (int)((M + t.mt - 1) / t.mt);
    return t;
}

// Built-in tiling for the GEMV kernels.
GemvTiling default_tiling(int op, int64_t M, int64_t N, int64_t K)
{
    const int mt = mt_for(M);
    const int64_t cpr = chunks_per_row(op, K);
    int cpl = cpr >= 256 ? 4 : (cpr >= 32 ? 2 : 1);
    while (mt * cpl > 8)
        cpl >>= 1;
    const int64_t slices = (cpr + 16 * cpl - 1) / (16 * cpl);
    const int64_t m_tiles = (M + mt - 1) / mt;
    // Aim at about four workgroups per compute unit (256 CUs).
    const int64_t target = 1024;
    int64_t blocks = (target + slices * m_tiles - 1) / (slices * m_tiles);
    if (blocks < 1)
        blocks = 1;
    int64_t rpw = (N + 4 * blocks - 1) / (4 * blocks);
    int gb = 4;
    while (gb * cpl > 16)
        gb >>= 1;
    if (rpw < 4 * gb) {
        gb = rpw <= 4 ? 1 : (rpw <= 8 ? 2 : gb);
    }
    rpw = (rpw + 4 * gb - 1) / (4 * gb) * (4 * gb);
    if (rpw > 4096)
        rpw = 4096;
    return make_tiling(op, M, N, K, cpl, gb, (int)rpw);
}

// Workspace layout: [per-op data, 256-aligned][counters].
size_t workspace_for(int op, int64_t M, int64_t N, const GemvTiling& t)
{
    if (t.slices <= 1)
        return 0;
    size_t data = op == 0 ? (size_t)M * (size_t)N * 4u
                          : (size_t)t.slices * (size_t)M * (size_t)N * 4u;
    size_t counters = (size_t)t.row_blocks * (size_t)t.m_tiles * 4u;
    return round_up(data, kAlign) + round_up(counters, kAlign);
}

size_t counters_offset(int op, int64_t M, int64_t N, const GemvTiling& t)
{
    size_t data = op == 0 ? (size_t)M * (size_t)N * 4u
                          : (size_t)t.slices * (size_t)M * (size_t)N * 4u;
    return round_up(data, kAlign);
}

// One device int per GPU for the packers' non-finite flag.
std::mutex g_flag_mu;
int* g_flag[64] = {nullptr};

int get_flag(int** out)
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
    *out = g_flag[dev];
    return QW_OK;
}

int read_flag(int* flag, hipStream_t st, int* host)
{
    hipError_t e = hipMemcpyAsync(host, flag, sizeof(int), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess)
        e = hipStreamSynchronize(st);
    return hip_status(e);
}

int run_w4a8(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
             int64_t K, float* Y, int32_t* acc, int8_t* xq, float* a_scale, void* workspace,
             size_t ws_bytes, const GemvTiling& t, bool debug, void* stream)
{
    if (!X || !Wq || !w_scale || !Y)
        return QW_ERR_NULL;
    int st = check_shape(M, N, K);
    if (st != QW_OK)
        return st;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y) ||
        !aligned16(workspace) || !aligned16(acc) || !aligned16(xq) || !aligned16(a_scale))
        return QW_ERR_ALIGN;
    const size_t need = workspace_for(0, M, N, t);
    if (need > 0 && (workspace == nullptr || ws_bytes < need))
        return QW_ERR_WORKSPACE;
    qw::W4A8Args a;
    a.X = X;
    a.Wq = static_cast<const uint8_t*>(Wq);
    a.w_scale = w_scale;
    a.Y = Y;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.rows_per_wave = t.rows_per_wave;
    a.acc_ws = need ? static_cast<int32_t*>(workspace) : nullptr;
    a.counters = need ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                                    counters_offset(0, M, N, t))
                      : nullptr;
    a.dbg_acc = acc;
    a.dbg_xq = xq;
    a.dbg_a = a_scale;
    return hip_status(qw::launch_gemv_w4a8(a, t, debug, static_cast<hipStream_t>(stream)));
}

int run_w8a16(const uint16_t* X, const void* Wq, const uint16_t* w_scale, int64_t M, int64_t N,
              int64_t K, uint16_t* Y, void* workspace, size_t ws_bytes, const GemvTiling& t,
              void* stream)
{
    if (!X || !Wq || !w_scale || !Y)
        return QW_ERR_NULL;
    int st = check_shape(M, N, K);
    if (st != QW_OK)
        return st;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Y) ||
        !aligned16(workspace))
        return QW_ERR_ALIGN;
    const size_t need = workspace_for(1, M, N, t);
    if (need > 0 && (workspace == nullptr || ws_bytes < need))
        return QW_ERR_WORKSPACE;
    qw::W8A16Args a;
    a.X = X;
    a.Wq = static_cast<const uint8_t*>(Wq);
    a.w_scale = w_scale;
    a.Y = Y;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.rows_per_wave = t.rows_per_wave;
    a.part_ws = need ? static_cast<float*>(workspace) : nullptr;
    a.counters = need ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                                    counters_offset(1, M, N, t))
                      : nullptr;
    return hip_status(qw::launch_gemv_w8a16(a, t, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

size_t qw_w4_packed_bytes(int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0)
        return 0;
    return (size_t)N * (size_t)(K / 2);
}

size_t qw_w8_packed_bytes(int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0)
        return 0;
    return (size_t)N * (size_t)K;
}

size_t qw_workspace_bytes(int op, int64_t M, int64_t N, int64_t K)
{
    if ((op != 0 && op != 1) || check_shape(M, N, K) != QW_OK)
        return 0;
    return workspace_for(op, M, N, default_tiling(op, M, N, K));
}

size_t qw_tiled_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int cpl, int gb,
                                int rows_per_wave)
{
    if ((op != 0 && op != 1) || check_shape(M, N, K) != QW_OK ||
        !tiling_ok(mt_for(M), cpl, gb, rows_per_wave))
        return 0;
    return workspace_for(op, M, N, make_tiling(op, M, N, K, cpl, gb, rows_per_wave));
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
    int* flag = nullptr;
    if ((st = get_flag(&flag)) != QW_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = qw::launch_fill_zero(reinterpret_cast<uint32_t*>(flag), 1, s);
    if (e == hipSuccess)
        e = qw::launch_pack_w4(W, (int)N, (int)K, static_cast<uint8_t*>(Wq), w_scale, flag, s);
    if (e != hipSuccess)
        return hip_status(e);
    int host = 0;
    if ((st = read_flag(flag, s, &host)) != QW_OK)
        return st;
    return host ? QW_ERR_NONFINITE : QW_OK;
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
    int* flag = nullptr;
    if ((st = get_flag(&flag)) != QW_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = qw::launch_fill_zero(reinterpret_cast<uint32_t*>(flag), 1, s);
    if (e == hipSuccess)
        e = qw::launch_pack_w8(W, (int)N, (int)K, static_cast<int8_t*>(Wq), w_scale_f16, flag, s);
    if (e != hipSuccess)
        return hip_status(e);
    int host = 0;
    if ((st = read_flag(flag, s, &host)) != QW_OK)
        return st;
    return host ? QW_ERR_NONFINITE : QW_OK;
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
    if (check_shape(M, N, K) != QW_OK)
        return (!X || !Wq || !w_scale || !Y) ? QW_ERR_NULL : QW_ERR_SHAPE;
    return run_w4a8(X, Wq, w_scale, M, N, K, Y, nullptr, nullptr, nullptr, workspace, ws_bytes,
                    default_tiling(0, M, N, K), false, stream);
}

int qw_gemv_w4a8_debug(const float* X, const void* Wq, const float* w_scale, int64_t M,
                       int64_t N, int64_t K, float* Y, int32_t* acc, int8_t* xq, float* a_scale,
                       void* workspace, size_t ws_bytes, void* stream)
{
    if (check_shape(M, N, K) != QW_OK)
        return (!X || !Wq || !w_scale || !Y) ? QW_ERR_NULL : QW_ERR_SHAPE;
    return run_w4a8(X, Wq, w_scale, M, N, K, Y, acc, xq, a_scale, workspace, ws_bytes,
                    default_tiling(0, M, N, K), true, stream);
}

int qw_gemv_w4a8_tiled(const float* X, const void* Wq, const float* w_scale, int64_t M,
                       int64_t N, int64_t K, float* Y, void* workspace, size_t ws_bytes, int cpl,
                       int gb, int rows_per_wave, void* stream)
{
    if (check_shape(M, N, K) != QW_OK)
        return (!X || !Wq || !w_scale || !Y) ? QW_ERR_NULL : QW_ERR_SHAPE;
    if (!tiling_ok(mt_for(M), cpl, gb, rows_per_wave))
        return QW_ERR_TILING;
    return run_w4a8(X, Wq, w_scale, M, N, K, Y, nullptr, nullptr, nullptr, workspace, ws_bytes,
                    make_tiling(0, M, N, K, cpl, gb, rows_per_wave), false, stream);
}

int gemv_w8a16(const uint16_t* X_f16, const void* Wq, const uint16_t* w_scale_f16, int64_t M,
               int64_t N, int64_t K, uint16_t* Y_f16, void* workspace, size_t ws_bytes,
               void* stream)
{
    if (check_shape(M, N, K) != QW_OK)
        return (!X_f16 || !Wq || !w_scale_f16 || !Y_f16) ? QW_ERR_NULL : QW_ERR_SHAPE;
    return run_w8a16(X_f16, Wq, w_scale_f16, M, N, K, Y_f16, workspace, ws_bytes,
                     default_tiling(1, M, N, K), stream);
}

int qw_gemv_w8a16_tiled(const uint16_t* X_f16, const void* Wq, const uint16_t* w_scale_f16,
                        int64_t M, int64_t N, int64_t K, uint16_t* Y_f16, void* workspace,
                        size_t ws_bytes, int cpl, int gb, int rows_per_wave, void* stream)
{
    if (check_shape(M, N, K) != QW_OK)
        return (!X_f16 || !Wq || !w_scale_f16 || !Y_f16) ? QW_ERR_NULL : QW_ERR_SHAPE;
    if (!tiling_ok(mt_for(M), cpl, gb, rows_per_wave))
        return QW_ERR_TILING;
    return run_w8a16(X_f16, Wq, w_scale_f16, M, N, K, Y_f16, workspace, ws_bytes,
                     make_tiling(1, M, N, K, cpl, gb, rows_per_wave), stream);
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
    return hip_status(qw::launch_codes_w8(static_cast<const int8_t*>(Wq), (int)N, (int)K, codes,
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

}  // extern "C"
