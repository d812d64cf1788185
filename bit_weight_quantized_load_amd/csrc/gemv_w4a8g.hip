// Group-wise W4A8 GEMV (M == 1): launchers of the producer-wave kernel (w4a8_prod.hpp)
// with one fp32 scale per output row and group of g consecutive k.  The group-wise
// scale is listed as future work in "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到
// 19.6 tok/s", section 后续优化方向; everything else is the row-wise path: INT4 codes in
// the same tile layout, the activation quantized per vector by producer waves, int8
// dots into int32.
#include "common.hpp"
#include "kernels.hpp"
#include "w4a8_prod.hpp"

namespace qw {

namespace {

template <int T, int NW, int P, int S, int LG>
hipError_t launch_g(const W4A8Args& a, const GemvTiling& t, hipStream_t st)
{
    hipLaunchKernelGGL((k_gemv_w4a8_prod<T, NW, P, S, LG, false>), dim3(t.blocks),
                       dim3(64 * (NW + P)), 0, st, a);
    return hipGetLastError();
}

// K <= 4096: 8 consumer + 2 producer waves or 4 + 4
template <int LG, int T>
hipError_t launch_g_w(const W4A8Args& a, const GemvTiling& t, hipStream_t st)
{
    if (t.nw == 8 && t.prod == 2) return launch_g<T, 8, 2, 1, LG>(a, t, st);
    if (t.nw == 4 && t.prod == 4) return launch_g<T, 4, 4, 1, LG>(a, t, st);
    return hipErrorInvalidValue;
}

// K split over S consumer waves of 5 or 6 tiles: 8 consumer + 8 producer waves (a wave's
// group scales take registers too: 7 tiles would spill)
template <int LG, int S>
hipError_t launch_g_s(const W4A8Args& a, const GemvTiling& t, hipStream_t st)
{
    if (t.nw != 8 || t.prod != 8)
        return hipErrorInvalidValue;
    switch (t.reg_cg) {
    case 5: return launch_g<5, 8, 8, S, LG>(a, t, st);
    case 6: return launch_g<6, 8, 8, S, LG>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

template <int LG>
hipError_t launch_g_any(const W4A8Args& a, const GemvTiling& t, hipStream_t st)
{
    switch (t.splitk) {
    case 2: return launch_g_s<LG, 2>(a, t, st);
    case 4: return launch_g_s<LG, 4>(a, t, st);
    case 8: return launch_g_s<LG, 8>(a, t, st);
    default: break;
    }
    switch (t.reg_cg) {
    case 1: return launch_g_w<LG, 1>(a, t, st);
    case 2: return launch_g_w<LG, 2>(a, t, st);
    case 3: return launch_g_w<LG, 3>(a, t, st);
    case 4: return launch_g_w<LG, 4>(a, t, st);
    case 5: return launch_g_w<LG, 5>(a, t, st);
    case 6: return launch_g_w<LG, 6>(a, t, st);
    case 7: return launch_g_w<LG, 7>(a, t, st);
    case 8: return launch_g_w<LG, 8>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t prod_guard_status_groupwise(unsigned* trips, bool clear)
{
    return read_prod_guard(trips, clear);
}

hipError_t launch_gemv_w4a8g(const W4A8Args& a, const GemvTiling& t, int group, hipStream_t st)
{
    if (t.u != 5 && t.u != 6)
        return hipErrorInvalidValue;
    switch (group) {
    case 32: return launch_g_any<1>(a, t, st);
    case 64: return launch_g_any<2>(a, t, st);
    case 128: return launch_g_any<4>(a, t, st);
    case 256: return launch_g_any<8>(a, t, st);
    case 512: return launch_g_any<16>(a, t, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qw
