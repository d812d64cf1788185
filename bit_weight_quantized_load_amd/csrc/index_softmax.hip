// IndexSoftmax: the integer softmax of the IntAttention summary (CSDN, MLSys 2026 paper),
// section 基准/方法设计, over int32 attention logits A [rows][L] -> UINT8 probabilities.
// Per row:
//   D  = rowMax(A) - A,  D' = min(D, c_int)                          (clipping)
//   idx = round(D' * n / c_int), n = 2^b - 1;  E = LUT[idx]           (table exponent)
//   P  = round(255 * E / sum E)                                       (integer normalisation)
// with LUT[i] = round(255 * exp(-c * i / n)), the last entry 0, and every rounding of a
// non-negative ratio half up.
//
// One workgroup per row, one pass over memory: the row is read once into registers (4 B
// per logit) and P written once (1 B).  No division per element: idx >= k exactly when
// D' >= T_k = ceil(c_int * (2k - 1) / (2n)) (host-computed thresholds, in LDS).  A float
// estimate round(D' * (n / c_int)) is within one of idx (its error is below 1e-5 of a
// step), and one comparison with the thresholds on each side makes it exact.  P depends
// on idx only, so after the row sum the 2^b probabilities round(255 * LUT[k] / sum) are
// computed once (one integer division per table entry) and gathered.
#include "common.hpp"
#include "kernels.hpp"

namespace qw {

namespace {

// Wave-wide maximum / sum of 32-bit integers (DPP within rows of 16, then across rows);
// lane 63 receives the result.
__device__ __forceinline__ int wave_max_i32_dpp(int v)
{
    v = max(v, __builtin_amdgcn_update_dpp(INT32_MIN, v, 0x128, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(INT32_MIN, v, 0x124, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(INT32_MIN, v, 0x122, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(INT32_MIN, v, 0x121, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(INT32_MIN, v, 0x142, 0xa, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(INT32_MIN, v, 0x143, 0xc, 0xf, false));
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint32_t wave_sum_u32_dpp(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// NW waves per row, V 16-byte loads (4 logits) per thread: L <= 256 * NW * V.  MAG: the
// index by one multiply-high (IndexSoftmaxArgs::magic) instead of the float estimate and
// its threshold corrections (half the vector instructions and two thirds of the LDS reads
// per logit).
template <int NW, int V, bool MAG>
__global__ __launch_bounds__(64 * NW) void k_index_softmax(const int32_t* __restrict__ A,
                                                           int64_t L, IndexSoftmaxArgs t,
                                                           uint8_t* __restrict__ P)
{
    constexpr int kThreads = 64 * NW;
    __shared__ uint32_t s_thr[64];   // T_1 .. T_n (index 0 unused)
    __shared__ uint32_t s_lut[64];   // E = LUT[idx]
    __shared__ uint32_t s_prob[64];  // P = round(255 * LUT[idx] / sum)
    __shared__ int s_red[NW];
    __shared__ uint32_t s_sum[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = (1 << t.b) - 1;
    if (tid <= n) {
        s_thr[tid] = t.thr[tid];
        s_lut[tid] = t.lut[tid];
    }
    const size_t row = blockIdx.x;
    const rsrc_t ar = make_rsrc(A + row * (size_t)L, (uint32_t)L * 4u);
    int4 a[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        a[i] = __builtin_bit_cast(int4, load16(ar, (uint32_t)(i * kThreads + tid) * 16u));
    // row maximum over the logits inside the row
    int mx = INT32_MIN;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int64_t e = 4 * (int64_t)(i * kThreads + tid);
        mx = max(mx, e < L ? a[i].x : INT32_MIN);
        mx = max(mx, e + 1 < L ? a[i].y : INT32_MIN);
        mx = max(mx, e + 2 < L ? a[i].z : INT32_MIN);
        mx = max(mx, e + 3 < L ? a[i].w : INT32_MIN);
    }
    mx = wave_max_i32_dpp(mx);
    if (lane == 0)
        s_red[wave] = mx;
    __syncthreads();
    mx = s_red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        mx = max(mx, s_red[w]);
    // table index of each logit (a byte each), and the row sum of the table values
    const uint32_t cint = (uint32_t)t.c_int;
    uint32_t idx[V];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int64_t e = 4 * (int64_t)(i * kThreads + tid);
        const int v4[4] = {a[i].x, a[i].y, a[i].z, a[i].w};
        uint32_t packed = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // mx >= v: the difference is exact as an unsigned 32-bit number
            uint32_t d = (uint32_t)mx - (uint32_t)v4[u];
            d = d < cint ? d : cint;
            uint32_t k;
            if constexpr (MAG) {
                k = __umulhi(__umul24(d, 2u * (uint32_t)n) + cint, t.magic) >> t.shift;
            } else {
                k = (uint32_t)((float)d * t.scale + 0.5f);
                k = k < (uint32_t)n ? k : (uint32_t)n;
                if (k > 0 && d < s_thr[k])
                    --k;
                else if (k < (uint32_t)n && d >= s_thr[k + 1])
                    ++k;
            }
            if (e + u < L)
                sum += s_lut[k];
            packed |= k << (8 * u);
        }
        idx[i] = packed;
    }
    sum = wave_sum_u32_dpp(sum);
    if (lane == 0)
        s_sum[wave] = sum;
    __syncthreads();
    sum = s_sum[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        sum += s_sum[w];
    // the row's probability for each table entry: round(255 * LUT[k] / sum), half up
    if (tid <= n)
        s_prob[tid] = (2u * 255u * s_lut[tid] + sum) / (2u * sum);
    __syncthreads();
    uint8_t* prow = P + row * (size_t)L;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int64_t e = 4 * (int64_t)(i * kThreads + tid);
        if (e >= L)
            continue;
        const uint32_t k = idx[i];
        const uint32_t b0 = s_prob[k & 0xff], b1 = s_prob[(k >> 8) & 0xff];
        const uint32_t b2 = s_prob[(k >> 16) & 0xff], b3 = s_prob[k >> 24];
        if (e + 3 < L && (L & 3) == 0) {
            *reinterpret_cast<uint32_t*>(prow + e) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
        } else {
            prow[e] = (uint8_t)b0;
            if (e + 1 < L) prow[e + 1] = (uint8_t)b1;
            if (e + 2 < L) prow[e + 2] = (uint8_t)b2;
            if (e + 3 < L) prow[e + 3] = (uint8_t)b3;
        }
    }
}

template <int NW, int V>
hipError_t launch_is(const int32_t* A, int64_t rows, int64_t L, const IndexSoftmaxArgs& t,
                     uint8_t* P, hipStream_t st)
{
    if (t.magic != 0)
        hipLaunchKernelGGL((k_index_softmax<NW, V, true>), dim3((unsigned)rows), dim3(64 * NW), 0, st,
                           A, L, t, P);
    else
        hipLaunchKernelGGL((k_index_softmax<NW, V, false>), dim3((unsigned)rows), dim3(64 * NW), 0,
                           st, A, L, t, P);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_index_softmax(const int32_t* A, int64_t rows, int64_t L,
                                const IndexSoftmaxArgs& t, uint8_t* P, hipStream_t st)
{
    if (L <= 1024)
        return launch_is<4, 1>(A, rows, L, t, P, st);
    if (L <= 4096)
        return launch_is<4, 4>(A, rows, L, t, P, st);
    if (L <= 16384)
        return launch_is<8, 8>(A, rows, L, t, P, st);
    return hipErrorInvalidValue;
}

}  // namespace qw
