// Launch-shape selection of the GEMV kernels (W4A8 and W8A16, every variant): shape
// limits, the check and construction of a launch shape, and the built-in shape per
// problem.  Included by api.hip inside its anonymous namespace; host code only.
#pragma once

// Largest K of the GEMVs: the streaming variant keeps one row of X (quantized codes
// for W4A8, f16 for W8A16) in LDS, so K is bounded by the LDS budget.
constexpr int64_t kMaxGemvK4 = 57344;
constexpr int64_t kMaxGemvK8 = 28672;

int check_gemv_shape(int bits, int64_t M, int64_t N, int64_t K)
{
    const int st = check_shape(M, N, K);
    if (st != QW_OK)
        return st;
    return K <= (bits == 4 ? kMaxGemvK4 : kMaxGemvK8) ? QW_OK : QW_ERR_SHAPE;
}

// Bytes of LDS activation storage per tile per row of X: 16 chunks x 32 INT8 codes
// (W4A8) or 32 chunks x 16 f16 values (W8A16).
int act_tile_bytes(int bits) { return bits == 4 ? 512 : 1024; }

int scale_lds_bytes(int bits, int nw) { return bits == 4 ? 4 * 64 * nw * 4 : 2 * 64 * nw * 2; }

// Launch-shape check.  u = 0: register variant (M == 1, K <= 4096); u = 1: eager
// variant (at most 16 tiles per wave, at most 4 rows of X per workgroup); u = 4 or 8:
// streaming LDS variant with u tiles per batch.  4, 8 or 16 waves per workgroup; at
// most 64 row groups per row run (the workgroup's output scales are staged in LDS); a
// workgroup's tiles addressable by one buffer resource.  splitk 2 or 4: LDS variant
// only, 4 or 8 waves, at most 16 row groups per row run.
bool tiling_ok(int bits, int64_t M, int u, int nw, int nwaves, int splitk,
               const qw::TileLayout& L)
{
    // producer variant (INT4, M == 1, K <= 4096): nw consumer and splitk producer waves
    // per workgroup, (8, 2), (6, 2), (5, 3) or (4, 4); nwaves = workgroups * nw; a
    // workgroup's tiles addressable by one buffer resource
    if (u == 5) {
        const bool pair = (nw == 8 && splitk == 2) || (nw == 6 && splitk == 2) ||
                          (nw == 5 && splitk == 3) || (nw == 4 && splitk == 4);
        if (bits != 4 || M != 1 || L.cg > qw::kRegCG || !pair || nwaves < nw || nwaves % nw != 0)
            return false;
        const int64_t blocks = nwaves / nw;
        const int64_t per_blk = ((int64_t)L.nrg + blocks - 1) / blocks;
        return per_blk * L.cg * 1024 < ((int64_t)1 << 31);
    }
    // producer variant with K split (INT4, M == 1): 8 consumer and 8 producer waves per
    // workgroup, K split over splitk = 2, 4 or 8 consumer waves of at most 7 tiles each,
    // at most 16 row groups per workgroup
    if (u == 6) {
        if (bits != 4 || M != 1 || nw != 8 || !(splitk == 2 || splitk == 4 || splitk == 8) ||
            nwaves < nw || nwaves % nw != 0 || (L.cg + splitk - 1) / splitk > 7)
            return false;
        const int64_t blocks = nwaves / nw;
        const int64_t per_blk = ((int64_t)L.nrg + blocks - 1) / blocks;
        return per_blk <= 16 && per_blk * L.cg * 1024 < ((int64_t)1 << 31);
    }
    // balanced long-K variant (INT8): nwaves workgroups (one per CU, more only past 16
    // row groups each) of nw == splitk waves, each taking a k-slice of every row group
    // of the workgroup, for 1, 2 or 4 rows of X (a grid row per such group of rows):
    // at M == 1 up to 16 waves with slices of at most 4 tiles, else up to 8 waves with
    // slices of at most 8 tiles (at most 5 when M >= 3)
    if (u == 7) {
        const int T = (L.cg + splitk - 1) / splitk;
        if (bits != 8 || nw != splitk || splitk < 1 || T > 8 || splitk > (T <= 4 && M == 1 ? 16 : 8) ||
            nwaves < 1)
            return false;
        const int64_t per = ((int64_t)L.nrg + nwaves - 1) / nwaves;
        const int64_t mtiles = M == 1 ? 1 : (M + 1) / 2;  // at least 2 rows of X per workgroup
        return per <= 16 && per * L.cg * 1024 < ((int64_t)1 << 31) &&
               (int64_t)nwaves * mtiles * 64 * splitk < ((int64_t)1 << 31);
    }
    if (u < 0 || u > 8 || u == 5 || u == 6)
        return false;
    // all in flight with K split over 2..8 (INT4) or 2..7 (INT8) waves of 8-tile slices:
    // one row run of at most 4 row groups per workgroup, M == 1, K <= 4096 * splitk
    if (u == 3) {
        const int64_t per = nwaves < 1 ? 0 : ((int64_t)L.nrg + nwaves - 1) / nwaves;
        return M == 1 && splitk >= 2 && splitk <= (bits == 4 ? 8 : 7) && L.cg <= 8 * splitk &&
               per >= 1 && per <= 4;
    }
    if ((u == 0 || u == 2) && !(M == 1 && L.cg <= qw::kRegCG))
        return false;
    // all in flight: 4 waves per workgroup with at most 4 (INT8) or 5 (INT4) row groups
    // per wave, or for INT4 8 waves with at most 3
    if (u == 2) {
        const int64_t per = nwaves < 1 ? 0 : ((int64_t)L.nrg + nwaves - 1) / nwaves;
        const int64_t cap = bits == 8 ? (nw == 4 ? 4 : 0) : (nw == 4 ? 5 : (nw == 8 ? 3 : 0));
        if (splitk != 1 || nwaves < 1 || per > cap)
            return false;
    }
    if (nw != 4 && nw != 8 && nw != 16)
        return false;
    if (splitk != 1 && splitk != 2 && splitk != 4)
        return false;
    if (splitk > 1 && (u < 4 || nw == 16))
        return false;
    if (nwaves < 1)
        return false;
    const int64_t per_wave = ((int64_t)L.nrg + nwaves - 1) / nwaves;
    if (per_wave > (splitk > 1 ? 16 : 64))
        return false;
    if (u == 1 && per_wave * L.cg > 16)
        return false;
    if ((int64_t)nw * per_wave * L.cg * 1024 >= ((int64_t)1 << 31))
        return false;
    (void)bits;
    return true;
}

GemvTiling make_tiling(int bits, int64_t M, int64_t N, int64_t K, int u, int nw, int nwaves,
                       int splitk = 1)
{
    const qw::TileLayout L = qw::tile_layout(bits, N, K);
    GemvTiling t;
    t.u = u;
    t.nw = nw;
    t.splitk = splitk;
    t.nwaves = nwaves;
    const int runs = nw / splitk > 0 ? nw / splitk : 1;  // row runs per workgroup
    t.blocks = (nwaves + runs - 1) / runs;
    t.tmax = 0;
    t.reg_cg = 0;
    t.prod = 0;
    if (u == 5 || u == 6) {
        // producer variant; u == 5: splitk carries the producer waves, every row of codes
        // in registers; u == 6: 8 producer waves, K split over splitk consumer waves of
        // reg_cg >= 5 tiles each.  LDS is static.
        t.prod = u == 5 ? splitk : 8;
        t.splitk = u == 5 ? 1 : splitk;
        t.blocks = nwaves / nw;
        t.reg_cg = u == 5 ? L.cg : std::max(5, (L.cg + splitk - 1) / splitk);
        t.mt = 1;
        t.m_tiles = 1;
        t.lds_bytes = 0;
        return t;
    }
    if (u == 7) {
        t.blocks = nwaves;
        t.reg_cg = (L.cg + splitk - 1) / splitk;  // tiles per k-slice
        t.mt = M == 1 ? 1 : (M >= 3 && t.reg_cg <= 5 ? 4 : 2);  // rows of X per workgroup
        t.m_tiles = (int)((M + t.mt - 1) / t.mt);
        t.lds_bytes = 0;
        return t;
    }
    const int scale_bytes = scale_lds_bytes(bits, nw);
    int tiles = 0, mt_cap = splitk > 1 ? 2 : 8;
    if (u == 3) {
        // one row run per workgroup of splitk waves; LDS: X (codes or f16) for 8 * splitk
        // tiles, then RPW rows' scales and partial sums
        const int per = (int)(((int64_t)L.nrg + nwaves - 1) / nwaves);
        t.tmax = per == 3 ? 4 : per;
        t.nw = splitk;
        t.blocks = nwaves;
        t.mt = 1;
        t.m_tiles = (int)M;
        const int R = bits == 4 ? 4 : 2;
        t.lds_bytes = 8 * splitk * act_tile_bytes(bits) + t.tmax * R * 4 + t.tmax * R * splitk * 4;
        return t;
    }
    if (u == 0) {
        t.reg_cg = L.cg;
        mt_cap = 1;
        tiles = bits == 4 ? L.cg : 0;  // W8A16 keeps X in registers, W4A8 stages codes
    } else if (u == 2) {
        // all in flight: at most 4 row groups per wave, X (codes or f16) staged in LDS
        t.reg_cg = L.cg;
        t.tmax = (int)(((int64_t)L.nrg + nwaves - 1) / nwaves);
        mt_cap = 1;
        tiles = L.cg;
    } else if (u == 1) {
        const int64_t per_wave = ((int64_t)L.nrg + nwaves - 1) / nwaves;
        t.tmax = per_wave * L.cg <= 8 ? 8 : 16;
        mt_cap = 4;
        tiles = L.cg;
    } else {
        const int slice = (L.cg + splitk - 1) / splitk;  // tiles per k-slice
        tiles = splitk * ((slice + u - 1) / u) * u;
    }
    // split-K partial sums: one int32 / fp32 per (run, row group, row of X, row, slice)
    const int per_wave = (int)(((int64_t)L.nrg + nwaves - 1) / nwaves);
    auto part_bytes = [&](int mt) {
        return splitk > 1 ? nw * per_wave * mt * (bits == 4 ? 4 : 2) * 4 : 0;
    };
    int mt = M >= 5 ? 8 : (M >= 3 ? 4 : (int)M);
    if (mt > mt_cap)
        mt = mt_cap;
    while (mt > 1 && mt * tiles * act_tile_bytes(bits) + scale_bytes + part_bytes(mt) > kMaxLds)
        mt >>= 1;
    t.mt = mt;
    t.lds_bytes = mt * tiles * act_tile_bytes(bits) + scale_bytes + part_bytes(mt);
    t.m_tiles = (int)((M + t.mt - 1) / t.mt);
    return t;
}

bool fits_lds(const GemvTiling& t) { return t.lds_bytes <= kMaxLds; }

// Compute units of the current device (one workgroup each in the producer variant),
// read once per device.
std::atomic<int> g_cus[64];

int device_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Built-in launch shape of the GEMV kernels (M == 1 for W4A8, M <= 2 for W8A16).
// Whether M rows of X with K > 4096 run the balanced long-K GEMV kernels (W4A8 from 2
// rows, W8A16 from 1) rather than the matrix-core ones: up to 8 rows (a grid row of
// workgroups per 4 rows, each reading all the weights), up to 16 when the weights are
// below 24 MB.  Measured at 16 rows: W4A8 18944 -> 3584 (34 MB) 41.3 us against 38.0
// for the 4-wave matrix-core kernel, 18944 -> 512 17.7 against 38.0; W8A16
// 8192 -> 2048 (17 MB) 17.2 against about 28.
bool long_k_rows(int bits, int64_t M, int64_t N, int64_t K)
{
    const int64_t wbytes = bits == 4 ? N * K / 2 : N * K;
    return K > 512 * qw::kRegCG && M <= 16 && (M <= 8 || wbytes < ((int64_t)24 << 20));
}

GemvTiling default_tiling(int bits, int64_t M, int64_t N, int64_t K)
{
    // Launch shapes picked by timing on MI355X at the decode shapes.  INT4 with
    // K <= 4096: activations in registers; 2048 waves (two 4-wave workgroups per CU) from
    // 2048 row groups up (7.95 us against 8.5 us at 3584 x 18944), 1024 waves (one
    // workgroup per CU) from 1024 (3584 -> 4608: 5.5 us against 6.8 us with one row
    // group per wave), else one row group per wave.  INT8 at M == 1 with K <= 4096: all weight tiles of a
    // wave in flight (12.0 us against 13.2 us at 3584 x 18944); otherwise the LDS
    // variant with 4-tile batches and about 4736 waves.  INT4 with K > 4096: the LDS variant with 4-tile batches and 8-wave
    // workgroups (one block of X per workgroup in the prologue); below 2048 row groups
    // (the 18944 -> 3584 down projection) each row group is split over two waves along
    // K, which measured 15.4 us against 19.5 us unsplit.
    const qw::TileLayout L = qw::tile_layout(bits, N, K);
    const int64_t nrg = L.nrg;
    auto waves_for = [&](int64_t target) {
        int64_t per = (nrg + target / 2) / target;
        per = per < 1 ? 1 : (per > 64 ? 64 : per);
        return (nrg + per - 1) / per;
    };
    // INT4 with K <= 4096: the producer variant.  From 2048 row groups one workgroup of 8
    // consumer and 2 producer waves per CU (3584 x 18944: 6.97 us against 8.11 us for the
    // register variant in the same session; 3584 x 152064: 41.9 against 42.5 us); below,
    // 4 consumer and 4 producer waves on at most one workgroup per two row groups
    // (3584 -> 3584: 3.28 against 4.32 us; 3584 -> 512: 3.02 against 4.16 us; 3584 -> 4608:
    // 3.87 against 4.72 us)
    // From 8192 to 16383 row groups (the fused gate|up projection 3584 -> 37888) two
    // workgroups per CU of 6 consumer and 2 producer waves: 12.16 against 13.14 us (at
    // 4736 row groups, 3584 -> 18944, slower: 7.38 against 7.10).  From
    // 1024 to 2047 row groups (the fused q|k|v 3584 -> 4608) 5 consumer and 3 producer
    // waves: 3.60 against 3.79 us.  (Measured with the timing order varied.)
    if (bits == 4 && M == 1 && L.cg <= qw::kRegCG) {
        const int cus = device_cus();
        if (nrg >= 8192 && nrg < 16384 && tiling_ok(bits, M, 5, 6, cus * 2 * 6, 2, L))
            return make_tiling(bits, M, N, K, 5, 6, cus * 2 * 6, 2);
        if (nrg >= 2048) {
            if (tiling_ok(bits, M, 5, 8, cus * 8, 2, L))
                return make_tiling(bits, M, N, K, 5, 8, cus * 8, 2);
        } else {
            const int blocks = (int)std::min<int64_t>(cus, std::max<int64_t>(1, nrg / 2));
            if (nrg >= 1024 && tiling_ok(bits, M, 5, 5, blocks * 5, 3, L))
                return make_tiling(bits, M, N, K, 5, 5, blocks * 5, 3);
            if (tiling_ok(bits, M, 5, 4, blocks * 4, 4, L))
                return make_tiling(bits, M, N, K, 5, 4, blocks * 4, 4);
        }
    }
    // INT4 with K > 4096: the producer variant with K split over 2, 4 or 8 consumer waves
    // where at most 16 row groups fall on a workgroup (18944 -> 3584: 7.9 us against 13.2 us
    // for the all-in-flight K-split variant)
    if (bits == 4 && M == 1 && L.cg > qw::kRegCG) {
        const int cus = device_cus();
        for (int S = 2; S <= 8; S *= 2)
            if (tiling_ok(bits, M, 6, 8, cus * 8, S, L))
                return make_tiling(bits, M, N, K, 6, 8, cus * 8, S);
    }
    if (bits == 4 && M == 1 && L.cg <= qw::kRegCG)
        return make_tiling(bits, M, N, K, 0, 4,
                           (int)(nrg >= 2048 ? 2048 : (nrg > 1024 ? 1024 : nrg)));
    if (bits == 8 && M == 1 && L.cg <= qw::kRegCG) {
        // every weight tile of a wave requested up front: one row group per wave, two
        // from 1024 to 2048 row groups (q/o-sized shapes), where that measured faster
        const int per = nrg >= 1024 && nrg <= 2048 ? 2 : 1;
        return make_tiling(bits, M, N, K, 2, 4, (int)((nrg + per - 1) / per));
    }
    // INT8 with K > 4096, M == 1 from 1024 row groups and 2 to 8 (16) rows always: the
    // balanced long-K variant, one workgroup per CU of min(8, ceil(CG / 4)) waves, one
    // k-slice each, 1, 2 or 4 rows of X per workgroup (at M == 1, 18944 -> 3584: 12.9 us
    // against 13.9 us for the LDS variant split over two waves; 18944 -> 4608: 16.7
    // against 19.3; 28672 -> 3584: 17.8 against 19.2; 8192 -> 2048: 5.1 against 5.9; at
    // 512 row groups, 18944 -> 1024, the all-in-flight split below stays faster: 6.0
    // against 6.9.  From 2 rows it replaces the LDS variant and the matrix-core kernels,
    // whose 128-row workgroups leave most CUs idle at these N: 18944 -> 3584 at 2, 4, 8
    // and 16 rows 14.3, 18.0, 32.7 and 62.0 us against 26.2, 82.0, 82.3 and 83.5)
    if (bits == 8 && long_k_rows(8, M, N, K) && (M >= 2 || nrg >= 1024)) {
        const int S = (int)std::min<int64_t>(8, (L.cg + 3) / 4);
        const int64_t nwg = std::max<int64_t>(std::min<int64_t>(device_cus(), nrg), (nrg + 15) / 16);
        if (tiling_ok(bits, M, 7, S, (int)nwg, S, L))
            return make_tiling(bits, M, N, K, 7, S, (int)nwg, S);
    }
    // M == 1 with K > 4096: all in flight with K split into 8-tile slices, one wave per
    // slice, where that measured faster: INT4 always (18944 -> 3584: 13.6 us against
    // 14.7 us; 18944 -> 512: 7.5 against 13.7), INT8 below 1024 row groups (18944 -> 512:
    // 4.3 us against 7.0)
    const int64_t slices = (L.cg + 7) / 8;
    if (M == 1 && slices >= 2 && slices <= (bits == 4 ? 8 : 7) && (bits == 4 || nrg < 1024)) {
        const int64_t rpw = bits == 4 && nrg >= 512 ? 4 : 1;
        const GemvTiling t = make_tiling(bits, M, N, K, 3, 4, (int)((nrg + rpw - 1) / rpw),
                                         (int)slices);
        if (t.lds_bytes <= kMaxLds)
            return t;
    }
    if (bits == 8 && M == 1 && nrg < 2048) {
        // long K, short N where neither form above applies: split K over two waves
        const GemvTiling t = make_tiling(bits, M, N, K, 4, 8, (int)nrg, 2);
        if (t.lds_bytes <= kMaxLds)
            return t;
    }
    if (bits == 8)
        return make_tiling(bits, M, N, K, 4, 4, (int)waves_for(4736));
    const GemvTiling t = nrg < 2048 ? make_tiling(bits, M, N, K, 4, 8, (int)nrg, 2)
                                    : make_tiling(bits, M, N, K, 4, 8, (int)waves_for(4096));
    if (t.lds_bytes <= kMaxLds)
        return t;
    // the longest rows of X: 4-wave workgroups, whose LDS holds one row of codes
    int64_t nwaves = nrg < 4096 ? nrg : 4096;
    while ((nrg + nwaves - 1) / nwaves > 64)
        nwaves *= 2;
    return make_tiling(bits, M, N, K, 8, 4, (int)(nwaves > nrg ? nrg : nwaves));
}
