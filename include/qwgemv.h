/*
 * qwgemv.h -- C ABI of the weight-quantized decode linear for AMD MI355X (gfx950).
 *
 * Two linears of single-batch LLM decode, each behind plain pointers and sizes:
 *
 *  W4A8  Row-wise symmetric INT4 weights with one fp32 scale per output row,
 *        activations quantized dynamically to INT8 per row of X, int8 x int8 dot
 *        products accumulated in int32, output = acc * w_scale[n] * a_scale[m].
 *        Source: "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s",
 *        sections 当前实现方式 (the three formulas) and 正确方向 (int8 dot into int32).
 *
 *  W8A16 Per-output-channel INT8 weights with an f16 scale, dequantized in registers
 *        against f16 activations, fp32 accumulation, f16 output.
 *        Source: ChatGLM2-6B W8A16 deployment on BM1684X (TPU-MLIR write-up),
 *        sections 2 (per-channel INT8 storage, F16 compute), 3 (f16 scale vector) and
 *        4 (load INT8, cast, multiply by the scale, multiply with the activation).
 *
 * Conventions for every function below:
 *  - Pointers are DEVICE pointers (memory of the current HIP device) unless a comment
 *    says otherwise.  The caller allocates and owns every buffer; the library never
 *    keeps a pointer past the call.
 *  - Matrices are row-major and contiguous: W and the packed weights are [N][K]
 *    (output rows n, input columns k), X is [M][K], Y is [M][N].
 *  - Every pointer must be 16-byte aligned.  K must be a positive multiple of 32 and
 *    at most 131072 for the packers, at most 57344 for gemv_w4a8 and 28672 for
 *    gemv_w8a16 (one row of X lives in on-chip LDS); M and N must be positive
 *    (M at most 65535).  Larger K returns QW_ERR_SHAPE.
 *  - fp16 values travel as their IEEE binary16 bit patterns in uint16_t.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.  Work is
 *    enqueued asynchronously on it and the call returns without synchronising,
 *    except for the two load-time packers (see below).
 *  - Arguments are validated on the host before any HIP call.  The return value is
 *    QW_OK or one of the error codes; nothing is enqueued when validation fails.
 *    Nothing throws across this interface.
 *  - Inputs must be finite.  The packers check and report QW_ERR_NONFINITE; for X
 *    the result of a non-finite activation is unspecified.
 */
#ifndef QWGEMV_H
#define QWGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    QW_OK = 0,
    QW_ERR_NULL = 1,       /* a required pointer is NULL                        */
    QW_ERR_SHAPE = 2,      /* M, N or K out of range, or K % 32 != 0            */
    QW_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned                  */
    QW_ERR_WORKSPACE = 4,  /* ws_bytes below qw_workspace_bytes()               */
    QW_ERR_NONFINITE = 5,  /* a packer met a non-finite weight or f16 overflow  */
    QW_ERR_HIP = 6,        /* a HIP runtime call or launch failed               */
    QW_ERR_TILING = 7      /* launch-shape arguments of a *_tiled call invalid  */
};

/* Bytes of the packed weights, and their layout.  The packed buffer is a sequence
   of 1 KB tiles.  A chunk is 16 bytes of one row: 32 INT4 codes (byte j holds
   k = 2j in its low nibble and k = 2j+1 in its high nibble, 4-bit two's complement)
   or 16 INT8 codes.  A tile covers 512 consecutive k of R rows: R = 4 rows of 16
   chunks (INT4) or R = 2 rows of 32 chunks (INT8).  Tile (rg, t) holds rows
   R*rg .. R*rg+R-1 and k 512t .. 512t+511; inside it, 16-byte slot
   (n % R) * (64/R) + (chunk % (64/R)) holds row n's chunk.  Tiles are stored row group
   by row group, in k order within a row group, so a wave of 64 lanes loading 16
   bytes each reads one tile as 1 KB of contiguous memory.  Rows past N and chunks
   past K are zero padding.  Size: ceil(N/4) * ceil(K/512) KB for INT4 and
   ceil(N/2) * ceil(K/512) KB for INT8, which is N*K/2 and N*K when N % 4 == 0
   (N % 2 == 0) and K is a multiple of 512.  Returns 0 for an invalid shape.
   qw_w4_codes / qw_w8_codes decode the layout back to codes. */
size_t qw_w4_packed_bytes(int64_t N, int64_t K);
size_t qw_w8_packed_bytes(int64_t N, int64_t K);

/* Workspace that gemv_w4a8 (op 0), gemv_w8a16 (op 1) or qw_gemm_w4a8_mfma and
   qw_gemv_w4a8_long_k (op 2) need for shape (M, N, K).  0 means the call needs none
   and accepts workspace == NULL: gemv_w4a8 at M == 1 (the GEMV finishes its rows
   inside one workgroup) and gemv_w8a16 at any M.  gemv_w4a8 with M >= 2 runs on the
   matrix cores (or, with K > 4096 and up to 16 rows, on the balanced long-K kernel)
   and needs align256(ceil(M/16) * ceil(K/64) * 1024) + align256(4 * M) bytes: the
   activation codes and scales, quantized once per call (in operand order for the
   matrix cores, row-major for the long-K kernel).  Its contents need
   no initialisation and are overwritten by every call; calls that share one
   workspace must not overlap in time. */
size_t qw_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/* Zero-fills a workspace with a kernel (no memset node, safe to capture). */
int qw_workspace_clear(void* workspace, size_t ws_bytes, void* stream);

/* Row-wise INT4 quantization and packing, done once at weight-load time
   ("Jetson Orin AGX 上的 INT4 量化推理实践", section 当前实现方式).
   W fp32 [N][K] -> Wq (qw_w4_packed_bytes, tile layout) and w_scale fp32 [N] with
   w_scale[n] = maxabs(W[n,:]) / 7 (fp32 division) and codes
   clamp(rint(W / w_scale), -7, 7) (round half to even); an all-zero row has scale 0.
   Synchronises `stream` once to read back a non-finite flag: not capturable. */
int quantize_pack_w4(const float* W, int64_t N, int64_t K, void* Wq, float* w_scale,
                     void* stream);

/* Per-output-channel INT8 quantization, done once at load time (ChatGLM2-6B W8A16
   write-up, sections 2 and 3).  W fp32 [N][K] -> Wq (qw_w8_packed_bytes, tile layout) and
   w_scale_f16 [N] = f16(maxabs(W[n,:]) / 127); codes clamp(rint(W / s16), -127, 127)
   are taken against the stored f16 scale.  A row whose f16 scale is 0 gets zero
   codes; a scale that overflows f16 is QW_ERR_NONFINITE.  Synchronises once.
   The three packers share one device flag per GPU: calls from several host threads
   are serialised inside the library (each call holds a lock from clearing the flag to
   reading it back), so each reports its own non-finite status. */
int quantize_pack_w8(const float* W, int64_t N, int64_t K, void* Wq, uint16_t* w_scale_f16,
                     void* stream);

/* Dynamic per-row INT8 activation quantization ("Jetson Orin AGX 上的 INT4 量化推理实践",
   section 当前实现方式).  X fp32 [M][K] -> Xq int8 [M][K] and a_scale fp32 [M] with
   a_scale[m] = maxabs(X[m,:]) / 127 and codes clamp(rint(X / a_scale), -127, 127).
   gemv_w4a8 runs the same computation in its prologue; the codes agree bit for bit. */
int quant_act_i8(const float* X, int64_t M, int64_t K, int8_t* Xq, float* a_scale,
                 void* stream);

/* W4A8 linear ("Jetson Orin AGX 上的 INT4 量化推理实践", sections 当前实现方式 and 正确方向).
   X fp32 [M][K], Wq from quantize_pack_w4, w_scale fp32 [N] -> Y fp32 [M][N] with
   Y[m][n] = ((float)acc[m][n] * w_scale[n]) * a_scale[m] and
   acc[m][n] = sum_k q[n][k] * xq[m][k] in int32, where xq and a_scale are exactly
   what quant_act_i8 computes.  M == 1: one GEMV kernel with the activation
   quantization fused into its prologue; workspace may be NULL.  M >= 2: the
   quantization runs once into `workspace` (at least qw_workspace_bytes(0, M, N, K)
   bytes, else QW_ERR_WORKSPACE), then an int8 matrix-core GEMM (from 33 rows, where
   the output has at least 96 tiles, the tiled GEMM of qw_gemm_w4a8_tile at the variant
   a model of the tiles per CU picks; from 20 rows its 128 by 32 tiles where there are
   at least 128 of them), or with
   K > 4096 and up to 8 rows (16 with packed weights below 24 MB) the balanced long-K
   GEMV kernel (qw_gemv_w4a8_long_k); results are the same bits as the GEMV's. */
int gemv_w4a8(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
              int64_t K, float* Y, void* workspace, size_t ws_bytes, void* stream);

/* gemv_w4a8 for callers that cannot allocate (code under HIP graph capture, tight
   serving loops, harnesses that forbid hipMalloc): the same computation and the same
   output bits as gemv_w4a8, but from two rows of X the activation codes and scales go
   to a fixed array of 8 MiB in device memory that the library holds on each GPU it runs
   on until the process ends, instead of a caller's workspace.  The call allocates
   nothing (no hipMalloc, hipFree or allocating library routine); the array's address is
   looked up once per device on the first call, with that device current.  Shapes whose
   workspace (qw_workspace_bytes(0, M, N, K)) exceeds 8 MiB return QW_ERR_WORKSPACE
   (e.g. M = 512 fits up to K = 16320, M = 64 up to K = 57344).  Every call on one GPU
   shares that GPU's array: calls that overlap in time on one GPU (several streams or
   host threads) race and must be serialised by the caller.  The array needs no
   initialisation: each call overwrites what it reads. */
int gemv_w4a8_noalloc(const float* X, const void* Wq, const float* w_scale, int64_t M,
                      int64_t N, int64_t K, float* Y, void* stream);

/* Group-wise INT4 scales ("Jetson Orin AGX 上的 INT4 量化推理实践", section 后续优化方向,
   which lists a group-wise scale as future work; the formula is this library's reading:
   the row-wise rule applied to each group).  One fp32 scale per output row n and group t
   of `group` consecutive k, group = 32, 64, 128, 256 or 512 with K a multiple of it:
     s[n][t] = maxabs(W[n][t*group .. t*group + group - 1]) / 7,
     q[n][k] = clamp(rint(W[n][k] / s[n][k / group]), -7, 7).
   Wq has the layout of quantize_pack_w4; w_scale has a device layout of
   qw_w4g_scale_bytes(N, K, group) bytes (0 for an invalid shape or group): for each
   group of 4 rows, each row, each group of a 512-k tile, the scales of that group in
   tile order, zero padded to a multiple of 4 tiles.  qw_w4g_scales decodes it to
   [N][K / group].  Non-finite weights: QW_ERR_NONFINITE (those rows keep zero scales).
   Synchronises once on `stream`, like the other packers. */
size_t qw_w4g_scale_bytes(int64_t N, int64_t K, int64_t group);
int quantize_pack_w4g(const float* W, int64_t N, int64_t K, int64_t group, void* Wq,
                      float* w_scale, void* stream);
int qw_w4g_scales(const float* w_scale, int64_t N, int64_t K, int64_t group, float* out,
                  void* stream);

/* Group-wise W4A8 linear, M == 1 (decode; QW_ERR_SHAPE otherwise).  X fp32 [1][K], Wq
   and w_scale from quantize_pack_w4g -> Y fp32 [1][N] with, for each output row,
     acc_t = sum over k in group t of q[n][k] * xq[k]   (int32, exact),
     Y[n]  = (sum over t of (float)acc_t * s[n][t]) * a_scale,
   the activation codes xq and scale a_scale being exactly those of quant_act_i8, and
   the sum over groups taken in fp32 (in an order of the kernel's choosing: the result
   lies within (K/group + 2) * 2^-24 * sum_t |acc_t * s[n][t]| * |a_scale| of the exact
   value).  K <= 4096, or K <= 24576 when the rows fit 16 groups of 4 rows per compute
   unit; else QW_ERR_SHAPE.  No workspace (may be NULL). */
int gemv_w4a8g(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
               int64_t K, int64_t group, float* Y, void* workspace, size_t ws_bytes,
               void* stream);

/* W8A16 linear (ChatGLM2-6B W8A16 write-up, section 4).  X f16 [M][K], Wq from
   quantize_pack_w8, w_scale_f16 [N] -> Y f16 [M][N] with
   Y[m][n] = f16(w_scale[n] * sum_k q[n][k] * x[m][k]), the sum in fp32.  The per-channel
   scale is applied after the sum, which equals dequantize-then-multiply up to fp32
   rounding.  M <= 2: GEMV kernel; M >= 3: f16 matrix-core GEMM on the exactly cast
   weights (from 33 rows, where the output has at least 96 tiles, the tiled GEMM of
   qw_gemm_w8a16_tile at the variant a model of the tiles per CU picks; from 12 rows
   its 128 by 32 tiles where there are at least 128 of them), except with K > 4096 and
   up to 8 rows (16 with weights below
   24 MB), where the balanced long-K GEMV variant runs (u = 7 of qw_gemv_w8a16_tiled).
   No workspace at any M (workspace may be NULL). */
int gemv_w8a16(const uint16_t* X_f16, const void* Wq, const uint16_t* w_scale_f16, int64_t M,
               int64_t N, int64_t K, uint16_t* Y_f16, void* workspace, size_t ws_bytes,
               void* stream);

/* ---- test and tuning helpers (not on the decode path) ---------------------- */

/* Device layout -> int8 codes [N][K] (device pointer). */
int qw_w4_codes(const void* Wq, int64_t N, int64_t K, int8_t* codes, void* stream);
int qw_w8_codes(const void* Wq, int64_t N, int64_t K, int8_t* codes, void* stream);

/* gemv_w4a8 that also writes the int32 accumulators acc [M][N], the activation
   codes xq [M][K] and scales a_scale [M] its prologue computed.  Any of the three
   extra pointers may be NULL. */
int qw_gemv_w4a8_debug(const float* X, const void* Wq, const float* w_scale, int64_t M,
                       int64_t N, int64_t K, float* Y, int32_t* acc, int8_t* xq,
                       float* a_scale, void* workspace, size_t ws_bytes, void* stream);

/* The GEMV kernels (any M up to 65535, rows of X in groups of up to 8 per workgroup)
   with an explicit launch shape instead of the built-in choice.  nw = waves per
   workgroup (4, 8 or 16); nwaves = row runs along N, which split the ceil(N/4) (INT4)
   or ceil(N/2) (INT8) row groups evenly.
     u = 0  activations in registers, two batches of whole row groups in flight (M == 1,
            K <= 4096, at most 64 row groups per run);
     u = 1  every weight load of a wave issued before its first dot product (at most 16
            tiles of 512 k per wave, M <= 4 per workgroup);
     u = 2  every weight tile of a wave requested right after X, activations in
            registers (M == 1, K <= 4096; nw 4 with at most 4 (INT8) or 5 (INT4) row
            groups per run, or for INT4 nw 8 with at most 3);
     u = 3  as u = 2 with K split into 8-tile slices, one wave per slice: splitk = 2..8
            (INT4) or 2..7 (INT8) waves per workgroup with K <= 4096 * splitk, one row
            run of at most 4 row groups per workgroup (nw is ignored, M == 1);
     u = 4, 8  activations read from LDS in batches of u tiles, two batches in flight;
            splitk = 2 or 4 splits each row run's tiles over that many waves of the
            workgroup (nw 4 or 8, at most 16 row groups per run), whose partial sums
            are added in on-chip memory;
     u = 5  (INT4, M == 1, K <= 4096) producer waves: each workgroup has nw consumer
            waves streaming weights and splitk producer waves quantizing X, with
            (nw, splitk) = (8, 2), (6, 2), (5, 3) or (4, 4); nwaves = workgroups * nw,
            and the row groups are split evenly over the workgroups, then over the
            consumer waves;
     u = 6  (INT4, M == 1) the producer-wave variant with K split: nw = 8 consumer and
            8 producer waves per workgroup, each row group's tiles split over splitk =
            2, 4 or 8 consumer waves (at most 7 tiles each, so K <= 3584 * splitk),
            whose int32 partial sums are added in on-chip memory; at most 16 row groups
            per workgroup (nwaves = workgroups * 8);
     u = 7  (INT8) balanced long-K variant: nwaves workgroups, which split the row
            groups evenly (at most 16 each), of nw == splitk waves; wave s takes k-slice
            s (ceil(CG / splitk) <= 8 tiles, CG = ceil(K / 512)) of every row group of
            its workgroup with that slice of X held in registers, for 1 (M == 1), 4
            (M >= 3 with slices of at most 5 tiles) or 2 rows of X per workgroup; at
            M == 1 up to 16 waves with slices of at most 4 tiles, else up to 8.  The
            slices' fp32 sums are added in slice order.
   splitk must be 1 unless stated.  Results do not depend on the launch shape, except
   that W8A16 with splitk > 1 adds its fp32 partial sums in a different order.
   QW_ERR_TILING for an invalid shape. */
int qw_gemv_w4a8_tiled(const float* X, const void* Wq, const float* w_scale, int64_t M,
                       int64_t N, int64_t K, float* Y, int u, int nw, int nwaves, int splitk,
                       void* stream);
int qw_gemv_w8a16_tiled(const uint16_t* X_f16, const void* Wq, const uint16_t* w_scale_f16,
                        int64_t M, int64_t N, int64_t K, uint16_t* Y_f16, int u, int nw,
                        int nwaves, int splitk, void* stream);

/* gemv_w4a8g with an explicit launch shape of the producer-wave kernel: u = 5 with
   (nw, splitk) = (8, 2) or (4, 4) consumer and producer waves (K <= 4096), or u = 6 with
   K split over splitk = 2, 4 or 8 waves of at most 6 tiles (see qw_gemv_w4a8_tiled).
   QW_ERR_TILING for an invalid shape. */
int qw_gemv_w4a8g_tiled(const float* X, const void* Wq, const float* w_scale, int64_t M,
                        int64_t N, int64_t K, int64_t group, float* Y, int u, int nw,
                        int nwaves, int splitk, void* stream);

/* The matrix-core kernels (the M >= 2 path of gemv_w4a8, M >= 3 of gemv_w8a16, outside
   the long-K rows above) at any
   M with an explicit launch shape: nw waves per workgroup (4 or 8), mb blocks of 16
   rows of X per workgroup (1, 2 or 4 for W4A8, not 4 with nw 4 and nbw 2; 1 or 2 for
   W8A16), nbw blocks of 16 output rows per wave (1 or 2; not 2 with nw 8 and mb 1 for
   W4A8, not 2 with nw 8 for W8A16).  W4A8 also takes mb = 0 (nbw 1, K <= 4096): the
   balanced kernel, one workgroup per CU and block of 16 rows of X, with that block's
   activation codes resident in on-chip memory; with nw 8 and nbw 2 and 17 to 1024 rows,
   one workgroup per CU over all blocks of X, the weights held in registers after one
   pass.  W8A16 takes mb = 0 too (nw 8, K <= 4096): the balanced kernel with one wave
   per 512-k step, whose f16 X operands stay in registers, with one block of 16 rows of X
   per workgroup (nbw 1, M <= 16) or two (nbw 2, M <= 1024; each INT8 weight converted
   once for both).  Rows of X are padded to a multiple of 16 with
   zeros.  The W4A8 one needs a workspace of qw_workspace_bytes(2, M, N, K) bytes (else
   QW_ERR_WORKSPACE).  Results do not depend on the launch shape; the W4A8 outputs equal
   gemv_w4a8's bit for bit.  QW_ERR_TILING for an invalid shape. */
int qw_gemm_w4a8_mfma(const float* X, const void* Wq, const float* w_scale, int64_t M,
                      int64_t N, int64_t K, float* Y, void* workspace, size_t ws_bytes, int nw,
                      int mb, int nbw, void* stream);

/* The balanced long-K W4A8 GEMV (Jetson Orin INT4 page, sections on the correct
   direction and the current implementation: INT4 weights widened to int8, 4-way int8
   dots into int32, output acc * weight scale * activation scale) at any M with an
   explicit launch shape: X is first quantized per row (as by quant_act_i8) into the
   workspace (qw_workspace_bytes(2, M, N, K) bytes, else QW_ERR_WORKSPACE); then
   `workgroups` workgroups (at most the row-group count, at most 16 row groups each)
   of `waves` waves (1..8) each take k-slices of ceil(ceil(K / 512) / waves) <= 8 tiles
   of every row group of their share, for 1, 2 or 4 rows of X per workgroup.  The int32
   sums are exact, so the outputs equal gemv_w4a8's bit for bit; gemv_w4a8 runs this
   kernel for 2 to 16 rows with K > 4096.  QW_ERR_TILING for an invalid shape. */
int qw_gemv_w4a8_long_k(const float* X, const void* Wq, const float* w_scale, int64_t M,
                        int64_t N, int64_t K, float* Y, void* workspace, size_t ws_bytes,
                        int waves, int workgroups, void* stream);
int qw_gemm_w8a16_mfma(const uint16_t* X_f16, const void* Wq, const uint16_t* w_scale_f16,
                       int64_t M, int64_t N, int64_t K, uint16_t* Y_f16, int nw, int mb,
                       int nbw, void* stream);

/* The tiled f16 matrix-core GEMM for many rows of X (ChatGLM2-6B W8A16 write-up,
   section 4; gemv_w8a16's computation, Y = f16(s16[n] * sum_k q x) with the fp32 sum on
   the matrix cores) at an explicit launch variant: one workgroup per output tile of
   rows of W by rows of X, staged through LDS by direct loads and multiplied from there:
   variant 0: 256 by 256, eight waves; 1: 256 by 128, eight waves; 2: 128 by 128, four
   waves; 3: 128 by 128, two groups of four waves splitting each stage's k; 4: 128 by 64,
   four waves; 5: 128 by 64, two groups of four waves; 6: 64 by 64, four waves; 7: as 5
   with stages of 128 bytes of weights per row instead of 64; 8: 128 by 32, four waves,
   stages of 128 bytes.  The INT8
   weights stay INT8 in LDS and each operand is cast to f16 after it is read.  Same
   arguments and limits as gemv_w8a16; no workspace.  QW_ERR_TILING for another
   variant. */
int qw_gemm_w8a16_tile(const uint16_t* X_f16, const void* Wq, const uint16_t* w_scale_f16,
                       int64_t M, int64_t N, int64_t K, uint16_t* Y_f16, int variant, void* stream);

/* The same tiled GEMM for W4A8 ("Jetson Orin AGX 上的 INT4 量化推理实践", sections
   当前实现方式 and 正确方向) on the int8 matrix cores: X is first quantized per row into
   the workspace (row-major codes, as quant_act_i8, each 16-byte group of codes in the
   order the INT4 unpack presents the weights), then the packed INT4 weights are staged
   in LDS as stored, each operand widened to int8 lanes after it is read and multiplied
   against the tile's rows of codes into int32; outputs are gemv_w4a8's bits.  Arguments, limits and workspace as gemv_w4a8 at
   M >= 2 (qw_workspace_bytes(2, M, N, K) bytes at any M); variants as
   qw_gemm_w8a16_tile. */
int qw_gemm_w4a8_tile(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
                      int64_t K, float* Y, void* workspace, size_t ws_bytes, int variant,
                      void* stream);

/* The launch variant of the tiled GEMM that gemv_w4a8 (bits 4) and gemv_w8a16 (bits 8)
   take on their matrix-core path (M >= 2 for W4A8, M >= 3 for W8A16, outside the long-K
   rows) for M rows of X and N rows of W on the current device, or -1 where the balanced
   matrix-core kernels run instead.  With no device visible the model assumes 256 CUs.
   A host-side query: no HIP call other than the device's CU count. */
int qw_tile_variant(int bits, int64_t M, int64_t N);

/* The two ablations the INT4 write-up times beside its INT4-weight / INT8-activation
   path ("Jetson Orin AGX 上的 INT4 量化推理实践", section 速度结果), as M == 1 GEMVs with
   K <= 4096 (QW_ERR_SHAPE otherwise); not part of the quantized linear itself.
   qw_gemv_f16: the FP16 baseline.  X16 f16 [1][K], W16 f16 [N][K] row-major (no
     packing) -> Y16 f16 [1][N] = f16(sum_k w * x), the sum in fp32.
   qw_gemv_w4f32: weight-only INT4 with float activations (sections 最初的问题 and
     问题原因): Wq and w_scale from quantize_pack_w4, X fp32 [1][K] -> Y fp32 [1][N] =
     w_scale[n] * sum_k (float)q[n][k] * x[k], each nibble sign-extended, converted to
     float and multiplied-added in fp32 (summation order of the kernel's choosing).
   rows_per_wave: rows (FP16) or groups of 4 rows (INT4) per wave, 1, 2 or 4, or 0 for
   the default (2 for FP16, 1 for INT4); QW_ERR_TILING otherwise. */
int qw_gemv_f16(const uint16_t* X16, const uint16_t* W16, int64_t M, int64_t N, int64_t K,
                uint16_t* Y16, int rows_per_wave, void* stream);
int qw_gemv_w4f32(const float* X, const void* Wq, const float* w_scale, int64_t M, int64_t N,
                  int64_t K, float* Y, int rows_per_wave, void* stream);

/* IndexSoftmax, the integer softmax of the IntAttention summary (CSDN, MLSys 2026 paper),
   section 基准/方法设计: int32 attention logits A [rows][L] (row-major, from an INT8
   QK^T) -> UINT8 probabilities P [rows][L].  Per row, with n = 2^b - 1:
     D = rowMax(A) - A,  D' = min(D, c_int),  idx = round(D' * n / c_int),
     E = LUT[idx],  LUT[i] = round(255 * exp(-c * i / n)) (LUT[n] = 0),
     P = round(255 * E / sum_row E)   (32-bit row sum),
   every rounding of a non-negative ratio half up.  The page recommends (b, c) = (5, 6.6);
   b = 4, 5 or 6, 1 <= L <= 16384 (the page's longest sequence), c_int >= 1 (QW_ERR_SHAPE otherwise); A and P 16-byte
   aligned.  One pass over memory: 4 bytes read and 1 written per logit.
   qw_index_cint gives c_int = round(c * sqrt(d) / (s_Q * s_K)) for head dimension d and
   the per-tensor scales of Q and K, or -1 when that is not a positive int32. */
int index_softmax(const int32_t* A, int64_t rows, int64_t L, int32_t c_int, int b, double c,
                  uint8_t* P, void* stream);
int32_t qw_index_cint(double c, int64_t d, double s_q, double s_k);
/* Test helper: the table index the IndexSoftmax kernel computes without a division,
   idx = (mulhi(2 n D' + c_int, magic) >> shift) = round(D' n / c_int) half up, exact for
   0 <= D' <= c_int.  Writes magic and shift and returns 1 when c_int < 2^24 and
   c_int (2n + 1) < 2^31 (the kernel then uses them); returns 0 otherwise (the kernel
   then takes a float estimate corrected by thresholds) or for b outside 4..6, c_int < 1
   or a NULL pointer. */
int qw_index_magic(int32_t c_int, int b, uint32_t* magic, int* shift);

/* Bandwidth reference (not part of the linear): a kernel that only streams `bytes`
   bytes (a multiple of 16) from src with 16-byte loads, each byte once, and writes one
   32-bit XOR of what it read per workgroup to sink (4-byte aligned, at least `blocks`
   words, or one per compute unit when `blocks` is 0).  A weight-streaming GEMV cannot be faster than this read of its weight
   bytes: decode is memory-bound and GEMV-dominated ("Jetson Orin AGX 上的 INT4
   量化推理实践", section 为什么这个结果有意义).  Launch shape: `blocks` workgroups
   (0: one per compute unit) of `waves` waves (1, 2, 4, 8 or 16; 0: 8), each lane with
   `loads_in_flight` loads requested before use (1, 2, 4, 8 or 16; 0: 4); the grid reads
   the buffer front to back as one moving window, each workgroup taking every blocks-th
   run of loads.  QW_ERR_SHAPE for 0, a non-multiple of 16 bytes or 2 GiB or more,
   QW_ERR_TILING for another launch shape. */
int qw_stream_read(const void* src, size_t bytes, uint32_t* sink, int waves, int blocks,
                   int loads_in_flight, void* stream);

/* Device status of the library on the current device, read synchronously into the HOST
   word *status, then cleared when `clear` is nonzero.  Bit QW_STATUS_PRODUCER_WAIT is set
   when, in some earlier gemv_w4a8 / gemv_w4a8g call at M == 1, a wave of the fused
   activation quantization stopped waiting for the other waves' partial maxima after its
   bounded wait ran out (it cannot happen in a correct run: every wave publishes its own
   maximum before waiting).  The call then finished normally but its activation codes may
   have come from a partial maximum.  Not a hot-path call: it synchronises the device. */
#define QW_STATUS_PRODUCER_WAIT 1u
int qw_device_status(uint32_t* status, int clear);

/* Text for a status code (static storage). */
const char* qw_status_str(int status);
/* The hipError_t of the last QW_ERR_HIP returned on this thread (0 if none). */
int qw_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QWGEMV_H */
