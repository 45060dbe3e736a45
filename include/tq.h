/*
 * tq.h - weight-only quantized linear layers for AMD Instinct MI355X (gfx950).
 *
 * Two packed weight formats, each multiplied against fp16 or bf16 activations
 * with fp32 accumulation:
 *
 *  - Ternary: every weight is one of {-1, 0, +1} times a per-output-row fp16
 *    scale; four 2-bit codes per byte.  Sources: page "Ternary quantized
 *    models in vLLM: reverse engineering, reconciliation and kernel
 *    optimization" (wzjinhao.cn/news/47283) - section 1 (tip: scaled sign
 *    function with a threshold), section 2.3 (the layer receives the packed
 *    uint8 weight, its fp16 scale and an optional bias, and never holds fp16
 *    weights), section 3.1 (threshold 0.7 * mean|w|, code table, bit order,
 *    fp16 scale), section 3.2 (row length ceil(K/4) bytes), section 4 (the
 *    layer's arithmetic: value = code - 1, dot product per output).
 *
 *  - W4A16: symmetric int4 with a fixed zero point of 8, eight codes per
 *    int32 along K, one fp16 scale per output row and group of 128 columns.
 *    Source: page "Model quantization - vLLM runtime quantization
 *    architecture" (notes.devxops.cn, 2026-05-14), section 5 steps (1) and
 *    (3): bits 4, group_size 128, sym, packed factor 8, weight [d_out, d_in/8],
 *    scales [d_out, d_in/128]; section 4.4: the prepare (create + load +
 *    post-process) then apply lifecycle this API follows.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers on the current HIP device (the
 *    library never calls hipSetDevice).  Tensors are row-major and contiguous.
 *  - fp16 and bf16 values are passed as 16-bit patterns (uint16_t / void*).
 *  - The caller owns every buffer; the library keeps no pointer after a call
 *    returns.  Buffers must stay alive until the work on `stream` completes.
 *  - Shapes: M = activation rows, N = output features (weight rows),
 *    K = input features.  A is [M, K], C is [M, N].
 *  - Errors the host can see return at once with nothing launched:
 *    TQ_ERR_NULL, TQ_ERR_SHAPE, TQ_ERR_ALIGN, TQ_ERR_DTYPE, TQ_ERR_GROUP,
 *    TQ_ERR_PATH.  A failed launch or HIP call returns TQ_ERR_HIP.
 *  - Prepare calls (pack / unpack) are SYNCHRONOUS: they wait for `stream`
 *    and report data errors (TQ_ERR_NONFINITE, TQ_ERR_RANGE,
 *    TQ_ERR_BAD_CODE).  They allocate nothing: their status flags live in
 *    the library's own device memory, one copy per device, so prepare calls
 *    on one device are serialized by a host mutex.
 *  - Apply calls (tq_gemm, tq_gemm_ws, w4a16_gemm) are ASYNCHRONOUS on
 *    `stream`, allocate nothing, never synchronize and are safe to capture in
 *    a HIP graph.  Faults during execution surface at the caller's next sync.
 *  - All results are deterministic: where K is split across workgroups the
 *    fp32 partial sums are added in a fixed order, split 0 first, whichever
 *    workgroup adds them.  The same inputs, path and workspace size give
 *    bit-identical outputs.
 *  - Workspaces (the *_ws and asym calls): the first TQ_WORKSPACE_FLAG_BYTES
 *    bytes of a workspace are per-tile arrival counters of the K split (the
 *    last split workgroup of an output tile to finish adds the partials
 *    itself, instead of a second kernel).  They must be zero before the
 *    workspace is first used; every call leaves them zero again, so a
 *    workspace that only this library writes needs clearing once.  The
 *    *_workspace_bytes queries include them; a workspace smaller than
 *    TQ_WORKSPACE_FLAG_BYTES counts as none.
 */
#ifndef TQ_H
#define TQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 6

/* Arrival counters at the front of every workspace (see above). */
#define TQ_WORKSPACE_FLAG_BYTES 16384

typedef enum tq_status {
    TQ_OK = 0,
    TQ_ERR_NULL = 1,       /* a required pointer is NULL */
    TQ_ERR_SHAPE = 2,      /* a size is <= 0 or violates a K constraint */
    TQ_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned */
    TQ_ERR_DTYPE = 4,      /* unknown activation dtype enum */
    TQ_ERR_GROUP = 5,      /* W4A16 group size other than 128 */
    TQ_ERR_NONFINITE = 6,  /* pack: a weight is NaN or infinite */
    TQ_ERR_RANGE = 7,      /* pack: a scale rounds to infinity in fp16 */
    TQ_ERR_BAD_CODE = 8,   /* unpack: a 2-bit field holds the unused 0b11 */
    TQ_ERR_HIP = 9,        /* a HIP runtime call or kernel launch failed */
    TQ_ERR_PATH = 10,      /* a forced kernel path cannot run this shape */
    TQ_ERR_SCRATCH = 11    /* tq_gemm_noalloc: the schedule needs more than its scratch */
} tq_status;

typedef enum tq_dtype {
    TQ_F16 = 0,            /* IEEE binary16 activations and outputs */
    TQ_BF16 = 1            /* bfloat16 activations and outputs */
} tq_dtype;

/* Kernel families the dispatcher chooses between (by M; see tq_select_path). */
typedef enum tq_path {
    TQ_PATH_AUTO = 0,        /* let the dispatcher choose */
    TQ_PATH_GEMV = 1,        /* small M: weight-streaming kernel, codes read once per call */
    TQ_PATH_STREAM_MFMA = 2, /* medium M: 64-row tiles, K split across workgroups */
    TQ_PATH_GEMM = 3         /* large M: LDS-tiled matrix-core GEMM (prefill; W4A16 also medium M) */
} tq_path;

/* ---------------------------------------------------------------- prepare */

/*
 * tq_pack - ternarize and pack fp32 weights.
 *   W          [N, K] fp32 (device).
 *   codes      [N, ceil(K/4)] uint8 (device, written).  Code of column 4j+k
 *              sits in bits 2k..2k+1 of byte j of its row; 00 = -1, 01 = 0,
 *              10 = +1; 11 is never written; tail fields of a row whose K is
 *              not a multiple of 4 are 01.
 *   scale_f16  [N] fp16 bit patterns (device, written).
 * Per row n (sums in fp64, sequential in ascending column order):
 *   S = sum |w|;  thr = 0.7 * (S / K);  kept = |w| > thr;  t = sign(w) if kept
 *   else 0;  scale = (sum of kept |w|) / (number kept), rounded once to fp16
 *   (round to nearest even), +0 for a row with nothing kept (an all-zero row).
 * Any N >= 1, K >= 1.  Errors: TQ_ERR_NONFINITE if any weight is NaN/Inf
 * (checked before anything is written), TQ_ERR_RANGE if a scale overflows
 * fp16 (outputs then hold partial results).  Synchronous.
 */
tq_status tq_pack(const float* W, int64_t N, int64_t K,
                  uint8_t* codes, uint16_t* scale_f16, hipStream_t stream);

/*
 * tq_unpack - decode packed ternary weights.
 *   t_out        [N, K] int8 in {-1, 0, +1} (device, written; may be NULL).
 *   wdq_f16_out  [N, K] fp16 bit patterns of t * scale (device, written; may
 *                be NULL).  The product is exact in fp16 with IEEE signs
 *                (-1 * +0 = -0, 0 * s = +0).
 * Errors: TQ_ERR_BAD_CODE if any field of columns 0..K-1 is 0b11 (outputs
 * then hold partial results; padding fields are not examined).  Synchronous.
 */
tq_status tq_unpack(const uint8_t* codes, const uint16_t* scale_f16, int64_t N, int64_t K,
                    int8_t* t_out, uint16_t* wdq_f16_out, hipStream_t stream);

/*
 * w4a16_pack - symmetric int4 quantization, group of 128 along K.
 *   W           [N, K] fp32 (device), K % group_size == 0.
 *   qweight     [N, K/8] int32 (device, written); nibble i (bits 4i..4i+3)
 *               of word j holds column 8j+i, as q = r + 8 in 0..15.
 *   scales_f16  [N, K/group_size] fp16 bit patterns (device, written).
 * Per (row, group): s = fp16(max|w| / 7) (fp64 divide, one rounding);
 * r = round-half-even(w / s) in fp64, clamped to [-8, 7]; r = 0 if s == 0.
 * Errors: TQ_ERR_GROUP unless group_size == 128; TQ_ERR_NONFINITE,
 * TQ_ERR_RANGE as for tq_pack.  Synchronous.
 */
tq_status w4a16_pack(const float* W, int64_t N, int64_t K, int64_t group_size,
                     int32_t* qweight, uint16_t* scales_f16, hipStream_t stream);

/*
 * w4a16_unpack - decode int4 weights.
 *   q_out        [N, K] uint8 codes 0..15 (device, written; may be NULL).
 *   wdq_f16_out  [N, K] fp16 bit patterns of (q - 8) * s rounded once to
 *                nearest even (device, written; may be NULL).
 * Synchronous.
 */
tq_status w4a16_unpack(const int32_t* qweight, const uint16_t* scales_f16,
                       int64_t N, int64_t K, int64_t group_size,
                       uint8_t* q_out, uint16_t* wdq_f16_out, hipStream_t stream);

/* ------------------------------------------------------------------ apply */

/*
 * tq_gemm - C = A * dequant(codes, scale)^T (+ bias), fp32 accumulation.
 *   A      [M, K] activations in `dt` (device, 16-byte aligned).
 *   codes  [N, K/4] packed ternary codes as written by tq_pack (16-byte aligned).
 *   scale_f16 [N] fp16 row scales.
 *   bias   [N] in `dt`, added in fp32 after scaling (may be NULL).
 *   C      [M, N] in `dt` (device, written), rounded once from fp32 to
 *          nearest even; overflow gives +-inf.
 * C[m, n] = scale[n] * sum_k A[m, k] * t[n, k] + bias[n]: the scale is
 * applied after accumulation (ternary page, section 4.2).  Requires
 * K % 64 == 0 (rows are whole 16-byte chunks) and K <= 2^22 (every product
 * call: tiles address their rows with 32-bit byte offsets; TQ_ERR_SHAPE
 * beyond).  A row of codes containing the
 * unused field 0b11 gives an unspecified result.  Asynchronous; allocates
 * nothing; graph-capturable.
 */
tq_status tq_gemm(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K,
                  const uint8_t* codes, const uint16_t* scale_f16, const void* bias,
                  void* C, hipStream_t stream);

/* tq_gemm with a forced kernel path (tests and benchmarks). */
tq_status tq_gemm_ex(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K,
                     const uint8_t* codes, const uint16_t* scale_f16, const void* bias,
                     void* C, hipStream_t stream, tq_path path);

/*
 * tq_gemm_ws - tq_gemm with a caller-owned workspace and a path choice.
 *   workspace        device buffer (16-byte aligned) of workspace_bytes
 *                    bytes, or NULL, whose first TQ_WORKSPACE_FLAG_BYTES
 *                    are zero (see the workspace rules above); the call may
 *                    overwrite the rest and the caller must not touch it
 *                    until the work on `stream` is done.  Calls that may
 *                    overlap must use different workspaces.
 *   workspace_bytes  at least tq_gemm_workspace_bytes(M, N, K, dt, path)
 *                    for the split-K schedule of the decode streaming
 *                    kernel (3 <= M <= 16, long K, where the small-M kernel
 *                    does not run; the query then reports 0), TQ_PATH_STREAM_MFMA and
 *                    TQ_PATH_GEMM; with less (or NULL) they run one
 *                    workgroup per output tile over all of K - correct,
 *                    slower when the output tiles leave compute units idle.
 *   path             TQ_PATH_AUTO or a forced kernel family (TQ_ERR_PATH if
 *                    it cannot run the shape: TQ_PATH_GEMV needs M <= 16).
 * With S > 1 splits the kernel writes S fp32 partials [S][M][N] into the
 * workspace (after the counters), summed in order z = 0 .. S-1: on
 * TQ_PATH_GEMV and TQ_PATH_GEMM by the last split of each output tile to
 * finish (for grids of up to TQ_WORKSPACE_FLAG_BYTES / 4 tiles), on
 * TQ_PATH_STREAM_MFMA by a second kernel, whose launch costs less there than
 * the tail of one workgroup reading every split of its tile.  On
 * TQ_PATH_STREAM_MFMA with K % 256 == 0 and N * K >= 200 * 2^20 the
 * workspace also holds the activations in the kernel's pair order (M * K * 2
 * bytes after the partials, written by a first kernel of the call); with a
 * workspace too small for both, the pairs are made inside the tiles, as
 * without a workspace.  Other arguments, results and errors as tq_gemm;
 * TQ_ERR_ALIGN for a misaligned workspace.  Asynchronous; allocates nothing;
 * graph-capturable.
 */
tq_status tq_gemm_ws(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K,
                     const uint8_t* codes, const uint16_t* scale_f16, const void* bias,
                     void* C, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, tq_path path);

/*
 * tq_gemm_noalloc - tq_gemm_ws for callers that cannot allocate memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Instead of a caller workspace it uses a scratch array in the
 * library's own device memory: tq_gemm_noalloc_scratch_bytes() bytes
 * (16 MiB) per device, held until the process ends.  The call takes the
 * schedule tq_gemm_ws would take with tq_gemm_workspace_bytes(M, N, K, dt,
 * path) bytes of workspace, and so gives bit-identical results; when that
 * schedule needs more than the scratch holds it returns TQ_ERR_SCRATCH with
 * nothing launched.  It calls no allocating routine.  Every call on a device
 * shares that device's scratch: its front holds the split arrival counters,
 * zero when the library is loaded and left zero by every call, and the
 * split partials behind them are fully rewritten by each call, so nothing
 * needs clearing; calls that may overlap on one device
 * (different streams, or threads) race and must be serialized by the
 * caller; calls in one stream's order are safe.  Other arguments, results
 * and errors as tq_gemm_ws.
 */
tq_status tq_gemm_noalloc(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K,
                          const uint8_t* codes, const uint16_t* scale_f16, const void* bias,
                          void* C, hipStream_t stream, tq_path path);

/* Bytes of the per-device scratch of tq_gemm_noalloc. */
size_t tq_gemm_noalloc_scratch_bytes(void);

/*
 * tq_gemm_workspace_bytes - workspace tq_gemm_ws needs for its fastest
 * schedule of this shape on the current device (0 when none is used).
 * Depends on the device's compute-unit count; query on the device that will
 * run the call.
 */
size_t tq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, tq_dtype dt, tq_path path);

/*
 * w4a16_gemm - C = A * dequant(qweight, scales)^T (+ bias), fp32 accumulation.
 *   qweight [N, K/8] int32 and scales_f16 [N, K/128] as written by
 *   w4a16_pack; group_size must be 128; K % 128 == 0; K <= 2^22 as for
 *   tq_gemm.
 * C[m, n] = sum_g s[n, g] * sum_{k in g} A[m, k] * (q[n, k] - 8) + bias[n]:
 * the group scale multiplies each group's fp32 partial sum.  Other arguments
 * as tq_gemm.  From M = 33 (M = 17 when K >= 8192), or with TQ_PATH_GEMM, a
 * GEMM runs on the matrix cores (256-row tiles from M = 256, 64-row tiles
 * below); without a workspace it needs K / 128 <= 128.  Other shapes run the
 * decode kernels over blocks of 16 rows.  Asynchronous; allocates nothing;
 * graph-capturable.
 */
tq_status w4a16_gemm(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K,
                     const int32_t* qweight, const uint16_t* scales_f16, int64_t group_size,
                     const void* bias, void* C, hipStream_t stream);

/* w4a16_gemm with a forced kernel path (tests and benchmarks). */
tq_status w4a16_gemm_ex(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K,
                        const int32_t* qweight, const uint16_t* scales_f16, int64_t group_size,
                        const void* bias, void* C, hipStream_t stream, tq_path path);

/*
 * w4a16_gemm_ws - w4a16_gemm with a caller-owned workspace and a path
 * choice (ABI 3).  The workspace rules are those of tq_gemm_ws: 16-byte
 * aligned device memory of workspace_bytes bytes or NULL, zero counters at
 * its front, the rest overwritten by the call, not shared by calls that may
 * overlap.  With at least
 * w4a16_gemm_workspace_bytes() bytes the fp16 streaming kernel (M above 4,
 * or shapes the M <= 4 kernel cannot take) may split the K groups across
 * workgroups (fp32 partials with the group scales applied, summed in order
 * by the tile's last split to finish, bias added there); with less it makes one pass over
 * K.  The M <= 4 kernel never splits, and the query reports 0 for it.  The
 * matrix-core GEMM splits the K groups the same way while its 128-column
 * tiles leave compute units idle (at most 16 splits) and always when K / 128
 * > 128 (each split holds at most 128 groups' scales), summed by a second
 * kernel; a shape that needs a
 * split the workspace cannot hold runs the decode kernels over blocks of 16
 * rows under TQ_PATH_AUTO and returns TQ_ERR_PATH under TQ_PATH_GEMM.  Row
 * blocks (M > 16) reuse the workspace in stream order.  Other arguments, results and errors as
 * w4a16_gemm; TQ_ERR_ALIGN for a misaligned workspace.
 */
tq_status w4a16_gemm_ws(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K,
                        const int32_t* qweight, const uint16_t* scales_f16, int64_t group_size,
                        const void* bias, void* C, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, tq_path path);

/*
 * w4a16_gemm_workspace_bytes - workspace w4a16_gemm_ws needs for its fastest
 * schedule of this shape on the current device (0 when none is used, or for
 * invalid arguments).
 */
size_t w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, tq_dtype dt, int64_t group_size);

/* ----------------------- W4A16 with zero points and activation order (ABI 4)
 *
 * The variant the page "Model quantization - vLLM runtime quantization
 * architecture" names in section 5, steps (0) and (3): a per-group zero
 * point beside the group scale, and optionally g_idx, the group of each
 * input column (activation ordering).  The quantizer is asymmetric
 * min-max over each group's range widened to include 0:
 *   s = fp16((max(0, hi) - min(0, lo)) / 15), z = clamp(rint(-min(0, lo) / s), 0, 15),
 *   q = clamp(rint(w / s) + z, 0, 15), dequantized weight (q - z) * s,
 * in fp64 with round-half-even (a zero scale gives z = 0 and q = 0).
 */

/*
 * w4a16_pack_asym - pack W [N, K] fp32 (device) with zero points.
 *   g_idx      int32 [K] or NULL: input column k belongs to group g_idx[k];
 *              every group must hold exactly 128 columns (else TQ_ERR_GROUP).
 *              The packed matrix stores the columns sorted by group, stably
 *              (ascending column within a group), so groups are contiguous.
 *   qweight    int32 [N, K/8], nibble i of word j = packed column 8j + i.
 *   scales_f16 [N, K/128]; zeros uint8 [N, K/128] (values 0..15).
 *   perm       int32 [K], required with g_idx: packed column i is input
 *              column perm[i] (not written without g_idx; the order is then
 *              the identity).
 * Synchronous.  Errors: TQ_ERR_NULL, TQ_ERR_GROUP (group_size != 128 or a
 * malformed g_idx), TQ_ERR_SHAPE (K % 128 != 0), TQ_ERR_ALIGN (W, qweight,
 * g_idx, perm 4-byte aligned; scales 2-byte), TQ_ERR_NONFINITE, TQ_ERR_RANGE.
 */
tq_status w4a16_pack_asym(const float* W, int64_t N, int64_t K, int64_t group_size, const int32_t* g_idx,
                          int32_t* qweight, uint16_t* scales_f16, uint8_t* zeros, int32_t* perm,
                          hipStream_t stream);

/*
 * w4a16_unpack_asym - codes q_out [N, K] in packed column order (nullable)
 * and dequantized weights wdq_f16_out [N, K] in the input column order
 * (nullable; (q - z) * s rounded once to fp16, placed at column perm[i], or
 * i without perm).  Synchronous.
 */
tq_status w4a16_unpack_asym(const int32_t* qweight, const uint16_t* scales_f16, const uint8_t* zeros,
                            const int32_t* perm, int64_t N, int64_t K, int64_t group_size, uint8_t* q_out,
                            uint16_t* wdq_f16_out, hipStream_t stream);

/*
 * w4a16_gemm_asym - C = A * dequant(qweight, scales, zeros)^T (+ bias), the
 * packed weights of w4a16_pack_asym.
 *   zeros  uint8 [N, K/128] or NULL (then the symmetric zero point 8).
 *   perm   int32 [K] or NULL: with it, A is first gathered into packed
 *          column order, A[:, perm], in the workspace after its counters, which is
 *          then required: at least w4a16_gemm_asym_workspace_bytes(..., 1)
 *          bytes for the fastest schedule, never less than the gathered
 *          activations (M * K * 2 bytes rounded up to 256; TQ_ERR_SHAPE
 *          otherwise).  perm must be the array the pack wrote; any other
 *          contents give unspecified results (indices are clamped into
 *          [0, K), so memory stays in bounds).
 *   path   TQ_PATH_AUTO, TQ_PATH_GEMV or TQ_PATH_GEMM (the matrix-core GEMM;
 *          with K / 128 > 128 it needs the workspace of the K split after
 *          the gathered activations, TQ_ERR_PATH otherwise).
 * The rest of the workspace serves the split-K schedule of w4a16_gemm_ws.
 * Asynchronous; allocates nothing; graph-capturable.
 */
tq_status w4a16_gemm_asym(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const int32_t* qweight,
                          const uint16_t* scales_f16, const uint8_t* zeros, const int32_t* perm, int64_t group_size,
                          const void* bias, void* C, void* workspace, size_t workspace_bytes, hipStream_t stream,
                          tq_path path);

/*
 * w4a16_gemm_asym_workspace_bytes - workspace of w4a16_gemm_asym's fastest
 * schedule: the counters, the gathered activations when with_perm, and the
 * split-K partials (0 for invalid arguments or when nothing is needed).
 */
size_t w4a16_gemm_asym_workspace_bytes(int64_t M, int64_t N, int64_t K, tq_dtype dt, int64_t group_size,
                                       int with_perm);

/* ----------------------------------------------------------- measurement
 *
 * Instruments for the benchmark, not part of the layer: they measure the
 * device, not compute a result.
 */

/*
 * tq_diag_stream_read - a plain streaming read of `bytes` bytes at `src`
 * (device, 16-byte aligned, bytes a positive multiple of 16) by at most
 * `blocks` workgroups of 256 lanes, each reading a contiguous share.  The
 * data are folded with XOR and nothing is stored unless a workgroup's fold
 * equals an improbable value; `sink` (device, at least `blocks` uint32)
 * takes those stores.  This is the HBM read ceiling one launch of that size
 * reaches.  Asynchronous.  TQ_ERR_SHAPE if blocks exceeds bytes / 16.
 */
tq_status tq_diag_stream_read(const void* src, size_t bytes, uint32_t* sink, int64_t blocks, hipStream_t stream);

/*
 * tq_diag_gemv - the M = 1 decode kernel of tq_gemm in a measurement form
 * (page "Ternary quantized models in vLLM ...", section 5.7: attributing
 * kernel time to unpacking).  variant 0 runs the kernel tq_gemm runs (same
 * result); 1 makes every workgroup read the codes of rows 0..15, so the
 * codes come from the cache, not HBM; 2 is 1 without the matrix-core
 * multiply (codes are loaded and unpacked only).  Outputs of variants 1 and
 * 2 are unspecified (C is still written, in bounds).  Arguments as tq_gemm;
 * TQ_ERR_PATH if M != 1 or the M = 1 kernel does not take the shape.
 */
tq_status tq_diag_gemv(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K,
                       const uint8_t* codes, const uint16_t* scale_f16, const void* bias,
                       void* C, hipStream_t stream, int variant);

/* ------------------------------------------------------------------ misc */

/*
 * tq_select_path - the dispatcher's choice for a shape (never TQ_PATH_AUTO).
 *   format: 0 = ternary, 1 = W4A16.  Decode-sized M (<= 16) streams the
 *   weights (they dominate the bytes moved); prefill-sized M (>= 256) is a
 *   dense contraction for the matrix cores (the decode / prefill split of
 *   the quantization decision tree on page "10.6 Quantization choice and vLLM
 *   in practice", section 10.6.1); ternary M in 17 .. 255, and ternary M in
 *   3 .. 16 with K % 256 != 0, take the medium path, 32- or 64-row tiles
 *   with K split across workgroups.  W4A16 takes its matrix-core GEMM from
 *   M = 33 (M = 17 when K >= 8192), 64-row tiles below 256 rows.
 */
tq_path tq_select_path(int format, int64_t M, int64_t N, int64_t K, tq_dtype dt);

/* Static string for a status code (never NULL). */
const char* tq_status_str(tq_status s);

/* TQ_ABI_VERSION of the loaded library. */
int tq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
