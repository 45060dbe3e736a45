// Internal launcher declarations shared by the libtq translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace tq {

// pack.hip
hipError_t launch_finite_scan(const float* W, int64_t total, int* flags, hipStream_t s);
hipError_t launch_ternary_pack(const float* W, int64_t N, int64_t K, uint8_t* codes, uint16_t* scale,
                               int* flags, hipStream_t s);
hipError_t launch_ternary_unpack(const uint8_t* codes, const uint16_t* scale, int64_t N, int64_t K,
                                 int8_t* t_out, uint16_t* wdq_out, int* flags, hipStream_t s);
hipError_t launch_w4_pack(const float* W, int64_t N, int64_t K, int32_t* qweight, uint16_t* scales,
                          int* flags, hipStream_t s);
hipError_t launch_w4_unpack(const int32_t* qweight, const uint16_t* scales, int64_t N, int64_t K,
                            uint8_t* q_out, uint16_t* wdq_out, hipStream_t s);
// W4A16 with zero points and activation order: the packed column order from
// g_idx (flags[3] on a malformed g_idx), then pack / unpack in that order.
hipError_t launch_w4a_order(const int32_t* g_idx, int64_t K, int32_t* perm, int* flags, hipStream_t s);
hipError_t launch_w4a_pack(const float* W, int64_t N, int64_t K, const int32_t* perm, int32_t* qweight,
                           uint16_t* scales, uint8_t* zeros, int* flags, hipStream_t s);
hipError_t launch_w4a_unpack(const int32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                             const int32_t* perm, int64_t N, int64_t K, uint8_t* q_out, uint16_t* wdq_out,
                             hipStream_t s);
// gemv.hip: A_perm[m, i] = A[m, perm[i]] (activation order), fp16/bf16 bits.
hipError_t launch_gather_columns(const uint16_t* A, const int32_t* perm, int64_t M, int64_t K, uint16_t* out,
                                 hipStream_t s);

// One bit per device ordinal (0..63): whether a per-function setting has been
// applied on that device.
struct DeviceFlags {
    std::atomic<uint64_t> bits{0};
};

// Allow `fn` up to `bytes` of dynamic LDS on the current device (once per
// device; repeating the call is harmless, so a race between threads is too).
inline hipError_t raise_lds_limit(const void* fn, int bytes, DeviceFlags& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
    if (bit && (done.bits.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    done.bits.fetch_or(bit, std::memory_order_relaxed);
    return hipSuccess;
}

// Arguments of one quantized linear-layer call (apply stage).
struct GemmArgs {
    const uint16_t* A;      // [M, K] fp16 / bf16 bit patterns
    int bf16;               // 0: fp16 activations and output, 1: bf16
    int64_t M, N, K;
    const void* wq;         // ternary codes [N, K/4] or W4 words [N, K/8]
    const uint16_t* scale;  // ternary [N]; W4 [N, K/128]
    const uint16_t* bias;   // [N] or nullptr
    uint16_t* C;            // [M, N]
    const uint8_t* zeros = nullptr;  // W4A16 zero points [N, K/128] (nullptr: symmetric, zero point 8)
};

// A call whose K range is split S ways: split z writes its fp32 partial sums
// (no row scale, no bias) to ws[z][M][N], and the S partials of each output
// are summed in order z = 0 .. S-1 before the row scale and bias, so the
// result does not depend on scheduling.  With `flags` the summing is done
// inside the kernel by the last split workgroup of each output tile to
// finish (a counter per tile, split_last_arrival); without, by a second
// launch (launch_splitk_reduce).
struct SplitArgs {
    GemmArgs g;
    float* ws;  // [S][M][N] fp32 partials, unused when S == 1
    int S;
    int scaled;  // 1: the partials already carry the weight scales (W4A16), the reduction adds only the bias
    int64_t ldc = 0;  // row stride of C in elements (0: N); the large-M kernel's column-split launches set it
    uint32_t* flags = nullptr;  // per-tile arrival counters, zero on entry and on exit (S > 1), or nullptr
};
hipError_t launch_splitk_reduce(const SplitArgs& sa, hipStream_t s);  // gemm.hip

// Arrival counters at the front of every caller workspace: kFlagBytes bytes,
// one 32-bit counter per output tile of a split call (kMaxFlags tiles; a
// call with more tiles falls back to the reduction launch).  They must be
// zero when a workspace is first used, and every call leaves them zero.
constexpr size_t kFlagBytes = 16384;
constexpr int64_t kMaxFlags = (int64_t)(kFlagBytes / 4);
// The counters to use for a split grid of `tiles` output tiles, or nullptr.
inline uint32_t* split_flags(uint32_t* flags, int S, int64_t tiles) {
    return (flags && S > 1 && tiles <= kMaxFlags) ? flags : nullptr;
}

// gemv.hip: small M (<= kGemvMaxM), weights streamed once per call.
constexpr int kGemvMaxM = 16;
// Largest K of a product call: the tiled kernels address up to 256 rows of
// a tile from a uniform base with 32-bit byte offsets (256 * 2K bytes).
constexpr int64_t kMaxK = (int64_t)1 << 22;
// With a workspace of gemv_workspace_bytes() the streaming kernel may split
// K (long-K, short-N shapes); without one it never does.
size_t gemv_workspace_bytes(const GemmArgs& a);
hipError_t launch_ternary_gemv(const GemmArgs& a, void* workspace, size_t workspace_bytes, hipStream_t s,
                               uint32_t* flags = nullptr);
hipError_t launch_ternary_gemv(const GemmArgs& a, hipStream_t s);         // picks the fastest eligible kernel
hipError_t launch_ternary_gemv_simple(const GemmArgs& a, hipStream_t s);  // any dtype, any K % 64 == 0
bool ternary_gemv_mfma_ok(const GemmArgs& a);                             // fp16, K % 256 == 0
// Measurement variants of the M = 1 kernel: 0 as dispatched, 1 codes read
// from the cache (every workgroup reads row-block 0), 2 as 1 without the
// matrix-core step.  hipErrorInvalidValue where the M = 1 kernel does not run.
hipError_t launch_ternary_gemv_variant(const GemmArgs& a, int variant, hipStream_t s);
// diag.hip: a plain streaming read of `bytes` (a multiple of 16) by `blocks`
// workgroups; sink[b] (blocks entries) is written only if workgroup b's
// XOR of the data equals an improbable value.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int64_t blocks, hipStream_t s);
// W4A16 small M: with a workspace of w4_gemv_workspace_bytes() the streaming
// kernel may split K; without one it never does.
size_t w4_gemv_workspace_bytes(const GemmArgs& a);
hipError_t launch_w4_gemv(const GemmArgs& a, void* workspace, size_t workspace_bytes, hipStream_t s,
                          uint32_t* flags = nullptr);
hipError_t launch_w4_gemv(const GemmArgs& a, hipStream_t s);         // picks the fastest eligible kernel
hipError_t launch_w4_gemv_simple(const GemmArgs& a, hipStream_t s);  // any dtype

// gemm.hip: LDS-tiled matrix-core GEMM, any M.
// Large M: K split S ways (gemm_splits) when `workspace` holds
// gemm_workspace_bytes(), else one pass over K.
hipError_t launch_ternary_gemm(const GemmArgs& a, void* workspace, size_t workspace_bytes, int compute_units,
                               hipStream_t s, uint32_t* flags = nullptr);
int gemm_splits(int64_t M, int64_t N, int64_t K, int compute_units);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int compute_units);
// gemm.hip: medium M (64-row tiles, K split across workgroups when the
// workspace allows; see medium_m_workspace_bytes).
int medium_m_splits(int64_t M, int64_t N, int64_t K, int compute_units);
size_t medium_m_workspace_bytes(int64_t M, int64_t N, int64_t K, int compute_units);
hipError_t launch_ternary_medium(const GemmArgs& a, void* workspace, size_t workspace_bytes, int compute_units,
                                 hipStream_t s);
hipError_t launch_ternary_medium_split(const SplitArgs& sa, bool paired, hipStream_t s);  // a given split count; paired: A holds pairs
// Compute units of the current device (cached per device ordinal).
int compute_units();
hipError_t launch_w4_gemm(const GemmArgs& a, void* workspace, size_t workspace_bytes, hipStream_t s,
                          uint32_t* flags = nullptr);
// gemm.hip: W4A16 prefill GEMM (any M, K % 128 == 0, at most 128 groups).
// gemm.hip: W4A16 matrix-core GEMM (17 <= M), K split across workgroups
// while the tiles leave compute units idle or a split would hold more than
// 128 groups; w4_prefill_ok tells whether a workspace of the given size lets
// it run (long K needs at least the minimum split's partials).
int w4_gemm_splits(int64_t M, int64_t N, int64_t K, int compute_units);
size_t w4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int compute_units);
bool w4_prefill_ok(const GemmArgs& a, size_t workspace_bytes);
hipError_t launch_w4_prefill(const GemmArgs& a, void* workspace, size_t workspace_bytes, hipStream_t s);

}  // namespace tq
