// extern "C" entry points of libtq: argument checks, the M-based dispatcher,
// and the synchronous prepare calls.  See include/tq.h for the contract.
//
// The library never calls hipSetDevice and keeps no state between calls: it
// works on the caller's current device and stream (page "Ternary quantized
// models in vLLM ...", section 5.1: a kernel bound to the wrong device
// ordinal is the first deployment failure it lists).

#include "tq.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "tq_internal.h"

// Status flags of the synchronous prepare calls, in the library's own device
// memory (one copy per device), so that a prepare call allocates nothing.
// Their address is looked up per device; prepare calls on one device share
// the flags and are therefore serialized by a per-device host mutex.
static __device__ __align__(16) int prepare_flags[4];

// Scratch memory of tq_gemm_noalloc: the split-K partials of the apply
// kernels, for callers that cannot allocate.  One copy per device, held
// until the process ends; every call on a device shares it.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Dispatcher thresholds on M (activation rows).  Decode-sized M is bound by
// streaming the packed weights; large M is a dense contraction for the matrix
// cores; in between, 64-row tiles with K split across workgroups.
constexpr int64_t kGemvMaxM = tq::kGemvMaxM;
constexpr int64_t kMediumMaxM = 256;  // M < 256: medium path

constexpr int kMaxDevices = 64;

// Device address of a file-scope __device__ symbol on the current device,
// looked up once per device (the symbol's name in host code is only a
// host-side stand-in, never a device address).
template <class T>
tq_status symbol_address(const T& sym, std::atomic<void*> (&cache)[kMaxDevices], void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_ERR_HIP;
    void* p = cache[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(sym)) != hipSuccess || !p) return TQ_ERR_HIP;
        cache[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return TQ_OK;
}

std::atomic<void*> prepare_flags_ptr[kMaxDevices];
std::atomic<void*> scratch_ptr[kMaxDevices];
std::mutex prepare_mutex[kMaxDevices];

// Status flags of one synchronous prepare call: holds the device's prepare
// mutex for the call's duration.
struct StatusWord {
    std::unique_lock<std::mutex> lock;
    int* dev = nullptr;
    tq_status init(hipStream_t s) {
        int d = 0;
        if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDevices) return TQ_ERR_HIP;
        lock = std::unique_lock<std::mutex>(prepare_mutex[d]);
        void* p = nullptr;
        const tq_status r = symbol_address(prepare_flags, prepare_flags_ptr, &p);
        if (r != TQ_OK) return r;
        dev = static_cast<int*>(p);
        if (hipMemsetAsync(dev, 0, 4 * sizeof(int), s) != hipSuccess) return TQ_ERR_HIP;
        return TQ_OK;
    }
    tq_status read(hipStream_t s, int out[4]) {
        if (hipMemcpyAsync(out, dev, 4 * sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess) return TQ_ERR_HIP;
        if (hipStreamSynchronize(s) != hipSuccess) return TQ_ERR_HIP;
        return TQ_OK;
    }
};

tq_status check_gemm_common(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const void* wq,
                            const uint16_t* scale, void* C) {
    if (!A || !wq || !scale || !C) return TQ_ERR_NULL;
    if (dt != TQ_F16 && dt != TQ_BF16) return TQ_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K <= 0 || K > tq::kMaxK) return TQ_ERR_SHAPE;
    if (!aligned16(A) || !aligned16(wq)) return TQ_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(C) & 1u) || (reinterpret_cast<uintptr_t>(scale) & 1u)) return TQ_ERR_ALIGN;
    return TQ_OK;
}

tq_status from_hip(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_ERR_HIP; }

// A caller workspace: tq::kFlagBytes of split arrival counters at its front
// (zero when first used; every call leaves them zero), then the bytes for
// partial sums and staging.  A workspace smaller than the counters counts as
// none.
struct Carved {
    uint32_t* flags = nullptr;
    void* data = nullptr;
    size_t bytes = 0;
};
Carved carve(void* ws, size_t bytes) {
    Carved c;
    if (!ws || bytes < tq::kFlagBytes) return c;
    c.flags = static_cast<uint32_t*>(ws);
    c.bytes = bytes - tq::kFlagBytes;
    if (c.bytes) c.data = static_cast<uint8_t*>(ws) + tq::kFlagBytes;
    return c;
}
// Caller bytes for `data` bytes of partials and staging (0: no workspace).
size_t with_flags(size_t data) { return data ? tq::kFlagBytes + data : 0; }

}  // namespace

extern "C" {

int tq_abi_version(void) { return TQ_ABI_VERSION; }

const char* tq_status_str(tq_status s) {
    switch (s) {
        case TQ_OK: return "ok";
        case TQ_ERR_NULL: return "a required pointer is NULL";
        case TQ_ERR_SHAPE: return "invalid shape (sizes must be positive; see K constraints)";
        case TQ_ERR_ALIGN: return "pointer not 16-byte aligned";
        case TQ_ERR_DTYPE: return "unknown activation dtype";
        case TQ_ERR_GROUP: return "W4A16 group size must be 128";
        case TQ_ERR_NONFINITE: return "a weight is NaN or infinite";
        case TQ_ERR_RANGE: return "a scale overflows fp16";
        case TQ_ERR_BAD_CODE: return "packed code field 0b11 (unused) found";
        case TQ_ERR_HIP: return "HIP runtime error or kernel launch failure";
        case TQ_ERR_PATH: return "forced kernel path cannot run this shape";
        case TQ_ERR_SCRATCH: return "the call needs more scratch memory than tq_gemm_noalloc holds";
    }
    return "unknown status";
}

tq_path tq_select_path(int format, int64_t M, int64_t N, int64_t K, tq_dtype dt) {
    (void)N; (void)dt;
    // Ternary rows that are not whole 256-column chunk-sets leave the decode
    // kernels only their per-lane FMA form; from three activation rows the
    // medium path's matrix-core tiles (any K % 64 == 0) are faster.
    if (format == 0 && M >= 3 && M <= kGemvMaxM && K % 256 != 0) return TQ_PATH_STREAM_MFMA;
    if (M <= kGemvMaxM) return TQ_PATH_GEMV;
    if (format == 1) {
        // W4A16: the matrix-core GEMM (64-row tiles below 256 rows, 256-row
        // tiles above) from 33 rows, and from 17 where K >= 8192; the small-M
        // kernels over blocks of 16 rows below that, where two passes over
        // short-K weights beat the GEMM's K loop (Llama-3-8B gate_up at
        // M = 17..32: 27-29 against 34 us).  A call whose K needs a split the
        // workspace cannot hold also takes the row blocks (w4a16_gemm_ws).
        if (K % 128 != 0 || (M <= 32 && K < 8192)) return TQ_PATH_GEMV;
        return TQ_PATH_GEMM;
    }
    if (M < kMediumMaxM) return TQ_PATH_STREAM_MFMA;
    return TQ_PATH_GEMM;
}

size_t tq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, tq_dtype dt, tq_path path) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 64 != 0 || K > tq::kMaxK) return 0;
    if (path == TQ_PATH_AUTO) path = tq_select_path(0, M, N, K, dt);
    if (path == TQ_PATH_STREAM_MFMA) return with_flags(tq::medium_m_workspace_bytes(M, N, K, tq::compute_units()));
    if (path == TQ_PATH_GEMM) return with_flags(tq::gemm_workspace_bytes(M, N, K, tq::compute_units()));
    if (path == TQ_PATH_GEMV && M <= kGemvMaxM) {
        const tq::GemmArgs a{nullptr, dt == TQ_BF16 ? 1 : 0, M, N, K, nullptr, nullptr, nullptr, nullptr};
        return with_flags(tq::gemv_workspace_bytes(a));
    }
    return 0;
}

// ---------------------------------------------------------------- prepare

tq_status tq_pack(const float* W, int64_t N, int64_t K, uint8_t* codes, uint16_t* scale_f16, hipStream_t stream) {
    if (!W || !codes || !scale_f16) return TQ_ERR_NULL;
    if (N <= 0 || K <= 0) return TQ_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(W) & 3u) || (reinterpret_cast<uintptr_t>(scale_f16) & 1u)) return TQ_ERR_ALIGN;
    if ((K % 64) == 0 && !aligned16(codes)) return TQ_ERR_ALIGN;
    StatusWord st;
    tq_status r = st.init(stream);
    if (r != TQ_OK) return r;
    int flags[4];
    if (tq::launch_finite_scan(W, N * K, st.dev, stream) != hipSuccess) return TQ_ERR_HIP;
    if ((r = st.read(stream, flags)) != TQ_OK) return r;
    if (flags[0]) return TQ_ERR_NONFINITE;
    if (tq::launch_ternary_pack(W, N, K, codes, scale_f16, st.dev, stream) != hipSuccess) return TQ_ERR_HIP;
    if ((r = st.read(stream, flags)) != TQ_OK) return r;
    if (flags[1]) return TQ_ERR_RANGE;
    return TQ_OK;
}

tq_status tq_unpack(const uint8_t* codes, const uint16_t* scale_f16, int64_t N, int64_t K, int8_t* t_out,
                    uint16_t* wdq_f16_out, hipStream_t stream) {
    if (!codes || !scale_f16) return TQ_ERR_NULL;
    if (N <= 0 || K <= 0) return TQ_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(scale_f16) & 1u) || (reinterpret_cast<uintptr_t>(wdq_f16_out) & 1u))
        return TQ_ERR_ALIGN;
    StatusWord st;
    tq_status r = st.init(stream);
    if (r != TQ_OK) return r;
    int flags[4];
    if (tq::launch_ternary_unpack(codes, scale_f16, N, K, t_out, wdq_f16_out, st.dev, stream) != hipSuccess)
        return TQ_ERR_HIP;
    if ((r = st.read(stream, flags)) != TQ_OK) return r;
    if (flags[2]) return TQ_ERR_BAD_CODE;
    return TQ_OK;
}

tq_status w4a16_pack(const float* W, int64_t N, int64_t K, int64_t group_size, int32_t* qweight,
                     uint16_t* scales_f16, hipStream_t stream) {
    if (!W || !qweight || !scales_f16) return TQ_ERR_NULL;
    if (group_size != 128) return TQ_ERR_GROUP;
    if (N <= 0 || K <= 0 || (K % 128) != 0) return TQ_ERR_SHAPE;
    if (!aligned16(W) || (reinterpret_cast<uintptr_t>(qweight) & 3u) || (reinterpret_cast<uintptr_t>(scales_f16) & 1u))
        return TQ_ERR_ALIGN;
    StatusWord st;
    tq_status r = st.init(stream);
    if (r != TQ_OK) return r;
    int flags[4];
    if (tq::launch_finite_scan(W, N * K, st.dev, stream) != hipSuccess) return TQ_ERR_HIP;
    if ((r = st.read(stream, flags)) != TQ_OK) return r;
    if (flags[0]) return TQ_ERR_NONFINITE;
    if (tq::launch_w4_pack(W, N, K, qweight, scales_f16, st.dev, stream) != hipSuccess) return TQ_ERR_HIP;
    if ((r = st.read(stream, flags)) != TQ_OK) return r;
    if (flags[1]) return TQ_ERR_RANGE;
    return TQ_OK;
}

tq_status w4a16_unpack(const int32_t* qweight, const uint16_t* scales_f16, int64_t N, int64_t K,
                       int64_t group_size, uint8_t* q_out, uint16_t* wdq_f16_out, hipStream_t stream) {
    if (!qweight || !scales_f16) return TQ_ERR_NULL;
    if (group_size != 128) return TQ_ERR_GROUP;
    if (N <= 0 || K <= 0 || (K % 128) != 0) return TQ_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(qweight) & 3u) || (reinterpret_cast<uintptr_t>(scales_f16) & 1u) ||
        (reinterpret_cast<uintptr_t>(wdq_f16_out) & 1u))
        return TQ_ERR_ALIGN;
    if (tq::launch_w4_unpack(qweight, scales_f16, N, K, q_out, wdq_f16_out, stream) != hipSuccess) return TQ_ERR_HIP;
    return from_hip(hipStreamSynchronize(stream));
}

// ------------------------------------------------------------------ apply

tq_status tq_gemm_ws(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                     const uint16_t* scale_f16, const void* bias, void* C, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, tq_path path) {
    tq_status r = check_gemm_common(A, dt, M, N, K, codes, scale_f16, C);
    if (r != TQ_OK) return r;
    if (K % 64 != 0) return TQ_ERR_SHAPE;
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 1u)) return TQ_ERR_ALIGN;
    if (workspace && !aligned16(workspace)) return TQ_ERR_ALIGN;
    if (path == TQ_PATH_AUTO) path = tq_select_path(0, M, N, K, dt);
    tq::GemmArgs a{static_cast<const uint16_t*>(A), dt == TQ_BF16 ? 1 : 0, M, N, K, codes, scale_f16,
                   static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(C)};
    const Carved w = carve(workspace, workspace_bytes);
    switch (path) {
        case TQ_PATH_GEMV:
            if (M > kGemvMaxM) return TQ_ERR_PATH;
            return from_hip(tq::launch_ternary_gemv(a, w.data, w.bytes, stream, w.flags));
        case TQ_PATH_STREAM_MFMA:
            return from_hip(tq::launch_ternary_medium(a, w.data, w.bytes, tq::compute_units(), stream));
        case TQ_PATH_GEMM:
            return from_hip(tq::launch_ternary_gemm(a, w.data, w.bytes, tq::compute_units(), stream, w.flags));
        default:
            return TQ_ERR_PATH;
    }
}

tq_status tq_gemm_ex(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                     const uint16_t* scale_f16, const void* bias, void* C, hipStream_t stream, tq_path path) {
    return tq_gemm_ws(A, dt, M, N, K, codes, scale_f16, bias, C, nullptr, 0, stream, path);
}

tq_status tq_gemm(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                  const uint16_t* scale_f16, const void* bias, void* C, hipStream_t stream) {
    return tq_gemm_ws(A, dt, M, N, K, codes, scale_f16, bias, C, nullptr, 0, stream, TQ_PATH_AUTO);
}

size_t tq_gemm_noalloc_scratch_bytes(void) { return kScratchBytes; }

tq_status tq_gemm_noalloc(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                          const uint16_t* scale_f16, const void* bias, void* C, hipStream_t stream, tq_path path) {
    tq_status r = check_gemm_common(A, dt, M, N, K, codes, scale_f16, C);
    if (r != TQ_OK) return r;
    if (K % 64 != 0) return TQ_ERR_SHAPE;
    const size_t need = tq_gemm_workspace_bytes(M, N, K, dt, path);
    if (need > kScratchBytes) return TQ_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0 && (r = symbol_address(scratch, scratch_ptr, &ws)) != TQ_OK) return r;
    return tq_gemm_ws(A, dt, M, N, K, codes, scale_f16, bias, C, ws, need, stream, path);
}

namespace {
// The W4A16 kernels for a resolved path.  TQ_PATH_GEMM that the workspace
// cannot serve (K long enough to need a split) falls back to the small-M
// kernels over blocks of 16 rows when the dispatcher chose it, and is
// refused when the caller forced it.
tq_status launch_w4_path(const tq::GemmArgs& a, tq_path path, bool chosen, void* workspace, size_t wsb,
                         hipStream_t stream, uint32_t* flags) {
    switch (path) {
        case TQ_PATH_GEMV:
            if (a.M > kGemvMaxM) return from_hip(tq::launch_w4_gemm(a, workspace, wsb, stream, flags));
            return from_hip(tq::launch_w4_gemv(a, workspace, wsb, stream, flags));
        case TQ_PATH_GEMM:
            if (tq::w4_prefill_ok(a, wsb)) return from_hip(tq::launch_w4_prefill(a, workspace, wsb, stream));
            if (!chosen) return TQ_ERR_PATH;
            if (a.M > kGemvMaxM) return from_hip(tq::launch_w4_gemm(a, workspace, wsb, stream, flags));
            return from_hip(tq::launch_w4_gemv(a, workspace, wsb, stream, flags));
        default:
            return TQ_ERR_PATH;
    }
}
}  // namespace

tq_status w4a16_gemm_ws(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const int32_t* qweight,
                        const uint16_t* scales_f16, int64_t group_size, const void* bias, void* C, void* workspace,
                        size_t workspace_bytes, hipStream_t stream, tq_path path) {
    tq_status r = check_gemm_common(A, dt, M, N, K, qweight, scales_f16, C);
    if (r != TQ_OK) return r;
    if (group_size != 128) return TQ_ERR_GROUP;
    if (K % 128 != 0) return TQ_ERR_SHAPE;
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 1u)) return TQ_ERR_ALIGN;
    if (workspace && !aligned16(workspace)) return TQ_ERR_ALIGN;
    const bool chosen = path == TQ_PATH_AUTO;
    if (chosen) path = tq_select_path(1, M, N, K, dt);
    tq::GemmArgs a{static_cast<const uint16_t*>(A), dt == TQ_BF16 ? 1 : 0, M, N, K, qweight, scales_f16,
                   static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(C)};
    const Carved w = carve(workspace, workspace_bytes);
    return launch_w4_path(a, path, chosen, w.data, w.bytes, stream, w.flags);
}

namespace {
// Bytes of partial sums a W4A16 call uses for its fastest schedule (no counters).
size_t w4_data_bytes(int64_t M, int64_t N, int64_t K, tq_dtype dt) {
    if (tq_select_path(1, M, N, K, dt) == TQ_PATH_GEMM) return tq::w4_gemm_workspace_bytes(M, N, K, tq::compute_units());
    const tq::GemmArgs a{nullptr, dt == TQ_BF16 ? 1 : 0, M < kGemvMaxM ? M : kGemvMaxM, N, K,
                         nullptr, nullptr, nullptr, nullptr};
    size_t b = tq::w4_gemv_workspace_bytes(a);
    if (M > kGemvMaxM && M % kGemvMaxM != 0) {  // the last block of M % 16 rows may split differently
        tq::GemmArgs t = a;
        t.M = M % kGemvMaxM;
        const size_t bt = tq::w4_gemv_workspace_bytes(t);
        if (bt > b) b = bt;
    }
    return b;
}
}  // namespace

size_t w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, tq_dtype dt, int64_t group_size) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || K > tq::kMaxK || group_size != 128) return 0;
    return with_flags(w4_data_bytes(M, N, K, dt));
}

tq_status w4a16_gemm_ex(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const int32_t* qweight,
                        const uint16_t* scales_f16, int64_t group_size, const void* bias, void* C,
                        hipStream_t stream, tq_path path) {
    return w4a16_gemm_ws(A, dt, M, N, K, qweight, scales_f16, group_size, bias, C, nullptr, 0, stream, path);
}

// ------------------------------------------- W4A16, zero points and act order

tq_status w4a16_pack_asym(const float* W, int64_t N, int64_t K, int64_t group_size, const int32_t* g_idx,
                          int32_t* qweight, uint16_t* scales_f16, uint8_t* zeros, int32_t* perm,
                          hipStream_t stream) {
    if (!W || !qweight || !scales_f16 || !zeros) return TQ_ERR_NULL;
    if (g_idx && !perm) return TQ_ERR_NULL;
    if (group_size != 128) return TQ_ERR_GROUP;
    if (N <= 0 || K <= 0 || (K % 128) != 0) return TQ_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(W) & 3u) || (reinterpret_cast<uintptr_t>(qweight) & 3u) ||
        (reinterpret_cast<uintptr_t>(scales_f16) & 1u) || (reinterpret_cast<uintptr_t>(g_idx) & 3u) ||
        (reinterpret_cast<uintptr_t>(perm) & 3u))
        return TQ_ERR_ALIGN;
    StatusWord st;
    tq_status r = st.init(stream);
    if (r != TQ_OK) return r;
    int flags[4];
    if (tq::launch_finite_scan(W, N * K, st.dev, stream) != hipSuccess) return TQ_ERR_HIP;
    if ((r = st.read(stream, flags)) != TQ_OK) return r;
    if (flags[0]) return TQ_ERR_NONFINITE;
    if (g_idx) {
        if (tq::launch_w4a_order(g_idx, K, perm, st.dev, stream) != hipSuccess) return TQ_ERR_HIP;
        if ((r = st.read(stream, flags)) != TQ_OK) return r;
        if (flags[3]) return TQ_ERR_GROUP;
    }
    if (tq::launch_w4a_pack(W, N, K, g_idx ? perm : nullptr, qweight, scales_f16, zeros, st.dev, stream) != hipSuccess)
        return TQ_ERR_HIP;
    if ((r = st.read(stream, flags)) != TQ_OK) return r;
    if (flags[1]) return TQ_ERR_RANGE;
    return TQ_OK;
}

tq_status w4a16_unpack_asym(const int32_t* qweight, const uint16_t* scales_f16, const uint8_t* zeros,
                            const int32_t* perm, int64_t N, int64_t K, int64_t group_size, uint8_t* q_out,
                            uint16_t* wdq_f16_out, hipStream_t stream) {
    if (!qweight || !scales_f16 || !zeros) return TQ_ERR_NULL;
    if (group_size != 128) return TQ_ERR_GROUP;
    if (N <= 0 || K <= 0 || (K % 128) != 0) return TQ_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(qweight) & 3u) || (reinterpret_cast<uintptr_t>(scales_f16) & 1u) ||
        (reinterpret_cast<uintptr_t>(perm) & 3u) || (reinterpret_cast<uintptr_t>(wdq_f16_out) & 1u))
        return TQ_ERR_ALIGN;
    if (tq::launch_w4a_unpack(qweight, scales_f16, zeros, perm, N, K, q_out, wdq_f16_out, stream) != hipSuccess)
        return TQ_ERR_HIP;
    return from_hip(hipStreamSynchronize(stream));
}

namespace {
// Workspace of the act-order gather: the activations in packed column order.
size_t gather_bytes(int64_t M, int64_t K) { return ((size_t)M * (size_t)K * 2 + 255) & ~(size_t)255; }
}  // namespace

size_t w4a16_gemm_asym_workspace_bytes(int64_t M, int64_t N, int64_t K, tq_dtype dt, int64_t group_size,
                                       int with_perm) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || K > tq::kMaxK || group_size != 128) return 0;
    return with_flags((with_perm ? gather_bytes(M, K) : 0) + w4_data_bytes(M, N, K, dt));
}

tq_status w4a16_gemm_asym(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const int32_t* qweight,
                          const uint16_t* scales_f16, const uint8_t* zeros, const int32_t* perm, int64_t group_size,
                          const void* bias, void* C, void* workspace, size_t workspace_bytes, hipStream_t stream,
                          tq_path path) {
    tq_status r = check_gemm_common(A, dt, M, N, K, qweight, scales_f16, C);
    if (r != TQ_OK) return r;
    if (group_size != 128) return TQ_ERR_GROUP;
    if (K % 128 != 0) return TQ_ERR_SHAPE;
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 1u)) return TQ_ERR_ALIGN;
    if (perm && (reinterpret_cast<uintptr_t>(perm) & 3u)) return TQ_ERR_ALIGN;
    if (workspace && !aligned16(workspace)) return TQ_ERR_ALIGN;
    const bool chosen = path == TQ_PATH_AUTO;
    if (chosen) path = tq_select_path(1, M, N, K, dt);
    if (path != TQ_PATH_GEMV && path != TQ_PATH_GEMM) return TQ_ERR_PATH;
    const uint16_t* a_eff = static_cast<const uint16_t*>(A);
    const Carved w = carve(workspace, workspace_bytes);  // counters, then [gathered activations][partials]
    uint8_t* ws = static_cast<uint8_t*>(w.data);
    size_t wsb = w.bytes;
    {  // a forced GEMM path that cannot run is refused before anything is launched
        const tq::GemmArgs probe{nullptr, dt == TQ_BF16 ? 1 : 0, M, N, K, nullptr, nullptr, nullptr, nullptr};
        const size_t gb = perm ? gather_bytes(M, K) : 0;
        if (path == TQ_PATH_GEMM && !chosen && !tq::w4_prefill_ok(probe, wsb > gb ? wsb - gb : 0)) return TQ_ERR_PATH;
    }
    if (perm) {  // gather the activations into packed column order, at the front of the workspace
        const size_t gb = gather_bytes(M, K);
        if (wsb < gb) return TQ_ERR_SHAPE;
        if (tq::launch_gather_columns(a_eff, perm, M, K, reinterpret_cast<uint16_t*>(ws), stream) != hipSuccess)
            return TQ_ERR_HIP;
        a_eff = reinterpret_cast<const uint16_t*>(ws);
        ws += gb;
        wsb -= gb;
    }
    tq::GemmArgs a{a_eff, dt == TQ_BF16 ? 1 : 0, M, N, K, qweight, scales_f16,
                   static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(C), zeros};
    void* rest = wsb ? ws : nullptr;
    return launch_w4_path(a, path, chosen, rest, wsb, stream, w.flags);
}

tq_status w4a16_gemm(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const int32_t* qweight,
                     const uint16_t* scales_f16, int64_t group_size, const void* bias, void* C, hipStream_t stream) {
    return w4a16_gemm_ex(A, dt, M, N, K, qweight, scales_f16, group_size, bias, C, stream, TQ_PATH_AUTO);
}

// ------------------------------------------------------------ measurement

tq_status tq_diag_stream_read(const void* src, size_t bytes, uint32_t* sink, int64_t blocks, hipStream_t stream) {
    if (!src || !sink) return TQ_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0 || blocks <= 0 || (int64_t)(bytes / 16) < blocks) return TQ_ERR_SHAPE;
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return TQ_ERR_ALIGN;
    return from_hip(tq::launch_stream_read(src, bytes, sink, blocks, stream));
}

tq_status tq_diag_gemv(const void* A, tq_dtype dt, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                       const uint16_t* scale_f16, const void* bias, void* C, hipStream_t stream, int variant) {
    tq_status r = check_gemm_common(A, dt, M, N, K, codes, scale_f16, C);
    if (r != TQ_OK) return r;
    if (K % 64 != 0) return TQ_ERR_SHAPE;
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 1u)) return TQ_ERR_ALIGN;
    if (variant < 0 || variant > 2) return TQ_ERR_PATH;
    tq::GemmArgs a{static_cast<const uint16_t*>(A), dt == TQ_BF16 ? 1 : 0, M, N, K, codes, scale_f16,
                   static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(C)};
    const hipError_t e = tq::launch_ternary_gemv_variant(a, variant, stream);
    return e == hipErrorInvalidValue ? TQ_ERR_PATH : from_hip(e);
}

}  // extern "C"
