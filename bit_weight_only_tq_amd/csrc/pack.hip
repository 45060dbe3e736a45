// Prepare-stage kernels: ternary and W4A16 pack / unpack.
//
// Ternary (page "Ternary quantized models in vLLM ...", section 1 tip and
// section 3.1): per output row, threshold 0.7 * mean|w|, t = sign(w) where
// |w| exceeds it, scale = mean |w| over the kept entries stored as fp16, four
// 2-bit codes t + 1 per byte (column 4j+k in bits 2k..2k+1 of byte j).
//
// W4A16 (page "Model quantization - vLLM runtime quantization architecture",
// section 5): symmetric int4, group of 128 along K, eight codes per int32,
// fp16 group scales; and the variant with per-group zero points and an
// optional activation order (g_idx) that section 5 (0) and (3) name.
//
// These results must be reproducible bit for bit, so every sum that decides
// a code is fp64 and runs sequentially in ascending column order in a single
// lane (one lane owns one row), divisions are IEEE fp64, and rounding to
// fp16 is done once, in software, from fp64.  This file is compiled with
// -ffp-contract=off.

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

// Status word bits written by the prepare kernels (plain stores of a
// constant; any number of lanes may write the same bit).
constexpr int kFlagNonFinite = 0;
constexpr int kFlagRange = 1;
constexpr int kFlagBadCode = 2;
constexpr int kFlagGroup = 3;

// ------------------------------------------------------------------ scans

// Marks flags[kFlagNonFinite] if any of the `total` floats is NaN or infinite.
__global__ __launch_bounds__(256) void finite_scan_kernel(const float* __restrict__ W, int64_t total,
                                                          int* __restrict__ flags) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const uint32_t u = __float_as_uint(W[i]);
        bad |= (u & 0x7F800000u) == 0x7F800000u;
    }
    if (bad) flags[kFlagNonFinite] = 1;
}

// ------------------------------------------------------------ ternary pack

constexpr int kPackRows = 64;   // one lane per row, one wave per block
constexpr int kPackCols = 64;   // columns staged per LDS tile

// Loads columns [k0, k0 + 64) of rows [row0, row0 + 64) into tile[r][c]
// (coalesced: consecutive lanes read consecutive columns of one row).
__device__ __forceinline__ void load_tile(float (*tile)[kPackCols + 1], const float* __restrict__ W,
                                          int64_t N, int64_t K, int64_t row0, int64_t k0, int lane) {
    const int64_t col = k0 + lane;
    for (int r = 0; r < kPackRows; ++r) {
        const int64_t row = row0 + r;
        tile[r][lane] = (row < N && col < K) ? W[row * K + col] : 0.0f;
    }
}

__global__ __launch_bounds__(64) void ternary_pack_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                          uint8_t* __restrict__ codes,
                                                          uint16_t* __restrict__ scale,
                                                          int* __restrict__ flags) {
    __shared__ float tile[kPackRows][kPackCols + 1];
    const int lane = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * kPackRows;
    const int64_t row = row0 + lane;
    const bool live = row < N;
    const int64_t rb = (K + 3) / 4;  // bytes per packed row

    // pass 1: S = sum |w| (sequential, ascending k)
    double S = 0.0;
    for (int64_t k0 = 0; k0 < K; k0 += kPackCols) {
        load_tile(tile, W, N, K, row0, k0, lane);
        __syncthreads();
        const int cn = (int)((K - k0) < kPackCols ? (K - k0) : kPackCols);
        for (int c = 0; c < cn; ++c) S += fabs((double)tile[lane][c]);
        __syncthreads();
    }
    const double thr = 0.7 * (S / (double)K);

    // pass 2: keep decisions, codes, kept sum and count
    double kept_sum = 0.0;
    int64_t kept = 0;
    const bool vec_store = (K % 64) == 0;  // whole 16-byte chunks per tile
    for (int64_t k0 = 0; k0 < K; k0 += kPackCols) {
        load_tile(tile, W, N, K, row0, k0, lane);
        __syncthreads();
        uint32_t words[4] = {0u, 0u, 0u, 0u};  // the 16 bytes of this tile's 64 columns
        for (int c = 0; c < kPackCols; ++c) {
            uint32_t code = 1u;  // padding beyond K: zero code 01
            if (k0 + c < K) {
                const double w = (double)tile[lane][c];
                const double a = fabs(w);
                if (a > thr) {
                    code = w > 0.0 ? 2u : 0u;
                    kept_sum += a;
                    ++kept;
                }
            }
            words[c >> 4] |= code << (2 * (c & 15));
        }
        if (live) {
            uint8_t* dst = codes + row * rb + k0 / 4;
            if (vec_store) {
                *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
            } else {
                const int64_t nb = (rb - k0 / 4) < 16 ? (rb - k0 / 4) : 16;
                for (int64_t b = 0; b < nb; ++b) dst[b] = (uint8_t)(words[b >> 2] >> (8 * (b & 3)));
            }
        }
        __syncthreads();
    }
    if (live) {
        const double s64 = kept > 0 ? kept_sum / (double)kept : 0.0;
        const uint16_t sb = f64_to_f16_rne(s64);
        if ((sb & 0x7FFFu) == 0x7C00u) flags[kFlagRange] = 1;
        scale[row] = sb;
    }
}

// ---------------------------------------------------------- ternary unpack

// One thread per packed byte (four columns).
__global__ __launch_bounds__(256) void ternary_unpack_kernel(const uint8_t* __restrict__ codes,
                                                             const uint16_t* __restrict__ scale,
                                                             int64_t N, int64_t K,
                                                             int8_t* __restrict__ t_out,
                                                             uint16_t* __restrict__ wdq_out,
                                                             int* __restrict__ flags) {
    const int64_t rb = (K + 3) / 4;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N * rb) return;
    const int64_t row = i / rb;
    const int64_t j = i - row * rb;
    const uint32_t byte = codes[i];
    const uint16_t s = scale[row];
    bool bad = false;
    for (int k = 0; k < 4; ++k) {
        const int64_t col = 4 * j + k;
        if (col >= K) break;
        const uint32_t f = (byte >> (2 * k)) & 3u;
        bad |= f == 3u;
        const int t = (int)f - 1;
        if (t_out) t_out[row * K + col] = (int8_t)t;
        if (wdq_out) {
            // t * s is exact in binary16: 0 * s keeps only the sign of s (IEEE
            // product sign rule), +1 * s = s, -1 * s flips the sign bit.
            const uint16_t v = t == 0 ? (uint16_t)(s & 0x8000u) : (t > 0 ? s : (uint16_t)(s ^ 0x8000u));
            wdq_out[row * K + col] = v;
        }
    }
    if (bad) flags[kFlagBadCode] = 1;
}

// ---------------------------------------------------------------- W4 pack

// One thread per output word (eight consecutive columns); the 16 threads of
// a 128-column group are 16 consecutive lanes (K % 128 == 0 keeps groups
// aligned to them), which share the group maximum through lane shuffles.
__global__ __launch_bounds__(256) void w4_pack_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                      int32_t* __restrict__ qweight,
                                                      uint16_t* __restrict__ scales,
                                                      int* __restrict__ flags) {
    const int64_t words = N * (K / 8);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = i < words;
    float w[8];
    float amax = 0.0f;
    if (live) {
        const float4 lo = reinterpret_cast<const float4*>(W)[2 * i];
        const float4 hi = reinterpret_cast<const float4*>(W)[2 * i + 1];
        w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
        w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(w[k]));
    } else {
        for (int k = 0; k < 8; ++k) w[k] = 0.0f;
    }
    // max over the 16 lanes of the group (max is exact: order does not matter)
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    if (!live) return;
    const uint16_t sb = f64_to_f16_rne((double)amax / 7.0);
    if ((sb & 0x7FFFu) == 0x7C00u) flags[kFlagRange] = 1;
    const double s = f16_bits_to_f64(sb);
    uint32_t word = 0u;
    for (int k = 0; k < 8; ++k) {
        int r = 0;
        if (s != 0.0) {
            double q = rint((double)w[k] / s);  // IEEE divide, round half to even
            q = q < -8.0 ? -8.0 : (q > 7.0 ? 7.0 : q);
            r = (int)q;
        }
        word |= (uint32_t)(r + 8) << (4 * k);
    }
    qweight[i] = (int32_t)word;
    if ((i & 15) == 0) scales[i >> 4] = sb;  // group index = word index / 16
}

// --------------------------------------------------------------- W4 unpack

// One thread per word: eight codes; dequant (q - 8) * s is exact in fp32 and
// rounded once to binary16.
__global__ __launch_bounds__(256) void w4_unpack_kernel(const int32_t* __restrict__ qweight,
                                                        const uint16_t* __restrict__ scales,
                                                        int64_t N, int64_t K,
                                                        uint8_t* __restrict__ q_out,
                                                        uint16_t* __restrict__ wdq_out) {
    const int64_t words = N * (K / 8);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const uint32_t word = (uint32_t)qweight[i];
    const float s = f16_bits_to_f32(scales[i >> 4]);
    for (int k = 0; k < 8; ++k) {
        const uint32_t q = (word >> (4 * k)) & 15u;
        if (q_out) q_out[8 * i + k] = (uint8_t)q;
        if (wdq_out) wdq_out[8 * i + k] = f32_to_f16_rne((float)((int)q - 8) * s);
    }
}

// ------------------------------------------ W4A16, zero points and g_idx

// Packed column order from g_idx: workgroup g places the columns of group g
// at 128g, 128g + 1, ... in ascending column order (a stable sort by group).
// Thread t counts the matches in its contiguous segment of the columns, an
// exclusive prefix sum over the threads gives each segment's first slot, and
// a second pass writes the columns.  Any other g_idx (an index out of range,
// a group without exactly 128 columns) sets flags[kFlagGroup]; slots past
// 128 are never written.
__global__ __launch_bounds__(256) void w4a_order_kernel(const int32_t* __restrict__ g_idx, int64_t K,
                                                        int32_t* __restrict__ perm, int* __restrict__ flags) {
    __shared__ int scan[256];
    const int64_t G = K / 128;
    const int64_t g = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t seg = (K + 255) / 256;
    const int64_t k0 = t * seg < K ? t * seg : K;
    const int64_t k1 = k0 + seg < K ? k0 + seg : K;
    int c = 0;
    bool bad = false;
    for (int64_t k = k0; k < k1; ++k) {
        const int32_t gk = g_idx[k];
        bad |= gk < 0 || (int64_t)gk >= G;
        c += (int64_t)gk == g;
    }
    scan[t] = c;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {  // inclusive Hillis-Steele scan
        const int v = t >= d ? scan[t - d] : 0;
        __syncthreads();
        scan[t] += v;
        __syncthreads();
    }
    int slot = scan[t] - c;
    for (int64_t k = k0; k < k1; ++k) {
        if ((int64_t)g_idx[k] == g) {
            if (slot < 128) perm[128 * g + slot] = (int32_t)k;
            ++slot;
        }
    }
    if (bad || (t == 255 && scan[255] != 128)) flags[kFlagGroup] = 1;
}

// One thread per output word (eight consecutive packed columns, gathered
// through perm when given); the 16 threads of a group share its minimum and
// maximum through lane shuffles (exact: order does not matter).  Range
// [min(0, lo), max(0, hi)], s = fp16((hi - lo) / 15), z = clamp(rint(-lo /
// s), 0, 15), q = clamp(rint(w / s) + z, 0, 15), all in fp64.
__global__ __launch_bounds__(256) void w4a_pack_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                       const int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ qweight,
                                                       uint16_t* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros,
                                                       int* __restrict__ flags) {
    const int64_t words = N * (K / 8);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = i < words;
    float w[8];
    float lo = 0.0f, hi = 0.0f;
    if (live) {
        const int64_t row = i / (K / 8);
        const int64_t c0 = (i % (K / 8)) * 8;
        const float* wr = W + row * K;
        for (int k = 0; k < 8; ++k) {
            w[k] = wr[perm ? (int64_t)perm[c0 + k] : c0 + k];
            lo = fminf(lo, w[k]);
            hi = fmaxf(hi, w[k]);
        }
    } else {
        for (int k = 0; k < 8; ++k) w[k] = 0.0f;
    }
    for (int off = 8; off >= 1; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, 16));
        hi = fmaxf(hi, __shfl_xor(hi, off, 16));
    }
    if (!live) return;
    const uint16_t sb = f64_to_f16_rne(((double)hi - (double)lo) / 15.0);
    if ((sb & 0x7FFFu) == 0x7C00u) flags[kFlagRange] = 1;
    const double s = f16_bits_to_f64(sb);
    int z = 0;
    if (s != 0.0) {
        double zz = rint(-(double)lo / s);
        zz = zz < 0.0 ? 0.0 : (zz > 15.0 ? 15.0 : zz);
        z = (int)zz;
    }
    uint32_t word = 0u;
    for (int k = 0; k < 8; ++k) {
        int q = 0;
        if (s != 0.0) {
            double qq = rint((double)w[k] / s) + (double)z;  // IEEE divide, round half to even
            qq = qq < 0.0 ? 0.0 : (qq > 15.0 ? 15.0 : qq);
            q = (int)qq;
        }
        word |= (uint32_t)q << (4 * k);
    }
    qweight[i] = (int32_t)word;
    if ((i & 15) == 0) {  // group index = word index / 16
        scales[i >> 4] = sb;
        zeros[i >> 4] = (uint8_t)z;
    }
}

// One thread per word: codes in packed order; dequant (q - z) * s is exact in
// fp32, rounded once to binary16 and stored at the input column perm[i].
__global__ __launch_bounds__(256) void w4a_unpack_kernel(const int32_t* __restrict__ qweight,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint8_t* __restrict__ zeros,
                                                         const int32_t* __restrict__ perm, int64_t N, int64_t K,
                                                         uint8_t* __restrict__ q_out,
                                                         uint16_t* __restrict__ wdq_out) {
    const int64_t words = N * (K / 8);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const uint32_t word = (uint32_t)qweight[i];
    const float s = f16_bits_to_f32(scales[i >> 4]);
    const int z = zeros[i >> 4];
    const int64_t row = i / (K / 8);
    const int64_t c0 = (i % (K / 8)) * 8;
    for (int k = 0; k < 8; ++k) {
        const uint32_t q = (word >> (4 * k)) & 15u;
        if (q_out) q_out[8 * i + k] = (uint8_t)q;
        if (wdq_out) {
            int64_t col = perm ? (int64_t)perm[c0 + k] : c0 + k;
            col = col < 0 || col >= K ? c0 + k : col;  // memory-safe for any perm contents
            wdq_out[row * K + col] = f32_to_f16_rne((float)((int)q - z) * s);
        }
    }
}

// ------------------------------------------------------------- launchers

static int grid_for(int64_t items, int block) {
    int64_t g = (items + block - 1) / block;
    return (int)(g < 1 ? 1 : g);
}

hipError_t launch_finite_scan(const float* W, int64_t total, int* flags, hipStream_t s) {
    int64_t g = (total + 255) / 256;
    if (g > 8192) g = 8192;
    if (g < 1) g = 1;
    finite_scan_kernel<<<(int)g, 256, 0, s>>>(W, total, flags);
    return hipGetLastError();
}

hipError_t launch_ternary_pack(const float* W, int64_t N, int64_t K, uint8_t* codes, uint16_t* scale,
                               int* flags, hipStream_t s) {
    ternary_pack_kernel<<<grid_for(N, kPackRows), kPackRows, 0, s>>>(W, N, K, codes, scale, flags);
    return hipGetLastError();
}

hipError_t launch_ternary_unpack(const uint8_t* codes, const uint16_t* scale, int64_t N, int64_t K,
                                 int8_t* t_out, uint16_t* wdq_out, int* flags, hipStream_t s) {
    const int64_t bytes = N * ((K + 3) / 4);
    ternary_unpack_kernel<<<grid_for(bytes, 256), 256, 0, s>>>(codes, scale, N, K, t_out, wdq_out, flags);
    return hipGetLastError();
}

hipError_t launch_w4_pack(const float* W, int64_t N, int64_t K, int32_t* qweight, uint16_t* scales,
                          int* flags, hipStream_t s) {
    w4_pack_kernel<<<grid_for(N * (K / 8), 256), 256, 0, s>>>(W, N, K, qweight, scales, flags);
    return hipGetLastError();
}

hipError_t launch_w4_unpack(const int32_t* qweight, const uint16_t* scales, int64_t N, int64_t K,
                            uint8_t* q_out, uint16_t* wdq_out, hipStream_t s) {
    w4_unpack_kernel<<<grid_for(N * (K / 8), 256), 256, 0, s>>>(qweight, scales, N, K, q_out, wdq_out);
    return hipGetLastError();
}

hipError_t launch_w4a_order(const int32_t* g_idx, int64_t K, int32_t* perm, int* flags, hipStream_t s) {
    w4a_order_kernel<<<(unsigned)(K / 128), 256, 0, s>>>(g_idx, K, perm, flags);
    return hipGetLastError();
}

hipError_t launch_w4a_pack(const float* W, int64_t N, int64_t K, const int32_t* perm, int32_t* qweight,
                           uint16_t* scales, uint8_t* zeros, int* flags, hipStream_t s) {
    w4a_pack_kernel<<<grid_for(N * (K / 8), 256), 256, 0, s>>>(W, N, K, perm, qweight, scales, zeros, flags);
    return hipGetLastError();
}

hipError_t launch_w4a_unpack(const int32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                             const int32_t* perm, int64_t N, int64_t K, uint8_t* q_out, uint16_t* wdq_out,
                             hipStream_t s) {
    w4a_unpack_kernel<<<grid_for(N * (K / 8), 256), 256, 0, s>>>(qweight, scales, zeros, perm, N, K, q_out, wdq_out);
    return hipGetLastError();
}

}  // namespace tq
