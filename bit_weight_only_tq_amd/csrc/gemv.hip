// Small-M (decode) kernels: every packed weight byte is read from HBM exactly
// once per call and unpacked in registers; activations (a few KB) come from
// the L2 cache.  One wave owns one output row at a time; its 64 lanes split K
// into 16-byte chunks of packed codes, and the lane partials are combined by
// a wave-wide reduction (DPP + lane shuffles).  No atomics, no split-K
// across waves: results are deterministic.
//
// Ternary layer arithmetic (page "Ternary quantized models in vLLM ...",
// section 4): value = code - 1, out = sum_k a_k * value_k, then the row
// scale is applied once after accumulation (section 4.2), in fp32.
// W4A16 (page "Model quantization - vLLM runtime quantization architecture",
// section 5): value = q - 8 with a per-(row, 128-column group) fp16 scale.

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

constexpr int kGemvWaves = 4;  // waves per block; one output row per wave

// --------------------------------------------------------------- ternary

// C[m, row] for all m < M (M <= MT).  A 16-byte chunk holds 64 codes:
// dword d of the chunk covers columns 16d .. 16d+15, field j (bits 2j..2j+1)
// being column 16d + j.
template <int MT, class T>
__global__ __launch_bounds__(kGemvWaves * kWave) void ternary_gemv_kernel(GemmArgs p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kGemvWaves + (threadIdx.x >> 6);
    if (row >= p.N) return;  // uniform per wave
    const int64_t K = p.K;
    const int64_t chunks = K / 64;
    const uint4* crow = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(p.wq) + row * (K / 4));
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

    for (int64_t c = lane; c < chunks; c += kWave) {
        const uint4 q = crow[c];
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < p.M) {
                const uint4* ap = reinterpret_cast<const uint4*>(p.A + m * K + c * 64);
#pragma unroll
                for (int d = 0; d < 8; ++d) {  // 8 columns per 16-byte activation load
                    const uint4 av = ap[d];
                    const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
                    const uint32_t cw = qw[d >> 1] >> (16 * (d & 1));
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint16_t h = (uint16_t)(aw[e >> 1] >> (16 * (e & 1)));
                        const float t = (float)((int)((cw >> (2 * e)) & 3u) - 1);
                        acc[m] = fmaf(t, T::to_f32(h), acc[m]);
                    }
                }
            }
        }
    }
    const float s = f16_bits_to_f32(p.scale[row]);
    const float b = p.bias ? T::to_f32(p.bias[row]) : 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (m < p.M) {
            const float v = wave_sum(acc[m]);
            if (lane == 0) p.C[m * p.N + row] = T::from_f32(v * s + b);
        }
    }
}

// ------------------------------------------------------------------- W4

// A 16-byte chunk holds four int32 words = 32 columns, all inside one
// 128-column group (a group is four chunks).
template <int MT, class T>
__global__ __launch_bounds__(kGemvWaves * kWave) void w4_gemv_kernel(GemmArgs p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kGemvWaves + (threadIdx.x >> 6);
    if (row >= p.N) return;
    const int64_t K = p.K;
    const int64_t chunks = K / 32;
    const uint4* wrow = reinterpret_cast<const uint4*>(static_cast<const int32_t*>(p.wq) + row * (K / 8));
    const uint16_t* srow = p.scale + row * (K / 128);
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

    for (int64_t c = lane; c < chunks; c += kWave) {
        const uint4 q = wrow[c];
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
        const float s = f16_bits_to_f32(srow[c >> 2]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < p.M) {
                const uint4* ap = reinterpret_cast<const uint4*>(p.A + m * K + c * 32);
                float part = 0.0f;
#pragma unroll
                for (int d = 0; d < 4; ++d) {  // word d: columns 8d .. 8d+7
                    const uint4 av = ap[d];
                    const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint16_t h = (uint16_t)(aw[e >> 1] >> (16 * (e & 1)));
                        const float v = (float)((int)((qw[d] >> (4 * e)) & 15u) - 8);
                        part = fmaf(v, T::to_f32(h), part);
                    }
                }
                acc[m] = fmaf(part, s, acc[m]);
            }
        }
    }
    const float b = p.bias ? T::to_f32(p.bias[row]) : 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (m < p.M) {
            const float v = wave_sum(acc[m]);
            if (lane == 0) p.C[m * p.N + row] = T::from_f32(v + b);
        }
    }
}

// ------------------------------------------------------------- launchers

hipError_t launch_ternary_gemv(const GemmArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.N + kGemvWaves - 1) / kGemvWaves));
    const dim3 block(kGemvWaves * kWave);
    if (a.M <= 1) {
        if (a.bf16) ternary_gemv_kernel<1, BF16><<<grid, block, 0, s>>>(a);
        else ternary_gemv_kernel<1, F16><<<grid, block, 0, s>>>(a);
    } else if (a.M <= 4) {
        if (a.bf16) ternary_gemv_kernel<4, BF16><<<grid, block, 0, s>>>(a);
        else ternary_gemv_kernel<4, F16><<<grid, block, 0, s>>>(a);
    } else {
        if (a.bf16) ternary_gemv_kernel<16, BF16><<<grid, block, 0, s>>>(a);
        else ternary_gemv_kernel<16, F16><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_w4_gemv(const GemmArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.N + kGemvWaves - 1) / kGemvWaves));
    const dim3 block(kGemvWaves * kWave);
    if (a.M <= 1) {
        if (a.bf16) w4_gemv_kernel<1, BF16><<<grid, block, 0, s>>>(a);
        else w4_gemv_kernel<1, F16><<<grid, block, 0, s>>>(a);
    } else if (a.M <= 4) {
        if (a.bf16) w4_gemv_kernel<4, BF16><<<grid, block, 0, s>>>(a);
        else w4_gemv_kernel<4, F16><<<grid, block, 0, s>>>(a);
    } else {
        if (a.bf16) w4_gemv_kernel<16, BF16><<<grid, block, 0, s>>>(a);
        else w4_gemv_kernel<16, F16><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace tq
