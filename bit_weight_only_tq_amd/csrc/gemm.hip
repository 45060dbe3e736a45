// Large-M (prefill) ternary GEMM on the CDNA4 matrix cores.
//
// C[m, n] = scale[n] * sum_k A[m, k] * t[n, k] (+ bias[n]), fp32 accumulation
// (page "Ternary quantized models in vLLM ...", section 4.2: ternary weights
// fed to the matrix units as fp16, fp32 accumulator, scale applied to the
// accumulator at the end; section 4.3: block / warp / thread tiling with
// asynchronous weight staging through shared memory).  Tiles here are sized
// for gfx950 (64-wide waves, 160 KB LDS), not for the page's 32x32 blocks.
//
// Block tile BM x BN = 128 x 256 outputs, K step BK = 64, four waves in a
// 2 x 2 arrangement, each wave owning 64 x 128 outputs = 4 x 8 tiles of
// v_mfma_f32_16x16x32_{f16,bf16}.
//
// Unpacking codes into matrix-core operands costs one VALU op per code: a
// pair of 2-bit fields is masked straight into the low mantissa bits of the
// constant MAGIC (1024.0 in fp16, 128.0 in bf16, whose unit in the last
// place is 1), giving the exact values MAGIC + c for c in {0, 1, 2}.  Since
// t = c - 1,  sum_k a_k t_k = sum_k a_k (MAGIC + c_k) - (MAGIC + 1) sum_k a_k,
// and the row sums of A are accumulated alongside (dot2 on the A fragments
// the wave already holds), so the correction is one FMA per output.
//
// A field pair extracted from bits 2i and 16+2i of a code dword covers
// columns i and i+8 of that dword's 16 columns, so K positions inside each
// 16-column group are stored in the order (0, 8, 1, 9, ..., 7, 15) for both
// operands in LDS; the contraction is invariant under that common reordering.

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int LDSK = BK + 8;     // padded LDS row (halves): 144 bytes, conflict-free 16-byte reads
constexpr int kThreads = 256;
constexpr int WM = 64;           // wave tile rows
constexpr int WN = 128;          // wave tile cols
constexpr int TM = WM / 16;      // 4 mfma tiles down
constexpr int TN = WN / 16;      // 8 mfma tiles across

template <class T> struct Mfma;
template <> struct Mfma<F16> {
    typedef f16x8 vec;
    static constexpr uint32_t kMagicPair = 0x64006400u;  // 1024.0 in both halves
    static constexpr float kBias = 1025.0f;              // MAGIC + 1
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
    }
    static constexpr uint32_t kOnePair = 0x3C003C00u;     // (1.0, 1.0)
};
template <> struct Mfma<BF16> {
    typedef bf16x8 vec;
    static constexpr uint32_t kMagicPair = 0x43004300u;  // 128.0 in both halves
    static constexpr float kBias = 129.0f;
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
    }
    static constexpr uint32_t kOnePair = 0x3F803F80u;
};

// Interleave two groups of 8 activation columns (lo = columns 0..7,
// hi = columns 8..15 of a 16-column group) into the LDS order
// (0, 8, 1, 9, ..., 7, 15): out dword i = (lo[i], hi[i]).
__device__ __forceinline__ void interleave16(const uint4& lo, const uint4& hi, uint32_t out[8]) {
    const uint32_t l[4] = {lo.x, lo.y, lo.z, lo.w};
    const uint32_t h[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // v_perm_b32(s0, s1, sel): bytes 0-3 of s1 are selectors 0-3, of s0 are 4-7
        out[2 * j] = __builtin_amdgcn_perm(h[j], l[j], 0x05040100u);      // (lo.low16, hi.low16)
        out[2 * j + 1] = __builtin_amdgcn_perm(h[j], l[j], 0x07060302u);  // (lo.high16, hi.high16)
    }
}

template <class T>
__global__ __launch_bounds__(kThreads) void ternary_gemm_kernel(GemmArgs p) {
    typedef typename Mfma<T>::vec vec;
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDSK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDSK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t rb = K / 4;  // code bytes per weight row
    const uint8_t* codes = static_cast<const uint8_t*>(p.wq);

    // global -> register staging: A = two (row, 16-column group) pieces of
    // 32 bytes per thread; B = one 16-byte chunk (64 codes) of row n0 + tid.
    const int a_grp = tid & 3;         // 16-column group within BK
    const int a_row0 = tid >> 2;       // rows a_row0 and a_row0 + 64
    uint4 a_reg[2][2];
    uint4 b_reg;
    const int64_t b_row = n0 + tid;

    auto load_global = [&](int64_t k0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t r = m0 + a_row0 + 64 * j;
            if (r < M) {
                const uint4* src = reinterpret_cast<const uint4*>(p.A + r * K + k0 + 16 * a_grp);
                a_reg[j][0] = src[0];
                a_reg[j][1] = src[1];
            } else {
                a_reg[j][0] = make_uint4(0, 0, 0, 0);
                a_reg[j][1] = make_uint4(0, 0, 0, 0);
            }
        }
        b_reg = (b_row < N) ? *reinterpret_cast<const uint4*>(codes + b_row * rb + k0 / 4)
                            : make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
    };

    const uint32_t magic_v = vgpr_const<Mfma<T>::kMagicPair>();
    const uint32_t mask3 = sgpr_const<0x00030003u>();
    auto store_lds = [&]() {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            uint32_t o[8];
            interleave16(a_reg[j][0], a_reg[j][1], o);
            uint4* dst = reinterpret_cast<uint4*>(As + (a_row0 + 64 * j) * LDSK + 16 * a_grp);
            dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
            dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
        const uint32_t bw[4] = {b_reg.x, b_reg.y, b_reg.z, b_reg.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {  // code dword d = columns 16d .. 16d+15
            uint32_t o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = ((bw[d] >> (2 * i)) & mask3) | magic_v;
            uint4* dst = reinterpret_cast<uint4*>(Bs + tid * LDSK + 16 * d);
            dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
            dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float rsum[TM] = {0.f, 0.f, 0.f, 0.f};  // partial row sums of A (row lane%16 of tile i)

    const int frag_row = lane & 15;
    const int frag_k = 8 * (lane >> 4);

    load_global(0);
    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        __syncthreads();
        store_lds();
        __syncthreads();
        if (k0 + BK < K) load_global(k0 + BK);
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            vec af[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const uint4 v = *reinterpret_cast<const uint4*>(As + (wm * WM + 16 * i + frag_row) * LDSK + ks + frag_k);
                af[i] = __builtin_bit_cast(vec, v);
                float r = rsum[i];
                r = Mfma<T>::dot2(v.x, Mfma<T>::kOnePair, r);
                r = Mfma<T>::dot2(v.y, Mfma<T>::kOnePair, r);
                r = Mfma<T>::dot2(v.z, Mfma<T>::kOnePair, r);
                r = Mfma<T>::dot2(v.w, Mfma<T>::kOnePair, r);
                rsum[i] = r;
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const uint4 v = *reinterpret_cast<const uint4*>(Bs + (wn * WN + 16 * j + frag_row) * LDSK + ks + frag_k);
                const vec bf = __builtin_bit_cast(vec, v);
#pragma unroll
                for (int i = 0; i < TM; ++i) acc[i][j] = Mfma<T>::mma(af[i], bf, acc[i][j]);
            }
        }
    }

    // full row sums: lanes l, l^16, l^32, l^48 hold the four K subsets of row l%16
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        rsum[i] += __shfl_xor(rsum[i], 16, kWave);
        rsum[i] += __shfl_xor(rsum[i], 32, kWave);
    }
    // epilogue: lane holds rows 4*(lane/16) + r (r = 0..3), column lane%16 of each tile
    const int out_col = lane & 15;
    const int out_row = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        float rs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) rs[r] = __shfl(rsum[i], out_row + r, kWave);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n0 + wn * WN + 16 * j + out_col;
            if (n >= N) continue;
            const float s = f16_bits_to_f32(p.scale[n]);
            const float b = p.bias ? T::to_f32(p.bias[n]) : 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * WM + 16 * i + out_row + r;
                if (m < M) {
                    const float v = acc[i][j][r] - Mfma<T>::kBias * rs[r];
                    p.C[m * N + n] = T::from_f32(v * s + b);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_ternary_gemm(const GemmArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    if (a.bf16) ternary_gemm_kernel<BF16><<<grid, kThreads, 0, s>>>(a);
    else ternary_gemm_kernel<F16><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

// W4A16 at large M: run the small-M kernel on successive blocks of 16
// activation rows (weights are re-read once per block).
hipError_t launch_w4_gemm(const GemmArgs& a, hipStream_t s) {
    for (int64_t m = 0; m < a.M; m += kGemvMaxM) {
        GemmArgs b = a;
        b.A = a.A + m * a.K;
        b.C = a.C + m * a.N;
        b.M = (a.M - m) < kGemvMaxM ? (a.M - m) : kGemvMaxM;
        hipError_t e = launch_w4_gemv(b, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tq
