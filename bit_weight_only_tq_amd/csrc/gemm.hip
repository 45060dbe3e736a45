// Large-M (prefill) ternary GEMM on the CDNA4 matrix cores.
//
// C[m, n] = scale[n] * sum_k A[m, k] * t[n, k] (+ bias[n]), fp32 accumulation
// (page "Ternary quantized models in vLLM ...", section 4.2: ternary weights
// fed to the matrix units as fp16, fp32 accumulator, scale applied to the
// accumulator at the end; section 4.3: block / warp / thread tiling with
// asynchronous weight staging through shared memory).  Tiles here are sized
// for gfx950 (64-wide waves, 160 KB LDS), not for the page's 32x32 blocks.
//
// Unpacking codes into matrix-core operands costs about one VALU op per
// code: a pair of 2-bit fields is masked straight into the low mantissa bits
// of the constant MAGIC (1024.0 in fp16, 128.0 in bf16, whose unit in the
// last place is 1), giving the exact values MAGIC + c for c in {0, 1, 2}.
// Since t = c - 1,
//   sum_k a_k t_k = sum_k a_k (MAGIC + c_k) - (MAGIC + 1) sum_k a_k,
// and the row sums of A are accumulated alongside with dot2, so the
// correction is one FMA per output.

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

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

// ------------------------------------------------------------------------
// v3 (K % 64 == 0): all global traffic is DMA (global_load_lds_dwordx4, no
// registers) into a 3-stage LDS ring issued two K-steps ahead:
//  - activations: 256 rows x 64 columns per stage, natural column order,
//    16-byte chunks XOR-swizzled (chunk c of row r at position c ^ (r % 8));
//  - codes: 256 weight rows x 16 bytes (64 columns) per stage.
// Codes are unpacked in registers into natural-order fp16 / bf16 pairs
// (f_2j, f_2j+1):  E = x & 0x33333333 (even fields), O = (x >> 2) & 0x33333333
// (odd fields), Y = byte-merge(E, O) per half dword, pair j = ((Y >> 4j) &
// 0x00030003) | MAGIC.  Block tile 256 x 256, K-step 64, eight waves (2 x 4)
// of 128 x 64 outputs; MFMA s of a K-step (s = 0, 1) takes 8-column chunk
// 2g + s for lane group g.  Row sums of A for the bias correction are split
// over the four waves sharing a row block (m-tiles wn and wn + 4).  The
// epilogue stages each wave's outputs through LDS so that every lane stores
// 16 contiguous bytes.
namespace v3 {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 512;
constexpr int WM = 128, WN = 64;
constexpr int TM = WM / 16, TN = WN / 16;
constexpr int kStages = 3;
constexpr int kABytes = BM * BK * 2;                // 32 KB, unpadded (swizzled)
constexpr int kBBytes = BN * BK / 4;                // 4 KB of codes
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kEpiLd = WN + 8;                      // epilogue staging row (halves)
constexpr int kEpiRows = 32;
constexpr int kEpiBytesPerWave = kEpiRows * kEpiLd * 2;
constexpr size_t kLdsBytes = (size_t)kStages * kStageBytes;
static_assert(8 * kEpiBytesPerWave + BM * 4 <= (int)kLdsBytes, "epilogue staging must fit in the ring");

// 16 bytes per lane, global -> LDS at M0 + 16 * lane (M0 must be wave-uniform).
// Issued through asm so that the compiler does not model the LDS write: its
// conservative tracking would otherwise wait for every DMA in flight before
// any LDS read, defeating the prefetch.  The kernel orders the DMA itself:
// explicit vmcnt waits before the barrier that publishes a stage, and the
// "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gptr), "s"(lds_addr) : "memory", "m0");
}

// Bare workgroup barrier: __syncthreads() would add a release fence that
// waits for every outstanding DMA, including the stage issued ahead.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <class T>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p) {
    typedef typename Mfma<T>::vec vec;
    extern __shared__ uint4 smem_v3[];
    uint8_t* lds = reinterpret_cast<uint8_t*>(smem_v3);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem_v3;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: lives in an SGPR
    const int wm = wave >> 2, wn = wave & 3;
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t rb = K / 4;
    const uint32_t magic_v = vgpr_const<Mfma<T>::kMagicPair>();
    const uint32_t mask3 = sgpr_const<0x00030003u>();
    const uint32_t mask33 = sgpr_const<0x33333333u>();

    // Activation DMA: wave w fills 1-KB blocks 4w .. 4w+3 of a stage (8 rows
    // each); lane l lands at chunk l % 8 of row l / 8, so it fetches global
    // chunk (l % 8) ^ (l / 8) of that row.  Rows past M re-read row M-1.
    const uint16_t* a_blk = p.A + m0 * K;
    uint32_t a_off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        int64_t r = 8 * (4 * wave + u) + (lane >> 3);
        if (m0 + r >= M) r = M - 1 - m0;
        a_off[u] = (uint32_t)(r * K + 8 * ((lane & 7) ^ (lane >> 3)));
    }
    // Code DMA (waves 0..3): lane l of wave w fetches the 16 bytes of weight
    // row n0 + 64w + l for the K-step.  Rows past N re-read row N-1.
    const uint8_t* b_blk = static_cast<const uint8_t*>(p.wq) + n0 * rb;
    uint32_t b_off;
    {
        int64_t n = 64 * (wave & 3) + lane;
        if (n0 + n >= N) n = N - 1 - n0;
        b_off = (uint32_t)(n * rb);
    }
    const bool b_issuer = wave < 4;
    auto issue = [&](int kstep, int stage) {
        const int64_t k0 = (int64_t)kstep * BK;
        const uint32_t dst = lds_base + (uint32_t)(stage * kStageBytes + 4096 * wave);
#pragma unroll
        for (int u = 0; u < 4; ++u) dma16(a_blk + k0 + a_off[u], dst + 1024u * u);
        if (b_issuer) dma16(b_blk + k0 / 4 + b_off, lds_base + (uint32_t)(stage * kStageBytes + kABytes + 1024 * wave));
    };
    // the stage issued before the last one has landed (per-wave DMA counts)
    auto wait_prev_stage = [&]() {
        if (b_issuer) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float rsum[2] = {0.f, 0.f};  // row sums for m-tiles wn and wn + 4

    // fragment row R = wm*128 + 16i + i16 (R % 8 == i16 % 8): chunk c at
    // byte R*128 + 16*(c ^ (i16 & 7)) of a stage
    const int frag_base = (wm * WM + i16) * (BK * 2);
    const int swz = i16 & 7;
    // code dword of tile j: row wn*64 + 16j + i16, bytes 4g .. 4g+3
    const int b_frag = kABytes + (wn * WN + i16) * 16 + 4 * g;

    const int nk = (int)(K / BK);
    issue(0, 0);
    issue(nk > 1 ? 1 : 0, 1);
    wait_prev_stage();
    stage_barrier();
    for (int kt = 0; kt < nk; ++kt) {
        const int stage = kt % kStages;
        // Unconditional so the per-wave counts stay exact: past the end the DMA
        // re-reads the last K-step into the stage nobody reads any more.
        issue(kt + 2 < nk ? kt + 2 : nk - 1, (kt + 2) % kStages);
        const uint8_t* sbase = lds + stage * kStageBytes;
        uint32_t E[TN], O[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint32_t x = *reinterpret_cast<const uint32_t*>(sbase + b_frag + 16 * 16 * j);
            E[j] = x & mask33;
            O[j] = (x >> 2) & mask33;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int chunk = (2 * g + s) ^ swz;
            vec af[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = __builtin_bit_cast(vec, *reinterpret_cast<const uint4*>(sbase + frag_base + i * 16 * (BK * 2) + 16 * chunk));
            uint4 bop[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const uint32_t y = __builtin_amdgcn_perm(O[j], E[j], s ? 0x07060302u : 0x05040100u);
                bop[j] = make_uint4((y & mask3) | magic_v, ((y >> 4) & mask3) | magic_v,
                                    ((y >> 8) & mask3) | magic_v, ((y >> 12) & mask3) | magic_v);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {  // this wave's share of the row sums: m-tiles wn, wn + 4
                const uint4 v = *reinterpret_cast<const uint4*>(sbase + frag_base + (wn + 4 * t) * 16 * (BK * 2) + 16 * chunk);
                float r = rsum[t];
                r = Mfma<T>::dot2(v.x, Mfma<T>::kOnePair, r);
                r = Mfma<T>::dot2(v.y, Mfma<T>::kOnePair, r);
                r = Mfma<T>::dot2(v.z, Mfma<T>::kOnePair, r);
                r = Mfma<T>::dot2(v.w, Mfma<T>::kOnePair, r);
                rsum[t] = r;
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const vec bf = __builtin_bit_cast(vec, bop[j]);
#pragma unroll
                for (int i = 0; i < TM; ++i) acc[i][j] = Mfma<T>::mma(af[i], bf, acc[i][j]);
            }
        }
        wait_prev_stage();  // stage kt + 1 (issued last iteration) has landed
        stage_barrier();    // ... for every wave, and nobody reads stage kt any more
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();        // the ring is idle from here on

    // row sums -> LDS
    float* rs_lds = reinterpret_cast<float*>(lds + 8 * kEpiBytesPerWave);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float r = rsum[t];
        r += __shfl_xor(r, 16, kWave);
        r += __shfl_xor(r, 32, kWave);
        if (g == 0) rs_lds[wm * WM + 16 * (wn + 4 * t) + i16] = r;
    }
    __syncthreads();

    // epilogue: per wave, 4 slabs of 32 rows x 64 columns through a private LDS area
    uint16_t* stg = reinterpret_cast<uint16_t*>(lds + wave * kEpiBytesPerWave);
    float sc[TN], bi[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + 16 * j + i16;
        const int64_t nc = n < N ? n : N - 1;
        sc[j] = f16_bits_to_f32(p.scale[nc]);
        bi[j] = p.bias ? T::to_f32(p.bias[nc]) : 0.0f;
    }
    const bool vec_ok = (N % 8) == 0;
#pragma unroll
    for (int slab = 0; slab < TM / 2; ++slab) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * slab + ii;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * ii + 4 * g + r;
                const float rs = rs_lds[wm * WM + 16 * i + 4 * g + r];
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    stg[row * kEpiLd + 16 * j + i16] = T::from_f32_fast((acc[i][j][r] - Mfma<T>::kBias * rs) * sc[j] + bi[j]);
            }
        }
        // each lane stores 16 contiguous bytes: row lane/8 + 8q, columns 8*(lane%8) .. +7
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = (lane >> 3) + 8 * q;
            const int col = 8 * (lane & 7);
            const int64_t m = m0 + wm * WM + 32 * slab + row;
            const int64_t n = n0 + wn * WN + col;
            if (m >= M) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(stg + row * kEpiLd + col);
            if (vec_ok && n + 8 <= N) {
                *reinterpret_cast<uint4*>(p.C + m * N + n) = v;
            } else {
                const uint16_t h[8] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16),
                                       (uint16_t)v.z, (uint16_t)(v.z >> 16), (uint16_t)v.w, (uint16_t)(v.w >> 16)};
                for (int e = 0; e < 8; ++e)
                    if (n + e < N) p.C[m * N + n + e] = h[e];
            }
        }
    }
}

}  // namespace v3


}  // namespace

template <class T>
static hipError_t launch_v3(const GemmArgs& a, hipStream_t s) {
    static DeviceFlags lds_limit_set;
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&v3::gemm_kernel<T>), (int)v3::kLdsBytes, lds_limit_set);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((a.N + v3::BN - 1) / v3::BN), (unsigned)((a.M + v3::BM - 1) / v3::BM));
    v3::gemm_kernel<T><<<grid, v3::kThreads, v3::kLdsBytes, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_ternary_gemm(const GemmArgs& a, hipStream_t s) {
    // the C ABI guarantees K % 64 == 0 (whole 16-byte code chunks per row)
    return a.bf16 ? launch_v3<BF16>(a, s) : launch_v3<F16>(a, s);
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
