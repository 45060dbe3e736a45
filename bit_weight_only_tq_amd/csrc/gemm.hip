// Large-M (prefill) ternary GEMM on the CDNA4 matrix cores.
//
// C[m, n] = scale[n] * sum_k A[m, k] * t[n, k] (+ bias[n]), fp32 accumulation
// (page "Ternary quantized models in vLLM ...", section 4.2: ternary weights
// fed to the matrix units as fp16, fp32 accumulator, scale applied to the
// accumulator at the end; section 4.3: block / warp / thread tiling with
// asynchronous weight staging through shared memory).  Tiles here are sized
// for gfx950 (64-wide waves, 160 KB LDS), not for the page's 32x32 blocks.
//
// Unpacking codes into matrix-core operands: a pair of 2-bit fields is
// masked straight into the low mantissa bits of the fp16 constant 1024
// (unit in the last place 1), giving the exact values 1024 + c for c in
// {0, 1, 2}, and one packed fp16 subtract of 1025 leaves the ternary value
// t = c - 1 itself (exact).  The matrix units therefore multiply every
// activation by -1, 0 or +1 and the fp32 sums hold only the terms of the
// result, so the error of an output scales with its own sum_k |a_k t_k|.
// bf16 activations take the same operand bits, which read as bf16 are
// -2^-7, 0, +2^-7; those kernels multiply their sums by 128 (exact).

#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

template <class T> struct Mfma;
template <> struct Mfma<F16> {
    typedef f16x8 vec;
    static constexpr float kUnit = 1.0f;  // value of the operand bits of +1
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<BF16> {
    typedef bf16x8 vec;
    static constexpr float kUnit = kBf16TernaryUnit;  // the operand bits of +1 read as bf16 are 2^-7
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

// Natural-order operand pairs of byte b of a code dword x (fields f_4b ..
// f_4b+3 at bits 0, 2, 4, 6 of the byte): one byte permute puts the byte in
// the low byte of both halves, a mask into 1024.0 keeps field 4b (low half)
// and 4b+1 (high half) at bits 0 and 2, or fields 4b+2 and 4b+3 at bits 4
// and 6, and one packed fp16 fma per pair scales each half by its own power
// of 4 and subtracts 1024/4^s + 1: (1024 + 4^s c) / 4^s - (1024/4^s + 1) =
// c - 1, exact.
struct NatConsts {
    f16x2 mul_lo, add_lo, mul_hi, add_hi;
};
__device__ __forceinline__ NatConsts nat_consts() {
    return NatConsts{f16x2{(_Float16)1.0f, (_Float16)0.25f}, f16x2{(_Float16)-1025.0f, (_Float16)-257.0f},
                     f16x2{(_Float16)0.0625f, (_Float16)0.015625f}, f16x2{(_Float16)-65.0f, (_Float16)-17.0f}};
}
__device__ __forceinline__ uint32_t nat_fma(uint32_t v, f16x2 mul, f16x2 add) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, v), mul, add));
}
// Operand of fields 8h .. 8h+7 of x (bytes 2h and 2h+1) in natural order.
template <int H>
__device__ __forceinline__ uint4 nat_quad(uint32_t x, uint32_t magic_v, const NatConsts& k) {
    const uint32_t p0 = __builtin_amdgcn_perm(x, x, 0x0C000C00u | (uint32_t)(2 * H) * 0x00010001u);
    const uint32_t p1 = __builtin_amdgcn_perm(x, x, 0x0C000C00u | (uint32_t)(2 * H + 1) * 0x00010001u);
    const uint32_t mlo = sgpr_const<0x000C0003u>(), mhi = sgpr_const<0x00C00030u>();
    return make_uint4(nat_fma((p0 & mlo) | magic_v, k.mul_lo, k.add_lo), nat_fma((p0 & mhi) | magic_v, k.mul_hi, k.add_hi),
                      nat_fma((p1 & mlo) | magic_v, k.mul_lo, k.add_lo), nat_fma((p1 & mhi) | magic_v, k.mul_hi, k.add_hi));
}

// Workgroup barrier without a release fence: __syncthreads() would wait for
// every outstanding DMA, including the stages issued ahead.  LDS reads and
// writes issued before it are waited for here (the hardware barrier does not
// wait for them, and the compiler may place register-only work, with the
// waits that feed it, after the barrier): a slot read before the barrier may
// be refilled by another wave's DMA right after it, and pairs written before
// it are read by other waves after it.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------------
// v3 (K % 64 == 0): all global traffic is DMA (global_load_lds_dwordx4, no
// registers) into a 3-stage LDS ring issued two K-steps ahead:
//  - activations: 256 rows x 64 columns per stage, natural column order,
//    16-byte chunks XOR-swizzled (chunk c of row r at position c ^ (r % 8));
//  - codes: 256 weight rows x 16 bytes (64 columns) per stage.
// Codes are unpacked in registers into natural-order pairs (f_2j, f_2j+1),
// five VALU instructions per four codes (nat_quad): a byte permute, two
// masks into 1024.0 and two packed fp16 fmas that leave the ternary values
// c - 1 themselves.  DMA addresses are the tile's base in SGPRs plus fixed
// 32-bit lane offsets, so the K loop does no 64-bit address arithmetic.
// Block tile 256 x 256 (128 x 256 for the last round of
// an unbalanced grid), K-step 64, eight waves (2 x 4) of 128 x 64 (64 x 64)
// outputs; MFMA s of a K-step (s = 0, 1) takes 8-column chunk 2g + s for
// lane group g.  The epilogue stages each wave's outputs through LDS so that
// every lane stores 16 contiguous bytes.  With a K split (blockIdx.z = split
// z of S, K-steps [z*nk/S, (z+1)*nk/S)) the fp32 partials (in units of the
// result) are stored straight from the accumulators instead.
namespace v3 {

constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 512;
constexpr int WN = 64;
constexpr int TN = WN / 16;
constexpr int kStages = 3;
constexpr int kBBytes = BN * BK / 4;                // 4 KB of codes
constexpr int kEpiLd = WN + 8;                      // epilogue staging row (halves)
constexpr int kEpiRows = 32;
constexpr int kEpiBytesPerWave = kEpiRows * kEpiLd * 2;

// Block tile height: 256 rows (two waves of 128 along M), or 128 (two of 64)
// for the last round of a grid that does not fill whole rounds.
template <int BM_>
struct Tile {
    static constexpr int BM = BM_;
    static constexpr int WM = BM / 2;               // rows per wave
    static constexpr int TM = WM / 16;              // m-tiles per wave
    static constexpr int AU = BM / 64;              // 1-KB activation DMA blocks per wave and stage
    static constexpr int kABytes = BM * BK * 2;     // unpadded (swizzled)
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr size_t kLdsBytes = (size_t)kStages * kStageBytes;
    static_assert(8 * kEpiBytesPerWave <= (int)kLdsBytes, "epilogue staging must fit in the ring");
};

template <class T, int BMT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(SplitArgs sa) {
    typedef typename Mfma<T>::vec vec;
    typedef Tile<BMT> G;
    constexpr int BM = G::BM, WM = G::WM, TM = G::TM, AU = G::AU;
    constexpr int kABytes = G::kABytes, kStageBytes = G::kStageBytes;
    const GemmArgs& p = sa.g;
    const int64_t ldc = sa.ldc ? sa.ldc : p.N;       // row stride of C
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
    const uint32_t magic_v = vgpr_const<kMagic2>();
    const NatConsts nk_c = nat_consts();

    // Activation DMA: wave w fills 1-KB blocks AU w .. AU w + AU-1 of a stage
    // (8 rows each); lane l lands at chunk l % 8 of row l / 8, so it fetches
    // global chunk (l % 8) ^ (l / 8) of that row.  Rows past M re-read row M-1.
    const uint16_t* a_blk = p.A + m0 * K;
    uint32_t a_off[AU];
#pragma unroll
    for (int u = 0; u < AU; ++u) {
        int64_t r = 8 * (AU * wave + u) + (lane >> 3);
        if (m0 + r >= M) r = M - 1 - m0;
        a_off[u] = (uint32_t)(2 * (r * K + 8 * ((lane & 7) ^ (lane >> 3))));  // bytes
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
        const uint32_t dst = lds_base + (uint32_t)(stage * kStageBytes + 1024 * AU * wave);
#pragma unroll
        for (int u = 0; u < AU; ++u) dma16s(a_blk + k0, a_off[u], dst + 1024u * u);
        if (b_issuer) dma16s(b_blk + k0 / 4, b_off, lds_base + (uint32_t)(stage * kStageBytes + kABytes + 1024 * wave));
    };
    // the stage issued before the last one has landed (per-wave DMA counts)
    auto wait_prev_stage = [&]() {
        if (b_issuer) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(AU + 1) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(AU) : "memory");
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragment row R = wm*128 + 16i + i16 (R % 8 == i16 % 8): chunk c at
    // byte R*128 + 16*(c ^ (i16 & 7)) of a stage
    const int frag_base = (wm * WM + i16) * (BK * 2);
    const int swz = i16 & 7;
    // code dword of tile j: row wn*64 + 16j + i16, bytes 4g .. 4g+3
    const int b_frag = kABytes + (wn * WN + i16) * 16 + 4 * g;

    // this split's K-steps [kb, kb + nk); the host keeps S <= K / BK
    const int nk_all = (int)(K / BK);
    const int kb = (int)((int64_t)blockIdx.z * nk_all / sa.S);
    const int nk = (int)((int64_t)(blockIdx.z + 1) * nk_all / sa.S) - kb;
    issue(kb, 0);
    issue(kb + (nk > 1 ? 1 : 0), 1);
    wait_prev_stage();
    stage_barrier();
    for (int kt = 0; kt < nk; ++kt) {
        const int stage = kt % kStages;
        // Unconditional so the per-wave counts stay exact: past the end the DMA
        // re-reads the last K-step into the stage nobody reads any more.
        issue(kb + (kt + 2 < nk ? kt + 2 : nk - 1), (kt + 2) % kStages);
        const uint8_t* sbase = lds + stage * kStageBytes;
        uint32_t X[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) X[j] = *reinterpret_cast<const uint32_t*>(sbase + b_frag + 16 * 16 * j);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int chunk = (2 * g + s) ^ swz;
            vec af[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = __builtin_bit_cast(vec, *reinterpret_cast<const uint4*>(sbase + frag_base + i * 16 * (BK * 2) + 16 * chunk));
            uint4 bop[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bop[j] = s ? nat_quad<1>(X[j], magic_v, nk_c) : nat_quad<0>(X[j], magic_v, nk_c);
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

    if (sa.S > 1) {  // fp32 partial of this split: 16 lanes store 64 contiguous bytes per row
        float* ws = sa.ws + (int64_t)blockIdx.z * M * N;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * WM + 16 * i + 4 * g + r;
                const int64_t m = m0 + row;
                if (m >= M) continue;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int64_t n = n0 + wn * WN + 16 * j + i16;
                    if (n < N) store_partial(ws + m * N + n, acc[i][j][r] * Mfma<T>::kUnit);
                }
            }
        // the last split of this tile to finish sums the partials and finishes it
        if (!sa.flags || !split_last_arrival(sa.flags, blockIdx.y * gridDim.x + blockIdx.x, sa.S,
                                             reinterpret_cast<uint32_t*>(lds)))
            return;
        float scz[TN], biz[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n0 + wn * WN + 16 * j + i16;
            const int64_t nc = n < N ? n : N - 1;
            scz[j] = f16_bits_to_f32(p.scale[nc]);
            biz[j] = p.bias ? T::to_f32(p.bias[nc]) : 0.0f;
        }
        // two m-tiles (32 outputs) per batch, both splits of a batch in flight
        const float* base = sa.ws + m0 * N + n0;
        constexpr int IB = TM < 2 ? TM : 2, E = IB * 4 * TN;
#pragma unroll
        for (int i0 = 0; i0 < TM; i0 += IB) {
            uint32_t off[E];
#pragma unroll
            for (int ii = 0; ii < IB; ++ii)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int64_t m = m0 + wm * WM + 16 * (i0 + ii) + 4 * g + r;
                        const int64_t n = n0 + wn * WN + 16 * j + i16;
                        off[(ii * 4 + r) * TN + j] = (uint32_t)(((m < M ? m : M - 1) - m0) * N + ((n < N ? n : N - 1) - n0));
                    }
            float sum[E];
            split_sums<E, 2>(base, M * N, off, sa.S, sum);
#pragma unroll
            for (int ii = 0; ii < IB; ++ii)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t m = m0 + wm * WM + 16 * (i0 + ii) + 4 * g + r;
                    if (m >= M) continue;
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int64_t n = n0 + wn * WN + 16 * j + i16;
                        if (n < N) p.C[m * ldc + n] = T::from_f32_fast(sum[(ii * 4 + r) * TN + j] * scz[j] + biz[j]);
                    }
                }
        }
        return;
    }

    // epilogue: per wave, 4 slabs of 32 rows x 64 columns through a private LDS area
    uint16_t* stg = reinterpret_cast<uint16_t*>(lds + wave * kEpiBytesPerWave);
    float sc[TN], bi[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + 16 * j + i16;
        const int64_t nc = n < N ? n : N - 1;
        sc[j] = f16_bits_to_f32(p.scale[nc]) * Mfma<T>::kUnit;
        bi[j] = p.bias ? T::to_f32(p.bias[nc]) : 0.0f;
    }
    const bool vec_ok = ((N | ldc) % 8) == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15u) == 0;
#pragma unroll
    for (int slab = 0; slab < TM / 2; ++slab) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * slab + ii;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * ii + 4 * g + r;
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    stg[row * kEpiLd + 16 * j + i16] = T::from_f32_fast(acc[i][j][r] * sc[j] + bi[j]);
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
                *reinterpret_cast<uint4*>(p.C + m * ldc + n) = v;
            } else {
                const uint16_t h[8] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16),
                                       (uint16_t)v.z, (uint16_t)(v.z >> 16), (uint16_t)v.w, (uint16_t)(v.w >> 16)};
                for (int e = 0; e < 8; ++e)
                    if (n + e < N) p.C[m * ldc + n + e] = h[e];
            }
        }
    }
}

}  // namespace v3

// ------------------------------------------------------------------------
// Medium M (17 .. 255 activation rows): 16TM x 256 tiles (TM m-tiles of 16
// rows, 256 weight rows) fed by the same DMA ring and register unpack as v3,
// but six stages deep (five K-steps in flight), so that a single workgroup
// per compute unit keeps enough loads outstanding.  Wave w computes all
// 16TM rows x columns 32w .. 32w+31.  With few row tiles the grid is also
// split along K (SplitArgs); with S = 1 the tile kernel finishes its outputs
// itself.
namespace mm {

constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 512;
constexpr int TN = 2;
constexpr int kStages = 6;
constexpr int kAhead = kStages - 1;
constexpr int kBBytes = BN * BK / 4;  // 4 KB of codes per stage
template <int TM> constexpr int a_bytes() { return 16 * TM * BK * 2; }
template <int TM> constexpr int stage_bytes() { return a_bytes<TM>() + kBBytes; }
template <int TM> constexpr size_t lds_bytes() { return (size_t)kStages * stage_bytes<TM>(); }

template <class T, int TM>
__global__ __launch_bounds__(kThreads) void tile_kernel(SplitArgs sa) {
    typedef typename Mfma<T>::vec vec;
    constexpr int BM = 16 * TM;
    constexpr int kABytes = a_bytes<TM>();
    constexpr int kStageBytes = stage_bytes<TM>();
    const GemmArgs& p = sa.g;
    extern __shared__ uint4 smem_mm[];
    uint8_t* lds = reinterpret_cast<uint8_t*>(smem_mm);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem_mm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int z = blockIdx.z;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t rb = K / 4;
    const int nk = (int)(K / BK);
    const int ks0 = (int)((int64_t)nk * z / sa.S);
    const int ks1 = (int)((int64_t)nk * (z + 1) / sa.S);  // > ks0: S <= nk
    const uint32_t magic_v = vgpr_const<kMagic2>();
    const NatConsts nk_c = nat_consts();

    // Activation DMA: waves 0 .. 2TM-1 fill the 1-KB blocks of a stage (8 rows
    // each); lane l lands at chunk l % 8 of row 8w + l / 8 and fetches global
    // chunk (l % 8) ^ (l / 8) of it.  Rows past M re-read row M-1.
    const bool a_issuer = wave < 2 * TM;
    uint32_t a_off;
    {
        int64_t r = 8 * (wave % (2 * TM)) + (lane >> 3);
        if (m0 + r >= M) r = M - 1 - m0;
        a_off = (uint32_t)(2 * (r * K + 8 * ((lane & 7) ^ (lane >> 3))));  // bytes
    }
    const uint16_t* a_blk = p.A + m0 * K;
    // Code DMA (waves 0..3): lane l of wave w fetches 16 bytes of weight row
    // n0 + 64w + l.  Rows past N re-read row N-1.
    const bool b_issuer = wave < 4;
    const uint8_t* b_blk = static_cast<const uint8_t*>(p.wq) + n0 * rb;
    uint32_t b_off;
    {
        int64_t n = 64 * (wave & 3) + lane;
        if (n0 + n >= N) n = N - 1 - n0;
        b_off = (uint32_t)(n * rb);
    }
    auto issue = [&](int kstep, int stage) {
        const int64_t k0 = (int64_t)kstep * BK;
        if (a_issuer) dma16s(a_blk + k0, a_off, lds_base + (uint32_t)(stage * kStageBytes + 1024 * wave));
        if (b_issuer) dma16s(b_blk + k0 / 4, b_off, lds_base + (uint32_t)(stage * kStageBytes + kABytes + 1024 * wave));
    };
    // the oldest stage in flight has landed: at most kAhead - 1 stages of
    // this wave's DMAs remain outstanding
    const int per_stage = (a_issuer ? 1 : 0) + (b_issuer ? 1 : 0);
    auto wait_oldest = [&]() {
        if (per_stage == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else if (per_stage == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    };
    static_assert(kAhead == 5, "wait counts above assume five K-steps in flight");

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int swz = i16 & 7;
    const int frag_base = i16 * (BK * 2);
    const int b_frag = kABytes + (32 * wave + i16) * 16 + 4 * g;

#pragma unroll
    for (int u = 0; u < kAhead; ++u) issue(ks0 + u < ks1 ? ks0 + u : ks1 - 1, u);
    wait_oldest();
    stage_barrier();
    for (int kt = ks0; kt < ks1; ++kt) {
        const int it = kt - ks0;
        const int stage = it % kStages;
        issue(kt + kAhead < ks1 ? kt + kAhead : ks1 - 1, (it + kAhead) % kStages);
        const uint8_t* sbase = lds + stage * kStageBytes;
        uint32_t X[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) X[j] = *reinterpret_cast<const uint32_t*>(sbase + b_frag + 16 * 16 * j);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int chunk = (2 * g + s) ^ swz;
            vec af[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = __builtin_bit_cast(vec, *reinterpret_cast<const uint4*>(sbase + frag_base + i * 16 * (BK * 2) + 16 * chunk));
            uint4 bop[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bop[j] = s ? nat_quad<1>(X[j], magic_v, nk_c) : nat_quad<0>(X[j], magic_v, nk_c);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const vec bf = __builtin_bit_cast(vec, bop[j]);
#pragma unroll
                for (int i = 0; i < TM; ++i) acc[i][j] = Mfma<T>::mma(af[i], bf, acc[i][j]);
            }
        }
        wait_oldest();      // stage of K-step kt + 1 has landed
        stage_barrier();    // ... for every wave, and nobody reads stage kt any more
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const bool final_out = sa.S == 1;
    float sc[TN], bi[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + 32 * wave + 16 * j + i16;
        const int64_t nc = n < N ? n : N - 1;
        sc[j] = f16_bits_to_f32(p.scale[nc]);
        bi[j] = p.bias ? T::to_f32(p.bias[nc]) : 0.0f;
    }
    float* wsz = final_out ? nullptr : sa.ws + (int64_t)z * M * N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * i + 4 * g + r;
            const int64_t m = m0 + row;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t n = n0 + 32 * wave + 16 * j + i16;
                if (n >= N) continue;
                const float v = acc[i][j][r] * Mfma<T>::kUnit;
                if (final_out) p.C[m * N + n] = T::from_f32_fast(v * sc[j] + bi[j]);
                else wsz[m * N + n] = v;
            }
        }
    }
}

// C[m, n] = (sum over z of ws[z][m][n]) * scale[n] + bias[n] (no scale when
// the partials carry it already); grid
// (ceil(N/256), reduce_rows(M)), each workgroup row striding over m.
constexpr int64_t kReduceMaxRows = 65535;
inline unsigned reduce_rows(int64_t M) { return (unsigned)(M < kReduceMaxRows ? M : kReduceMaxRows); }
template <class T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(SplitArgs sa) {
    const GemmArgs& p = sa.g;
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= p.N) return;
    const int64_t MN = p.M * p.N;
    const float sc = sa.scaled ? 1.0f : f16_bits_to_f32(p.scale[n]);
    const float b = p.bias ? T::to_f32(p.bias[n]) : 0.0f;
    for (int64_t m = blockIdx.y; m < p.M; m += gridDim.y) {
        const float* src = sa.ws + m * p.N + n;
        // eight partials in flight at a time, summed in split order z = 0, 1, ...
        float s = 0.0f;
        for (int z0 = 0; z0 < sa.S; z0 += 8) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = z0 + j < sa.S ? src[(int64_t)(z0 + j) * MN] : 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (z0 + j < sa.S) s += v[j];
        }
        p.C[m * p.N + n] = T::from_f32_fast(s * sc + b);
    }
}

}  // namespace mm


// ------------------------------------------------------------------------
// Medium M, K % 256 == 0 (fp16 or bf16): 16TM activation rows x 256 weight
// rows per workgroup, eight waves of 32 weight rows each, optional K split,
// with 256-column K-steps in an LDS ring filled R - 1 steps ahead, so that
// each barrier covers 8TM MFMAs per wave and every DMA instruction reads
// whole row segments:
//  - codes: 256 rows x 64 bytes per step, 16 rows per instruction (lane l:
//    row l/4, 16-byte chunk l%4); chunk c of row r sits at c ^ ((r/4) % 4)
//    so that the 64 lanes' dword reads of a fragment hit 64 different banks;
//  - activations: 16TM rows x 512 bytes per step, 2 rows per instruction
//    (lane l: row l/32, chunk l%32); chunk c of row r at c ^ (r % 16).
// Codes are unpacked with the in-place field scheme of the decode kernels
// (tern_pair: one v_and_or_b32 and one packed fp16 fma per operand
// register).  That needs the activations paired to match the fields, which
// is done once per K-step for the whole workgroup, in place in the ring
// slot: thread t owns the 16-column groups (row t/16 + 32p, group t%16) and
// rewrites each group's two 16-byte chunks (columns 16G..16G+7 and 16G+8..)
// as its pairs for fields 0..3 and 4..7, keeping the chunk positions
// (c ^ (r % 16)).  The pairing of step k+1 shares a phase with the MFMAs of
// step k, so one barrier per step still suffices:
//   issue DMA of step k + R - 1; pair step k + 1; contract step k;
//   wait for the DMA of step k + 2; barrier,
// with R = 4 ring slots for 32 activation rows and 3 for 64 (LDS).
// Sub-step u, half h of a K-step: lane group g contracts 16-column group
// G = 4u + g, fields 4h..4h+3, against code dword g of row chunk u.
namespace mm3 {

constexpr int BN = 256;
constexpr int BK = 256;
constexpr int kThreads = 512;
constexpr int TN = 2;
constexpr int kBBytes = BN * (BK / 4);  // 16 KB of codes per step
template <int TM> constexpr int a_bytes() { return 16 * TM * BK * 2; }
template <int TM> constexpr int stage_bytes() { return a_bytes<TM>() + kBBytes; }
template <int TM> constexpr int slots() { return TM == 2 ? 4 : 3; }
template <int TM> constexpr size_t lds_bytes() { return (size_t)slots<TM>() * stage_bytes<TM>(); }

// In-place pairing of one 16-column group of one activation row.
__device__ __forceinline__ void prep_group(uint8_t* row, int G, int swz) {
    uint4* p0 = reinterpret_cast<uint4*>(row + 16 * ((2 * G) ^ swz));
    uint4* p1 = reinterpret_cast<uint4*>(row + 16 * ((2 * G + 1) ^ swz));
    uint4 av[2] = {*p0, *p1};  // columns 16G .. 16G+7, 16G+8 .. 16G+15
    uint4 f03, f47;
    act_pairs16<0>(av, f03, f47);
    *p0 = f03;
    *p1 = f47;
}

// PAIRED: A already holds the pairs (pair_activations_kernel), so the
// in-place pairing of every K-step is skipped.
// The in-place pairing of prep_group, once per call for the whole of A:
// thread e pairs 16-column group e % (K / 16) of row e / (K / 16) (K % 16
// == 0, A and out 16-byte aligned).
__global__ __launch_bounds__(256) void pair_activations_kernel(const uint16_t* __restrict__ A, int64_t M, int64_t K,
                                                               uint16_t* __restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= M * (K / 16)) return;
    const uint4* src = reinterpret_cast<const uint4*>(A) + 2 * e;
    uint4 av[2] = {src[0], src[1]};
    uint4 f03, f47;
    act_pairs16<0>(av, f03, f47);
    uint4* dst = reinterpret_cast<uint4*>(out) + 2 * e;
    dst[0] = f03;
    dst[1] = f47;
}

template <class T, int TM, bool PAIRED>
__global__ __launch_bounds__(kThreads) void tile_kernel(SplitArgs sa) {
    typedef typename Mfma<T>::vec vec;
    constexpr int BM = 16 * TM;
    constexpr int kABytes = a_bytes<TM>();
    constexpr int kStageBytes = stage_bytes<TM>();
    constexpr int R = slots<TM>();
    constexpr int P = TM + 2;  // DMAs per wave per K-step
    const GemmArgs& p = sa.g;
    extern __shared__ uint4 smem_mm3[];
    uint8_t* lds = reinterpret_cast<uint8_t*>(smem_mm3);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem_mm3;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int z = blockIdx.z;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t rb = K / 4;
    const int nk = (int)(K / BK);
    const int ks0 = (int)((int64_t)nk * z / sa.S);
    const int ks1 = (int)((int64_t)nk * (z + 1) / sa.S);  // > ks0: S <= nk
    const uint32_t magic_v = vgpr_const<kMagic2>();

    // byte offsets of each lane's rows from the tile's first activation row
    // and first weight row
    const uint16_t* a_blk = p.A + m0 * K;
    uint32_t a_dma[TM];
#pragma unroll
    for (int u = 0; u < TM; ++u) {
        const int r = 2 * (wave * TM + u) + (lane >> 5);
        const int64_t m = m0 + r < M ? r : M - 1 - m0;
        a_dma[u] = (uint32_t)(2 * (m * K + 8 * ((lane & 31) ^ (r & 15))));
    }
    const uint8_t* b_blk = static_cast<const uint8_t*>(p.wq) + n0 * rb;
    uint32_t b_dma[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int r = 16 * (2 * wave + u) + (lane >> 2);
        const int64_t n = n0 + r < N ? r : N - 1 - n0;
        b_dma[u] = (uint32_t)(n * rb + 16 * ((lane & 3) ^ ((r >> 2) & 3)));
    }
    auto issue = [&](int kstep, int slot) {
        const uint32_t st = lds_base + (uint32_t)(slot * kStageBytes);
#pragma unroll
        for (int u = 0; u < TM; ++u) dma16s(a_blk + (int64_t)kstep * BK, a_dma[u], st + 1024u * (wave * TM + u));
#pragma unroll
        for (int u = 0; u < 2; ++u)
            dma16s(b_blk + (int64_t)kstep * (BK / 4), b_dma[u], st + kABytes + 1024u * (2 * wave + u));
    };
    auto clamp_step = [&](int k) { return k < ks1 ? k : ks1 - 1; };

    // pairing units of this thread: row tid/16 + 32q, group tid%16
    auto prep = [&](int slot) {
#pragma unroll
        for (int q = 0; q < TM / 2; ++q) {
            const int r = (tid >> 4) + 32 * q;
            prep_group(lds + slot * kStageBytes + r * 512, tid & 15, r & 15);
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    int b_off[TN], b_swz[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int row = 32 * wave + 16 * j + i16;
        b_off[j] = kABytes + row * 64 + 4 * g;
        b_swz[j] = (row >> 2) & 3;
    }

    // prologue: steps 0 .. R-2 in flight, step 0 prepped, step 1 landed
#pragma unroll
    for (int u = 0; u < R - 1; ++u) issue(clamp_step(ks0 + u), u);
    if constexpr (R == 4) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * P) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(P) : "memory");
    stage_barrier();
    if constexpr (!PAIRED) prep(0);
    if constexpr (R == 4) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(P) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    stage_barrier();
    for (int kt = ks0; kt < ks1; ++kt) {
        const int it = kt - ks0;
        // Unconditional so the per-wave counts stay exact: past the end the DMA
        // re-reads the last K-step into a slot nobody reads any more.
        issue(clamp_step(kt + R - 1), (it + R - 1) % R);
        if constexpr (!PAIRED) {
            if (kt + 1 < ks1) prep((it + 1) % R);
        }
        const uint8_t* sbase = lds + (it % R) * kStageBytes;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t x[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) x[j] = *reinterpret_cast<const uint32_t*>(sbase + b_off[j] + 16 * (u ^ b_swz[j]));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q = 2 * (4 * u + g) + h;
                vec af[TM];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[i] = __builtin_bit_cast(vec, *reinterpret_cast<const uint4*>(sbase + (16 * i + i16) * 512 +
                                                                                   16 * (q ^ i16)));
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const uint4 bw = h == 0 ? tern_quad<0>(x[j], magic_v) : tern_quad<4>(x[j], magic_v);
                    const vec bf = __builtin_bit_cast(vec, bw);
#pragma unroll
                    for (int i = 0; i < TM; ++i) acc[i][j] = Mfma<T>::mma(af[i], bf, acc[i][j]);
                }
            }
        }
        // the DMA of step kt + 2 has landed (only steps kt + 3 .. may remain)
        if constexpr (R == 4) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(P) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        stage_barrier();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const bool final_out = sa.S == 1;
    float sc[TN], bi[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + 32 * wave + 16 * j + i16;
        const int64_t nc = n < N ? n : N - 1;
        sc[j] = f16_bits_to_f32(p.scale[nc]);
        bi[j] = p.bias ? T::to_f32(p.bias[nc]) : 0.0f;
    }
    float* wsz = final_out ? nullptr : sa.ws + (int64_t)z * M * N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * i + 4 * g + r;
            const int64_t m = m0 + row;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t n = n0 + 32 * wave + 16 * j + i16;
                if (n >= N) continue;
                const float v = acc[i][j][r] * Mfma<T>::kUnit;
                if (final_out) p.C[m * N + n] = T::from_f32_fast(v * sc[j] + bi[j]);
                else wsz[m * N + n] = v;
            }
        }
    }
}

}  // namespace mm3


// ------------------------------------------------------------------------
// W4A16 at large M (prefill): the DMA ring of v3 with int4 codes.
//
// C[m, n] = sum_g s[n, g] * sum_{k in g} A[m, k] (q[n, k] - z[n, g]) (+ bias)
// (page "Model quantization - vLLM runtime quantization architecture",
// section 5: INT4 weights, fp16 group scales of 128 columns, and a GEMM
// kernel consuming them; page "10.6 Quantization choice ...", section
// 10.6.1: prefill is the compute-bound GEMM regime).
//
// Block tile 256 x 128, K-step 64 (half a group), eight waves (2 x 4) of
// 128 x 32 outputs (8 x 2 tiles of v_mfma_f32_16x16x32).  Per stage the ring
// holds 256 activation rows x 64 columns (natural order, 16-byte chunks
// XOR-swizzled as in v3) and 128 weight rows x 32 bytes of codes (8 words).
// A code word holds 8 consecutive columns, one MFMA operand: byte d of the
// word is moved to both halves of a dword (v_perm), its two nibbles masked
// into the mantissa of 1024 (1024 + q, 1024 + 16 q), and one packed fma by
// (1, 1/16) with -(1024 + z, 64 + z) leaves (q_2d - z, q_2d+1 - z) exactly -
// natural order, so the activations need no pairing.  bf16 activations take
// the same exact integers converted to bf16.  The MFMAs of a group run into
// group accumulators whose first MFMA takes zero as its accumulator input
// (no reset instructions; the loop walks a whole group, two K-steps, per
// iteration); at the group's end each is scaled by s[n, g] (fp32) into the
// output accumulators, so every product is exact and the scale is applied
// once per group, as the format defines.
// The block's scales (and zero points) are copied to LDS once, before the
// K loop, so the loop's only global traffic is the DMA whose per-wave counts
// the stage waits rely on; that bounds K at 128 groups (16384 columns).
namespace w4p {

constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kThreads = 512;
constexpr int kStages = 3;
constexpr int kBBytes = BN * BK / 2;        // 4 KB: 128 rows x 32 bytes
constexpr int kMaxGroups = 128;             // groups per split (scales held in LDS)

// Block tile BM x 128: BM = 256 (eight waves of 128 x 32) for prefill,
// BM = 64 (eight waves of 64 x 16) for 17 <= M < 256, where a 256-row tile
// would mostly multiply padding.
template <int BM>
struct Tile {
    static constexpr int WM = BM == 256 ? 128 : 64;
    static constexpr int WN = BM == 256 ? 32 : 16;
    static constexpr int kWaveCols = BN / WN;
    static constexpr int TM = WM / 16, TN = WN / 16;
    static constexpr int AU = BM / 64;                  // 1-KB activation DMA blocks per wave and stage
    static constexpr int kABytes = BM * BK * 2;
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr int kRingBytes = kStages * kStageBytes;
    static constexpr int kEpiLd = WN + 8;               // epilogue staging row (halves)
    static constexpr int kEpiBytesPerWave = 32 * kEpiLd * 2;
    static_assert((BM / WM) * kWaveCols == 8, "eight waves");
    static_assert(8 * kEpiBytesPerWave <= kRingBytes, "epilogue staging must fit in the ring");
};

template <int BM>
__host__ __device__ constexpr size_t lds_bytes(int64_t groups, bool asym) {
    return (size_t)Tile<BM>::kRingBytes + (size_t)BN * groups * 2 + (asym ? (size_t)BN * groups : 0);
}

// (q_2d - z, q_2d+1 - z) of code word x as exact fp16, natural order.
template <int D>
__device__ __forceinline__ uint32_t nat_w4_pair(uint32_t x, uint32_t mask_v, uint32_t magic_v, f16x2 mul, f16x2 add) {
    const uint32_t y = __builtin_amdgcn_perm(x, x, 0x0C000C00u | (uint32_t)D | ((uint32_t)D << 16));
    const f16x2 v = __builtin_bit_cast(f16x2, (y & mask_v) | magic_v);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v, mul, add));
}

template <class T>
__device__ __forceinline__ uint4 nat_w4_quad(uint32_t x, uint32_t mask_v, uint32_t magic_v, f16x2 mul, f16x2 add) {
    const uint4 h = make_uint4(nat_w4_pair<0>(x, mask_v, magic_v, mul, add), nat_w4_pair<1>(x, mask_v, magic_v, mul, add),
                               nat_w4_pair<2>(x, mask_v, magic_v, mul, add), nat_w4_pair<3>(x, mask_v, magic_v, mul, add));
    if constexpr (std::is_same<T, F16>::value) return h;
    else return make_uint4(f16x2_to_bf16x2(h.x), f16x2_to_bf16x2(h.y), f16x2_to_bf16x2(h.z), f16x2_to_bf16x2(h.w));
}

// -(1024 + z) in the low half, -(64 + z) in the high half
__device__ __forceinline__ f16x2 w4_nat_sub(uint32_t z) {
    return __builtin_bit_cast(f16x2, (0xE400u + z) | ((0xD400u + 16u * z) << 16));
}

// Split z of S (gridDim.z) covers groups [z G / S, (z + 1) G / S) and, when
// S > 1, stores fp32 partials (scales applied, no bias) for
// launch_splitk_reduce; the host keeps every split within kMaxGroups.
template <class T, bool ASYM, int BM>
__global__ __launch_bounds__(kThreads) void gemm_kernel(SplitArgs sa) {
    typedef typename Mfma<T>::vec vec;
    typedef Tile<BM> TL;
    constexpr int WM = TL::WM, WN = TL::WN, TM = TL::TM, TN = TL::TN, AU = TL::AU;
    constexpr int kABytes = TL::kABytes, kStageBytes = TL::kStageBytes, kRingBytes = TL::kRingBytes;
    constexpr int kEpiLd = TL::kEpiLd, kEpiBytesPerWave = TL::kEpiBytesPerWave;
    const GemmArgs& p = sa.g;
    extern __shared__ uint4 smem_w4p[];
    uint8_t* lds = reinterpret_cast<uint8_t*>(smem_w4p);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem_w4p;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / TL::kWaveCols, wn = wave % TL::kWaveCols;
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int G = (int)(K / 128);
    const int z = blockIdx.z;
    const int g_lo = (int)((int64_t)G * z / sa.S);
    const int Gs = (int)((int64_t)G * (z + 1) / sa.S) - g_lo;  // groups of this split, 1 .. kMaxGroups
    const int64_t rowb = K / 2;  // code bytes per weight row
    uint16_t* sc_lds = reinterpret_cast<uint16_t*>(lds + kRingBytes);   // [BN][Gs]
    uint8_t* zp_lds = lds + kRingBytes + (size_t)BN * Gs * 2;            // [BN][Gs]

    // the block's group scales (and zero points) of this split -> LDS; rows
    // past N re-read row N-1
    for (int e = tid; e < BN * Gs; e += kThreads) {
        const int r = e / Gs, gl = e - r * Gs;
        const int64_t n = n0 + r < N ? n0 + r : N - 1;
        sc_lds[e] = p.scale[n * G + g_lo + gl];
        if constexpr (ASYM) zp_lds[e] = p.zeros[n * G + g_lo + gl];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Activation DMA: as v3, wave w fills 1-KB blocks AU w .. AU w + AU-1 of a
    // stage (8 rows each), lane l at chunk l % 8 of row l / 8, fetching global
    // chunk (l % 8) ^ (l / 8).  Rows past M re-read row M-1.
    const uint16_t* a_blk = p.A + m0 * K;
    uint32_t a_off[AU];
#pragma unroll
    for (int u = 0; u < AU; ++u) {
        int64_t r = 8 * (AU * wave + u) + (lane >> 3);
        if (m0 + r >= M) r = M - 1 - m0;
        a_off[u] = (uint32_t)(2 * (r * K + 8 * ((lane & 7) ^ (lane >> 3))));  // bytes
    }
    // Code DMA (waves 0..3, 256 lanes): lane L = 64 w + l fetches bytes
    // 16 (L % 2) .. +15 of the K-step's 32 bytes of weight row n0 + L / 2,
    // landing at 32 (L / 2) + 16 (L % 2).  Rows past N re-read row N-1.
    const uint8_t* b_blk = static_cast<const uint8_t*>(p.wq) + n0 * rowb;
    const bool b_issuer = wave < 4;
    uint32_t b_off;
    {
        const int L = 64 * (wave & 3) + lane;
        const int64_t n = n0 + (L >> 1) < N ? (L >> 1) : N - 1 - n0;
        b_off = (uint32_t)(n * rowb + 16 * (L & 1));
    }
    auto issue = [&](int kstep, int stage) {
        const int64_t k0 = (int64_t)kstep * BK;
        const uint32_t dst = lds_base + (uint32_t)(stage * kStageBytes + 1024 * AU * wave);
#pragma unroll
        for (int u = 0; u < AU; ++u) dma16s(a_blk + k0, a_off[u], dst + 1024u * u);
        if (b_issuer) dma16s(b_blk + k0 / 2, b_off, lds_base + (uint32_t)(stage * kStageBytes + kABytes + 1024 * wave));
    };
    auto wait_prev_stage = [&]() {
        if (b_issuer) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(AU + 1) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(AU) : "memory");
    };

    f32x4 acc[TM][TN], accg[TM][TN];  // accg: each group's first MFMA starts from zero
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int frag_base = (wm * WM + i16) * (BK * 2);
    const int swz = i16 & 7;
    int nloc[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) nloc[j] = wn * WN + 16 * j + i16;
    const uint32_t magic_v = vgpr_const<kMagic2>();
    const uint32_t mask_v = sgpr_const<0x00F0000Fu>();
    const f16x2 mul = __builtin_bit_cast(f16x2, 0x2C003C00u);  // (1, 1/16)
    f16x2 add[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) add[j] = w4_nat_sub(8u);

    const int kb = 2 * g_lo, nk = 2 * Gs;  // this split's K-steps kb .. kb + nk - 1 (nk >= 2)
    issue(kb, 0);
    issue(kb + 1, 1);
    wait_prev_stage();
    __syncthreads();  // the scales in LDS and stage 0, for every wave
    const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < nk; kt += 2) {  // local group gl = kt / 2: K-steps kt and kt + 1
        const int gl = kt >> 1;
        if constexpr (ASYM) {
#pragma unroll
            for (int j = 0; j < TN; ++j) add[j] = w4_nat_sub(zp_lds[nloc[j] * Gs + gl]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = kt + h;
            const int stage = k % kStages;
            issue(kb + (k + 2 < nk ? k + 2 : nk - 1), (k + 2) % kStages);
            const uint8_t* sbase = lds + stage * kStageBytes;
            uint2 bw[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) bw[j] = *reinterpret_cast<const uint2*>(sbase + kABytes + nloc[j] * 32 + 8 * g);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int chunk = (2 * g + s) ^ swz;
                vec af[TM];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[i] = __builtin_bit_cast(vec, *reinterpret_cast<const uint4*>(sbase + frag_base + i * 16 * (BK * 2) + 16 * chunk));
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const vec bf = __builtin_bit_cast(vec, nat_w4_quad<T>(s ? bw[j].y : bw[j].x, mask_v, magic_v, mul, add[j]));
                    // the group's first MFMA starts from zero (an inline operand, no reset)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        accg[i][j] = Mfma<T>::mma(af[i], bf, h == 0 && s == 0 ? zero4 : accg[i][j]);
                }
            }
            if (h == 1) {  // end of group gi: scale into the outputs
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const float sc = f16_bits_to_f32(sc_lds[nloc[j] * Gs + gl]);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc, accg[i][j][r], acc[i][j][r]);
                }
            }
            wait_prev_stage();  // stage k + 1 has landed
            stage_barrier();    // ... for every wave, and nobody reads stage k any more
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();        // the ring is idle from here on

    if (sa.S > 1) {  // fp32 partial of this split: 16 lanes store 64 contiguous bytes per row
        float* ws = sa.ws + (int64_t)z * M * N;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * WM + 16 * i + 4 * g + r;
                if (m >= M) continue;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int64_t n = n0 + nloc[j];
                    if (n < N) ws[m * N + n] = acc[i][j][r];
                }
            }
        return;
    }

    // epilogue: per wave, slabs of 32 rows x WN columns through a private LDS area
    uint16_t* stg = reinterpret_cast<uint16_t*>(lds + wave * kEpiBytesPerWave);
    float bi[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + nloc[j];
        bi[j] = p.bias ? T::to_f32(p.bias[n < N ? n : N - 1]) : 0.0f;
    }
    const bool vec_ok = (N % 8) == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15u) == 0;
#pragma unroll
    for (int slab = 0; slab < TM / 2; ++slab) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * slab + ii;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * ii + 4 * g + r;
#pragma unroll
                for (int j = 0; j < TN; ++j) stg[row * kEpiLd + 16 * j + i16] = T::from_f32_fast(acc[i][j][r] + bi[j]);
            }
        }
        // each lane stores 16 contiguous bytes: WN / 8 lanes per row
        constexpr int kLanesPerRow = WN / 8, kRowsPerPass = 64 / kLanesPerRow;
#pragma unroll
        for (int q = 0; q < 32 / kRowsPerPass; ++q) {
            const int row = lane / kLanesPerRow + kRowsPerPass * q;
            const int col = 8 * (lane % kLanesPerRow);
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

}  // namespace w4p

}  // namespace

hipError_t launch_splitk_reduce(const SplitArgs& sa, hipStream_t s) {
    const GemmArgs& a = sa.g;
    const dim3 grid((unsigned)((a.N + 255) / 256), mm::reduce_rows(a.M));
    if (a.bf16) mm::splitk_reduce_kernel<BF16><<<grid, 256, 0, s>>>(sa);
    else mm::splitk_reduce_kernel<F16><<<grid, 256, 0, s>>>(sa);
    return hipGetLastError();
}

template <class T, int BM>
static hipError_t launch_v3(const SplitArgs& sa, hipStream_t s) {
    typedef v3::Tile<BM> G;
    static DeviceFlags lds_limit_set;
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&v3::gemm_kernel<T, BM>), (int)G::kLdsBytes, lds_limit_set);
    if (e != hipSuccess) return e;
    const GemmArgs& a = sa.g;
    const dim3 grid((unsigned)((a.N + v3::BN - 1) / v3::BN), (unsigned)((a.M + BM - 1) / BM), (unsigned)sa.S);
    SplitArgs k = sa;
    k.flags = split_flags(sa.flags, sa.S, (int64_t)grid.x * grid.y);
    v3::gemm_kernel<T, BM><<<grid, v3::kThreads, G::kLdsBytes, s>>>(k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (sa.S > 1 && !k.flags) e = launch_splitk_reduce(sa, s);
    return e;
}

// One pass over K whose 256 x 256 tiles leave the last round of workgroups
// partly filled: the first n1 columns of 256-row tiles make whole rounds,
// and the other columns run as 128 x 256 tiles in a second launch, which
// writes its own columns of C (row stride N).  Returns the column split n1
// (a multiple of 256), or 0 when the grid already fills whole rounds, the
// remainder is more than half a round, or the shape is too small.
int64_t gemm_tail_split(int64_t M, int64_t N, int compute_units) {
    const int64_t cus = compute_units > 0 ? compute_units : 1;
    const int64_t mt = (M + 255) / 256, nt = (N + v3::BN - 1) / v3::BN;
    const int64_t tiles = mt * nt;
    const int64_t full = tiles / cus * cus;
    if (tiles <= cus || tiles == full || (tiles - full) * 2 > cus) return 0;
    const int64_t n1 = full / mt;  // whole columns of tiles within the full rounds
    if (n1 <= 0 || n1 >= nt) return 0;
    return n1 * v3::BN;
}

template <class T>
static hipError_t launch_v3_auto(const SplitArgs& sa, int compute_units, hipStream_t s) {
    const GemmArgs& a = sa.g;
    const int64_t n1 = sa.S == 1 ? gemm_tail_split(a.M, a.N, compute_units) : 0;
    if (n1 == 0) return launch_v3<T, 256>(sa, s);
    SplitArgs head = sa, tail = sa;
    head.g.N = n1;
    head.ldc = a.N;
    tail.g.N = a.N - n1;
    tail.ldc = a.N;
    tail.g.wq = static_cast<const uint8_t*>(a.wq) + n1 * (a.K / 4);
    tail.g.scale = a.scale + n1;
    tail.g.bias = a.bias ? a.bias + n1 : nullptr;
    tail.g.C = a.C + n1;
    hipError_t e = launch_v3<T, 256>(head, s);
    if (e != hipSuccess) return e;
    return launch_v3<T, 128>(tail, s);
}

// K split of the large-M kernel.  One 256 x 256 workgroup fills a compute
// unit (the LDS ring takes 108 KB), so a grid of T tiles runs in
// ceil(T / CUs) rounds of nk K-steps each.  When T leaves compute units idle,
// S splits shorten each round to ceil(nk / S) K-steps at the price of
// writing S * M * N fp32 partials and re-reading them (by the last split of
// each tile, or a second launch without arrival counters; charged 3 us
// either way).  The split count minimises that estimate, with one K-step
// taken as 1.5 us (a 256 x 256 x 64 step at about 1 PFLOP/s over the whole
// chip) and the partials moving at 4 TB/s; each split keeps at least 16
// K-steps.
int gemm_splits(int64_t M, int64_t N, int64_t K, int compute_units) {
    const int64_t tiles = ((N + v3::BN - 1) / v3::BN) * ((M + v3::Tile<256>::BM - 1) / v3::Tile<256>::BM);
    const int64_t nk = K / v3::BK;
    const int64_t cus = compute_units > 0 ? compute_units : 1;
    const double step_us = 1.5, partial_bytes_per_us = 4.0e6, launch_us = 3.0;
    int best = 1;
    double best_us = (double)((tiles + cus - 1) / cus) * (double)nk * step_us;
    for (int S = 2; S <= 8 && nk / S >= 16; ++S) {
        const double us = (double)((tiles * S + cus - 1) / cus) * (double)((nk + S - 1) / S) * step_us +
                          2.0 * S * (double)M * (double)N * 4.0 / partial_bytes_per_us + launch_us;
        if (us < best_us) { best_us = us; best = S; }
    }
    return best;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int compute_units) {
    const int S = gemm_splits(M, N, K, compute_units);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// Large M with an optional workspace: the split count of gemm_splits when
// `workspace` holds gemm_workspace_bytes(), a single pass over K otherwise.
hipError_t launch_ternary_gemm(const GemmArgs& a, void* workspace, size_t workspace_bytes, int compute_units,
                               hipStream_t s, uint32_t* flags) {
    // the C ABI guarantees K % 64 == 0 (whole 16-byte code chunks per row)
    SplitArgs sa{a, static_cast<float*>(workspace), gemm_splits(a.M, a.N, a.K, compute_units)};
    sa.flags = flags;
    if (sa.S > 1 && (!workspace || workspace_bytes < gemm_workspace_bytes(a.M, a.N, a.K, compute_units))) sa.S = 1;
    return a.bf16 ? launch_v3_auto<BF16>(sa, compute_units, s) : launch_v3_auto<F16>(sa, compute_units, s);
}

// Split count of the medium-M kernels.
//  K % 256 == 0 (mm3): one workgroup fills a compute unit (the ring takes
//  96 or 144 KB of LDS), so the split count is the largest that keeps the
//  T tiles x S splits within one round on the compute units (at most 16,
//  each split keeping two K-steps); measured on the Llama-3-70B shapes at
//  M = 17 .. 64 this beat both fewer splits (longer K loops) and more (a
//  second round), the fp32 partials costing little in comparison.
//  Otherwise (mm): none when the row x column tiles already cover three
//  quarters of the compute units, else enough splits to give every compute
//  unit a workgroup, each split keeping >= 8 K-steps.
int medium_m_splits(int64_t M, int64_t N, int64_t K, int compute_units) {
    const int64_t tm = M <= 32 ? 2 : 4;
    const int64_t tiles = ((N + mm::BN - 1) / mm::BN) * ((M + 16 * tm - 1) / (16 * tm));
    const int64_t cus = compute_units > 0 ? compute_units : 1;
    if (K % mm3::BK == 0) {
        int64_t S = cus / tiles;
        const int64_t nk = K / mm3::BK;
        if (S > 16) S = 16;
        if (S > nk / 2) S = nk / 2;
        return S < 1 ? 1 : (int)S;
    }
    if (4 * tiles >= 3 * cus) return 1;
    int64_t S = (cus + tiles - 1) / tiles;
    const int64_t smax = (K / mm::BK) / 8;
    if (S > smax) S = smax;
    return S < 1 ? 1 : (int)S;
}

// With a workspace, large shapes pair the activations once per call
// (pair_activations_kernel, into the workspace after the split partials)
// instead of in every workgroup's K-steps: the pairing costs each of the
// (N / 256) x (K / 256) workgroup K-steps about a microsecond per thousand,
// the extra launch about 2.5 us, so it pays from N K ~ 2e8 (Llama-3-70B
// gate_up and down, not qkv and o).
constexpr int64_t kMediumPairMinNK = int64_t(200) << 20;

static bool medium_paired(int64_t N, int64_t K) { return K % mm3::BK == 0 && N * K >= kMediumPairMinNK; }

static size_t medium_partial_bytes(int64_t M, int64_t N, int64_t K, int compute_units) {
    const int S = medium_m_splits(M, N, K, compute_units);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

size_t medium_m_workspace_bytes(int64_t M, int64_t N, int64_t K, int compute_units) {
    const size_t part = medium_partial_bytes(M, N, K, compute_units);
    if (!medium_paired(N, K)) return part;
    return ((part + 255) & ~size_t(255)) + (size_t)M * (size_t)K * 2;
}

template <class T, int TM>
static hipError_t launch_mm(const SplitArgs& sa, hipStream_t s) {
    static DeviceFlags lds_limit_set;
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&mm::tile_kernel<T, TM>), (int)mm::lds_bytes<TM>(),
                                   lds_limit_set);
    if (e != hipSuccess) return e;
    const GemmArgs& a = sa.g;
    const dim3 grid((unsigned)((a.N + mm::BN - 1) / mm::BN), (unsigned)((a.M + 16 * TM - 1) / (16 * TM)), (unsigned)sa.S);
    mm::tile_kernel<T, TM><<<grid, mm::kThreads, mm::lds_bytes<TM>(), s>>>(sa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (sa.S > 1) e = launch_splitk_reduce(sa, s);
    return e;
}

template <class T, int TM, bool PAIRED>
static hipError_t launch_mm3(const SplitArgs& sa, hipStream_t s) {
    static DeviceFlags lds_limit_set;
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&mm3::tile_kernel<T, TM, PAIRED>),
                                   (int)mm3::lds_bytes<TM>(), lds_limit_set);
    if (e != hipSuccess) return e;
    const GemmArgs& a = sa.g;
    if (sa.S < 1 || sa.S > a.K / mm3::BK) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((a.N + mm3::BN - 1) / mm3::BN), (unsigned)((a.M + 16 * TM - 1) / (16 * TM)), (unsigned)sa.S);
    mm3::tile_kernel<T, TM, PAIRED><<<grid, mm3::kThreads, mm3::lds_bytes<TM>(), s>>>(sa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (sa.S > 1) e = launch_splitk_reduce(sa, s);
    return e;
}

// Medium M with an optional workspace: S splits when `workspace` holds
// medium_m_workspace_bytes(), a single pass over K otherwise.
hipError_t launch_ternary_medium(const GemmArgs& a, void* workspace, size_t workspace_bytes, int compute_units,
                                 hipStream_t s) {
    SplitArgs sa{a, static_cast<float*>(workspace), medium_m_splits(a.M, a.N, a.K, compute_units)};
    const size_t part = medium_partial_bytes(a.M, a.N, a.K, compute_units);
    const bool paired = medium_paired(a.N, a.K) && workspace &&
                        workspace_bytes >= medium_m_workspace_bytes(a.M, a.N, a.K, compute_units);
    if (sa.S > 1 && (!workspace || workspace_bytes < part)) sa.S = 1;
    if (paired) {
        uint16_t* pa = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + ((part + 255) & ~size_t(255)));
        const int64_t n = a.M * (a.K / 16);
        mm3::pair_activations_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a.A, a.M, a.K, pa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        sa.g.A = pa;
    }
    return launch_ternary_medium_split(sa, paired, s);
}

hipError_t launch_ternary_medium_split(const SplitArgs& sa, bool paired, hipStream_t s) {
    const GemmArgs& a = sa.g;
    const bool small = a.M <= 32;
    if (a.K % mm3::BK == 0) {
        if (paired) {
            if (a.bf16) return small ? launch_mm3<BF16, 2, true>(sa, s) : launch_mm3<BF16, 4, true>(sa, s);
            return small ? launch_mm3<F16, 2, true>(sa, s) : launch_mm3<F16, 4, true>(sa, s);
        }
        if (a.bf16) return small ? launch_mm3<BF16, 2, false>(sa, s) : launch_mm3<BF16, 4, false>(sa, s);
        return small ? launch_mm3<F16, 2, false>(sa, s) : launch_mm3<F16, 4, false>(sa, s);
    }
    if (a.bf16) return small ? launch_mm<BF16, 2>(sa, s) : launch_mm<BF16, 4>(sa, s);
    return small ? launch_mm<F16, 2>(sa, s) : launch_mm<F16, 4>(sa, s);
}

// W4A16 GEMM plan: the 256-row tile from M = 256, the 64-row tile below;
// K split S ways (fp32 partials, launch_splitk_reduce) while the tiles leave
// compute units idle (at most 16 splits, at least one group each), and at
// least enough splits that none holds more than kMaxGroups groups' scales.
static int w4_gemm_bm(int64_t M) { return M >= 256 ? 256 : 64; }

static int w4_gemm_min_splits(int64_t K) {
    const int64_t G = K / 128;
    return (int)((G + w4p::kMaxGroups - 1) / w4p::kMaxGroups);
}

int w4_gemm_splits(int64_t M, int64_t N, int64_t K, int compute_units) {
    const int64_t G = K / 128;
    const int bm = w4_gemm_bm(M);
    const int64_t tiles = ((N + w4p::BN - 1) / w4p::BN) * ((M + bm - 1) / bm);
    const int64_t cus = compute_units > 0 ? compute_units : 1;
    int64_t S = cus / tiles;
    if (S > 16) S = 16;
    if (S > G) S = G;
    const int smin = w4_gemm_min_splits(K);
    if (S < smin) S = smin;
    return S < 1 ? 1 : (int)S;
}

size_t w4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int compute_units) {
    const int S = w4_gemm_splits(M, N, K, compute_units);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

bool w4_prefill_ok(const GemmArgs& a, size_t workspace_bytes) {
    if (a.K % 128 != 0 || a.K < 128) return false;
    const int smin = w4_gemm_min_splits(a.K);
    return smin == 1 || (smin <= 16 && smin <= a.K / 128 &&
                         workspace_bytes >= (size_t)smin * (size_t)a.M * (size_t)a.N * sizeof(float));
}

template <class T, bool ASYM, int BM>
static hipError_t launch_w4p(const SplitArgs& sa, hipStream_t s) {
    static DeviceFlags lds_limit_set;
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&w4p::gemm_kernel<T, ASYM, BM>),
                                   (int)w4p::lds_bytes<BM>(w4p::kMaxGroups, ASYM), lds_limit_set);
    if (e != hipSuccess) return e;
    const GemmArgs& a = sa.g;
    const int64_t G = a.K / 128;
    if (a.K % 128 != 0 || sa.S < 1 || sa.S > G || (G + sa.S - 1) / sa.S > w4p::kMaxGroups) return hipErrorInvalidValue;
    const int64_t gs_max = (G + sa.S - 1) / sa.S;
    const dim3 grid((unsigned)((a.N + w4p::BN - 1) / w4p::BN), (unsigned)((a.M + BM - 1) / BM), (unsigned)sa.S);
    w4p::gemm_kernel<T, ASYM, BM><<<grid, w4p::kThreads, w4p::lds_bytes<BM>(gs_max, ASYM), s>>>(sa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return sa.S > 1 ? launch_splitk_reduce(sa, s) : hipSuccess;
}

template <int BM>
static hipError_t launch_w4p_bm(const SplitArgs& sa, hipStream_t s) {
    if (sa.g.zeros) return sa.g.bf16 ? launch_w4p<BF16, true, BM>(sa, s) : launch_w4p<F16, true, BM>(sa, s);
    return sa.g.bf16 ? launch_w4p<BF16, false, BM>(sa, s) : launch_w4p<F16, false, BM>(sa, s);
}

hipError_t launch_w4_prefill(const GemmArgs& a, void* workspace, size_t workspace_bytes, hipStream_t s) {
    if (!w4_prefill_ok(a, workspace ? workspace_bytes : 0)) return hipErrorInvalidValue;
    SplitArgs sa{a, static_cast<float*>(workspace), w4_gemm_splits(a.M, a.N, a.K, compute_units()), 1};
    const size_t need = (size_t)sa.S * (size_t)a.M * (size_t)a.N * sizeof(float);
    if (sa.S > 1 && (!workspace || workspace_bytes < need)) sa.S = w4_gemm_min_splits(a.K);  // fits: w4_prefill_ok
    return w4_gemm_bm(a.M) == 256 ? launch_w4p_bm<256>(sa, s) : launch_w4p_bm<64>(sa, s);
}

// W4A16 at large M where the prefill kernel does not take the shape (more
// than 128 groups): the small-M kernels on successive blocks of 16
// activation rows (weights are re-read once per block).
hipError_t launch_w4_gemm(const GemmArgs& a, void* workspace, size_t workspace_bytes, hipStream_t s,
                          uint32_t* flags) {
    for (int64_t m = 0; m < a.M; m += kGemvMaxM) {
        GemmArgs b = a;
        b.A = a.A + m * a.K;
        b.C = a.C + m * a.N;
        b.M = (a.M - m) < kGemvMaxM ? (a.M - m) : kGemvMaxM;
        // the blocks run in stream order, so they may share one workspace
        // (each leaves the arrival counters zero for the next)
        hipError_t e = launch_w4_gemv(b, workspace, workspace_bytes, s, flags);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tq
