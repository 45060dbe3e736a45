// Small-M (decode, M <= 16) kernels: every packed weight byte is read from
// HBM exactly once per call and unpacked in registers; activations (a few KB
// to a few hundred KB) come from the L2 cache.  The matrix-core kernels give
// each wave a fixed share of K for 16-row blocks of weights and sum the wave
// partials in LDS in a fixed order; the streaming kernels may also split K
// across workgroups (with a caller workspace), and a second kernel then sums
// the partials in a fixed order.  No atomics: results are deterministic for
// a given shape, path and workspace size.  Dispatch: the small-M kernels for
// M <= 2 (ternary; M <= 4 where the grid has few waves per SIMD, and always
// for bf16) and M <= 4 (W4A16), the streaming kernels above that (fp16),
// the per-lane FMA kernels for the shapes the others cannot take.
//
// Ternary layer arithmetic (page "Ternary quantized models in vLLM ...",
// section 4): value = code - 1, out = sum_k a_k * value_k, then the row
// scale is applied once after accumulation (section 4.2), in fp32.
// W4A16 (page "Model quantization - vLLM runtime quantization architecture",
// section 5): value = q - 8 with a per-(row, 128-column group) fp16 scale.

#include <algorithm>
#include <type_traits>

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
            if (lane == 0) p.C[m * p.N + row] = T::from_f32_fast(v * s + b);
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
    const uint8_t* zrow = p.zeros ? p.zeros + row * (K / 128) : nullptr;
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

    for (int64_t c = lane; c < chunks; c += kWave) {
        const uint4 q = wrow[c];
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
        const float s = f16_bits_to_f32(srow[c >> 2]);
        const int zp = zrow ? (int)zrow[c >> 2] : 8;
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
                        const float v = (float)((int)((qw[d] >> (4 * e)) & 15u) - zp);
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
            if (lane == 0) p.C[m * p.N + row] = T::from_f32_fast(v + b);
        }
    }
}

// ------------------------------------------------ ternary, matrix cores
//
// fp16 activations, M <= 16, K % 256 == 0.  The multiply-accumulates run on
// v_mfma_f32_16x16x32_f16 with M padded to 16 rows, so every M up to 16
// costs the same; the VALU only unpacks codes, at two ops per pair of codes.
//
// Unpack: a code dword x holds fields f_0..f_15 (f_j at bits 2j, column j of
// its 16).  Masking one field of each 16-bit half into the mantissa of the
// fp16 constant 1024 (0x6400, unit in the last place 1) gives, in one
// v_and_or_b32, the pair P_i = (1024 + 4^s f_i, 1024 + 4^s f_{i+8}) with
// s = i for fields in bits 0..9 (i = 0..4); fields in bits 10..15 are shifted
// down by 10 first (s = i - 5).  One packed fp16 fma, P_i * 4^-s - (1024 /
// 4^s + 1), then gives the ternary values (t_i, t_{i+8}) = f - 1 exactly
// (tern_pair).  The activations are paired the same way, (a_i, a_{i+8}), and
// not scaled, so every product a_k t_k is exact and the fp32 sums hold only
// the terms of the result: the error of a row scales with its own
// sum_k |a_k t_k| however few codes are nonzero.
//
// Work split: a block owns 16R weight rows (R blocks of 16, one per MFMA
// column tile) and all of K; its W waves take every W-th 256-column
// chunk-set.  Lane l = 16g + i loads 16 bytes (64 codes) of row i of each
// row block, chunk 4cs + g, and the 64 activations of row m = i of that
// chunk; MFMA j of a chunk-set contracts code dword j/2, fields
// 4(j%2)..4(j%2)+3 and their partners.  Wave partials meet in LDS and are
// summed in a fixed order: deterministic, no atomics.

template <int R, int W>
__global__ __launch_bounds__(W * kWave) void ternary_gemv_mfma_kernel(GemmArgs p) {
    __shared__ f32x4 red[W][R][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int64_t N = p.N, K = p.K;
    const int M = (int)p.M;
    const int64_t rb = K / 4;
    const int CS = (int)(K / 256);
    const int64_t n_base = (int64_t)blockIdx.x * (16 * R);
    const uint8_t* codes = static_cast<const uint8_t*>(p.wq);
    const bool a_live = i16 < M;
    const uint16_t* a_row = p.A + (int64_t)(a_live ? i16 : 0) * K;

    const uint8_t* crow[R];
    bool rlive[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = n_base + 16 * r + i16;
        rlive[r] = n < N;
        crow[r] = codes + (rlive[r] ? n : 0) * rb;
    }

    f32x4 acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t magic_v = vgpr_const<kMagic2>();

    uint4 q[R], qn[R];
    int cs = wave;
    if (cs < CS) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            q[r] = rlive[r] ? *reinterpret_cast<const uint4*>(crow[r] + (int64_t)(4 * cs + g) * 16)
                            : make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
    }
    for (; cs < CS; cs += W) {
        const int chunk = 4 * cs + g;
        // prefetch the next chunk-set's codes
        const int csn = cs + W;
        if (csn < CS) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                qn[r] = rlive[r] ? *reinterpret_cast<const uint4*>(crow[r] + (int64_t)(4 * csn + g) * 16)
                                 : make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
        }
        uint4 av[8];
        if (a_live) {
            const uint4* ap = reinterpret_cast<const uint4*>(a_row + (int64_t)chunk * 64);
#pragma unroll
            for (int e = 0; e < 8; ++e) av[e] = ap[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) av[e] = make_uint4(0u, 0u, 0u, 0u);
        }
#define TQ_MFMA_J(D, I0)                                                                              \
    {                                                                                                 \
        const uint4 aw = make_uint4(act_pair<D, I0>(av), act_pair<D, I0 + 1>(av), act_pair<D, I0 + 2>(av), \
                                    act_pair<D, I0 + 3>(av));                                         \
        const f16x8 aop = __builtin_bit_cast(f16x8, aw);                                              \
        _Pragma("unroll") for (int r = 0; r < R; ++r) {                                               \
            const uint4 bw = tern_quad<I0>(dword_of(q[r], D), magic_v);                               \
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, __builtin_bit_cast(f16x8, bw), acc[r], 0, 0, 0); \
        }                                                                                             \
    }
        TQ_MFMA_J(0, 0)
        TQ_MFMA_J(0, 4)
        TQ_MFMA_J(1, 0)
        TQ_MFMA_J(1, 4)
        TQ_MFMA_J(2, 0)
        TQ_MFMA_J(2, 4)
        TQ_MFMA_J(3, 0)
        TQ_MFMA_J(3, 4)
#undef TQ_MFMA_J
        if (csn < CS) {
#pragma unroll
            for (int r = 0; r < R; ++r) q[r] = qn[r];
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    for (int e = threadIdx.x; e < R * kWave; e += W * kWave) {
        const int r = e / kWave;
        const int l = e % kWave;
        f32x4 s = red[0][r][l];
#pragma unroll
        for (int w = 1; w < W; ++w) s += red[w][r][l];
        const int64_t n = n_base + 16 * r + (l & 15);
        if (n >= N) continue;
        const float sc = f16_bits_to_f32(p.scale[n]);
        const float b = p.bias ? F16::to_f32(p.bias[n]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * (l >> 4) + i;
            if (m < M) p.C[(int64_t)m * N + n] = F16::from_f32_fast(s[i] * sc + b);
        }
    }
}

// Same arithmetic, latency-first schedule (fp16, M <= 4, M * K <= 28672).
//
// Block = W waves over 16R weight rows and all of K; wave w owns chunk-sets
// w*CSW .. w*CSW + CSW-1 (256 columns each) of every row.  Waves are
// independent until the final reduction: each pairs the activations of its
// own columns in a private LDS area, so no barrier sits between the code
// loads and the contraction.
// 1. Each lane loads the activations of its prep units first (16 columns of
//    one activation row per unit, M*CSW/4 units per lane), then the wave
//    issues all its code loads in the order step 3 consumes them.  Every
//    load is unconditional (addresses clamped, surplus results discarded):
//    the compiler keeps this issue order, and the in-order completion
//    counter lets each use wait only for the loads it needs - the pairing
//    waits for the activations only.  The epilogue's row scale and bias are
//    loaded here too.
// 2. While the codes are in flight the wave writes its paired activations
//    to its LDS area in MFMA operand order - dword
//    ((m * 4 CSW + chunk) * 32 + 8 d + i) = pair (d, i) of row m.
// 3. The wave contracts its chunk-sets as their codes land.  Lanes of
//    activation rows m >= M skip the LDS read (their output rows are never
//    stored).
// 4. Wave partials meet in LDS; after one barrier a fixed-order sum, then the
//    row scale and bias.

// LDS layout of the kernel below (byte offsets): per wave, paired
// activations [M][4 CSW chunks][128 bytes]; after the W wave areas, the wave
// partials [W][R][64 lanes][16 bytes].
struct GemvLds {
    int64_t wave_bytes, red, total;
    __host__ __device__ GemvLds(int64_t M, int csw, int W, int R) {
        wave_bytes = M * csw * 512;
        red = W * wave_bytes;
        total = red + (int64_t)W * R * 64 * 16;
    }
};
static inline size_t gemv_lds_bytes(int64_t M, int csw, int W, int R) { return (size_t)GemvLds(M, csw, W, R).total; }

template <int R, int CSW, int UPT>
__global__ __launch_bounds__(1024) void ternary_gemv_lds_kernel(GemmArgs p) {
    extern __shared__ uint4 smem[];
    uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int64_t N = p.N, K = p.K;
    const int M = (int)p.M;
    const int64_t rb = K / 4;
    const int CS = (int)(K / 256);
    const int64_t n_base = (int64_t)blockIdx.x * (16 * R);
    const uint8_t* codes = static_cast<const uint8_t*>(p.wq);
    const int cs0 = wave * CSW;
    const int cnt = CS - cs0 < CSW ? CS - cs0 : CSW;  // >= 1 for every wave of the launch
    const GemvLds L(M, CSW, W, R);
    uint32_t* aps = reinterpret_cast<uint32_t*>(lds + wave * L.wave_bytes);   // this wave's pairs
    f32x4* red = reinterpret_cast<f32x4*>(lds + L.red);                      // [W][R][64]

    // 1a. activation loads: unit u = lane + 64 j covers columns
    //     256 cs0 + 16 c .. +15 of activation row m, where u = m * per + c
    const int per = cnt * 16;
    const int units = M * per;  // a multiple of 16
    uint4 av[UPT][8];
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
        const int u = lane + j * kWave;
        const int uc = u < units ? u : units - 1;
        const int m = (uc >= per) + (uc >= 2 * per) + (uc >= 3 * per);  // M <= 4
        const int c = uc - m * per;
        const uint4* src = reinterpret_cast<const uint4*>(p.A + (int64_t)m * K + (int64_t)cs0 * 256 + 16 * c);
        av[j][0] = src[0];
        av[j][1] = src[1];
    }
    // 1b. all code loads of this wave, in the order step 3 consumes them (rows
    //     past N re-read row N-1, chunk-sets past the wave's share re-read its
    //     first one; both are ignored)
    const uint8_t* crow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = n_base + 16 * r + i16;
        crow[r] = codes + (n < N ? n : N - 1) * rb;
    }
    uint4 q[CSW][R];
#pragma unroll
    for (int s = 0; s < CSW; ++s) {
        const int cs = (s < cnt) ? cs0 + s : cs0;
#pragma unroll
        for (int r = 0; r < R; ++r) q[s][r] = *reinterpret_cast<const uint4*>(crow[r] + (int64_t)(4 * cs + g) * 16);
    }
    // 1c. row scale and bias of the output this thread finishes in step 4
    //     (thread e < 64R: row n_base + 16 (e / 64) + e % 16)
    float sc_e, bi_e;
    {
        const int e = (int)threadIdx.x % (R * kWave);
        const int64_t n = n_base + 16 * (e / kWave) + (e & 15);
        const int64_t nc = n < N ? n : N - 1;
        sc_e = f16_bits_to_f32(p.scale[nc]);
        bi_e = p.bias ? F16::to_f32(p.bias[nc]) : 0.0f;
    }
    // 2. paired activations of this wave's columns to its LDS area
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
        const int u = lane + j * kWave;
        const bool live = u < units;
        const int uc = live ? u : units - 1;
        const int m = (uc >= per) + (uc >= 2 * per) + (uc >= 3 * per);
        const int c = uc - m * per;
        uint4 w0, w1;
        act_pairs16<0>(av[j], w0, w1);
        if (live) {
            uint4* dst = reinterpret_cast<uint4*>(aps + ((int64_t)(m * 4 * CSW + (c >> 2)) * 32 + 8 * (c & 3)));
            dst[0] = w0;
            dst[1] = w1;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes are complete

    // 3. contract
    f32x4 acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool a_live = i16 < M;
    const uint32_t magic_v = vgpr_const<kMagic2>();
#pragma unroll
    for (int s = 0; s < CSW; ++s) {
        if (s < cnt) {
            // Lanes of rows m >= M only feed output rows that are never
            // stored (row m of the product depends on row m of A alone), so
            // they skip the LDS read and keep an arbitrary register value.
            uint4 aw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) aw[e] = opaque_uint4();
            if (a_live) {
                const uint4* arow = reinterpret_cast<const uint4*>(aps + (int64_t)(i16 * 4 * CSW + 4 * s + g) * 32);
#pragma unroll
                for (int e = 0; e < 8; ++e) aw[e] = arow[e];
            }
#define TQ_MFMA_L(D, I0)                                                                              \
    {                                                                                                 \
        const f16x8 aop = __builtin_bit_cast(f16x8, aw[2 * (D) + (I0) / 4]);                          \
        _Pragma("unroll") for (int r = 0; r < R; ++r) {                                               \
            const uint4 bw = tern_quad<I0>(dword_of(q[s][r], D), magic_v);                            \
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, __builtin_bit_cast(f16x8, bw), acc[r], 0, 0, 0); \
        }                                                                                             \
    }
            TQ_MFMA_L(0, 0)
            TQ_MFMA_L(0, 4)
            TQ_MFMA_L(1, 0)
            TQ_MFMA_L(1, 4)
            TQ_MFMA_L(2, 0)
            TQ_MFMA_L(2, 4)
            TQ_MFMA_L(3, 0)
            TQ_MFMA_L(3, 4)
#undef TQ_MFMA_L
        }
    }

    // 4. wave partials -> LDS, fixed-order sum
#pragma unroll
    for (int r = 0; r < R; ++r) red[(wave * R + r) * kWave + lane] = acc[r];
    __syncthreads();
    if ((int)threadIdx.x < R * kWave) {  // R <= W
        const int e = (int)threadIdx.x;
        const int r = e / kWave;
        const int l = e % kWave;
        f32x4 sum = red[r * kWave + l];
        for (int w = 1; w < W; ++w) sum += red[(w * R + r) * kWave + l];
        const int64_t n = n_base + 16 * r + (l & 15);
        if (n < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * (l >> 4) + i;
                if (m < M) p.C[(int64_t)m * N + n] = F16::from_f32_fast(sum[i] * sc_e + bi_e);
            }
        }
    }
}

// Matrix-core step and output unit for activation type T.  Both types
// take the same exact ternary operand (tern_pair): fp16 reads it as -1, 0,
// +1; bf16 reads the same bits as -2^-7, 0, +2^-7, so a bf16 kernel's fp32
// sums are 2^-7 times the result and kUnit (128) restores it exactly.
template <class T>
__device__ __forceinline__ f32x4 sm_mma(uint4 a, uint4 b, f32x4 c) {
    if constexpr (std::is_same<T, F16>::value)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <class T>
constexpr float ternary_unit() { return std::is_same<T, F16>::value ? 1.0f : kBf16TernaryUnit; }

// Small-M form of the kernel above (fp16 or bf16, M <= 4, K a multiple of 256 CSW,
// N a multiple of 16 R, W = K / (256 CSW) waves), with MT in {1, 2, 4}
// activation rows held at compile time (rows M .. MT-1 re-read row M-1 and
// are never stored):
// * unit c (16 columns) of row m's part of a wave's pair area is 32
//   contiguous bytes at 32 c, and only lanes 16g + m (m < M: row m of the
//   matrix-core operand) read it back;
// * every global address is a wave-uniform base plus a 32-bit lane offset
//   and a compile-time displacement, and no count depends on M at run time.
// The bias is read from a valid address whether or not one is given, so the
// load needs no branch (a branch there makes the compiler wait for every
// outstanding load, codes included, before it).
//
// VAR selects a measurement variant (the dispatcher always runs VAR = 0):
// 1 reads row-block 0's codes in every workgroup, so the codes come from the
// cache instead of HBM; 2 does that and also drops the matrix-core step
// (the unpacked operands are kept alive but not multiplied).  Their outputs
// are meaningless; they split a call's time into HBM, unpack and MAC parts.
template <class T, int R, int CSW, int MT, int VAR = 0>
__global__ __launch_bounds__(1024) void ternary_gemv_m1_kernel(GemmArgs p) {
    extern __shared__ uint4 smem[];
    constexpr int U = CSW / 4;            // 16-column activation units per lane and row
    constexpr int kRowLds = CSW * 512;    // pair bytes of one activation row
    uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int M = (int)p.M;
    const uint32_t rb = (uint32_t)(p.K / 4);
    const int64_t n_base = (int64_t)blockIdx.x * (16 * R);
    const int cs0 = wave * CSW;
    uint8_t* aps = lds + wave * (MT * kRowLds);                           // this wave's pairs
    float* red = reinterpret_cast<float*>(lds + W * (MT * kRowLds));      // [W][R][MT][16]

    // 1. loads in the order they are consumed: activations, row scale and
    //    bias of the output this thread may finish, then all codes
    const uint8_t* abase = reinterpret_cast<const uint8_t*>(p.A) + (int64_t)cs0 * 512;
    uint4 av[MT][U][8];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int mr = m < M ? m : M - 1;
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const uint8_t* src = abase + (int64_t)mr * (p.K * 2) + 2048 * j + (uint64_t)(uint32_t)(32 * lane);
            av[m][j][0] = *reinterpret_cast<const uint4*>(src);
            av[m][j][1] = *reinterpret_cast<const uint4*>(src + 16);
        }
    }
    // output of thread t (< 16 R MT) in step 4: row-block t / (16 MT),
    // activation row (t / 16) % MT, weight row n_base + 16 (t / (16 MT)) + t % 16
    const int te = (int)threadIdx.x % (16 * R * MT);
    const int64_t n_e = n_base + 16 * (te / (16 * MT)) + (te & 15);
    const uint16_t* bsrc = p.bias ? p.bias : p.scale;
    const uint16_t sc_bits = p.scale[n_e];
    const uint16_t bi_bits = bsrc[n_e];
    const int64_t n_codes = VAR == 0 ? n_base : 0;
    const uint8_t* cbase = static_cast<const uint8_t*>(p.wq) + n_codes * rb + (int64_t)cs0 * 64;
    const uint32_t lo = (uint32_t)i16 * rb + 16u * (uint32_t)g;
    uint4 q[CSW][R];
#pragma unroll
    for (int s = 0; s < CSW; ++s) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            q[s][r] = *reinterpret_cast<const uint4*>(cbase + (int64_t)r * 16 * rb + 64 * s + (uint64_t)lo);
    }

    // 2. paired activations of this wave's columns to LDS
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            uint4 w0, w1;
            act_pairs16<0>(av[m][j], w0, w1);
            uint4* dst = reinterpret_cast<uint4*>(aps + m * kRowLds + 32 * (lane + 64 * j));
            dst[0] = w0;
            dst[1] = w1;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes are complete

    // 3. contract; lanes 16g + m (m < M) read row m of the operand, the
    //    others keep an arbitrary value (their output rows are never stored)
    f32x4 acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t magic_v = vgpr_const<kMagic2>();
    const bool a_live = MT == 1 ? i16 == 0 : i16 < M;
#pragma unroll
    for (int s = 0; s < CSW; ++s) {
        uint4 aw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) aw[e] = opaque_uint4();
        if (a_live) {
            const uint4* arow = reinterpret_cast<const uint4*>(aps + (MT == 1 ? 0 : i16 * kRowLds) + (4 * s + g) * 128);
#pragma unroll
            for (int e = 0; e < 8; ++e) aw[e] = arow[e];
        }
#define TQ_MFMA_1(D, I0)                                                                              \
    {                                                                                                 \
        const uint4 aop = aw[2 * (D) + (I0) / 4];                                                     \
        _Pragma("unroll") for (int r = 0; r < R; ++r) {                                               \
            const uint4 bw = tern_quad<I0>(dword_of(q[s][r], D), magic_v);                            \
            if constexpr (VAR == 2) asm volatile("" :: "v"(bw.x), "v"(bw.y), "v"(bw.z), "v"(bw.w), "v"(aop.x)); \
            else acc[r] = sm_mma<T>(aop, bw, acc[r]);                                                 \
        }                                                                                             \
    }
        TQ_MFMA_1(0, 0)
        TQ_MFMA_1(0, 4)
        TQ_MFMA_1(1, 0)
        TQ_MFMA_1(1, 4)
        TQ_MFMA_1(2, 0)
        TQ_MFMA_1(2, 4)
        TQ_MFMA_1(3, 0)
        TQ_MFMA_1(3, 4)
#undef TQ_MFMA_1
    }

    // 4. rows 0 .. MT-1 of each wave's partials -> LDS; fixed-order sum
    //    (component i of lane i16 < 16: activation row i)
    if (g == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < MT; ++i) red[((wave * R + r) * MT + i) * 16 + i16] = acc[r][i];
    }
    __syncthreads();
    if ((int)threadIdx.x < 16 * R * MT) {
        const int t = (int)threadIdx.x;
        const int i = (t / 16) % MT;
        float sum = red[t];
        for (int w = 1; w < W; ++w) sum += red[w * (16 * R * MT) + t];
        const float bi = p.bias ? T::to_f32(bi_bits) : 0.0f;
        const float sc = f16_bits_to_f32(sc_bits) * ternary_unit<T>();
        if (i < M) p.C[(int64_t)i * p.N + n_e] = T::from_f32_fast(sum * sc + bi);
    }
}

// Same arithmetic, streaming schedule (fp16 or bf16 activations AT, M <= 16,
// K / 256 <= 16 CSW).
//
// One workgroup per compute unit walks T consecutive 16-row blocks.  Wave w
// owns chunk-sets w*CSW .. w*CSW + CSW-1 (256 columns each) of all of them,
// so the activation operand of its MFMAs never changes: it is built once, in
// registers, from the activations of its columns (lane 16g + i: row i,
// chunk 4cs + g).  The wave issues its activation loads, then the code loads
// of all T row-blocks, then builds the operand while the codes are in
// flight, and contracts each row-block as its codes land (in-order
// completion), one accumulator per row-block.  Wave partials meet in LDS
// once, at the end, and are summed in a fixed order.
//
// The operand layout puts 16 activation rows on neighbouring lanes, so
// loading it directly would touch a different 128-byte line with every lane.
// Instead each chunk-set's 512-byte row slices are copied global -> LDS by
// DMA, two rows per instruction (lane l: row 2e + l/32, bytes 16 (l % 32)
// ..), MR/2 instructions for the MR >= M rows (4, 8 or 16; rows past M
// re-read row M-1), into the wave's own LDS area, and read back in operand
// order.  The area holds CSW x MR rows x 32 slots of 16 bytes, slot q of row
// r at q ^ (r % 16), which keeps the operand reads free of bank conflicts;
// the same area later takes the wave's partial sums.
//
// Every workgroup reads the activations of its whole K range (M * K * 2
// bytes), so for short, wide matrices the grid may also split K: workgroup
// (x, z) covers chunk-sets z*CS/S .. (z+1)*CS/S - 1 of its row-blocks and
// stores fp32 partials (S = gridDim.y divides CS); the last split of each
// row-block to finish sums them (step 6; launch_splitk_reduce instead when
// no arrival counters are given).
__host__ __device__ constexpr int stream_wave_lds(int csw, int mr, int t) {  // bytes of one wave's LDS area
    return t * 1024 > csw * mr * 512 ? t * 1024 : csw * mr * 512;
}

template <class AT, int CSW, int T, int MR>
__global__ __launch_bounds__(1024) void ternary_gemv_stream_kernel(SplitArgs sa) {
    const GemmArgs& p = sa.g;
    extern __shared__ uint4 smem[];
    constexpr int kArea = stream_wave_lds(CSW, MR, T);
    f32x4* red = reinterpret_cast<f32x4*>(smem);  // wave w, row-block t: red[w * kArea / 16 + 64 t + lane]
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int64_t N = p.N, K = p.K;
    const int M = (int)p.M;
    const int64_t rb = K / 4;
    const int CS = (int)(K / 256);
    const int64_t n_base = (int64_t)blockIdx.x * (16 * T);
    const uint8_t* codes = static_cast<const uint8_t*>(p.wq);
    uint8_t* area = reinterpret_cast<uint8_t*>(smem) + wave * kArea;
    const uint32_t area_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem + wave * kArea;
    const int csz = CS / sa.S;                       // chunk-sets of this split
    const int cs_end = ((int)blockIdx.y + 1) * csz;
    const int cs0 = (int)blockIdx.y * csz + wave * CSW;
    const int cnt = cs_end - cs0 < CSW ? cs_end - cs0 : CSW;  // >= 1 for every wave of the launch

    // row scale and bias bits of the output this thread finishes in step 5
    // (thread e < 64T: row n_base + 16 (e / 64) + e % 16); without a bias the
    // scale is read twice, so that no branch splits the load phase
    uint16_t sc_bits, bi_bits;
    {
        const int e = (int)threadIdx.x % (T * kWave);
        const int64_t n = n_base + 16 * (e / kWave) + (e & 15);
        const int64_t nc = n < N ? n : N - 1;
        sc_bits = p.scale[nc];
        bi_bits = (p.bias ? p.bias : p.scale)[nc];
    }
    // Global addresses are a wave-uniform base plus a 32-bit lane offset (the
    // plan keeps 16 T rows of codes and 16 rows of activations below 4 GiB).
    // 1. activation slices -> the wave's LDS area by DMA, two rows per
    //    instruction (rows past M re-read row M-1; operand rows m >= M only
    //    feed outputs that are never stored)
    const uint8_t* a_base = reinterpret_cast<const uint8_t*>(p.A);
#pragma unroll
    for (int s = 0; s < CSW; ++s) {
        const int cs = (s == 0 || s < cnt) ? cs0 + s : cs0;
        const uint8_t* a_cs = a_base + (int64_t)cs * 512;
#pragma unroll
        for (int e = 0; e < MR / 2; ++e) {
            const int r0 = 2 * e + (lane >> 5);
            const int r = r0 < M ? r0 : M - 1;
            const int piece = (lane & 31) ^ (r0 & 15);
            const uint32_t off = (uint32_t)r * (uint32_t)(2 * K) + 16u * (uint32_t)piece;
            dma16s(a_cs, off, area_lds + (uint32_t)(s * MR * 512 + e * 1024));
        }
    }
    // 2. code loads of all row-blocks, in the order step 4 consumes them (rows
    //    past N re-read row N-1, chunk-sets past the wave's share re-read its
    //    first one; both are ignored)
    const uint8_t* c_blk = codes + n_base * rb;
    uint4 q[T][CSW];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int64_t n = n_base + 16 * t + i16;
        const uint32_t roff = (uint32_t)((n < N ? n : N - 1) - n_base) * (uint32_t)rb + 16u * (uint32_t)g;
#pragma unroll
        for (int s = 0; s < CSW; ++s) {
            const int cs = (s == 0 || s < cnt) ? cs0 + s : cs0;
            q[t][s] = *reinterpret_cast<const uint4*>(c_blk + (int64_t)cs * 64 + roff);
        }
    }

    // 3. wait for the activation DMA only (the T * CSW code loads issued after
    //    it may still be in flight: completion is in order), read the operand
    //    rows and pair them (pair (d, i) of a chunk in dword 8 d + i)
    static_assert(T * CSW <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(T * CSW) : "memory");
    const int rd_row = i16 & (MR - 1);
    uint4 aw[CSW][8];
#pragma unroll
    for (int s = 0; s < CSW; ++s) {
        uint4 av[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            av[e] = *reinterpret_cast<const uint4*>(area + s * MR * 512 + rd_row * 512 +
                                                    16 * ((8 * g + e) ^ (rd_row & 15)));
        act_pairs16<0>(av, aw[s][0], aw[s][1]);
        act_pairs16<1>(av, aw[s][2], aw[s][3]);
        act_pairs16<2>(av, aw[s][4], aw[s][5]);
        act_pairs16<3>(av, aw[s][6], aw[s][7]);
    }

    // 4. contract each row-block as its codes land
    const uint32_t magic_v = vgpr_const<kMagic2>();
    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        f32x4 a4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < CSW; ++s) {
            if (s == 0 || s < cnt) {  // cnt >= 1: the first chunk-set is unconditional
#define TQ_MFMA_S(D, I0)                                                                              \
    {                                                                                                 \
        const uint4 bw = tern_quad<I0>(dword_of(q[t][s], D), magic_v);                                \
        a4 = sm_mma<AT>(aw[s][2 * (D) + (I0) / 4], bw, a4);                                           \
    }
                TQ_MFMA_S(0, 0)
                TQ_MFMA_S(0, 4)
                TQ_MFMA_S(1, 0)
                TQ_MFMA_S(1, 4)
                TQ_MFMA_S(2, 0)
                TQ_MFMA_S(2, 4)
                TQ_MFMA_S(3, 0)
                TQ_MFMA_S(3, 4)
#undef TQ_MFMA_S
            }
        }
        acc[t] = a4;
    }

    // 5. wave partials -> LDS, fixed-order sum; split partials carry the
    //    bf16 unit, so the reduction treats both types alike
#pragma unroll
    for (int t = 0; t < T; ++t) red[wave * (kArea / 16) + t * kWave + lane] = acc[t];
    __syncthreads();
    if ((int)threadIdx.x < T * kWave) {  // T <= W
        const int e = (int)threadIdx.x;
        const int t = e / kWave;
        const int l = e % kWave;
        f32x4 sum = red[t * kWave + l];
        for (int w = 1; w < W; ++w) sum += red[w * (kArea / 16) + t * kWave + l];
        const int64_t n = n_base + 16 * t + (l & 15);
        if (n < N && sa.S > 1) {
            float* part = sa.ws + (int64_t)blockIdx.y * M * N;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * (l >> 4) + i;
                if (m < M) store_partial(part + (int64_t)m * N + n, sum[i] * ternary_unit<AT>());
            }
        } else if (n < N) {
            const float sc_e = f16_bits_to_f32(sc_bits) * ternary_unit<AT>();
            const float bi_e = p.bias ? AT::to_f32(bi_bits) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * (l >> 4) + i;
                if (m < M) p.C[(int64_t)m * N + n] = AT::from_f32_fast(sum[i] * sc_e + bi_e);
            }
        }
    }
    // 6. with a split, the last workgroup of this row block to finish sums
    //    the S partials in split order and finishes the outputs
    if (sa.S == 1 || !sa.flags) return;
    if (!split_last_arrival(sa.flags, blockIdx.x, sa.S, reinterpret_cast<uint32_t*>(smem))) return;
    if ((int)threadIdx.x < T * kWave) {
        const int e = (int)threadIdx.x;
        const int l = e % kWave;
        const int64_t n = n_base + 16 * (e / kWave) + (l & 15);
        const int64_t nc = n < N ? n : N - 1;
        uint32_t off[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * (l >> 4) + i;
            off[i] = (uint32_t)((m < M ? m : M - 1) * N + nc);
        }
        float sum[4];
        split_sums<4, 4>(sa.ws, (int64_t)M * N, off, sa.S, sum);
        if (n < N) {
            const float sc_e = f16_bits_to_f32(sc_bits);
            const float bi_e = p.bias ? AT::to_f32(bi_bits) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * (l >> 4) + i;
                if (m < M) p.C[(int64_t)m * N + n] = AT::from_f32_fast(sum[i] * sc_e + bi_e);
            }
        }
    }
}

// ------------------------------------------------------ W4A16, matrix cores
//
// fp16 activations, M <= 16, K % 128 == 0.  A code word x (int32) holds
// nibbles q_0 .. q_7 (q_i at bits 4i: column 8j + i of word j).  Masking one
// nibble of each 16-bit half into the mantissa of the fp16 constant 1024
// (0x6400, unit in the last place 1) gives a pair of exact values in one
// v_and_or_b32:
//   (x & 0x000F000F) | magic = (1024 + q_0, 1024 + q_4),
//   (x & 0x00F000F0) | magic = (1024 + 16 q_1, 1024 + 16 q_5),
// and with y = x >> 8 the pairs (q_2, q_6) and (16 q_3, 16 q_7) the same way.
// One packed fp16 add of -(1024 + 8), or fma by 1/16 with -(64 + 8), leaves
// the weight values q - 8 exactly (zero point 8; w4_quad), and the
// activations are paired to match - (a_0, a_4), (a_1, a_5), (a_2, a_6),
// (a_3, a_7) - so one MFMA contracts one word of each of 16 rows with exact
// products and no offset in the sums.  The group scale s[n, g] then
// multiplies the group's fp32 sum (page "Model quantization - vLLM runtime
// quantization architecture", section 5: group_size 128).
//
// Work split: a block owns 16R weight rows and all of K; its W waves take
// every W-th 128-column group.  Lane l = 16h + i loads 16 bytes (32 codes,
// group columns 32h .. 32h+31) of row i of each row block, the row scales,
// and the 32 activations of row m = i at those columns; MFMA d contracts
// code word d of every lane.  The next group's loads are issued before the
// current group is contracted.  Wave partials meet in LDS and are summed in
// a fixed order.

template <int R, int W>
__global__ __launch_bounds__(W * kWave) void w4_gemv_mfma_kernel(GemmArgs p) {
    __shared__ f32x4 red[W][R][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int h = lane >> 4;
    const int i16 = lane & 15;
    const int64_t N = p.N, K = p.K;
    const int M = (int)p.M;
    const int G = (int)(K / 128);
    const int64_t rowb = K / 2;         // code bytes per row
    const int64_t n_base = (int64_t)blockIdx.x * (16 * R);
    const uint8_t* codes = static_cast<const uint8_t*>(p.wq);
    const bool a_live = i16 < M;
    const uint16_t* arow = p.A + (int64_t)(a_live ? i16 : 0) * K;

    const uint8_t* crow[R];
    const uint16_t* srow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t n = n_base + 16 * r + i16;
        n = n < N ? n : N - 1;  // rows past N re-read row N-1; ignored
        crow[r] = codes + n * rowb + 16 * h;
        srow[r] = p.scale + n * G;
    }
    auto load = [&](int gi, uint4 (&q)[R], uint16_t (&sc)[R], uint4 (&av)[4]) {
#pragma unroll
        for (int r = 0; r < R; ++r) q[r] = *reinterpret_cast<const uint4*>(crow[r] + (int64_t)gi * 64);
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r] = srow[r][gi];
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = opaque_uint4();
        if (a_live) {
            const uint4* ap = reinterpret_cast<const uint4*>(arow + (int64_t)gi * 128 + 32 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) av[e] = ap[e];
        }
    };

    f32x4 acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t magic_v = vgpr_const<kMagic2>();
    const f16x2 k0 = __builtin_bit_cast(f16x2, kW4Sub0Sym), k1 = __builtin_bit_cast(f16x2, kW4Sub1Sym);

    uint4 q[R], qn[R], av[4], avn[4];
    uint16_t sc[R], scn[R];
    int gi = wave;
    if (gi < G) load(gi, q, sc, av);
    for (; gi < G; gi += W) {
        const int gn = gi + W < G ? gi + W : gi;  // past the end: re-read, unused
        load(gn, qn, scn, avn);
        uint4 aop[4];  // activation operands of the four code words
#pragma unroll
        for (int d = 0; d < 4; ++d) aop[d] = w4_act_quad(av[d]);  // columns 8d .. 8d+7 of this lane's 32
#pragma unroll
        for (int r = 0; r < R; ++r) {
            f32x4 ag = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint4 bw = w4_quad(dword_of(q[r], d), magic_v, k0, k1);
                ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, aop[d]), __builtin_bit_cast(f16x8, bw), ag, 0, 0, 0);
            }
            const float s = f16_bits_to_f32(sc[r]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[r][i] = fmaf(s, ag[i], acc[r][i]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) { q[r] = qn[r]; sc[r] = scn[r]; }
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = avn[e];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    for (int e = threadIdx.x; e < R * kWave; e += W * kWave) {
        const int r = e / kWave;
        const int l = e % kWave;
        f32x4 sum = red[0][r][l];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += red[w][r][l];
        const int64_t n = n_base + 16 * r + (l & 15);
        if (n >= N) continue;
        const float b = p.bias ? F16::to_f32(p.bias[n]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * (l >> 4) + i;
            if (m < M) p.C[(int64_t)m * N + n] = F16::from_f32_fast(sum[i] + b);
        }
    }
}

// W4A16 at M <= 4 (fp16 or bf16, K = 128 G with GSW in {4, 8} groups per wave and
// 4 <= W = G / GSW <= 16 waves, N a multiple of 16 R), in the form of
// ternary_gemv_m1_kernel; MT in {1, 2, 4} activation rows are held, rows
// M .. MT-1 re-read row M-1 and are never stored:
// * wave w owns groups g0 = w GSW .. g0 + GSW - 1.  Lane l = 16h + i loads 16
//   bytes (group columns 32h .. 32h + 31) of row i of each group, and MFMA d
//   of a group contracts code word d of every lane (columns 32h + 8d ..);
// * unit u (8 columns) of the wave's columns is word u % 4 of lane slot
//   (u / 4) % 4 of group u / 16, so lane l pairs units l + 64 j of every
//   activation row m: (a_0, a_4), (a_1, a_5), (a_2, a_6), (a_3, a_7), 16
//   bytes at 16 u of row m's part of the wave's LDS area;
// * lanes 16h + m (m < M) read row m's operand back; each group's four MFMAs
//   start from zero on exact weight values q - z (w4_quad), and component i
//   (activation row i) of the group's fp32 sum is scaled by s[n, g] into the
//   row result (scales of a wave are GSW consecutive halves of a row: GSW / 4
//   8-byte loads);
// * rows 0 .. MT-1 of the wave results meet in LDS; one barrier, a
//   fixed-order sum.
// ASYM: per-(row, group) zero points z (uint8, [N, K/128]) instead of 8: the
// packed constants -(1024 + z), -(64 + z) are built per row and group.
// bf16: the exact fp16 integers are converted to bf16 (w4_quad_bf16).
template <class T, int R, int GSW, bool ASYM, int MT>
__global__ __launch_bounds__(1024) void w4_gemv_m1_kernel(GemmArgs p) {
    constexpr bool kBf = std::is_same<T, BF16>::value;
    extern __shared__ uint4 smem[];
    constexpr int U = GSW / 4;            // 8-column units per lane and row
    constexpr int kRowLds = GSW * 256;    // pair bytes of one activation row
    uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int h = lane >> 4;
    const int i16 = lane & 15;
    const int M = (int)p.M;
    const uint32_t rb = (uint32_t)(p.K / 2);         // code bytes per row
    const int64_t G = p.K / 128;
    const int64_t n_base = (int64_t)blockIdx.x * (16 * R);
    const int g0 = wave * GSW;
    uint8_t* aps = lds + wave * (MT * kRowLds);                           // this wave's pairs
    float* red = reinterpret_cast<float*>(lds + W * (MT * kRowLds));      // [W][R][MT][16]

    // 1. loads in the order they are consumed: activations, scales, zero
    //    points, bias of the output this thread may finish, codes
    const uint8_t* abase = reinterpret_cast<const uint8_t*>(p.A) + (int64_t)g0 * 256;
    uint4 av[MT][U];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int mr = m < M ? m : M - 1;
        const uint8_t* arow = abase + (int64_t)mr * (p.K * 2);
#pragma unroll
        for (int j = 0; j < U; ++j) av[m][j] = *reinterpret_cast<const uint4*>(arow + 1024 * j + (uint64_t)(uint32_t)(16 * lane));
    }
    uint2 scw[R][U];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint16_t* srow = p.scale + (n_base + 16 * r + i16) * G + g0;
#pragma unroll
        for (int j = 0; j < U; ++j) scw[r][j] = *reinterpret_cast<const uint2*>(srow + 4 * j);
    }
    uint32_t zw[R][U];
    if constexpr (ASYM) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint8_t* zrow = p.zeros + (n_base + 16 * r + i16) * G + g0;
#pragma unroll
            for (int j = 0; j < U; ++j) zw[r][j] = *reinterpret_cast<const uint32_t*>(zrow + 4 * j);
        }
    }
    // output of thread t (< 16 R MT) in step 4: row-block t / (16 MT),
    // activation row (t / 16) % MT, weight row n_base + 16 (t / (16 MT)) + t % 16
    const int te = (int)threadIdx.x % (16 * R * MT);
    const int64_t n_e = n_base + 16 * (te / (16 * MT)) + (te & 15);
    const uint16_t bi_bits = (p.bias ? p.bias : p.scale)[n_e];
    const uint8_t* cbase = static_cast<const uint8_t*>(p.wq) + n_base * rb + (int64_t)g0 * 64;
    const uint32_t lo = (uint32_t)i16 * rb + 16u * (uint32_t)h;
    uint4 q[GSW][R];
#pragma unroll
    for (int gi = 0; gi < GSW; ++gi) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            q[gi][r] = *reinterpret_cast<const uint4*>(cbase + (int64_t)r * 16 * rb + 64 * gi + (uint64_t)lo);
    }

    // 2. activation pairs of this lane's units to LDS
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int j = 0; j < U; ++j)
            *reinterpret_cast<uint4*>(aps + m * kRowLds + 16 * (lane + 64 * j)) = w4_act_quad(av[m][j]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes are complete

    // 3. contract group by group; lanes 16h + m (m < M) read row m's operand,
    //    the others keep an arbitrary value (their output rows are never
    //    stored)
    float res[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < MT; ++i) res[r][i] = 0.0f;
    const uint32_t magic_v = vgpr_const<kMagic2>();
    const bool a_live = MT == 1 ? i16 == 0 : i16 < M;
#pragma unroll
    for (int gi = 0; gi < GSW; ++gi) {
        uint4 aw[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) aw[d] = opaque_uint4();
        if (a_live) {
            const uint4* arow = reinterpret_cast<const uint4*>(aps + (MT == 1 ? 0 : i16 * kRowLds) + 16 * (16 * gi + 4 * h));
#pragma unroll
            for (int d = 0; d < 4; ++d) aw[d] = arow[d];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            W4Sub k{__builtin_bit_cast(f16x2, kW4Sub0Sym), __builtin_bit_cast(f16x2, kW4Sub1Sym)};
            if constexpr (ASYM) k = w4_sub((zw[r][gi / 4] >> (8 * (gi % 4))) & 0xFFu);
            f32x4 ag = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t x = dword_of(q[gi][r], d);
                const uint4 bw = kBf ? w4_quad_bf16(x, magic_v, k.k0, k.k1) : w4_quad(x, magic_v, k.k0, k.k1);
                ag = sm_mma<T>(aw[d], bw, ag);
            }
            const uint2 sw = scw[r][gi / 4];
            const uint32_t sd = (gi % 4) < 2 ? sw.x : sw.y;
            const float s = f16_bits_to_f32((uint16_t)(sd >> (16 * (gi % 2))));
#pragma unroll
            for (int i = 0; i < MT; ++i) res[r][i] = fmaf(s, ag[i], res[r][i]);
        }
    }

    // 4. rows 0 .. MT-1 of the wave results -> LDS; fixed-order sum
    if (h == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < MT; ++i) red[((wave * R + r) * MT + i) * 16 + i16] = res[r][i];
    }
    __syncthreads();
    if ((int)threadIdx.x < 16 * R * MT) {
        const int t = (int)threadIdx.x;
        const int i = (t / 16) % MT;
        float sum = red[t];
        for (int w = 1; w < W; ++w) sum += red[w * (16 * R * MT) + t];
        const float bi = p.bias ? T::to_f32(bi_bits) : 0.0f;
        if (i < M) p.C[(int64_t)i * p.N + n_e] = T::from_f32_fast(sum + bi);
    }
}

// W4A16, streaming schedule (fp16 or bf16, 3 <= M <= 16): the arithmetic above with
// the work split of the ternary streaming kernel.  One workgroup walks T
// consecutive 16-row blocks; wave w owns groups w*GSW .. w*GSW + GSW-1 (128
// columns each) of its K range, so it builds the activation operands once
// and contracts every row-block against them.
// Activations reach the wave's LDS area by DMA, four 256-byte row slices per
// instruction (lane l: row 4e + l/16, 16-byte slot l%16, slot q of row r at
// q ^ (r % 16)), MR/4 instructions for the MR >= M rows; each lane then reads
// its four operand chunks (row i, slots 4h .. 4h+3).  Issue order: bias bits
// and group scales, activation DMA, the code words of all row-blocks, then
// one vmcnt wait for the DMA only.  With S = gridDim.y > 1 splits of the groups
// the workgroup stores fp32 partials (group scales applied), and the last
// split of each row-block to finish sums them and adds the bias
// (launch_splitk_reduce instead when no arrival counters are given).
// ASYM: per-(row, group) zero points z instead of 8, loaded with the scales
// before the DMA; each row-block builds its packed constants -(1024 + z),
// -(64 + z) per group, so the operand is q - z exactly.
__host__ __device__ constexpr int w4_stream_wave_lds(int gsw, int mr, int t) {  // bytes of one wave's LDS area
    return t * 1024 > gsw * mr * 256 ? t * 1024 : gsw * mr * 256;
}

template <class AT, int GSW, int T, int MR, bool ASYM>
__global__ __launch_bounds__(1024) void w4_gemv_stream_kernel(SplitArgs sa) {
    constexpr bool kBf = std::is_same<AT, BF16>::value;  // bf16: exact integers converted to bf16
    const GemmArgs& p = sa.g;
    extern __shared__ uint4 smem[];
    constexpr int kArea = w4_stream_wave_lds(GSW, MR, T);
    f32x4* red = reinterpret_cast<f32x4*>(smem);  // wave w, row-block t: red[w * kArea / 16 + 64 t + lane]
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 4;
    const int i16 = lane & 15;
    const int64_t N = p.N, K = p.K;
    const int M = (int)p.M;
    const int G = (int)(K / 128);
    const int64_t rowb = K / 2;  // code bytes per row
    const int64_t n_base = (int64_t)blockIdx.x * (16 * T);
    const uint8_t* codes = static_cast<const uint8_t*>(p.wq);
    uint8_t* area = reinterpret_cast<uint8_t*>(smem) + wave * kArea;
    const uint32_t area_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem + wave * kArea;
    const int gsz = G / sa.S;  // groups of this split
    const int g_end = ((int)blockIdx.y + 1) * gsz;
    const int g0 = (int)blockIdx.y * gsz + wave * GSW;
    const int cnt = g_end - g0 < GSW ? g_end - g0 : GSW;  // >= 1 for every wave of the launch

    // bias bits of the output this thread finishes (thread e < 64T: row
    // n_base + 16 (e / 64) + e % 16); read from the scales when absent, so
    // that no branch splits the load phase
    uint16_t bi_bits;
    {
        const int e = (int)threadIdx.x % (T * kWave);
        const int64_t n = n_base + 16 * (e / kWave) + (e & 15);
        const int64_t nc = n < N ? n : N - 1;
        bi_bits = (p.bias ? p.bias : p.scale)[nc];
    }
    // group scales (and zero points) of all row-blocks, first: the codes are
    // waited for in order, so loads issued after them would hold up
    // row-block 0.  Each such load costs the address unit about as much as a
    // code load (one lane per row, so 64 cache lines), hence few of them: one
    // load serves four row-blocks (lane 16 j + r fetches row r of row-block
    // 4 c + j; rows past the workgroup's are clamped and unused) and, with
    // two groups per wave, both groups (a dword of scales, a halfword of zero
    // points: the plan takes two groups per wave only when G and the groups
    // per split are even and the arrays aligned, so g0 is even and the pair
    // lies in the row).  After the wait, lane shuffles hand each value to the
    // lanes that use it.
    static_assert(GSW == 1 || GSW == 2, "one or two groups per wave");
    using ScaleT = std::conditional_t<GSW == 2, uint32_t, uint16_t>;
    using ZeroT = std::conditional_t<GSW == 2, uint16_t, uint8_t>;
    constexpr int TC = (T + 3) / 4;
    ScaleT scl[TC];
    ZeroT zpl[TC];
#pragma unroll
    for (int c = 0; c < TC; ++c) {
        const int64_t n = n_base + 16 * (4 * c + h) + i16;
        const int64_t o = (n < N ? n : N - 1) * G + g0;
        scl[c] = *reinterpret_cast<const ScaleT*>(p.scale + o);
        if constexpr (ASYM) zpl[c] = *reinterpret_cast<const ZeroT*>(p.zeros + o);
    }
    // Global addresses are a wave-uniform base plus a 32-bit lane offset (the
    // plan keeps 16 T rows of codes and 16 rows of activations below 4 GiB).
    // 1. activation slices -> LDS by DMA (rows past M re-read row M-1)
    const uint8_t* a_base = reinterpret_cast<const uint8_t*>(p.A);
#pragma unroll
    for (int s = 0; s < GSW; ++s) {
        const int gi = (s == 0 || s < cnt) ? g0 + s : g0;
        const uint8_t* a_g = a_base + (int64_t)gi * 256;
#pragma unroll
        for (int e = 0; e < MR / 4; ++e) {
            const int r0 = 4 * e + (lane >> 4);
            const int r = r0 < M ? r0 : M - 1;
            const int piece = (lane & 15) ^ (r0 & 15);
            const uint32_t off = (uint32_t)r * (uint32_t)(2 * K) + 16u * (uint32_t)piece;
            dma16s(a_g, off, area_lds + (uint32_t)(s * MR * 256 + e * 1024));
        }
    }
    // 2. code words of all row-blocks (rows past N re-read row N-1, groups
    //    past the wave's share re-read its first; both ignored)
    const uint8_t* c_blk = codes + n_base * rowb;
    uint4 q[T][GSW];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int64_t n = n_base + 16 * t + i16;
        const uint32_t roff = (uint32_t)((n < N ? n : N - 1) - n_base) * (uint32_t)rowb + 16u * (uint32_t)h;
#pragma unroll
        for (int s = 0; s < GSW; ++s) {
            const int gi = (s == 0 || s < cnt) ? g0 + s : g0;
            q[t][s] = *reinterpret_cast<const uint4*>(c_blk + (int64_t)gi * 64 + roff);
        }
    }

    // 3. wait for the DMA only (completion is in order), build the operands
    static_assert(T * GSW <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(T * GSW) : "memory");
    const int rd_row = i16 & (MR - 1);
    uint4 aop[GSW][4];
#pragma unroll
    for (int s = 0; s < GSW; ++s) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
            aop[s][d] = w4_act_quad(*reinterpret_cast<const uint4*>(area + s * MR * 256 + rd_row * 256 +
                                                                    16 * ((4 * h + d) ^ (rd_row & 15))));
    }

    // the empty asm statements keep the compiler from consuming the loaded
    // values, with a wait of their own, before the wait above
    int sc[T][GSW], zp[T][GSW];
#pragma unroll
    for (int c = 0; c < TC; ++c) {
        int sv = (int)scl[c];
        asm volatile("" : "+v"(sv));
        int zv = 0;
        if constexpr (ASYM) {
            zv = (int)zpl[c];
            asm volatile("" : "+v"(zv));
        }
#pragma unroll
        for (int j = 0; j < 4 && 4 * c + j < T; ++j) {
            const int t = 4 * c + j;
            const int sx = __shfl(sv, 16 * j + i16);
            const int zx = ASYM ? __shfl(zv, 16 * j + i16) : 0;
#pragma unroll
            for (int s = 0; s < GSW; ++s) {
                sc[t][s] = (sx >> (16 * s)) & 0xFFFF;
                zp[t][s] = (zx >> (8 * s)) & 0xFF;
            }
        }
    }

    // 4. contract each row-block as its codes land
    const uint32_t magic_v = vgpr_const<kMagic2>();
    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        f32x4 a4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < GSW; ++s) {
            if (s == 0 || s < cnt) {  // cnt >= 1: the first group is unconditional
                W4Sub k{__builtin_bit_cast(f16x2, kW4Sub0Sym), __builtin_bit_cast(f16x2, kW4Sub1Sym)};
                if constexpr (ASYM) k = w4_sub((uint32_t)zp[t][s]);
                f32x4 ag = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t x = dword_of(q[t][s], d);
                    const uint4 bw = kBf ? w4_quad_bf16(x, magic_v, k.k0, k.k1) : w4_quad(x, magic_v, k.k0, k.k1);
                    ag = sm_mma<AT>(aop[s][d], bw, ag);
                }
                const float sv = f16_bits_to_f32((uint16_t)sc[t][s]);
#pragma unroll
                for (int i = 0; i < 4; ++i) a4[i] = fmaf(sv, ag[i], a4[i]);
            }
        }
        acc[t] = a4;
    }

    // 5. wave partials -> LDS (each wave's own area), fixed-order sum
#pragma unroll
    for (int t = 0; t < T; ++t) red[wave * (kArea / 16) + t * kWave + lane] = acc[t];
    __syncthreads();
    if ((int)threadIdx.x < T * kWave) {  // T <= W
        const int e = (int)threadIdx.x;
        const int t = e / kWave;
        const int l = e % kWave;
        f32x4 sum = red[t * kWave + l];
        for (int w = 1; w < W; ++w) sum += red[w * (kArea / 16) + t * kWave + l];
        const int64_t n = n_base + 16 * t + (l & 15);
        if (n < N && sa.S > 1) {
            float* part = sa.ws + (int64_t)blockIdx.y * M * N;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * (l >> 4) + i;
                if (m < M) store_partial(part + (int64_t)m * N + n, sum[i]);
            }
        } else if (n < N) {
            const float b = p.bias ? AT::to_f32(bi_bits) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * (l >> 4) + i;
                if (m < M) p.C[(int64_t)m * N + n] = AT::from_f32_fast(sum[i] + b);
            }
        }
    }
    // 6. with a split, the last workgroup of this row block to finish sums
    //    the S partials (which carry the group scales) in split order
    if (sa.S == 1 || !sa.flags) return;
    if (!split_last_arrival(sa.flags, blockIdx.x, sa.S, reinterpret_cast<uint32_t*>(smem))) return;
    if ((int)threadIdx.x < T * kWave) {
        const int e = (int)threadIdx.x;
        const int l = e % kWave;
        const int64_t n = n_base + 16 * (e / kWave) + (l & 15);
        const int64_t nc = n < N ? n : N - 1;
        uint32_t off[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * (l >> 4) + i;
            off[i] = (uint32_t)((m < M ? m : M - 1) * N + nc);
        }
        float sum[4];
        split_sums<4, 4>(sa.ws, (int64_t)M * N, off, sa.S, sum);
        if (n < N) {
            const float b = p.bias ? AT::to_f32(bi_bits) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * (l >> 4) + i;
                if (m < M) p.C[(int64_t)m * N + n] = AT::from_f32_fast(sum[i] + b);
            }
        }
    }
}

// ------------------------------------------------------------- launchers

template <int R, int W>
static void launch_gemv_mfma(const GemmArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.N + 16 * R - 1) / (16 * R)));
    ternary_gemv_mfma_kernel<R, W><<<grid, W * kWave, 0, s>>>(a);
}

template <int R>
static void launch_gemv_mfma_w(const GemmArgs& a, hipStream_t s) {
    const int64_t cs = a.K / 256;
    if (cs >= 16) launch_gemv_mfma<R, 8>(a, s);
    else if (cs >= 8) launch_gemv_mfma<R, 4>(a, s);
    else if (cs >= 4) launch_gemv_mfma<R, 2>(a, s);
    else launch_gemv_mfma<R, 1>(a, s);
}

bool ternary_gemv_mfma_ok(const GemmArgs& a) { return !a.bf16 && a.M <= kGemvMaxM && a.K % 256 == 0; }

#ifndef TQ_GEMV_MIN_CSW
#define TQ_GEMV_MIN_CSW 4
#endif
constexpr int kGemvMinCsw = TQ_GEMV_MIN_CSW;  // fewest chunk-sets per wave
constexpr int64_t kGemvLdsMaxMK = 28672;      // a' (M*K*2 bytes) within 56 KB
constexpr int kGemvLdsMaxBytes = 160 * 1024;  // the CU's LDS

struct GemvPlan {
    int csw, waves, rows16, upt;
    size_t lds;
};

// Shape rule for the LDS kernel: the fewest chunk-sets per wave CSW in
// {1, 2, 4, 8} (at least kGemvMinCsw) that keeps the block within 16 waves;
// R 16-row blocks per workgroup (the activation prep is shared by R times
// more rows).
static bool gemv_lds_plan(const GemmArgs& a, GemvPlan* pl) {
    if (a.bf16 || a.M > 4 || a.K % 256 != 0 || a.M * a.K > kGemvLdsMaxMK) return false;
    const int64_t cs = a.K / 256;
    int c = kGemvMinCsw;
    while (c > 1 && (cs + c / 2 - 1) / (c / 2) <= 4) c /= 2;  // keep at least 4 waves when K is short
    while (c <= 8 && (cs + c - 1) / c > 16) c *= 2;
    if (c > 8) return false;
    pl->csw = c;
    pl->waves = (int)((cs + c - 1) / c);
    const int64_t nrb = (a.N + 15) / 16;
    // two 16-row blocks per workgroup: for M = 2 once 256 workgroups remain;
    // for M = 1 only on very tall matrices (measured: slower at 1792
    // row-blocks, faster at 3584)
    pl->rows16 = (c <= 4 && pl->waves >= 2 && (a.M > 1 ? nrb >= 512 : nrb >= 3072)) ? 2 : 1;
    pl->upt = (int)((a.M * c + 3) / 4);  // <= 4: CSW = 8 only for K > 4096 * 4, where M * K <= 28672 keeps M = 1
    pl->lds = gemv_lds_bytes(a.M, c, pl->waves, pl->rows16);
    return pl->lds <= (size_t)kGemvLdsMaxBytes;
}

template <int R, int CSW, int UPT>
static hipError_t launch_gemv_lds(const GemmArgs& a, const GemvPlan& pl, hipStream_t s) {
    static DeviceFlags lds_limit_set;
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&ternary_gemv_lds_kernel<R, CSW, UPT>),
                                   kGemvLdsMaxBytes, lds_limit_set);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((a.N + 16 * R - 1) / (16 * R)));
    ternary_gemv_lds_kernel<R, CSW, UPT><<<grid, dim3(pl.waves * kWave), pl.lds, s>>>(a);
    return hipGetLastError();
}

template <int R, int CSW>
static hipError_t launch_gemv_lds_upt(const GemmArgs& a, const GemvPlan& pl, hipStream_t s) {
    switch (pl.upt) {
        case 1: return launch_gemv_lds<R, CSW, 1>(a, pl, s);
        case 2: return launch_gemv_lds<R, CSW, 2>(a, pl, s);
        case 3: return launch_gemv_lds<R, CSW, 3>(a, pl, s);
        default: return launch_gemv_lds<R, CSW, 4>(a, pl, s);
    }
}

// Shape rule for the M = 1 kernel: CSW = 4 chunk-sets per wave (8 when that
// would need more than 16 waves), every wave a full share of K, at least 4
// waves; two 16-row blocks per workgroup on the same very tall matrices as
// the LDS kernel, and with CSW = 8 once that still fills the compute units.
// Anything else runs the LDS kernel.
struct GemvM1Plan {
    int csw, waves, rows16, mt;
    size_t lds;
};
#ifndef TQ_TERNARY_SMALL_MAX_M
#define TQ_TERNARY_SMALL_MAX_M 4
#endif
constexpr int64_t kTernarySmallMaxM = TQ_TERNARY_SMALL_MAX_M;  // largest M the small-M kernel takes

#ifndef TQ_M1_R2_MIN
#define TQ_M1_R2_MIN 3072
#endif
constexpr int64_t kM1TwoBlockRows16 = TQ_M1_R2_MIN;  // 16-row blocks from which R = 2

static bool gemv_m1_plan(const GemmArgs& a, GemvM1Plan* pl) {
    if (a.M < 1 || a.M > kTernarySmallMaxM || a.K % 1024 != 0 || a.N % 16 != 0) return false;
    const int64_t cs = a.K / 256;
    const int c = cs > 64 ? 8 : 4;
    if (cs % c != 0 || cs / c < 4 || cs / c > 16) return false;
    pl->csw = c;
    pl->waves = (int)(cs / c);
    const int64_t nrb = a.N / 16;
    pl->rows16 = (c == 4 && nrb >= kM1TwoBlockRows16 && nrb % 2 == 0) ? 2 : 1;
    // Eight chunk-sets per wave take 78 VGPRs (6 waves per SIMD), so only one
    // 14-wave workgroup fits a compute unit; with two row-blocks each, one
    // round of workgroups covers the grid when it has at least 2 per CU.
    if (c == 8 && nrb % 2 == 0 && nrb >= 2 * (int64_t)compute_units()) pl->rows16 = 2;
    pl->mt = a.M == 1 ? 1 : a.M == 2 ? 2 : 4;
    // With four rows held a wave carries ~390 VALU instructions instead of
    // ~250: it wins where the grid has few waves per SIMD (Llama-3-8B o and
    // qkv, and down, which the streaming kernel must split along K) and loses
    // where it has many (gate_up: 7 per SIMD, 14.0 against 10.3 us).
    if (a.M >= 3 && nrb / pl->rows16 * pl->waves > 16 * (int64_t)compute_units()) return false;
    pl->lds = (size_t)pl->waves * pl->mt * c * 512 + (size_t)pl->waves * pl->rows16 * pl->mt * 64;
    return pl->lds <= (size_t)kGemvLdsMaxBytes;
}

template <class T, int R, int CSW, int MT, int VAR>
static hipError_t launch_gemv_m1_k(const GemmArgs& a, const GemvM1Plan& pl, hipStream_t s) {
    static DeviceFlags lds_limit_set;
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&ternary_gemv_m1_kernel<T, R, CSW, MT, VAR>),
                                   kGemvLdsMaxBytes, lds_limit_set);
    if (e != hipSuccess) return e;
    if (a.N % (16 * R) != 0 || a.K != (int64_t)pl.waves * CSW * 256 || a.M > MT) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(a.N / (16 * R)));
    ternary_gemv_m1_kernel<T, R, CSW, MT, VAR><<<grid, dim3(pl.waves * kWave), pl.lds, s>>>(a);
    return hipGetLastError();
}

template <class T, int R, int CSW, int VAR>
static hipError_t launch_gemv_m1_t(const GemmArgs& a, const GemvM1Plan& pl, hipStream_t s) {
    if (pl.mt == 1) return launch_gemv_m1_k<T, R, CSW, 1, VAR>(a, pl, s);
    if (VAR != 0) return hipErrorInvalidValue;  // measurement variants: M = 1 only
    if (pl.mt == 2) return launch_gemv_m1_k<T, R, CSW, 2, 0>(a, pl, s);
    return launch_gemv_m1_k<T, R, CSW, 4, 0>(a, pl, s);
}

template <int R, int CSW, int VAR = 0>
static hipError_t launch_gemv_m1(const GemmArgs& a, const GemvM1Plan& pl, hipStream_t s) {
    return a.bf16 ? launch_gemv_m1_t<BF16, R, CSW, VAR>(a, pl, s) : launch_gemv_m1_t<F16, R, CSW, VAR>(a, pl, s);
}

template <int VAR>
static hipError_t launch_gemv_m1_plan(const GemmArgs& a, const GemvM1Plan& m1, hipStream_t s) {
    if (m1.csw == 8 && m1.rows16 == 2) return launch_gemv_m1<2, 8, VAR>(a, m1, s);
    if (m1.csw == 8) return launch_gemv_m1<1, 8, VAR>(a, m1, s);
    return m1.rows16 == 2 ? launch_gemv_m1<2, 4, VAR>(a, m1, s) : launch_gemv_m1<1, 4, VAR>(a, m1, s);
}

// Measurement variants of the M = 1 kernel (see ternary_gemv_m1_kernel):
// variant 0 is the kernel the dispatcher runs, 1 reads cached codes, 2 also
// skips the matrix-core step.  Shapes the M = 1 kernel does not take fail.
hipError_t launch_ternary_gemv_variant(const GemmArgs& a, int variant, hipStream_t s) {
    GemvM1Plan m1;
    if (a.M != 1 || !gemv_m1_plan(a, &m1)) return hipErrorInvalidValue;
    if (variant == 0) return launch_gemv_m1_plan<0>(a, m1, s);
    if (variant == 1) return launch_gemv_m1_plan<1>(a, m1, s);
    if (variant == 2) return launch_gemv_m1_plan<2>(a, m1, s);
    return hipErrorInvalidValue;
}

// Streaming kernel: fp16, 3 <= M <= 16, at most 32 chunk-sets (8192
// columns) per workgroup (one or two per wave, at most 16 waves); for M <= 2
// the LDS kernel is faster, its per-wave activation prep being cheaper than
// building the operand in every wave.  T row-blocks per workgroup: the
// fewest (any count from 1) that keep the grid within one workgroup per
// compute unit (at most 8; at most 4 with two chunk-sets per wave, for
// registers; at most the wave count, which the final reduction needs).  The waves' LDS areas must fit the compute
// unit's LDS, which rules out two chunk-sets per wave for M > 8.  S splits of
// K when a workspace allows.
struct StreamPlan {
    int csw, waves, t, S, mr;
    size_t lds;
};

int compute_units() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev].store(v, std::memory_order_relaxed);
    return v;
}

// Geometry of the streaming kernel with K split S ways (false if it does not
// fit: S must divide the chunk-sets, a split keeps at least four).
// Row-blocks per workgroup for the streaming kernels: the fewest that keep
// the grid (S splits) within one workgroup per compute unit, at most tmax
// (registers) and at most the wave count (the final reduction).  Any count
// from 1 to tmax is instantiated, so that e.g. 1792 row-blocks take 7 per
// workgroup and fill 256 compute units instead of 224 with 8.
static int stream_rows_per_wg(int64_t nrb, int S, int64_t cus, int tmax, int waves) {
    const int cap = tmax < waves ? tmax : waves;
    for (int t = 1; t <= cap; ++t)
        if ((nrb + t - 1) / t * S <= cus) return t;
    // No count fits one round: the largest power of two within the cap (a
    // capped count in between would only make each of the rounds longer).
    int t = 1;
    while (2 * t <= cap) t *= 2;
    return t;
}

static bool stream_geometry(const GemmArgs& a, int S, int64_t cus, StreamPlan* pl) {
    const int64_t cs_all = a.K / 256;
    if (S < 1 || cs_all % S != 0) return false;
    const int64_t cs = cs_all / S;
    if (cs > 32 || (S > 1 && cs < 4)) return false;
    pl->S = S;
    pl->csw = cs <= 16 ? 1 : 2;
    pl->waves = (int)((cs + pl->csw - 1) / pl->csw);
    const int64_t nrb = (a.N + 15) / 16;
    pl->mr = a.M <= 4 ? 4 : a.M <= 8 ? 8 : 16;
    pl->t = stream_rows_per_wg(nrb, S, cus, pl->csw == 1 ? 8 : 4, pl->waves);
    pl->lds = (size_t)pl->waves * stream_wave_lds(pl->csw, pl->mr, pl->t);
    return pl->lds <= (size_t)kGemvLdsMaxBytes;
}

// Bytes one compute unit moves, as a cost: per workgroup the activations of
// its K range (M * K/S * 2), its codes and, with a split, its fp32 partials
// (written, then read back by the reduction), times the workgroups queued per
// compute unit; a split also adds the reduction launch, counted as 160 KB
// (what a compute unit takes in over the ~2.4 us a launch costs at the
// measured ~65 KB/us per compute unit).
static int64_t stream_cost(const GemmArgs& a, const StreamPlan& pl, int64_t cus) {
    const int64_t kr = a.K / pl.S;
    const int64_t per_wg = 2 * a.M * kr + (int64_t)pl.t * 16 * (kr / 4) +
                           (pl.S > 1 ? (int64_t)pl.t * 16 * a.M * 8 : 0);
    const int64_t nrb = (a.N + 15) / 16;
    const int64_t wgs = (nrb + pl.t - 1) / pl.t * pl.S;
    return (wgs + cus - 1) / cus * per_wg + (pl.S > 1 ? 160 * 1024 : 0);
}

// Cheapest streaming plan whose split fits `ws_bytes` of workspace.
static bool gemv_stream_plan(const GemmArgs& a, size_t ws_bytes, StreamPlan* pl) {
    // K <= 2^20 keeps the kernel's 32-bit lane offsets in range (the
    // geometry already bounds K far lower)
    if (a.M < 3 || a.M > kGemvMaxM || a.K % 256 != 0 || a.K > (int64_t(1) << 20)) return false;
    const int64_t cus = compute_units();
    bool found = false;
    int64_t best = 0;
    for (int S = 1; S <= 16; ++S) {
        StreamPlan c;
        if (!stream_geometry(a, S, cus, &c)) continue;
        if (S > 1 && ws_bytes < (size_t)S * (size_t)a.M * (size_t)a.N * sizeof(float)) continue;
        const int64_t cost = stream_cost(a, c, cus);
        if (!found || cost < best) {
            *pl = c;
            best = cost;
            found = true;
        }
    }
    return found;
}

size_t gemv_workspace_bytes(const GemmArgs& a) {
    GemvM1Plan m1;
    if (gemv_m1_plan(a, &m1)) return 0;  // the small-M kernel never splits K
    StreamPlan pl;
    if (!gemv_stream_plan(a, SIZE_MAX, &pl) || pl.S == 1) return 0;
    return (size_t)pl.S * (size_t)a.M * (size_t)a.N * sizeof(float);
}

template <class AT, int CSW, int T, int MR>
static hipError_t launch_gemv_stream_at(const SplitArgs& sa, const StreamPlan& pl, hipStream_t s) {
    static DeviceFlags lds_limit_set;
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&ternary_gemv_stream_kernel<AT, CSW, T, MR>),
                                   kGemvLdsMaxBytes, lds_limit_set);
    if (e != hipSuccess) return e;
    if (pl.lds != (size_t)pl.waves * stream_wave_lds(CSW, MR, T)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((sa.g.N + 16 * T - 1) / (16 * T)), (unsigned)sa.S);
    SplitArgs k = sa;
    k.flags = split_flags(sa.flags, sa.S, grid.x);
    ternary_gemv_stream_kernel<AT, CSW, T, MR><<<grid, dim3(pl.waves * kWave), pl.lds, s>>>(k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return sa.S > 1 && !k.flags ? launch_splitk_reduce(sa, s) : hipSuccess;
}

template <int CSW, int T, int MR>
static hipError_t launch_gemv_stream(const SplitArgs& sa, const StreamPlan& pl, hipStream_t s) {
    return sa.g.bf16 ? launch_gemv_stream_at<BF16, CSW, T, MR>(sa, pl, s) : launch_gemv_stream_at<F16, CSW, T, MR>(sa, pl, s);
}

template <int MR>
static hipError_t launch_gemv_stream_mr(const SplitArgs& sa, const StreamPlan& sp, hipStream_t s) {
    if (sp.csw == 1) {
        switch (sp.t) {
            case 1: return launch_gemv_stream<1, 1, MR>(sa, sp, s);
            case 2: return launch_gemv_stream<1, 2, MR>(sa, sp, s);
            case 3: return launch_gemv_stream<1, 3, MR>(sa, sp, s);
            case 4: return launch_gemv_stream<1, 4, MR>(sa, sp, s);
            case 5: return launch_gemv_stream<1, 5, MR>(sa, sp, s);
            case 6: return launch_gemv_stream<1, 6, MR>(sa, sp, s);
            case 7: return launch_gemv_stream<1, 7, MR>(sa, sp, s);
            default: return launch_gemv_stream<1, 8, MR>(sa, sp, s);
        }
    }
    if constexpr (MR == 16) {
        return hipErrorInvalidValue;  // 16 waves x 16 KB of activations exceed the LDS: the plan never asks for it
    } else {
        switch (sp.t) {
            case 1: return launch_gemv_stream<2, 1, MR>(sa, sp, s);
            case 2: return launch_gemv_stream<2, 2, MR>(sa, sp, s);
            case 3: return launch_gemv_stream<2, 3, MR>(sa, sp, s);
            default: return launch_gemv_stream<2, 4, MR>(sa, sp, s);
        }
    }
}

static hipError_t launch_gemv_stream_t(const SplitArgs& sa, const StreamPlan& sp, hipStream_t s) {
    if (sp.mr == 4) return launch_gemv_stream_mr<4>(sa, sp, s);
    if (sp.mr == 8) return launch_gemv_stream_mr<8>(sa, sp, s);
    return launch_gemv_stream_mr<16>(sa, sp, s);
}

hipError_t launch_ternary_gemv(const GemmArgs& a, hipStream_t s) { return launch_ternary_gemv(a, nullptr, 0, s); }

hipError_t launch_ternary_gemv(const GemmArgs& a, void* workspace, size_t workspace_bytes, hipStream_t s,
                               uint32_t* flags) {
    GemvM1Plan m1;
    if (gemv_m1_plan(a, &m1)) return launch_gemv_m1_plan<0>(a, m1, s);
    StreamPlan sp;
    if (gemv_stream_plan(a, workspace ? workspace_bytes : 0, &sp))
        return launch_gemv_stream_t(SplitArgs{a, static_cast<float*>(workspace), sp.S, 0, 0, flags}, sp, s);
    GemvPlan pl;
    if (gemv_lds_plan(a, &pl)) {
        if (pl.rows16 == 2) {
            switch (pl.csw) {
                case 1: return launch_gemv_lds_upt<2, 1>(a, pl, s);
                case 2: return launch_gemv_lds_upt<2, 2>(a, pl, s);
                default: return launch_gemv_lds_upt<2, 4>(a, pl, s);
            }
        }
        switch (pl.csw) {
            case 1: return launch_gemv_lds_upt<1, 1>(a, pl, s);
            case 2: return launch_gemv_lds_upt<1, 2>(a, pl, s);
            case 4: return launch_gemv_lds_upt<1, 4>(a, pl, s);
            default: return launch_gemv_lds_upt<1, 8>(a, pl, s);
        }
    }
    if (ternary_gemv_mfma_ok(a)) {
        if (a.M <= 4) launch_gemv_mfma_w<2>(a, s);
        else launch_gemv_mfma_w<4>(a, s);
        return hipGetLastError();
    }
    return launch_ternary_gemv_simple(a, s);
}

hipError_t launch_ternary_gemv_simple(const GemmArgs& a, hipStream_t s) {
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

template <int R, int W>
static hipError_t launch_w4_mfma(const GemmArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.N + 16 * R - 1) / (16 * R)));
    w4_gemv_mfma_kernel<R, W><<<grid, W * kWave, 0, s>>>(a);
    return hipGetLastError();
}

// fp16, 3 <= M <= 16 (for M <= 2 the FMA kernel is faster: its loads are
// all in flight at once, while this kernel prefetches one group ahead): W
// waves over the K/128 groups (at most 16), two 16-row blocks per workgroup
// while at least 512 workgroups remain.
template <int R>
static hipError_t launch_w4_mfma_w(const GemmArgs& a, hipStream_t s) {
    const int64_t G = a.K / 128;
    if (G >= 16) return launch_w4_mfma<R, 16>(a, s);
    if (G >= 8) return launch_w4_mfma<R, 8>(a, s);
    if (G >= 4) return launch_w4_mfma<R, 4>(a, s);
    if (G >= 2) return launch_w4_mfma<R, 2>(a, s);
    return launch_w4_mfma<R, 1>(a, s);
}

// W4A16 streaming plan: as the ternary one, over 128-column groups.  S
// divides the groups, a workgroup takes at most 32 (one or two per wave, at
// most 16 waves), a split keeps at least four; T row-blocks per workgroup
// (at most 8, 6 with two groups per wave and zero points; at most the wave
// count);
// the waves' LDS areas must fit.  The cost is the same estimate of bytes per
// compute unit: activations (M * K/S * 2), codes, split partials, plus
// 160 KB for the reduction launch.
struct W4StreamPlan {
    int gsw, waves, t, S, mr;
    size_t lds;
};

// Two groups per wave read their scales and zero points in pairs: the pair
// offset row * G + g0 must be even (G and the groups per split even, so g0 is
// too) and the arrays aligned to the pair's size.
static bool w4_pairs_ok(const GemmArgs& a, int S) {
    const int64_t g_all = a.K / 128;
    return g_all % 2 == 0 && (g_all / S) % 2 == 0 && (reinterpret_cast<uintptr_t>(a.scale) & 3u) == 0 &&
           (reinterpret_cast<uintptr_t>(a.zeros) & 1u) == 0;
}

static bool w4_stream_geometry(const GemmArgs& a, int S, int64_t cus, W4StreamPlan* pl) {
    const int64_t g_all = a.K / 128;
    if (S < 1 || g_all % S != 0) return false;
    const int64_t gs = g_all / S;
    if (gs > 32 || (S > 1 && gs < 4)) return false;
    pl->S = S;
    pl->gsw = gs <= 16 ? 1 : 2;
    if (pl->gsw == 2 && !w4_pairs_ok(a, S)) return false;
    pl->waves = (int)((gs + pl->gsw - 1) / pl->gsw);
    pl->mr = a.M <= 4 ? 4 : a.M <= 8 ? 8 : 16;
    const int64_t nrb = (a.N + 15) / 16;
    // registers: with two groups per wave and zero points, 7 or more
    // row-blocks spill (126 VGPRs and 20 bytes of scratch at 7)
    pl->t = stream_rows_per_wg(nrb, S, cus, (pl->gsw == 2 && a.zeros) ? 6 : 8, pl->waves);
    pl->lds = (size_t)pl->waves * w4_stream_wave_lds(pl->gsw, pl->mr, pl->t);
    return pl->lds <= (size_t)kGemvLdsMaxBytes;
}

static int64_t w4_stream_cost(const GemmArgs& a, const W4StreamPlan& pl, int64_t cus) {
    const int64_t kr = a.K / pl.S;
    const int64_t per_wg = 2 * a.M * kr + (int64_t)pl.t * 16 * (kr / 2) + (pl.S > 1 ? (int64_t)pl.t * 16 * a.M * 8 : 0);
    const int64_t nrb = (a.N + 15) / 16;
    const int64_t wgs = (nrb + pl.t - 1) / pl.t * pl.S;
    return (wgs + cus - 1) / cus * per_wg + (pl.S > 1 ? 160 * 1024 : 0);
}

static bool w4_stream_plan(const GemmArgs& a, size_t ws_bytes, W4StreamPlan* pl) {
    // K <= 2^20 keeps the kernel's 32-bit lane offsets in range (the
    // geometry already bounds K far lower)
    if (a.M < 1 || a.M > kGemvMaxM || a.K % 128 != 0 || a.K > (int64_t(1) << 20)) return false;
    const int64_t cus = compute_units();
    bool found = false;
    int64_t best = 0;
    for (int S = 1; S <= 16; ++S) {
        W4StreamPlan c;
        if (!w4_stream_geometry(a, S, cus, &c)) continue;
        if (S > 1 && ws_bytes < (size_t)S * (size_t)a.M * (size_t)a.N * sizeof(float)) continue;
        const int64_t cost = w4_stream_cost(a, c, cus);
        if (!found || cost < best) {
            *pl = c;
            best = cost;
            found = true;
        }
    }
    return found;
}

// Whether the streaming kernel serves this call, and with which plan.  At
// M = 1 the per-lane kernel (one wave per row) fills the chip on its own; the
// streaming kernel wins there only without a K split (whose reduction is a
// second launch) and with a workgroup for every compute unit, so M = 1 never
// uses a workspace.  From M = 2 on it wins whenever it has a plan.
static bool w4_use_stream(const GemmArgs& a, size_t ws_bytes, W4StreamPlan* sp) {
    if (!w4_stream_plan(a, a.M == 1 ? 0 : ws_bytes, sp)) return false;
    if (a.M >= 2) return true;
    const int64_t nrb = (a.N + 15) / 16;
    return sp->S == 1 && (nrb + sp->t - 1) / sp->t >= compute_units();
}


template <class AT, int GSW, int T, int MR, bool ASYM>
static hipError_t launch_w4_stream_at(const SplitArgs& sa, const W4StreamPlan& pl, hipStream_t s) {
    if constexpr (ASYM && GSW == 2 && T > 6) {
        return hipErrorInvalidValue;  // the plan never asks for it (registers)
    } else {
        static DeviceFlags lds_limit_set;
        hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&w4_gemv_stream_kernel<AT, GSW, T, MR, ASYM>),
                                       kGemvLdsMaxBytes, lds_limit_set);
        if (e != hipSuccess) return e;
        if (pl.lds != (size_t)pl.waves * w4_stream_wave_lds(GSW, MR, T)) return hipErrorInvalidValue;
        if (GSW == 2 && !w4_pairs_ok(sa.g, sa.S)) return hipErrorInvalidValue;
        const dim3 grid((unsigned)((sa.g.N + 16 * T - 1) / (16 * T)), (unsigned)sa.S);
        SplitArgs k = sa;
        k.flags = split_flags(sa.flags, sa.S, grid.x);
        w4_gemv_stream_kernel<AT, GSW, T, MR, ASYM><<<grid, dim3(pl.waves * kWave), pl.lds, s>>>(k);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        return sa.S > 1 && !k.flags ? launch_splitk_reduce(sa, s) : hipSuccess;
    }
}

template <int GSW, int T, int MR, bool ASYM>
static hipError_t launch_w4_stream_k(const SplitArgs& sa, const W4StreamPlan& pl, hipStream_t s) {
    return sa.g.bf16 ? launch_w4_stream_at<BF16, GSW, T, MR, ASYM>(sa, pl, s)
                     : launch_w4_stream_at<F16, GSW, T, MR, ASYM>(sa, pl, s);
}

template <int GSW, int T, int MR>
static hipError_t launch_w4_stream(const SplitArgs& sa, const W4StreamPlan& pl, hipStream_t s) {
    return sa.g.zeros ? launch_w4_stream_k<GSW, T, MR, true>(sa, pl, s) : launch_w4_stream_k<GSW, T, MR, false>(sa, pl, s);
}

template <int MR>
static hipError_t launch_w4_stream_mr(const SplitArgs& sa, const W4StreamPlan& pl, hipStream_t s) {
    if (pl.gsw == 1) {
        switch (pl.t) {
            case 1: return launch_w4_stream<1, 1, MR>(sa, pl, s);
            case 2: return launch_w4_stream<1, 2, MR>(sa, pl, s);
            case 3: return launch_w4_stream<1, 3, MR>(sa, pl, s);
            case 4: return launch_w4_stream<1, 4, MR>(sa, pl, s);
            case 5: return launch_w4_stream<1, 5, MR>(sa, pl, s);
            case 6: return launch_w4_stream<1, 6, MR>(sa, pl, s);
            case 7: return launch_w4_stream<1, 7, MR>(sa, pl, s);
            default: return launch_w4_stream<1, 8, MR>(sa, pl, s);
        }
    }
    switch (pl.t) {
        case 1: return launch_w4_stream<2, 1, MR>(sa, pl, s);
        case 2: return launch_w4_stream<2, 2, MR>(sa, pl, s);
        case 3: return launch_w4_stream<2, 3, MR>(sa, pl, s);
        case 4: return launch_w4_stream<2, 4, MR>(sa, pl, s);
        case 5: return launch_w4_stream<2, 5, MR>(sa, pl, s);
        case 6: return launch_w4_stream<2, 6, MR>(sa, pl, s);
        case 7: return launch_w4_stream<2, 7, MR>(sa, pl, s);
        default: return launch_w4_stream<2, 8, MR>(sa, pl, s);
    }
}

static hipError_t launch_w4_stream_t(const SplitArgs& sa, const W4StreamPlan& pl, hipStream_t s) {
    if (pl.mr == 4) return launch_w4_stream_mr<4>(sa, pl, s);
    if (pl.mr == 8) return launch_w4_stream_mr<8>(sa, pl, s);
    return launch_w4_stream_mr<16>(sa, pl, s);
}

hipError_t launch_w4_gemv(const GemmArgs& a, hipStream_t s) { return launch_w4_gemv(a, nullptr, 0, s); }

// Shape rule for the W4A16 M = 1 kernel: GSW = 4 groups per wave (8 when
// that would need more than 16 waves), every wave a full share of K, at
// least 4 waves, scales 8-byte and zero points 4-byte aligned (a wave reads
// aligned runs of them); two 16-row blocks per workgroup when one-block
// workgroups would hold more than 8 waves per SIMD.  Other shapes take the
// kernels below.
struct W4M1Plan {
    int gsw, waves, rows16, mt;
    size_t lds;
};
#ifndef TQ_W4_SMALL_MAX_M
#define TQ_W4_SMALL_MAX_M 4
#endif
constexpr int64_t kW4SmallMaxM = TQ_W4_SMALL_MAX_M;  // largest M the small-M kernel takes

static bool w4_m1_plan(const GemmArgs& a, W4M1Plan* pl) {
    if (a.M < 1 || a.M > kW4SmallMaxM || a.K % 512 != 0 || a.N % 16 != 0) return false;
    if ((reinterpret_cast<uintptr_t>(a.scale) & 7u) != 0 || (reinterpret_cast<uintptr_t>(a.zeros) & 3u) != 0)
        return false;
    const int64_t G = a.K / 128;
    const int c = G > 64 ? 8 : 4;
    if (G % c != 0 || G / c < 4 || G / c > 16) return false;
    pl->gsw = c;
    pl->waves = (int)(G / c);
    const int64_t nrb = a.N / 16;
    pl->rows16 = (nrb % 2 == 0 && nrb * pl->waves > 32 * (int64_t)compute_units()) ? 2 : 1;
    pl->mt = a.M == 1 ? 1 : a.M == 2 ? 2 : 4;
    pl->lds = (size_t)pl->waves * pl->mt * c * 256 + (size_t)pl->waves * pl->rows16 * pl->mt * 64;
    return pl->lds <= (size_t)kGemvLdsMaxBytes;
}

template <class T, int R, int GSW, bool ASYM, int MT>
static hipError_t launch_w4_m1_k(const GemmArgs& a, const W4M1Plan& pl, hipStream_t s) {
    static DeviceFlags lds_limit_set;
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&w4_gemv_m1_kernel<T, R, GSW, ASYM, MT>),
                                   kGemvLdsMaxBytes, lds_limit_set);
    if (e != hipSuccess) return e;
    if (a.N % (16 * R) != 0 || a.K != (int64_t)pl.waves * GSW * 128 || a.M > MT) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(a.N / (16 * R)));
    w4_gemv_m1_kernel<T, R, GSW, ASYM, MT><<<grid, dim3(pl.waves * kWave), pl.lds, s>>>(a);
    return hipGetLastError();
}

template <class T, int R, int GSW, bool ASYM>
static hipError_t launch_w4_m1_mt(const GemmArgs& a, const W4M1Plan& pl, hipStream_t s) {
    if (pl.mt == 1) return launch_w4_m1_k<T, R, GSW, ASYM, 1>(a, pl, s);
    if (pl.mt == 2) return launch_w4_m1_k<T, R, GSW, ASYM, 2>(a, pl, s);
    return launch_w4_m1_k<T, R, GSW, ASYM, 4>(a, pl, s);
}

template <class T, int R, int GSW>
static hipError_t launch_w4_m1_t(const GemmArgs& a, const W4M1Plan& pl, hipStream_t s) {
    return a.zeros ? launch_w4_m1_mt<T, R, GSW, true>(a, pl, s) : launch_w4_m1_mt<T, R, GSW, false>(a, pl, s);
}

template <int R, int GSW>
static hipError_t launch_w4_m1(const GemmArgs& a, const W4M1Plan& pl, hipStream_t s) {
    return a.bf16 ? launch_w4_m1_t<BF16, R, GSW>(a, pl, s) : launch_w4_m1_t<F16, R, GSW>(a, pl, s);
}

size_t w4_gemv_workspace_bytes(const GemmArgs& a) {
    W4M1Plan m1;
    if (w4_m1_plan(a, &m1)) return 0;  // the small-M kernel never splits K
    W4StreamPlan pl;
    if (a.M == 1 || !w4_stream_plan(a, SIZE_MAX, &pl) || pl.S == 1) return 0;
    return (size_t)pl.S * (size_t)a.M * (size_t)a.N * sizeof(float);
}

static hipError_t launch_w4_m1_plan(const GemmArgs& a, const W4M1Plan& m1, hipStream_t s) {
    if (m1.gsw == 8) return m1.rows16 == 2 ? launch_w4_m1<2, 8>(a, m1, s) : launch_w4_m1<1, 8>(a, m1, s);
    return m1.rows16 == 2 ? launch_w4_m1<2, 4>(a, m1, s) : launch_w4_m1<1, 4>(a, m1, s);
}

hipError_t launch_w4_gemv(const GemmArgs& a, void* workspace, size_t workspace_bytes, hipStream_t s,
                          uint32_t* flags) {
    W4M1Plan m1;
    if (w4_m1_plan(a, &m1)) return launch_w4_m1_plan(a, m1, s);
    W4StreamPlan sp;
    if (w4_use_stream(a, workspace ? workspace_bytes : 0, &sp))
        return launch_w4_stream_t(SplitArgs{a, static_cast<float*>(workspace), sp.S, 1, 0, flags}, sp, s);
    // bf16 shapes the streaming kernel cannot take: the small-M kernel over
    // blocks of kW4SmallMaxM rows, reading the weights once per block, which
    // still beats the per-lane FMA kernel several times over
    if (a.bf16 && a.M > kW4SmallMaxM) {
        GemmArgs b = a;
        b.M = kW4SmallMaxM;
        if (w4_m1_plan(b, &m1)) {
            for (int64_t m0 = 0; m0 < a.M; m0 += kW4SmallMaxM) {
                b.A = a.A + m0 * a.K;
                b.C = a.C + m0 * a.N;
                b.M = std::min<int64_t>(kW4SmallMaxM, a.M - m0);
                W4M1Plan pb;
                if (!w4_m1_plan(b, &pb)) return hipErrorInvalidValue;
                const hipError_t e = launch_w4_m1_plan(b, pb, s);
                if (e != hipSuccess) return e;
            }
            return hipSuccess;
        }
    }
    if (!a.bf16 && a.M >= 3 && a.M <= kGemvMaxM && !a.zeros) {  // zero point 8 only
        const int64_t nrb = (a.N + 15) / 16;
        return nrb >= 1024 ? launch_w4_mfma_w<2>(a, s) : launch_w4_mfma_w<1>(a, s);
    }
    return launch_w4_gemv_simple(a, s);
}

// A_perm[m, i] = A[m, perm[i]], the index clamped into [0, K) (an index out
// of range takes column i), so any perm contents stay in bounds.  K % 8 == 0
// and a 16-byte aligned output.  Thread t of block (x, y) owns columns
// 8c .. 8c+7, c = 256 x + t: it loads their eight indices once and gathers
// them from rows y R, y R + gridDim.y R, ... (R consecutive rows each: 1
// while M is small, so that the grid still has M blocks per 2048 columns),
// storing each row's eight values as one 16-byte write.  A row of A is at
// most a few tens of KB, so the scattered 2-byte reads of a row hit the
// cache after the first.

__global__ __launch_bounds__(256) void gather_columns_kernel(const uint16_t* __restrict__ A,
                                                             const int32_t* __restrict__ perm, int64_t M,
                                                             int64_t K, int R, uint16_t* __restrict__ out) {
    const int64_t c0 = 8 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (c0 >= K) return;
    int64_t k[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t v = perm[c0 + j];
        k[j] = v < 0 || v >= K ? c0 + j : v;
    }
    for (int64_t m0 = (int64_t)blockIdx.y * R; m0 < M; m0 += (int64_t)gridDim.y * R) {
        for (int r = 0; r < R; ++r) {
            const int64_t m = m0 + r;
            if (m >= M) break;
            const uint16_t* src = A + m * K;
            uint16_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = src[k[j]];
            *reinterpret_cast<uint4*>(out + m * K + c0) =
                make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16), v[4] | ((uint32_t)v[5] << 16),
                           v[6] | ((uint32_t)v[7] << 16));
        }
    }
}

// Large M: block b owns rows b R .. b R + R - 1, R = kGatherLdsBytes / (2 K)
// rows (at most 8): they are copied to LDS with 16-byte loads, then each
// thread gathers eight columns at a time from LDS (indices loaded once for
// the block's rows) and stores 16 bytes per row.  The global traffic is the
// rows read once and written once; the scattered reads stay on chip.  Same
// index clamp and alignment as above; A 16-byte aligned.
constexpr int kGatherLdsBytes = 64 << 10;

__global__ __launch_bounds__(256) void gather_columns_lds_kernel(const uint16_t* __restrict__ A,
                                                                 const int32_t* __restrict__ perm, int64_t M,
                                                                 int64_t K, int R, uint16_t* __restrict__ out) {
    extern __shared__ uint4 smem_gather[];
    const uint16_t* rows = reinterpret_cast<const uint16_t*>(smem_gather);
    const int64_t m0 = (int64_t)blockIdx.x * R;
    const int nr = (int)(M - m0 < R ? M - m0 : R);
    const int64_t chunks = K / 8;  // 16-byte chunks per row
    const uint4* src = reinterpret_cast<const uint4*>(A + m0 * K);
    for (int64_t e = threadIdx.x; e < nr * chunks; e += 256) smem_gather[e] = src[e];
    __syncthreads();
    for (int64_t c = threadIdx.x; c < chunks; c += 256) {
        int32_t k[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t v = perm[8 * c + j];
            k[j] = (int32_t)(v < 0 || v >= K ? 8 * c + j : v);
        }
        for (int r = 0; r < nr; ++r) {
            const uint16_t* row = rows + (int64_t)r * K;
            uint16_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = row[k[j]];
            *reinterpret_cast<uint4*>(out + (m0 + r) * K + 8 * c) =
                make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16), v[4] | ((uint32_t)v[5] << 16),
                           v[6] | ((uint32_t)v[7] << 16));
        }
    }
}

hipError_t launch_gather_columns(const uint16_t* A, const int32_t* perm, int64_t M, int64_t K, uint16_t* out,
                                 hipStream_t s) {
    if (K % 8 != 0 || (reinterpret_cast<uintptr_t>(out) & 15u) != 0) return hipErrorInvalidValue;
    if (M <= 0 || K <= 0) return hipSuccess;
    if (M > 64 && 2 * K <= kGatherLdsBytes && (reinterpret_cast<uintptr_t>(A) & 15u) == 0) {
        int64_t R = kGatherLdsBytes / (2 * K);
        if (R > 8) R = 8;
        static DeviceFlags lds_limit_set;
        hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&gather_columns_lds_kernel), kGatherLdsBytes,
                                       lds_limit_set);
        if (e != hipSuccess) return e;
        const size_t lds = (size_t)R * (size_t)K * 2;
        gather_columns_lds_kernel<<<(unsigned)((M + R - 1) / R), 256, lds, s>>>(A, perm, M, K, (int)R, out);
        return hipGetLastError();
    }
    const int R = M <= 64 ? 1 : 8;
    const int64_t gy = (M + R - 1) / R;
    const dim3 grid((unsigned)((K / 8 + 255) / 256), (unsigned)(gy < 65535 ? gy : 65535));
    gather_columns_kernel<<<grid, 256, 0, s>>>(A, perm, M, K, R, out);
    return hipGetLastError();
}

hipError_t launch_w4_gemv_simple(const GemmArgs& a, hipStream_t s) {
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
