// Device helpers shared by the HIP kernels of libtq (gfx950, wave64).
//
// Conversions are written from the IEEE-754 format definitions on integer
// bit patterns, so their rounding never depends on the hardware mode
// register: binary16 = 1 sign, 5 exponent (bias 15), 10 fraction bits;
// bfloat16 = the top half of binary32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// fp64 -> binary16 bit pattern, rounded once to nearest, ties to even.
// Magnitudes that round past 65504 give infinity; NaN gives 0x7E00.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a >= 0x7FF0000000000000ull)  // inf or NaN
        return (uint16_t)(a > 0x7FF0000000000000ull ? 0x7E00u : (sign | 0x7C00u));
    const int e = (int)(a >> 52) - 1023;  // exponent of a normal double
    if (e < -25) return (uint16_t)sign;   // below half the smallest subnormal (2^-25)
    const uint64_t m = (a & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;  // 53-bit significand
    int E = e < -14 ? -14 : e;            // binade of the result (subnormals share -14)
    const int shift = 42 + E - e;         // 52 - 10 + (E - e): to units of 2^(E-10)
    uint64_t r = m >> shift;
    const uint64_t rem = m & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (r & 1))) ++r;
    if (r == 2048) { ++E; r = 1024; }     // carried into the next binade
    if (E + 15 >= 31) return (uint16_t)(sign | 0x7C00u);
    const uint32_t bits = (E == -14) ? (uint32_t)r : ((uint32_t)(E + 15) << 10) + (uint32_t)(r - 1024);
    return (uint16_t)(sign | bits);
}

// binary32 -> binary16 bit pattern, round to nearest even (same construction).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x7F800000u) return (uint16_t)(a > 0x7F800000u ? 0x7E00u : (sign | 0x7C00u));
    const int e = (int)(a >> 23) - 127;
    if (e < -25) return (uint16_t)sign;
    const uint32_t m = (a & 0x007FFFFFu) | 0x00800000u;  // 24-bit significand
    int E = e < -14 ? -14 : e;
    const int shift = 13 + E - e;  // 23 - 10 + (E - e), in [13, 24]
    uint32_t r = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (r & 1))) ++r;
    if (r == 2048) { ++E; r = 1024; }
    if (E + 15 >= 31) return (uint16_t)(sign | 0x7C00u);
    const uint32_t bits = (E == -14) ? r : ((uint32_t)(E + 15) << 10) + (r - 1024);
    return (uint16_t)(sign | bits);
}

// binary32 -> bfloat16 bit pattern, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Exact value of a binary16 bit pattern.
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
    return (double)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// Constants the compiler cannot fold back into literals.  A VOP3 instruction
// on this target reads at most one scalar value and no literal, so with both
// operands of (x & mask) | magic as literals the compiler splits the pattern
// into v_and_b32 + v_or_b32; with the mask in an SGPR and the magic in a VGPR
// it selects a single v_and_or_b32.  Only the constants are opaque: the
// arithmetic stays visible to the compiler, which therefore still inserts
// the wait states a matrix instruction needs after a VALU write.
template <uint32_t C>
__device__ __forceinline__ uint32_t sgpr_const() {
    uint32_t r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(C));
    return r;
}
template <uint32_t C>
__device__ __forceinline__ uint32_t vgpr_const() {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(C));
    return r;
}

// A register value the compiler treats as defined but whose contents are
// whatever the registers hold: no instruction is emitted.  For operands whose
// results are discarded.
__device__ __forceinline__ uint4 opaque_uint4() {
    uint4 v;
    asm volatile("" : "=v"(v.x), "=v"(v.y), "=v"(v.z), "=v"(v.w));
    return v;
}

// Activation element type tags.
// from_f32 rounds in software (mode-independent); from_f32_fast uses the
// hardware conversion, which rounds to nearest even under the default mode
// register and keeps fp16 subnormals.  The output stores use the latter:
// the software rounding cost about 15 instructions per value in epilogues
// that one wave runs while the others wait.
struct F16 {
    static __device__ __forceinline__ float to_f32(uint16_t h) { return f16_bits_to_f32(h); }
    static __device__ __forceinline__ uint16_t from_f32(float x) { return f32_to_f16_rne(x); }
    static __device__ __forceinline__ uint16_t from_f32_fast(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
};
struct BF16 {
    static __device__ __forceinline__ float to_f32(uint16_t h) { return bf16_bits_to_f32(h); }
    static __device__ __forceinline__ uint16_t from_f32(float x) { return f32_to_bf16_rne(x); }
    static __device__ __forceinline__ uint16_t from_f32_fast(float x) { return f32_to_bf16_rne(x); }
};

// ---- fp16 a' unpack of ternary codes (the scheme is laid out at the
// matrix-core GEMV in gemv.hip): field I of a code dword x, masked into the
// mantissa of 1024.0, is the pair (1024 + 4^s c_I, 1024 + 4^s c_{I+8}),
// s = I for I < 5 and I - 5 (after x >> 10) otherwise; the activations of
// the same columns are paired and pre-scaled by 1 / 4^s to match.

constexpr uint32_t kMagic2 = 0x64006400u;  // (1024.0, 1024.0) as fp16

template <int I>
__device__ __forceinline__ uint32_t field_pair(uint32_t x, uint32_t y, uint32_t magic_v) {
    if constexpr (I < 5) return (x & sgpr_const<(0x00030003u << (2 * I))>()) | magic_v;
    else return (y & sgpr_const<(0x00030003u << (2 * (I - 5)))>()) | magic_v;
}

// 1 / 4^s for field I, as an fp16 pair.
template <int I>
__device__ __forceinline__ f16x2 inv_mult() {
    constexpr int s = I < 5 ? I : I - 5;
    const _Float16 v = (_Float16)(1.0f / (float)(1 << (2 * s)));
    return f16x2{v, v};
}

// -(1024 + 4^s) for field I in both halves (the code-01 pattern, negated).
template <int I>
__device__ __forceinline__ constexpr uint32_t neg_one_pattern() {
    constexpr int s = I < 5 ? I : I - 5;
    return 0xE400E400u | (0x00010001u << (2 * s));
}

// a' pair for field I of code dword D: (a[16D+I], a[16D+I+8]) / 4^s(I).
template <int D, int I>
__device__ __forceinline__ uint32_t a_pair(const uint4 av[8]) {
    const uint4& lo4 = av[2 * D];
    const uint4& hi4 = av[2 * D + 1];
    constexpr int c = I / 2;
    const uint32_t lo = c == 0 ? lo4.x : c == 1 ? lo4.y : c == 2 ? lo4.z : lo4.w;
    const uint32_t hi = c == 0 ? hi4.x : c == 1 ? hi4.y : c == 2 ? hi4.z : hi4.w;
    const uint32_t pr = __builtin_amdgcn_perm(hi, lo, (I & 1) ? 0x07060302u : 0x05040100u);
    const f16x2 v = __builtin_bit_cast(f16x2, pr) * inv_mult<I>();
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t dword_of(const uint4& q, int d) {
    return d == 0 ? q.x : d == 1 ? q.y : d == 2 ? q.z : q.w;
}

template <int I>
__device__ __forceinline__ constexpr uint32_t one_pattern() {  // (1024 + 4^s) in both halves
    constexpr int s = I < 5 ? I : I - 5;
    return 0x64006400u | (0x00010001u << (2 * s));
}

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

// Sum over the 16 lanes of each DPP row (lanes 16r .. 16r+15); every lane of
// the row receives its row's total.  Steps: swap neighbours, swap pairs,
// mirror half-rows, mirror rows.  All 64 lanes must be active.
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
    return v;
}

// Sum over the 64 lanes of a wave; every lane receives the total: the row
// sums, then two exchanges across rows.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    return v;
}

}  // namespace tq
