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

// ---- exact ternary operands for the matrix cores (the scheme is laid out
// at the matrix-core GEMV in gemv.hip).  Field I of a code dword x, masked
// into the mantissa of 1024.0, is the pair (1024 + 4^s c_I, 1024 + 4^s
// c_{I+8}), s = I for I < 5 and I - 5 (after x >> 10) otherwise.  One packed
// fp16 fma, v * 4^-s - (1024 / 4^s + 1), turns each half into c - 1, the
// ternary value itself, without rounding: v * 4^-s = 1024 / 4^s + c is exact
// and so is the difference.  The activations of the same columns are paired
// to match but not scaled, so the matrix units multiply a_k by -1, 0 or +1
// and the fp32 sums carry no offset that would later cancel.
//
// Read as bfloat16, the fp16 bit patterns of -1, 0 and +1 (0xBC00, 0, 0x3C00)
// are -2^-7, 0 and +2^-7: the same operand feeds the bf16 matrix cores, and
// the bf16 kernels multiply their fp32 sums by 128 (exact).

constexpr uint32_t kMagic2 = 0x64006400u;  // (1024.0, 1024.0) as fp16
constexpr float kBf16TernaryUnit = 128.0f;  // 1 / (bf16 value of the fp16 pattern of +1)

template <int I>
__device__ __forceinline__ uint32_t field_pair(uint32_t x, uint32_t y, uint32_t magic_v) {
    if constexpr (I < 5) return (x & sgpr_const<(0x00030003u << (2 * I))>()) | magic_v;
    else return (y & sgpr_const<(0x00030003u << (2 * (I - 5)))>()) | magic_v;
}

// (t_I, t_{I+8}) of code dword x (y = x >> 10) as exact fp16 values.
template <int I>
__device__ __forceinline__ uint32_t tern_pair(uint32_t x, uint32_t y, uint32_t magic_v) {
    constexpr int s = I < 5 ? I : I - 5;
    constexpr float kAdd = -(float)((1024 >> (2 * s)) + 1);
    constexpr float kMul = 1.0f / (float)(1 << (2 * s));
    const f16x2 v = __builtin_bit_cast(f16x2, field_pair<I>(x, y, magic_v));
    const f16x2 add = f16x2{(_Float16)kAdd, (_Float16)kAdd};
    if constexpr (s == 0) {
        return __builtin_bit_cast(uint32_t, v + add);
    } else {
        const f16x2 mul = f16x2{(_Float16)kMul, (_Float16)kMul};
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v, mul, add));
    }
}

// Four exact operand dwords of code dword x for fields I0 .. I0+3.
template <int I0>
__device__ __forceinline__ uint4 tern_quad(uint32_t x, uint32_t magic_v) {
    const uint32_t y = x >> 10;
    return make_uint4(tern_pair<I0>(x, y, magic_v), tern_pair<I0 + 1>(x, y, magic_v),
                      tern_pair<I0 + 2>(x, y, magic_v), tern_pair<I0 + 3>(x, y, magic_v));
}

// Activation pair matching field I of code dword D: (a[16D+I], a[16D+I+8]),
// 16-bit patterns (fp16 or bf16) of 16 consecutive columns per two uint4.
template <int D, int I>
__device__ __forceinline__ uint32_t act_pair(const uint4 av[8]) {
    const uint4& lo4 = av[2 * D];
    const uint4& hi4 = av[2 * D + 1];
    constexpr int c = I / 2;
    const uint32_t lo = c == 0 ? lo4.x : c == 1 ? lo4.y : c == 2 ? lo4.z : lo4.w;
    const uint32_t hi = c == 0 ? hi4.x : c == 1 ? hi4.y : c == 2 ? hi4.z : hi4.w;
    return __builtin_amdgcn_perm(hi, lo, (I & 1) ? 0x07060302u : 0x05040100u);
}

// The eight activation pairs of 16 columns (fields 0..3, then 4..7).
template <int D>
__device__ __forceinline__ void act_pairs16(const uint4 av[8], uint4& f03, uint4& f47) {
    f03 = make_uint4(act_pair<D, 0>(av), act_pair<D, 1>(av), act_pair<D, 2>(av), act_pair<D, 3>(av));
    f47 = make_uint4(act_pair<D, 4>(av), act_pair<D, 5>(av), act_pair<D, 6>(av), act_pair<D, 7>(av));
}

__device__ __forceinline__ uint32_t dword_of(const uint4& q, int d) {
    return d == 0 ? q.x : d == 1 ? q.y : d == 2 ? q.z : q.w;
}

// ---- exact W4A16 operands.  Nibble q_i of a code word x sits at bits 4i;
// masked into the mantissa of 1024.0, (x & 0x000F000F) | magic = (1024 + q_0,
// 1024 + q_4) and (x & 0x00F000F0) | magic = (1024 + 16 q_1, 1024 + 16 q_5),
// and with x >> 8 the pairs (q_2, q_6) and (q_3, q_7).  One packed fp16
// add or fma per pair subtracts 1024 + z (or scales by 1/16 and subtracts
// 64 + z), leaving q - z exactly (integers of magnitude <= 15).  The
// activations are paired to match: (a_0, a_4), (a_1, a_5), (a_2, a_6),
// (a_3, a_7).
struct W4Sub {
    f16x2 k0, k1;  // -(1024 + z), -(64 + z) in both halves
};
__device__ __forceinline__ W4Sub w4_sub(uint32_t z) {  // z in 0..15
    // -(1024 + z): sign, exponent 10, fraction z; -(64 + z): exponent 6,
    // fraction 16 z (unit in the last place 1/16)
    const uint32_t a = 0xE400u + z, b = 0xD400u + 16u * z;
    return W4Sub{__builtin_bit_cast(f16x2, a | (a << 16)), __builtin_bit_cast(f16x2, b | (b << 16))};
}
constexpr uint32_t kW4Sub0Sym = 0xE408E408u;  // -(1024 + 8), both halves
constexpr uint32_t kW4Sub1Sym = 0xD480D480u;  // -(64 + 8), both halves

__device__ __forceinline__ uint4 w4_quad(uint32_t x, uint32_t magic_v, f16x2 k0, f16x2 k1) {
    const uint32_t y = x >> 8;
    const f16x2 sixteenth = f16x2{(_Float16)0.0625f, (_Float16)0.0625f};
    const f16x2 v0 = __builtin_bit_cast(f16x2, (x & sgpr_const<0x000F000Fu>()) | magic_v);
    const f16x2 v1 = __builtin_bit_cast(f16x2, (x & sgpr_const<0x00F000F0u>()) | magic_v);
    const f16x2 v2 = __builtin_bit_cast(f16x2, (y & sgpr_const<0x000F000Fu>()) | magic_v);
    const f16x2 v3 = __builtin_bit_cast(f16x2, (y & sgpr_const<0x00F000F0u>()) | magic_v);
    return make_uint4(__builtin_bit_cast(uint32_t, v0 + k0), __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v1, sixteenth, k1)),
                      __builtin_bit_cast(uint32_t, v2 + k0), __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v3, sixteenth, k1)));
}

// bf16 form: the exact fp16 integers converted to bf16 through fp32 (every
// integer of magnitude <= 15 is exact in all three formats).
__device__ __forceinline__ uint32_t f16x2_to_bf16x2(uint32_t v) {
    const f16x2 h = __builtin_bit_cast(f16x2, v);
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(float)h.x, (__bf16)(float)h.y});
}
__device__ __forceinline__ uint4 w4_quad_bf16(uint32_t x, uint32_t magic_v, f16x2 k0, f16x2 k1) {
    const uint4 h = w4_quad(x, magic_v, k0, k1);
    return make_uint4(f16x2_to_bf16x2(h.x), f16x2_to_bf16x2(h.y), f16x2_to_bf16x2(h.z), f16x2_to_bf16x2(h.w));
}

// Activation pairs of one code word's eight columns (v: columns 8d .. 8d+7).
__device__ __forceinline__ uint4 w4_act_quad(const uint4& v) {
    return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                      __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
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
// The same from a wave-uniform base address (an SGPR pair) plus a 32-bit
// per-lane byte offset: no 64-bit vector address arithmetic per load.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds_addr) : "memory", "m0");
}

// Split-K completion inside the kernel.  Every split workgroup of an output
// tile stores its fp32 partials (store_partial) and then counts itself in
// flags[tile]; the one that brings the count to S is the last, resets the
// counter (every call leaves the counters zero, as the next call needs them)
// and goes on to sum the S partials in split order (split_sum), the same
// order and arithmetic as the separate reduction kernel, so the result does
// not depend on which split finishes last.
// Coherence across the XCDs (each has its own L2) comes from the accesses
// themselves, not from fences: the partials are stored and loaded at device
// scope (write-through stores, loads served from the device's coherence
// point), the counter is a device-scope atomic, and each wave waits for its
// partial stores to complete before the barrier that precedes the count.
// A fence would write back or drop the whole L2 of the XCD instead.
// Called by every thread of a one-dimensional workgroup after its last use
// of LDS; `word` is a 32-bit LDS word for the broadcast.  Nothing waits on
// another workgroup.
__device__ __forceinline__ void store_partial(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool split_last_arrival(uint32_t* flags, uint32_t tile, int S, uint32_t* word) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t seen = __hip_atomic_fetch_add(flags + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = seen == (uint32_t)(S - 1);
        if (last) __hip_atomic_store(flags + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *word = last ? 1u : 0u;
    }
    __syncthreads();
    return *word != 0u;
}

// Sums of the S partials of E outputs in split order z = 0 .. S-1 (the
// reduction kernel's arithmetic: 0 + p_0 + p_1 + ...): output e of slab z is
// base[z * MN + off[e]].  Rounds of R splits issue all R * E loads before
// using any, so a round costs one memory latency.  Every off[e] must address
// an element of the slab, also for outputs the caller then drops.
template <int E, int R>
__device__ __forceinline__ void split_sums(const float* base, int64_t MN, const uint32_t (&off)[E], int S,
                                           float (&out)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = 0.0f;
    for (int z0 = 0; z0 < S; z0 += R) {
        float v[R][E];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float* slab = base + (int64_t)(z0 + r < S ? z0 + r : S - 1) * MN;
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[r][e] = __hip_atomic_load(slab + off[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (z0 + r < S) {
#pragma unroll
                for (int e = 0; e < E; ++e) out[e] += v[r][e];
            }
    }
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
