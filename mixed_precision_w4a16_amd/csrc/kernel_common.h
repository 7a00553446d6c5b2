// Device-side building blocks shared by the kernels of libw4a16 (internal header): vector
// types, the constants every kernel uses, buffer resources and the fp16 decode of 4-bit codes.
#ifndef W4A16_KERNEL_COMMON_H
#define W4A16_KERNEL_COMMON_H

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16 __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u3 __attribute__((ext_vector_type(3)));

constexpr int kThreads = 256;                 // 4 waves of 64
constexpr int kWaves = 4;
constexpr int kGroup = 128;                   // K rows per tile = one scale group

// Raw buffer resources: base, size in bytes, gfx9 dword-access flags.  Loads past `bytes`
// return zero, which masks the rows of A beyond M for free.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

constexpr int kNonTemporal = 2;    // cache policy: streaming, evict first (weights, read once)
constexpr int kDeviceScope = 16;   // cache policy sc1: write through / read past the XCD's L2

// Offset for loads that must not touch memory: above every buffer the kernels read (they
// check that theirs lie below it), so the range check turns the load into a zero.
constexpr uint32_t kOutside = 0x80000000u;

// Opaque copy of a uniform value: offsets derived from it are computed where they are used.
// Without it the compiler hoists every loop-invariant store offset of the epilogue out of the
// main loop and keeps them all live there.
__device__ __forceinline__ uint32_t opaque(uint32_t x)
{
    asm volatile("" : "+s"(x));
    return x;
}

// A value the compiler must keep in a VGPR and cannot treat as a known constant.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// (a & m) | o in one VALU op (v_and_or_b32) when m and o are in VGPRs (in_vgpr): gfx9 VOP3
// encodings take no literal and read at most one SGPR, so given two constants the compiler
// would split it into v_and + v_or.  Written in C, not inline asm: a matrix instruction that
// reads a VGPR as an operand needs two wait states after the VALU write of it, and the
// compiler's hazard recognizer inserts them only for instructions it knows (an inline-asm
// write right before the MFMA was read stale now and then).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o)
{
    return (a & m) | o;
}

// 8 codes -> 8 fp16 values q - z, in MFMA B-operand order (see pack.cpp for the nibbles).
// 9 VALU ops per 8 weights: 4 mask-and-OR, 1 shift, 2 packed adds, 2 packed FMAs.  `zsub`
// is 1024 + z and `zadd` is 960 - (1024 + z) = -(64 + z), both exact in fp16: the low nibbles
// give 1024 + q, the high ones 1024 + 16q, so (1024 + q) - zsub and (1024 + 16q) / 16 + zadd
// are q - z exactly.  The symmetric format passes z = 8: 1032 and -72.
__device__ __forceinline__ h8 dequant8(uint32_t w, uint32_t mlo, uint32_t mhi, uint32_t magic,
                                       h2 zsub, h2 zadd)
{
    const uint32_t w8 = w >> 8;
    const uint32_t x0 = and_or(w, mlo, magic);     // k0, k1: fp16 1024 + q
    const uint32_t x1 = and_or(w, mhi, magic);     // k2, k3: fp16 1024 + 16 q
    const uint32_t x2 = and_or(w8, mlo, magic);    // k4, k5
    const uint32_t x3 = and_or(w8, mhi, magic);    // k6, k7
    const h2 mul = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
    const h2 y0 = __builtin_bit_cast(h2, x0) - zsub;                                // q - z
    const h2 y1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, x1), mul, zadd); // q - z
    const h2 y2 = __builtin_bit_cast(h2, x2) - zsub;
    const h2 y3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, x3), mul, zadd);
    h8 r;
    r[0] = y0[0]; r[1] = y0[1]; r[2] = y1[0]; r[3] = y1[1];
    r[4] = y2[0]; r[5] = y2[1]; r[6] = y3[0]; r[7] = y3[1];
    return r;
}

// 8 weights, decoded and scaled: fp16(s * (q - z)), one rounding.
__device__ __forceinline__ h8 dequant8_scaled(uint32_t w, h2 s, uint32_t mlo, uint32_t mhi,
                                              uint32_t magic, h2 zsub, h2 zadd)
{
    const uint32_t w8 = w >> 8;
    const uint32_t x0 = and_or(w, mlo, magic);
    const uint32_t x1 = and_or(w, mhi, magic);
    const uint32_t x2 = and_or(w8, mlo, magic);
    const uint32_t x3 = and_or(w8, mhi, magic);
    const h2 mul = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
    const h2 y0 = (__builtin_bit_cast(h2, x0) - zsub) * s;
    const h2 y1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, x1), mul, zadd) * s;
    const h2 y2 = (__builtin_bit_cast(h2, x2) - zsub) * s;
    const h2 y3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, x3), mul, zadd) * s;
    h8 r;
    r[0] = y0[0]; r[1] = y0[1]; r[2] = y1[0]; r[3] = y1[1];
    r[4] = y2[0]; r[5] = y2[1]; r[6] = y3[0]; r[7] = y3[1];
    return r;
}

// 8 codes -> raw fp16 values in MFMA B-operand order, 5 VALU ops (4 mask-and-OR, 1 shift) and
// no arithmetic: codes 0, 1, 4, 5 (the low nibble of a byte, the last 4 mantissa bits) ORed into
// the exponent field of 1024 (0x6400) read as 1024 + q; codes 2, 3, 6, 7 (the high nibble, 4
// bits further up) ORed into the field of 64 (0x5400) read as 64 + q.  The matrix instruction
// sums A * raw; the symmetric format's offsets, 1032 and 72 at those positions (raw8 of code 8
// everywhere, raw_offsets() below), are summed against the same A by a second chain and
// subtracted from the first (see the kernels).  mag_lo = 0x64006400, mag_hi = 0x54005400.
__device__ __forceinline__ h8 raw8(uint32_t w, uint32_t mlo, uint32_t mhi, uint32_t mag_lo,
                                   uint32_t mag_hi)
{
    const uint32_t w8 = w >> 8;
    const u4 x = {and_or(w, mlo, mag_lo), and_or(w, mhi, mag_hi), and_or(w8, mlo, mag_lo),
                  and_or(w8, mhi, mag_hi)};
    return __builtin_bit_cast(h8, x);
}

// raw8 of eight codes 8: {1032, 1032, 72, 72, 1032, 1032, 72, 72}
__device__ __forceinline__ h8 raw_offsets()
{
    return __builtin_bit_cast(h8, u4{0x64086408u, 0x54805480u, 0x64086408u, 0x54805480u});
}

// Decode constants (zsub, zadd) of the symmetric format, z = 8.
__device__ __forceinline__ h2 sym_zsub()
{
    return h2{static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
}
__device__ __forceinline__ h2 sym_zadd()
{
    return h2{static_cast<_Float16>(-72.0f), static_cast<_Float16>(-72.0f)};
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ uint16_t float_to_half_bits(float x)
{
    // v_cvt_f16_f32: one rounding, nearest-even in the default mode
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

}  // namespace

#endif  // W4A16_KERNEL_COMMON_H
