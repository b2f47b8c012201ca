// Dropout draws for the attention kernels: Philox4x32-10 and the keep masks.
//
// The reading-notes page (section 其他算子) has dropout zero attention weights at
// random and keep the generator's state for the backward pass, without naming a
// generator.  Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011) is counter based, so
// that state is just (seed, offset), and the backward pass regenerates any draw
// from its coordinates.
//
// Draws are 16 bits wide, so one call (128 bits) covers eight keys of one query
// row.  For head unit bh, query row i and key j = 16a + 8b + 4c + w (b, c in
// {0, 1}, w in 0..3), the draw is the 16-bit half 4b + w (the low half of output
// word 0 first) of the call at counter (2a + c, i, bh, offset) under the key
// (seed mod 2^32, seed >> 32); the pair is kept iff the draw >= t = floor(p 2^16).
// That assignment matches the MFMA accumulator layout of the kernels: the keys
// 16a + 4c + {0..3, 8..11} of one row sit in one lane, in the order of a packed
// bf16x8 operand, so output word m decides the operand's dword m.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct PhiloxOut {
    uint32_t w[4];
};

// Round multipliers and key-schedule (Weyl) increments of Philox4x32.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

// Ten rounds.  A round takes the full 64-bit products of counter words 0 and
// 2 with the two multipliers; the new state is (hi(M1 c2) ^ c1 ^ k0,
// lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)).  The key grows by the Weyl
// increments before every round after the first.
// (m0, m1: the two multipliers, passed in so that a kernel short of scalar
// registers can hold them in vector registers.)
__device__ __forceinline__ PhiloxOut philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                   uint32_t k0, uint32_t k1, uint32_t m0 = kPhiloxM0,
                                                   uint32_t m1 = kPhiloxM1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        const uint64_t p0 = (uint64_t)m0 * c0;
        const uint64_t p1 = (uint64_t)m1 * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    return PhiloxOut{{c0, c1, c2, c3}};
}

typedef unsigned short phx_u16x2 __attribute__((ext_vector_type(2)));

// Dropout of one packed pair of non-negative bf16 weights by one output
// word: in each 16-bit half, the weight stays where the draw u >= t and
// becomes +0 where it is dropped.  t2 holds t in both halves.  With
// x = max(t - u, 0), which is 0 exactly when u >= t, and z = max(1 - x, 0)
// (1 when kept, 0 when dropped), the weight's bit pattern times z is the
// result; each step is one packed 16-bit integer instruction.
__device__ __forceinline__ uint32_t drop_pair(uint32_t pair, uint32_t word, uint32_t t2) {
    const phx_u16x2 u = __builtin_bit_cast(phx_u16x2, word);
    const phx_u16x2 t = __builtin_bit_cast(phx_u16x2, t2);
    const phx_u16x2 x = __builtin_elementwise_sub_sat(t, u);
    const phx_u16x2 z = __builtin_elementwise_sub_sat((phx_u16x2)1, x);
    return __builtin_bit_cast(uint32_t, (phx_u16x2)(__builtin_bit_cast(phx_u16x2, pair) * z));
}

}  // namespace fa
