// Device-side helpers shared by the gfx950 kernels of libspecverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlock = 32;       // quantization block length (hidden axis)
constexpr int kTileRows = 16;    // vocab rows per MFMA tile (N of the 16x16x32 MFMA)

// Four int8 codes packed in a dword -> four exact fp16 values, by the exponent-bias ("magic
// number") integer-to-float conversion (2^23 for fp32; here 2^10, the fp16 form that weight-only
// quantized GEMMs use to expand int8 and int4 codes).
// Each byte is biased to u = q + 128 (xor 0x80), placed under the fp16 exponent of 1024
// (bit pattern 0x64uu = 1024 + u, exact since the ulp at 1024 is 1), and 1152 = 1024 + 128
// is subtracted; the result q is an integer in [-128, 127], exact in fp16.
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, f16x2& lo, f16x2& hi) {
    const uint32_t u = w ^ 0x80808080u;
    const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // [u0,64,u1,64]
    const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // [u2,64,u3,64]
    const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = __builtin_bit_cast(f16x2, a) - bias;
    hi = __builtin_bit_cast(f16x2, b) - bias;
}

// Eight int8 codes (two dwords, k order preserved) -> f16x8 MFMA operand.
__device__ __forceinline__ f16x8 i8x8_to_f16x8(u32x2 w) {
    f16x2 p0, p1, p2, p3;
    i8x4_to_f16(w.x, p0, p1);
    i8x4_to_f16(w.y, p2, p3);
    f16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f2h(float f) {            // round to nearest even
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Workgroup barrier that orders LDS accesses only: global loads and stores in flight are not
// waited for (a plain __syncthreads() also waits for every outstanding global store).  For
// barriers across which only LDS data is exchanged.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Maximum of a 32-bit unsigned value over the 64 lanes of a wave, returned to every lane: DPP
// steps within quads, half rows and rows, then row broadcasts carry each row's maximum into the
// last row, whose lane 63 holds the wave's maximum (max is idempotent, so lanes combined twice
// do no harm).  All lanes of the wave must be active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Argmax order: larger value first, then lower index.  -0.0 == +0.0.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Reduce (value, index) over each aligned group of `width` lanes; every lane of the
// group ends with the group's best.
template <int WIDTH>
__device__ __forceinline__ void argmax_group(float& v, int& i) {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) {
        const float ov = __shfl_xor(v, off, WIDTH);
        const int oi = __shfl_xor(i, off, WIDTH);
        if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// Merge two partial log-sum-exp states (max m, sum of exp(z - m)) into (m, l); an empty state
// has m = -inf.
__device__ __forceinline__ void lse_merge(float& m, float& l, float om, float ol) {
    const float M = fmaxf(m, om);
    l = (m == -INFINITY ? 0.0f : l * __expf(m - M)) + (om == -INFINITY ? 0.0f : ol * __expf(om - M));
    m = M;
}

// lse_merge over each aligned group of `width` lanes (xor butterfly); every lane of the group
// ends with the group's state.
template <int WIDTH>
__device__ __forceinline__ void lse_merge_group(float& m, float& l) {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) {
        const float om = __shfl_xor(m, off, WIDTH);
        const float ol = __shfl_xor(l, off, WIDTH);
        lse_merge(m, l, om, ol);
    }
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
// 3", SC'11): ten rounds of two 32x32 -> 64-bit products, the high halves folded into the
// other two words with the key, the key advancing by the Weyl increments between rounds.
struct Philox4 { uint32_t w[4]; };
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                  uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
    }
    return Philox4{{c0, c1, c2, c3}};
}

// Word i (0..3) of a Philox block, with selects rather than a dynamic register index.
__device__ __forceinline__ uint32_t philox_word(const Philox4& r, int i) {
    return i == 0 ? r.w[0] : i == 1 ? r.w[1] : i == 2 ? r.w[2] : r.w[3];
}

// A 32-bit word -> (floor(w / 2^9) + 1/2) / 2^23, strictly inside (0, 1) and exact in fp32.
__device__ __forceinline__ float uniform01(uint32_t w) {
    return ((float)(w >> 9) + 0.5f) * (1.0f / 8388608.0f);
}

// Gumbel(0, 1) noise from a uniform: -log(-log u).
__device__ __forceinline__ float gumbel(float u) {
    return -__logf(-__logf(u));
}

}  // namespace sv
