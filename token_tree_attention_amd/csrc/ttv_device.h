// Device-side helpers shared by the verification kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "treeverify.h"

#define TTV_WAVE 64

// ---- bounds checks of the debug build --------------------------------------
// Compiled with TTV_DEBUG defined (libtreeverify_debug.so), TTV_DCHECK(cond,
// site) checks a bound on the device: a failure counts in this translation
// unit's debug word, records the first failing site (TTV_SITE_*), and yields
// false so the caller skips or redirects the access it guards; nothing traps.
// ttv_debug_report (abi.hip) sums the words of every translation unit.
// Without TTV_DEBUG the check is the constant true and compiles to nothing.
#ifdef TTV_DEBUG
static __device__ unsigned int ttv_debug_word[2];  // failures, first failing site
__device__ __noinline__ static void ttv_debug_fail(int site) {
    if (atomicAdd(&ttv_debug_word[0], 1u) == 0u) atomicExch(&ttv_debug_word[1], (unsigned int)site);
}
#define TTV_DCHECK(cond, site) ((cond) ? true : (ttv_debug_fail(site), false))
// Host reader of this translation unit's word (and reset), for ttv_debug_report.
#define TTV_DEBUG_TU(name)                                                                      \
    extern "C" int ttv_debug_take_##name(unsigned int* out, int reset) {                       \
        if (hipMemcpyFromSymbol(out, HIP_SYMBOL(ttv_debug_word), 2 * sizeof(unsigned int)) !=   \
            hipSuccess)                                                                         \
            return TTV_EHIP;                                                                    \
        if (reset) {                                                                            \
            const unsigned int zero[2] = {0u, 0u};                                              \
            if (hipMemcpyToSymbol(HIP_SYMBOL(ttv_debug_word), zero, sizeof zero) != hipSuccess) \
                return TTV_EHIP;                                                                \
        }                                                                                       \
        return TTV_OK;                                                                          \
    }
#else
#define TTV_DCHECK(cond, site) true
#define TTV_DEBUG_TU(name)
#endif

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 ttv_bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float ttv_f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t ttv_u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t ttv_u32x2;
typedef _Float16 ttv_f16x4 __attribute__((ext_vector_type(4)));

// ---- bf16 <-> fp32 -------------------------------------------------------

__device__ __forceinline__ float ttv_bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float ttv_bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round fp32 to bf16, nearest-even (finite inputs).
__device__ __forceinline__ uint32_t ttv_f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Round fp64 to fp32 to odd: nearest-even first, one step back toward zero
// where that went away from zero, and the lowest bit set whenever the result
// is inexact.  Rounding this to bf16 (nearest-even) equals rounding d to bf16
// directly, since fp32 keeps 16 more fraction bits (no double rounding).
__device__ __forceinline__ float ttv_f64_to_f32_odd(double d) {
    const float f = (float)d;
    const double back = (double)f;
    uint32_t u = __float_as_uint(f);
    if (back != d) {
        if (fabs(back) > fabs(d)) u -= 1u;
        u |= 1u;
    }
    return __uint_as_float(u);
}

// Round fp64 to bf16, nearest-even.
__device__ __forceinline__ uint32_t ttv_f64_to_bf16_bits(double d) {
    return ttv_f32_to_bf16_bits(ttv_f64_to_f32_odd(d));
}

__device__ __forceinline__ double ttv_bf16_bits_to_f64(uint32_t h) {
    return (double)__uint_as_float(h << 16);
}

__device__ __forceinline__ uint32_t ttv_pack_bf16x2(float lo, float hi) {
    return ttv_f32_to_bf16_bits(lo) | (ttv_f32_to_bf16_bits(hi) << 16);
}

// ---- ordered keys for argmax ---------------------------------------------

// Map float bits to an unsigned key with the same order; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t ttv_order_key(uint32_t fbits) {
    if (fbits == 0x80000000u) fbits = 0u;
    return (fbits & 0x80000000u) ? ~fbits : (fbits | 0x80000000u);
}

// 64-bit argmax key: larger value wins, then smaller index.
__device__ __forceinline__ uint64_t ttv_argmax_key(uint32_t fbits, uint32_t idx) {
    return ((uint64_t)ttv_order_key(fbits) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint32_t ttv_key_index(uint64_t key) {
    return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull);
}

// ---- wave reductions ------------------------------------------------------

__device__ __forceinline__ uint64_t ttv_wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
        uint32_t olo = __shfl_xor(lo, off, TTV_WAVE);
        uint32_t ohi = __shfl_xor(hi, off, TTV_WAVE);
        uint64_t o = ((uint64_t)ohi << 32) | olo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ int ttv_div_up(int a, int b) { return (a + b - 1) / b; }
