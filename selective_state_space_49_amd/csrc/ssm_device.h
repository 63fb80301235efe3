// ssm_device.h -- device helpers shared by the scan and decode kernels (gfx950).
//
// Element types: float, or bfloat16 kept as its 16 raw bits (uint16_t). Widening
// a bfloat16 is exact (its bits are the top half of a float32); narrowing rounds
// to nearest even with the hardware conversion (v_cvt_pk_bf16_f32 on gfx950).
//
// Rows of B and C are the same for every channel of a (batch, step), so every
// lane of a wave needs the same values. They are read through a constant-address
// -space pointer: with a wave-uniform address the compiler issues scalar loads
// (s_load_dwordxN) and widens in the scalar unit, and the multiply-adds take the
// values straight from SGPRs, costing no vector instructions. The arrays are
// read-only for the whole kernel, which the constant address space requires.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

typedef uint16_t bf16_bits;
typedef __attribute__((address_space(4))) const uint32_t cu32;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
    __bf16 r = (__bf16)v;                 // round to nearest even (hardware convert)
    return __builtin_bit_cast(uint16_t, r);
}

template <typename IO> struct Io;
template <> struct Io<float> {
    static __device__ __forceinline__ float ld(const float *p) { return *p; }
    static __device__ __forceinline__ void st(float *p, float v) { *p = v; }
};
template <> struct Io<bf16_bits> {
    static __device__ __forceinline__ float ld(const bf16_bits *p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ void st(bf16_bits *p, float v) { *p = f32_to_bf16(v); }
};

// Element at a wave-uniform row pointer plus a per-lane 32-bit byte offset. Keeping
// the lane part a zero-extended 32-bit value lets the compiler use the global
// load/store form with a scalar 64-bit base and a vector 32-bit offset, so walking
// rows costs scalar adds only.
template <typename IO>
__device__ __forceinline__ float ld_row(const IO *row, uint32_t byte_off) {
    return Io<IO>::ld((const IO *)((const char *)row + byte_off));
}
template <typename IO>
__device__ __forceinline__ void st_row(IO *row, uint32_t byte_off, float v) {
    Io<IO>::st((IO *)((char *)row + byte_off), v);
}

// Element e (wave-uniform) of a float / bf16 array through the scalar path. A bf16
// value is taken out of a dword load, so a bf16 base must be 4-byte aligned.
template <typename IO> struct Uniform;
template <> struct Uniform<float> {
    static __device__ __forceinline__ float ld(const float *base, int64_t e) {
        return __uint_as_float(((cu32 *)base)[e]);
    }
};
template <> struct Uniform<bf16_bits> {
    static __device__ __forceinline__ float ld(const bf16_bits *base, int64_t e) {
        const uint32_t w = ((cu32 *)base)[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

// Row b of a [batch][L][N] array (B or C) read through the scalar path, from the
// array's (4-byte aligned) start p and the row's first element e0 = b L N. With bf16
// and N odd (N = 1) a row starts at an odd element whenever b L is odd; the base is
// then rounded down to an even element and the index carries the parity. With N even
// or fp32 the row start is aligned and no parity is kept.
template <typename IO, int N, bool ODD = (sizeof(IO) == 2 && (N & 1) != 0)> struct UniRow;
template <typename IO, int N> struct UniRow<IO, N, false> {
    const IO *base;
    __device__ __forceinline__ UniRow(const void *p, int64_t e0) : base((const IO *)p + e0) {}
    __device__ __forceinline__ float ld(int64_t e) const { return Uniform<IO>::ld(base, e); }
};
template <typename IO, int N> struct UniRow<IO, N, true> {
    const IO *base;
    int64_t par;
    __device__ __forceinline__ UniRow(const void *p, int64_t e0)
        : base((const IO *)p + (e0 & ~(int64_t)1)), par(e0 & 1) {}
    __device__ __forceinline__ float ld(int64_t e) const { return Uniform<IO>::ld(base, e + par); }
};

// Hardware base-2 exponential (v_exp_f32) and reciprocal (v_rcp_f32).
__device__ __forceinline__ float e2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// silu(z) = z / (1 + exp(-z)), with exp(-z) = 2^(-z log2 e).
__device__ __forceinline__ float silu(float z) { return z * rcp(1.0f + e2(-z * kLog2e)); }

// sin and cos of 2*pi*r for r in revolutions, reduced to [0, 1) first.
__device__ __forceinline__ float fract(float r) { return __builtin_amdgcn_fractf(r); }
__device__ __forceinline__ float sin_rev(float r) { return __builtin_amdgcn_sinf(r); }
__device__ __forceinline__ float cos_rev(float r) { return __builtin_amdgcn_cosf(r); }

constexpr float kInv2Pi = 0.15915494309189535f;
constexpr double kInv2PiD = 0.15915494309189533577;

}  // namespace ssm
