// Device-side building blocks for the spectral causal convolution kernels (gfx950).
//
// Complex values are float2 (x = real, y = imaginary).  Transforms use the forward kernel
// W_n = exp(-2*pi*i/n) and are unscaled in both directions; the inverse uses conj(W_n).
// Register DFTs below take their input x[0..R-1] in natural order and return X[0..R-1]
// in natural order, X_k = sum_n x_n W_R^{nk} (or W_R^{-nk} when INV).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sc {

// ------------------------------------------------------------------ complex helpers

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 conjf2(float2 a) { return make_float2(a.x, -a.y); }
// a * b
__device__ __forceinline__ float2 cmul(float2 a, float2 b)
{
    return make_float2(__builtin_fmaf(a.x, b.x, -a.y * b.y), __builtin_fmaf(a.x, b.y, a.y * b.x));
}
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b)
{
    return make_float2(__builtin_fmaf(a.x, b.x, a.y * b.y), __builtin_fmaf(a.y, b.x, -a.x * b.y));
}
// a * b, or a * conj(b) when INV
template <bool INV>
__device__ __forceinline__ float2 cmul_dir(float2 a, float2 b)
{
    return INV ? cmulc(a, b) : cmul(a, b);
}
// multiply by -i (forward) or +i (inverse): the W_4^1 factor
template <bool INV>
__device__ __forceinline__ float2 mul_w4(float2 a)
{
    return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
}

// sqrt(1/2), cos(pi/8), sin(pi/8)
#define SC_R2 0.70710678118654752440f
#define SC_C8 0.92387953251128675613f
#define SC_S8 0.38268343236508977173f

// multiply by W_8^1 = (1 - i)/sqrt2 (forward) or W_8^-1 = (1 + i)/sqrt2 (inverse)
template <bool INV>
__device__ __forceinline__ float2 mul_w8(float2 a)
{
    return INV ? make_float2((a.x - a.y) * SC_R2, (a.x + a.y) * SC_R2)
               : make_float2((a.x + a.y) * SC_R2, (a.y - a.x) * SC_R2);
}
// multiply by W_8^3 = (-1 - i)/sqrt2 (forward) or W_8^-3 = (-1 + i)/sqrt2 (inverse)
template <bool INV>
__device__ __forceinline__ float2 mul_w8_3(float2 a)
{
    return INV ? make_float2(-(a.x + a.y) * SC_R2, (a.x - a.y) * SC_R2)
               : make_float2((a.y - a.x) * SC_R2, -(a.x + a.y) * SC_R2);
}
// multiply by the constant (c, -s) in the forward direction, (c, s) in the inverse
template <bool INV>
__device__ __forceinline__ float2 mul_cs(float2 a, float c, float s)
{
    return INV ? make_float2(__builtin_fmaf(a.x, c, -a.y * s), __builtin_fmaf(a.y, c, a.x * s))
               : make_float2(__builtin_fmaf(a.x, c, a.y * s), __builtin_fmaf(a.y, c, -a.x * s));
}

// ------------------------------------------------------------------ register DFTs

template <bool INV>
__device__ __forceinline__ void dft2(float2& a, float2& b)
{
    float2 t = a;
    a = cadd(t, b);
    b = csub(t, b);
}

// in place: (a0, a1, a2, a3) -> (X0, X1, X2, X3)
template <bool INV>
__device__ __forceinline__ void dft4(float2& a0, float2& a1, float2& a2, float2& a3)
{
    float2 t0 = cadd(a0, a2), t1 = csub(a0, a2);
    float2 t2 = cadd(a1, a3), t3 = mul_w4<INV>(csub(a1, a3));
    a0 = cadd(t0, t2);
    a2 = csub(t0, t2);
    a1 = cadd(t1, t3);
    a3 = csub(t1, t3);
}

// decimation in frequency: x -> (x_n + x_{n+4}, (x_n - x_{n+4}) W_8^n), then two DFT_4
template <bool INV>
__device__ __forceinline__ void dft8(float2* a)
{
    float2 u0 = cadd(a[0], a[4]), w0 = csub(a[0], a[4]);
    float2 u1 = cadd(a[1], a[5]), w1 = mul_w8<INV>(csub(a[1], a[5]));
    float2 u2 = cadd(a[2], a[6]), w2 = mul_w4<INV>(csub(a[2], a[6]));
    float2 u3 = cadd(a[3], a[7]), w3 = mul_w8_3<INV>(csub(a[3], a[7]));
    dft4<INV>(u0, u1, u2, u3);
    dft4<INV>(w0, w1, w2, w3);
    a[0] = u0; a[2] = u1; a[4] = u2; a[6] = u3;
    a[1] = w0; a[3] = w1; a[5] = w2; a[7] = w3;
}

// 16 = 4 x 4, decimation in frequency:
//   X[4 k1 + k2] = sum_{n1} W_4^{n1 k1} W_16^{n1 k2} sum_{n2} x[n1 + 4 n2] W_4^{n2 k2}
template <bool INV>
__device__ __forceinline__ void dft16(float2* a)
{
    // column DFTs over n2 for each n1: (a[n1], a[n1+4], a[n1+8], a[n1+12]) -> k2 = 0..3
    dft4<INV>(a[0], a[4], a[8], a[12]);
    dft4<INV>(a[1], a[5], a[9], a[13]);
    dft4<INV>(a[2], a[6], a[10], a[14]);
    dft4<INV>(a[3], a[7], a[11], a[15]);
    // now a[n1 + 4 k2] = T[n1][k2]; apply W_16^{n1 k2}
    a[5] = mul_cs<INV>(a[5], SC_C8, SC_S8);          // n1=1,k2=1: W16^1
    a[9] = mul_w8<INV>(a[9]);                        // n1=1,k2=2: W16^2
    a[13] = mul_cs<INV>(a[13], SC_S8, SC_C8);        // n1=1,k2=3: W16^3
    a[6] = mul_w8<INV>(a[6]);                        // n1=2,k2=1: W16^2
    a[10] = mul_w4<INV>(a[10]);                      // n1=2,k2=2: W16^4
    a[14] = mul_w8_3<INV>(a[14]);                    // n1=2,k2=3: W16^6
    a[7] = mul_cs<INV>(a[7], SC_S8, SC_C8);          // n1=3,k2=1: W16^3
    a[11] = mul_w8_3<INV>(a[11]);                    // n1=3,k2=2: W16^6
    a[15] = mul_cs<INV>(a[15], -SC_C8, -SC_S8);      // n1=3,k2=3: W16^9 = -W16^1
    // row DFTs over n1 for each k2: (a[4k2], a[4k2+1], a[4k2+2], a[4k2+3]) -> k1
    dft4<INV>(a[0], a[1], a[2], a[3]);
    dft4<INV>(a[4], a[5], a[6], a[7]);
    dft4<INV>(a[8], a[9], a[10], a[11]);
    dft4<INV>(a[12], a[13], a[14], a[15]);
    // now a[4 k2 + k1] = X[4 k1 + k2]: transpose the 4x4 index to natural order
    float2 t;
    t = a[1]; a[1] = a[4]; a[4] = t;
    t = a[2]; a[2] = a[8]; a[8] = t;
    t = a[3]; a[3] = a[12]; a[12] = t;
    t = a[6]; a[6] = a[9]; a[9] = t;
    t = a[7]; a[7] = a[13]; a[13] = t;
    t = a[11]; a[11] = a[14]; a[14] = t;
}

template <int R, bool INV>
__device__ __forceinline__ void dft(float2* a)
{
    if constexpr (R == 16) dft16<INV>(a);
    else if constexpr (R == 8) dft8<INV>(a);
    else if constexpr (R == 4) dft4<INV>(a[0], a[1], a[2], a[3]);
    else if constexpr (R == 2) dft2<INV>(a[0], a[1]);
}

// ------------------------------------------------------------------ storage types

// A raw buffer descriptor over `count` elements starting at p[first].  Loads outside it
// return 0 and stores outside it are dropped by the hardware; offsets are 32-bit.
struct Span {
    __amdgpu_buffer_rsrc_t rs;
};
template <class T>
__device__ __forceinline__ Span make_span(const T* p, int64_t first, int64_t count)
{
    int64_t bytes = count * (int64_t)sizeof(T);
    if (bytes > 0x7fffffff) bytes = 0x7fffffff;
    if (bytes < 0) bytes = 0;
    return Span{__builtin_amdgcn_make_buffer_rsrc((void*)(p + first), (short)0, (int)bytes, 0x00020000)};
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// round two floats to bfloat16 (nearest, ties to even) and pack them, a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    const f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

struct f32_io {
    typedef float T;
    static constexpr int SIZE = 4;
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, int64_t i, float x) { p[i] = x; }
    // Element OOB sits at byte offset 2^31, past every descriptor's range: it reads 0.
    static constexpr int OOB = (int)(0x80000000u / 4);
    __device__ __forceinline__ static float load(const Span& s, int i)
    {
        return __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(s.rs, (int)((uint32_t)i * 4u), 0, 0));
    }
    __device__ __forceinline__ static void store(const Span& s, int i, float x)
    {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), s.rs, i * 4, 0, 0);
    }
    // element i + j with j a uniform (scalar) offset
    __device__ __forceinline__ static float load_at(const Span& s, int i, int j)
    {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(s.rs, i * 4, j * 4, 0));
    }
    // two consecutive outputs at element i (8-byte aligned)
    __device__ __forceinline__ static void store2(const Span& s, int i, float a, float b)
    {
        const u32x2_t w = {__float_as_uint(a), __float_as_uint(b)};
        __builtin_amdgcn_raw_buffer_store_b64(w, s.rs, i * 4, 0, 0);
    }
};

// bfloat16 storage: widen exactly on load, round to nearest even on store
struct bf16_io {
    typedef uint16_t T;
    static constexpr int SIZE = 2;
    __device__ __forceinline__ static float load(const uint16_t* p, int64_t i)
    {
        return __uint_as_float(((uint32_t)p[i]) << 16);
    }
    __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float x)
    {
        p[i] = (uint16_t)pack_bf16x2(x, 0.f);
    }
    static constexpr int OOB = (int)(0x80000000u / 2);
    __device__ __forceinline__ static float load(const Span& s, int i)
    {
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b16(s.rs, (int)((uint32_t)i * 2u), 0, 0);
        return __uint_as_float(w << 16);
    }
    __device__ __forceinline__ static void store(const Span& s, int i, float x)
    {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)pack_bf16x2(x, 0.f), s.rs, i * 2, 0, 0);
    }
    __device__ __forceinline__ static float load_at(const Span& s, int i, int j)
    {
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b16(s.rs, i * 2, j * 2, 0);
        return __uint_as_float(w << 16);
    }
    __device__ __forceinline__ static void store2(const Span& s, int i, float a, float b)
    {
        __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(a, b), s.rs, i * 2, 0, 0);
    }
};

}  // namespace sc
