// Decimation-in-time radix-16 and radix-4 butterflies with tangent-merged twiddles
// (Linzer and Feig's scaled-twiddle FFT), for the fused kernels of sc_fused4k.hip (M = 4096)
// and sc_fused_dit.hip (M = 1024, 2048).  A twiddle T = c (1 + i t), t = tan of T's angle, is merged
// into the butterfly adds: a +- T y = a +- c (y + i t y), 6 fused multiply-adds for both
// outputs instead of 4 for the product and 4 for the sums.  Where c is 0 (T = +-i) the tables
// hold c = 2^-40, t = +-2^40, which keeps c (y + i t y) accurate to fp32 round-off.
#pragma once

#include "sc_device.h"

namespace sc {
namespace dit {

// T = c (1 + i t)
struct TC {
    float c, t;
};

// y (1 + i t)
__device__ __forceinline__ float2 rot(float2 y, float t)
{
    return make_float2(__builtin_fmaf(-t, y.y, y.x), __builtin_fmaf(t, y.x, y.y));
}

// Y[q] = sum_m W4^{m q} T^m y_m (W4 = -i forward, +i inverse) with T = c1 (1 + i t1),
// T^2 = c2 (1 + i t2), in place: 24 fused multiply-adds.
template <bool INV>
__device__ __forceinline__ void dft4t(float2& y0, float2& y1, float2& y2, float2& y3, TC T, TC T2)
{
    const float2 u = rot(y2, T2.t), w = rot(y3, T2.t);
    const float2 e0 = make_float2(__builtin_fmaf(T2.c, u.x, y0.x), __builtin_fmaf(T2.c, u.y, y0.y));
    const float2 e1 = make_float2(__builtin_fmaf(-T2.c, u.x, y0.x), __builtin_fmaf(-T2.c, u.y, y0.y));
    const float2 p0 = make_float2(__builtin_fmaf(T2.c, w.x, y1.x), __builtin_fmaf(T2.c, w.y, y1.y));
    const float2 p1 = make_float2(__builtin_fmaf(-T2.c, w.x, y1.x), __builtin_fmaf(-T2.c, w.y, y1.y));
    const float2 a = rot(p0, T.t), b = rot(p1, T.t);
    y0 = make_float2(__builtin_fmaf(T.c, a.x, e0.x), __builtin_fmaf(T.c, a.y, e0.y));
    y2 = make_float2(__builtin_fmaf(-T.c, a.x, e0.x), __builtin_fmaf(-T.c, a.y, e0.y));
    // W4 T p1 = W4 c b: forward (c b.y, -c b.x), inverse (-c b.y, c b.x)
    const float s = INV ? -T.c : T.c;
    y1 = make_float2(__builtin_fmaf(s, b.y, e1.x), __builtin_fmaf(-s, b.x, e1.y));
    y3 = make_float2(__builtin_fmaf(-s, b.y, e1.x), __builtin_fmaf(s, b.x, e1.y));
}

// The first two outputs (q = 0, 1) only: 20 fused multiply-adds.
template <bool INV>
__device__ __forceinline__ void dft4t_lo(float2& y0, float2& y1, float2 y2, float2 y3, TC T, TC T2)
{
    const float2 u = rot(y2, T2.t), w = rot(y3, T2.t);
    const float2 e0 = make_float2(__builtin_fmaf(T2.c, u.x, y0.x), __builtin_fmaf(T2.c, u.y, y0.y));
    const float2 e1 = make_float2(__builtin_fmaf(-T2.c, u.x, y0.x), __builtin_fmaf(-T2.c, u.y, y0.y));
    const float2 p0 = make_float2(__builtin_fmaf(T2.c, w.x, y1.x), __builtin_fmaf(T2.c, w.y, y1.y));
    const float2 p1 = make_float2(__builtin_fmaf(-T2.c, w.x, y1.x), __builtin_fmaf(-T2.c, w.y, y1.y));
    const float2 a = rot(p0, T.t), b = rot(p1, T.t);
    y0 = make_float2(__builtin_fmaf(T.c, a.x, e0.x), __builtin_fmaf(T.c, a.y, e0.y));
    const float s = INV ? -T.c : T.c;
    y1 = make_float2(__builtin_fmaf(s, b.y, e1.x), __builtin_fmaf(-s, b.x, e1.y));
}

// x[k2] = sum_{n2} A^{n2} x[n2] W16^{n2 k2} (natural order in and out) from the item's
// twiddle pairs tw = {B, B^2, F_0, F_0^2, .., F_3, F_3^2}, B = A^4, F_p = A W16^p:
//   n2 = n1 + 4 m, k2 = p + 4 q;  columns C_{n1}[p] = sum_m W4^{m p} B^m x[n1 + 4 m],
//   rows X[p + 4 q] = sum_{n1} W4^{n1 q} F_p^{n1} C_{n1}[p].
// With HALF only X[0..7] are formed (x[8..15] are left undefined).
template <bool INV, bool HALF = false>
__device__ __forceinline__ void dit16(float2 (&x)[16], const TC (&tw)[10])
{
#pragma unroll
    for (int n1 = 0; n1 < 4; ++n1) dft4t<INV>(x[n1], x[n1 + 4], x[n1 + 8], x[n1 + 12], tw[0], tw[1]);
    float2 o[16];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if constexpr (HALF) {
            dft4t_lo<INV>(x[4 * p], x[4 * p + 1], x[4 * p + 2], x[4 * p + 3], tw[2 + 2 * p],
                          tw[3 + 2 * p]);
            o[p] = x[4 * p];
            o[p + 4] = x[4 * p + 1];
        } else {
            dft4t<INV>(x[4 * p], x[4 * p + 1], x[4 * p + 2], x[4 * p + 3], tw[2 + 2 * p],
                       tw[3 + 2 * p]);
#pragma unroll
            for (int q = 0; q < 4; ++q) o[p + 4 * q] = x[4 * p + q];
        }
    }
#pragma unroll
    for (int k = 0; k < (HALF ? 8 : 16); ++k) x[k] = o[k];
}

// an item's 10 twiddle pairs: 5 16-byte loads through the table's buffer descriptor
__device__ __forceinline__ void load_tw(__amdgpu_buffer_rsrc_t rs, int entry, TC (&tw)[10])
{
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const auto d = __builtin_amdgcn_raw_buffer_load_b128(rs, entry * 8 + 16 * i, 0, 0);
        const float4 f = __builtin_bit_cast(float4, d);
        tw[2 * i] = TC{f.x, f.y};
        tw[2 * i + 1] = TC{f.z, f.w};
    }
}


// Y[q] = sum_m W8^{m q} T^m y_m in place (natural order), from the six pairs
// tw = {T^2, T^4, U_0, U_1, U_2, U_3}, U_p = T W8^p: the even and the odd inputs through
// dft4t with T^2, then Y[p] = E[p] + U_p O[p] and Y[p + 4] = E[p] - U_p O[p], each pair of
// outputs 6 fused multiply-adds.
template <bool INV>
__device__ __forceinline__ void dft8t(float2 (&y)[8], const TC (&tw)[6])
{
    float2 e0 = y[0], e1 = y[2], e2 = y[4], e3 = y[6];
    float2 o0 = y[1], o1 = y[3], o2 = y[5], o3 = y[7];
    dft4t<INV>(e0, e1, e2, e3, tw[0], tw[1]);
    dft4t<INV>(o0, o1, o2, o3, tw[0], tw[1]);
    const float2 e[4] = {e0, e1, e2, e3}, o[4] = {o0, o1, o2, o3};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const TC u = tw[2 + p];
        const float2 r = rot(o[p], u.t);
        y[p] = make_float2(__builtin_fmaf(u.c, r.x, e[p].x), __builtin_fmaf(u.c, r.y, e[p].y));
        y[p + 4] = make_float2(__builtin_fmaf(-u.c, r.x, e[p].x), __builtin_fmaf(-u.c, r.y, e[p].y));
    }
}

}  // namespace dit
}  // namespace sc
