// Fused in-LDS causal convolution for 512 < L <= 1024 (transform length M = 1024), gfx950.
//
// The method and data flow of the general fused kernel (sc_fused.hip): z = v + i g, the two
// branches u^b_n = z_n W_N^{b n} (N = 2M) transformed side by side by 64 threads each (one
// wave per branch), the unpack of V G into the half-length real-output inverse spectrum Y,
// one length-M inverse, the first `head` outputs by direct summation ("Caracal: Causal
// Architecture via Spectral Mixing", key designs 1-2 and the real-FFT improvement its
// limitations name).  The transforms are organised as in the M = 4096 kernel
// (sc_fused4k.hip), with passes of radix 4, 16 and 16 in decimation in time:
//
//   n = n'' + 16 n2 + 256 n1,  k = k1 + 4 k2 + 64 k3  (n1, k1 < 4; n2, k2, n'', k3 < 16)
//   pass 1 (registers): y1[n''+16 n2][k1] = sum_{n1} x[n] W4^{n1 k1}
//   pass 2: y2[n''][k1+4k2] = sum_{n2} W64^{n2 k1} y1[n''+16 n2][k1] W16^{n2 k2}
//   pass 3: X[m + 64 k3] = sum_{n''} W1024^{n'' m} y2[n''][m] W16^{n'' k3},  m = k1 + 4 k2
//
// Thread tau holds elements tau + 64 q (q < 16) at the input, so the radix-4 groups of pass 1
// (q, q + 4, q + 8, q + 12) sit in its registers and pass 1 needs no exchange; after pass 3
// it holds bins tau + 64 q, the order the unpack of the M = 4096 kernel takes.  Branch 1's
// rotation W_N^n = W_N^{n''} W_128^{n2} W_8^{n1} goes into the twiddles: W_8 is pass 1's
// constant base, W_128^{2k1+1} and W_2048^{2m+1} are the bases of passes 2 and 3.  All
// twiddles are merged into the butterflies (sc_dit.h).
//
// LDS (float2 units): pass 1 writes y1[n'][k1] at n' + 272 k1, pass 2 reads it (item
// (n'', k1) = (tau % 16, tau / 16)) and writes y2[n''][m] at m + 66 n'', pass 3 reads that;
// Y of the inverse at ypos(k), the mirror exchange of the unpack after Y.  Every access
// pattern of a wave hits 32 different bank pairs per 32 lanes (8-byte accesses serve 32
// lanes per cycle).  17.9 KB per workgroup of 128 threads: eight workgroups per CU.

#include "sc_device.h"
#include "sc_dit.h"
#include "sc_fft_lds.h"
#include "sc_internal.h"

namespace sc {

namespace f1k {

constexpr int M = 1024, TB = 64, FT = 128;
constexpr int REGION = 1088;   // one branch unit's pass layouts (positions < 1072)
constexpr int XCH = 1040;      // mirror exchange [unit][8][64], after Y (positions < 1040)

__device__ __forceinline__ int ypos(int k) { return (k >> 1) + (k & 1) * (M / 2 + 16); }
__device__ __forceinline__ int p1pos(int np, int k1) { return np + 272 * k1; }
__device__ __forceinline__ int p2pos(int npp, int m) { return m + 66 * npp; }

}  // namespace f1k

template <class IO, bool REV>
__global__ __launch_bounds__(128) void fused1k_kernel(const typename IO::T* __restrict__ v,
                                                      const typename IO::T* __restrict__ g,
                                                      typename IO::T* __restrict__ r, int L,
                                                      int head, int pair_store,
                                                      const float2* __restrict__ tab, int64_t pf)
{
    using namespace f1k;
    using namespace dit;
    __shared__ float2 lds[2 * REGION];
    __shared__ float hbuf[2 * HEAD_MAX];

    const auto trs = __builtin_amdgcn_make_buffer_rsrc((void*)tab, (short)0, DIT1K_TABLE_FLOAT2 * 8,
                                                       0x00020000);
    const int tid = threadIdx.x, tau = tid & (TB - 1);
    const int unit = __builtin_amdgcn_readfirstlane(tid >> 6);   // one wave per unit
    const int64_t ch = blockIdx.x;
    const Span vs = make_span(v, ch * L, L);
    const Span gs = make_span(g, ch * L, L);

    // 1. z_n = v_n + i g_n, n = tau + 64 q (0 past L)
    float2 x[16];
    if (L == M) {
        const int vb = REV ? L - 1 - tau - TB * 15 : tau;
#pragma unroll
        for (int q = 0; q < 16; ++q)
            x[q] = make_float2(IO::load_at(vs, vb, TB * (REV ? 15 - q : q)),
                               IO::load_at(gs, tau, TB * q));
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int n = tau + TB * q;
            const bool in = n < L;
            const int e = in ? n : IO::OOB;
            const int ev = in ? (REV ? L - 1 - n : n) : IO::OOB;
            x[q] = make_float2(IO::load(vs, ev), IO::load(gs, e));
        }
    }
    if (unit == 0 && tau < head) {
        hbuf[tau] = x[0].x;
        hbuf[HEAD_MAX + tau] = x[0].y;
    }

    float2* const reg = lds + unit * REGION;
    const int npp = tau & 15, k1 = tau >> 4;   // the pass-2 item of this thread

    // pass 1 (forward or inverse): the four radix-4 groups of registers q0, q0 + 4, q0 + 8,
    // q0 + 12 (n' = tau + 64 q0), branch 1 with its constant twiddle base, written to LDS
    auto pass1 = [&](float2* dst, bool twiddled, auto inv_tag) {
        constexpr bool INV = decltype(inv_tag)::value;
        TC t1{1.0f, 0.0f}, t2{1.0f, 0.0f};
        if (twiddled) {
            const float4 f = __builtin_bit_cast(
                float4, __builtin_amdgcn_raw_buffer_load_b128(trs, DIT1K_P1B1 * 8, 0, 0));
            t1 = TC{f.x, f.y};
            t2 = TC{f.z, f.w};
        }
#pragma unroll
        for (int q0 = 0; q0 < 4; ++q0) {
            float2 a = x[q0], b = x[q0 + 4], c = x[q0 + 8], d = x[q0 + 12];
            if (twiddled) dft4t<INV>(a, b, c, d, t1, t2);
            else dft4<INV>(a, b, c, d);
            const int np = tau + TB * q0;
            dst[p1pos(np, 0)] = a;
            dst[p1pos(np, 1)] = b;
            dst[p1pos(np, 2)] = c;
            dst[p1pos(np, 3)] = d;
        }
    };
    // pass 2, item (n'', k1): its inputs y1[n'' + 16 n2][k1] (read before a barrier), then the
    // butterfly and y2[n''][k1 + 4 k2] written
    auto pass2_read = [&](const float2* buf) {
#pragma unroll
        for (int n2 = 0; n2 < 16; ++n2) x[n2] = buf[p1pos(npp + 16 * n2, k1)];
    };
    auto pass2_write = [&](float2* buf, int var, auto inv_tag) {
        constexpr bool INV = decltype(inv_tag)::value;
        TC tw[10];
        load_tw(trs, DIT1K_P2 + (var * 4 + k1) * 10, tw);
        dit16<INV>(x, tw);
#pragma unroll
        for (int k2 = 0; k2 < 16; ++k2) buf[p2pos(npp, k1 + 4 * k2)] = x[k2];
    };

    // 2. forward transform of branch `unit`
    pass1(reg, unit == 1, std::false_type{});
    __syncthreads();
    pass2_read(reg);
    __syncthreads();
    pass2_write(reg, unit, std::false_type{});
    __syncthreads();
    {
        TC tw[10];
        load_tw(trs, DIT1K_P3 + (unit * TB + tau) * 10, tw);
#pragma unroll
        for (int n = 0; n < 16; ++n) x[n] = reg[p2pos(n, tau)];
        __syncthreads();
        dit16<false>(x, tw);   // x[q] = Z_{2 (tau + 64 q) + unit}
    }

    // 3. unpack.  The mirror thread needs registers 4..7 and 12..15 of this one.
    float2* xch = lds + XCH + unit * 8 * TB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xch[i * TB + tau] = x[4 + i];
        xch[(4 + i) * TB + tau] = x[12 + i];
    }
    __syncthreads();
    const int mir = (TB - tau - unit) & (TB - 1);
    float2 q1[4], p2[4];   // Z^b at the mirror's registers 15 - q and 7 - q
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        q1[q] = xch[(7 - q) * TB + mir];
        p2[q] = xch[(3 - q) * TB + mir];
    }
    const bool zero = unit == 0 && tau == 0;   // bins 0 and M/2 live in this thread alone
    if (zero) {
        q1[0] = x[0];
        q1[1] = x[15];
        q1[2] = x[14];
        q1[3] = x[13];
        p2[0] = x[8];
        p2[1] = x[7];
        p2[2] = x[6];
        p2[3] = x[5];
    }
    float2 yk[4], ymk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int k = 2 * (tau + TB * q) + unit;
        // bins k, N-k, M-k, M+k; 4 X = -i (P + Q)(P - Q) with P = Z_k, Q = conj Z_{N-k}
        const float2 pa = x[q], qa = conjf2(q1[q]), pb = p2[q], qb = conjf2(x[q + 8]);
        const float2 s1 = cadd(pa, qa), d1 = csub(pa, qa), s2 = cadd(pb, qb), d2 = csub(pb, qb);
        const float2 x1 = make_float2(__builtin_fmaf(s1.x, d1.y, s1.y * d1.x),
                                      __builtin_fmaf(s1.y, d1.y, -s1.x * d1.x));   // 4 X_k
        const float2 x2 = make_float2(__builtin_fmaf(s2.x, d2.y, s2.y * d2.x),
                                      __builtin_fmaf(s2.y, d2.y, -s2.x * d2.x));   // 4 X_{M-k}
        const float2 sm = make_float2(x1.x + x2.x, x1.y - x2.y);
        const float2 df = make_float2(x1.x - x2.x, x1.y + x2.y);
        // T = W_N^{-k} D = c (D + i t D);  Y_k = S + i T,  Y_{M-k} = conj(S - i T)
        const float2 ct = __builtin_bit_cast(
            float2, __builtin_amdgcn_raw_buffer_load_b64(trs, k * 8, DIT1K_UNP * 8, 0));
        const float2 u = rot(df, ct.y);
        yk[q] = make_float2(__builtin_fmaf(-ct.x, u.y, sm.x), __builtin_fmaf(ct.x, u.x, sm.y));
        ymk[q] = make_float2(__builtin_fmaf(ct.x, u.y, sm.x), __builtin_fmaf(ct.x, u.x, -sm.y));
    }
    if (zero) {
        // Y_{M/2} from bins M/2 and 3M/2 (registers 4 and 12) in place of the absent Y_M
        const float2 pa = x[4], qa = conjf2(x[12]);
        const float2 s1 = cadd(pa, qa), d1 = csub(pa, qa);
        const float2 x1 = make_float2(__builtin_fmaf(s1.x, d1.y, s1.y * d1.x),
                                      __builtin_fmaf(s1.y, d1.y, -s1.x * d1.x));
        // with both bins pairs equal, S = (2 Re, 0), D = (0, 2 Im) and W_N^{-M/2} = i, so
        // Y = S + i (i D) = (2 Re 4X, -2 Im 4X)
        ymk[0] = make_float2(2.f * x1.x, -2.f * x1.y);
    }
    // ypos(k) = yb + 64 q, ypos(M - k) = ym - 64 q for k = 2 (tau + 64 q) + unit
    float2* ybuf = lds;
    const int yb = tau + unit * (M / 2 + 16);
    const int ym = M / 2 - tau - unit + unit * (M / 2 + 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        ybuf[yb + TB * q] = yk[q];
        ybuf[q == 0 && zero ? M / 4 : ym - TB * q] = ymk[q];   // ypos(M / 2) = M / 4
    }
    __syncthreads();

    // 4. inverse transform (unit 0) of Y; unit 1 computes the direct head meanwhile
    const Span rs = make_span(r, ch * L, L);
    auto put = [&](int t, float a) { IO::store(rs, REV ? L - 1 - t : t, a); };
    uint2 touched = make_uint2(0u, 0u);
    static_assert(M * sizeof(typename IO::T) <= 128 * TB, "unit 1 covers a channel's lines");
    if (unit == 0) {
#pragma unroll
        for (int q = 0; q < 16; ++q) x[q] = ybuf[ypos(tau + TB * q)];
    }
    __syncthreads();
    if (unit == 0) {
        pass1(lds, false, std::true_type{});
    } else {
        direct_head<TB>(hbuf, 1, 1, L, head, tau, [&](int, int t, float a) { put(t, a); });
        // the inputs of the channel pf ahead, which will run in this workgroup's place (same
        // XCD for pf a multiple of 8): one 128-byte line of v and of g per thread
        if (pf > 0 && ch + pf < (int64_t)gridDim.x)
            touched = touch_line(v, g, (ch + pf) * L, (int64_t)L, tau);
    }
    __syncthreads();
    if (unit == 0) pass2_read(lds);
    __syncthreads();
    if (unit == 0) pass2_write(lds, 2, std::true_type{});
    __syncthreads();
    if (unit == 0) {
        TC tw[10];
        load_tw(trs, DIT1K_P3 + (2 * TB + tau) * 10, tw);
#pragma unroll
        for (int n = 0; n < 16; ++n) x[n] = lds[p2pos(n, tau)];
        dit16<true, true>(x, tw);
        // 5. x[q] = 8 M y_m, m = tau + 64 q (q < 8): r_{2m} = Re, r_{2m+1} = Im
        const float scale = 1.0f / (8.0f * (float)M);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int t = 2 * (tau + TB * q);
            if (t >= head && t < L) {
                const float a = x[q].x * scale, b = x[q].y * scale;
                if (t + 1 < L) {
                    if (pair_store) {
                        if (REV) IO::store2(rs, L - 2 - t, b, a);
                        else IO::store2(rs, t, a, b);
                    } else {
                        put(t, a);
                        put(t + 1, b);
                    }
                } else {
                    put(t, a);
                }
            }
        }
    }
    if (unit == 1) keep_touched(touched, pf, rs);
}

template <class IO, bool REV>
static hipError_t launch1k(const void* v, const void* g, void* r, int64_t nch, int L, int head,
                           bool pair, const float2* tab, hipStream_t stream)
{
    if (!grid_ok(nch, f1k::FT)) return hipErrorInvalidValue;
    // the next generation's inputs touched into the L2 of the XCD that will run it
    static int64_t resident[16];
    const int64_t pf =
        resident_workgroups((const void*)fused1k_kernel<IO, REV>, f1k::FT, resident) / 8 * 8;
    hipLaunchKernelGGL((fused1k_kernel<IO, REV>), dim3((unsigned)nch), dim3(f1k::FT), 0, stream,
                       (const typename IO::T*)v, (const typename IO::T*)g, (typename IO::T*)r, L,
                       head, pair ? 1 : 0, tab, pf);
    return hipGetLastError();
}

hipError_t launch_fused1k(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                          int head, bool pair_store, bool rev, const float2* tab,
                          hipStream_t stream)
{
    if (L <= 512 || L > 1024 || head > HEAD_MAX) return hipErrorInvalidValue;
    if (st == Store::F32)
        return rev ? launch1k<f32_io, true>(v, g, r, nch, L, head, pair_store, tab, stream)
                   : launch1k<f32_io, false>(v, g, r, nch, L, head, pair_store, tab, stream);
    return rev ? launch1k<bf16_io, true>(v, g, r, nch, L, head, pair_store, tab, stream)
               : launch1k<bf16_io, false>(v, g, r, nch, L, head, pair_store, tab, stream);
}

}  // namespace sc
