// Fused in-LDS causal convolution for 512 < L <= 2048 (transform length M = 1024 or 2048),
// gfx950.
//
// The method and data flow of the general fused kernel (sc_fused.hip): z = v + i g, the two
// branches u^b_n = z_n W_N^{b n} (N = 2M) transformed side by side by TB = M/16 threads each,
// the unpack of V G into the half-length real-output inverse spectrum Y, one length-M
// inverse, the first `head` outputs by direct summation ("Caracal: Causal Architecture via
// Spectral Mixing", key designs 1-2 and the real-FFT improvement its limitations name).  The
// transforms are organised as in the M = 4096 kernel (sc_fused4k.hip), with passes of radix
// R1 = M/256 (4 or 8), 16 and 16 in decimation in time:
//
//   n = n'' + 16 n2 + 256 n1,  k = k1 + R1 k2 + TB k3  (n1, k1 < R1; n2, k2, n'', k3 < 16)
//   pass 1 (registers): y1[n''+16 n2][k1] = sum_{n1} x[n] W_R1^{n1 k1}
//   pass 2: y2[n''][k1+R1 k2] = sum_{n2} W_{16 R1}^{n2 k1} y1[n''+16 n2][k1] W16^{n2 k2}
//   pass 3: X[m + TB k3] = sum_{n''} W_M^{n'' m} y2[n''][m] W16^{n'' k3},  m = k1 + R1 k2
//
// Thread tau holds elements tau + TB q (q < 16) at the input, so the radix-R1 groups of pass
// 1 (q0 + (16/R1) n1) sit in its registers and pass 1 needs no exchange; after pass 3 it
// holds bins tau + TB q, the order the unpack of the M = 4096 kernel takes.  Branch 1's
// rotation W_N^n = W_N^{n''} W_{32 R1}^{n2} W_{2 R1}^{n1} goes into the twiddles: W_{2 R1}
// is pass 1's constant base, W_{32 R1}^{2k1+1} and W_{2M}^{2m+1} are the bases of passes 2
// and 3.  All twiddles are merged into the butterflies (sc_dit.h).
//
// LDS (float2 units): pass 1 writes y1[n'][k1] at n' + 272 k1, pass 2 reads it (item
// (n'', k1) = (tau % 16, tau / 16)) and writes y2[n''][m] at m + (TB + 2) n'', pass 3 reads
// that; Y of the inverse at ypos(k), the mirror exchange of the unpack after Y.  Each access
// pattern hits 32 different bank pairs per 32 lanes (8-byte accesses serve 32 lanes per
// cycle).  M = 1024: 17.7 KB per workgroup of 128 threads, eight workgroups per CU; M = 2048:
// 35 KB per workgroup of 256 threads, four per CU.

#include "sc_device.h"
#include "sc_dit.h"
#include "sc_fft_lds.h"
#include "sc_internal.h"

namespace sc {

namespace fdit {

template <int M>
struct Shape {
    static constexpr int TB = M / 16, FT = 2 * TB, R1 = M / 256, G = 16 / R1;
    static constexpr int P2S = TB + 2;   // y2[n''][m] at m + P2S n''
    // one branch unit's pass layouts (positions < 272 R1 - 16 and < M + 30)
    static constexpr int REGION = 272 * R1 - 16 > M + 32 ? 272 * R1 - 16 : M + 32;
    static constexpr int XCH = M + 16;   // mirror exchange [unit][8][TB], after Y
    // the table's parts (sc_internal.h)
    static constexpr int T_P1B1 = DIT_P1B1, T_P2 = dit_p2(M), T_P3 = dit_p3(M);
    static constexpr int T_UNP = dit_unp(M), T_SIZE = dit_table_size(M);
    static_assert(R1 == 4 || R1 == 8, "M = 1024 or 2048");
    static_assert(XCH + 16 * TB <= 2 * REGION, "the exchange fits the two regions");
};

template <int M>
__device__ __forceinline__ int ypos(int k) { return (k >> 1) + (k & 1) * (M / 2 + 16); }

}  // namespace fdit

template <int M, class IO, bool REV>
__global__ __launch_bounds__(M / 8) void fused_dit_kernel(const typename IO::T* __restrict__ v,
                                                         const typename IO::T* __restrict__ g,
                                                         typename IO::T* __restrict__ r, int L,
                                                         int head, int pair_store,
                                                         const float2* __restrict__ tab,
                                                         int64_t pf)
{
    using namespace dit;
    using S = fdit::Shape<M>;
    constexpr int TB = S::TB, R1 = S::R1, G = S::G;
    __shared__ float2 lds[2 * S::REGION];
    __shared__ float hbuf[2 * HEAD_MAX];

    const auto trs = __builtin_amdgcn_make_buffer_rsrc((void*)tab, (short)0, S::T_SIZE * 8,
                                                       0x00020000);
    const int tid = threadIdx.x, tau = tid & (TB - 1);
    const int unit = __builtin_amdgcn_readfirstlane(tid / TB);   // uniform per wave
    const int64_t ch = blockIdx.x;
    const Span vs = make_span(v, ch * L, L);
    const Span gs = make_span(g, ch * L, L);

    // 1. z_n = v_n + i g_n, n = tau + TB q (0 past L)
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

    float2* const reg = lds + unit * S::REGION;
    const int npp = tau & 15, k1 = tau >> 4;   // the pass-2 item of this thread

    // pass 1 (forward or inverse): the G radix-R1 groups of registers q0 + G n1
    // (n' = tau + TB q0), branch 1 with its constant twiddle base, written to LDS
    auto pass1 = [&](float2* dst, bool twiddled, auto inv_tag) {
        constexpr bool INV = decltype(inv_tag)::value;
        TC tw[6];
        if (twiddled) {
#pragma unroll
            for (int i = 0; i < (R1 == 4 ? 1 : 3); ++i) {
                const float4 f = __builtin_bit_cast(
                    float4, __builtin_amdgcn_raw_buffer_load_b128(trs, S::T_P1B1 * 8 + 16 * i, 0, 0));
                tw[2 * i] = TC{f.x, f.y};
                tw[2 * i + 1] = TC{f.z, f.w};
            }
        }
#pragma unroll
        for (int q0 = 0; q0 < G; ++q0) {
            float2 y[R1];
#pragma unroll
            for (int n1 = 0; n1 < R1; ++n1) y[n1] = x[q0 + G * n1];
            if constexpr (R1 == 4) {
                if (twiddled) dft4t<INV>(y[0], y[1], y[2], y[3], tw[0], tw[1]);
                else dft4<INV>(y[0], y[1], y[2], y[3]);
            } else {
                if (twiddled) dft8t<INV>(y, tw);
                else dft8<INV>(y);
            }
            const int np = tau + TB * q0;
#pragma unroll
            for (int kk = 0; kk < R1; ++kk) dst[np + 272 * kk] = y[kk];
        }
    };
    // pass 2, item (n'', k1): its inputs y1[n'' + 16 n2][k1] (read before a barrier), then the
    // butterfly and y2[n''][k1 + R1 k2] written
    auto pass2_read = [&](const float2* buf) {
#pragma unroll
        for (int n2 = 0; n2 < 16; ++n2) x[n2] = buf[npp + 16 * n2 + 272 * k1];
    };
    auto pass2_write = [&](float2* buf, int var, auto inv_tag) {
        constexpr bool INV = decltype(inv_tag)::value;
        TC tw[10];
        load_tw(trs, S::T_P2 + (var * R1 + k1) * 10, tw);
        dit16<INV>(x, tw);
#pragma unroll
        for (int k2 = 0; k2 < 16; ++k2) buf[k1 + R1 * k2 + S::P2S * npp] = x[k2];
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
        load_tw(trs, S::T_P3 + (unit * TB + tau) * 10, tw);
#pragma unroll
        for (int n = 0; n < 16; ++n) x[n] = reg[tau + S::P2S * n];
        __syncthreads();
        dit16<false>(x, tw);   // x[q] = Z_{2 (tau + TB q) + unit}
    }

    // 3. unpack.  The mirror thread needs registers 4..7 and 12..15 of this one.
    float2* xch = lds + S::XCH + unit * 8 * TB;
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
            float2, __builtin_amdgcn_raw_buffer_load_b64(trs, k * 8, S::T_UNP * 8, 0));
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
    // ypos(k) = yb + TB q, ypos(M - k) = ym - TB q for k = 2 (tau + TB q) + unit
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
    // The inverse alternates between the two regions, unit 1's being free now: pass 1 writes
    // region 1 while Y in region 0 may still be read, pass 2 reads region 1 and writes region
    // 0, so neither needs a barrier between its reads and its writes.
    if (unit == 0) {
#pragma unroll
        for (int q = 0; q < 16; ++q) x[q] = ybuf[fdit::ypos<M>(tau + TB * q)];
        pass1(lds + S::REGION, false, std::true_type{});
    } else {
        direct_head<TB>(hbuf, 1, 1, L, head, tau, [&](int, int t, float a) { put(t, a); });
        // the inputs of the channel pf ahead, which will run in this workgroup's place (same
        // XCD for pf a multiple of 8): one 128-byte line of v and of g per thread
        if (pf > 0 && ch + pf < (int64_t)gridDim.x)
            touched = touch_line(v, g, (ch + pf) * L, (int64_t)L, tau);
    }
    __syncthreads();
    if (unit == 0) {
        pass2_read(lds + S::REGION);
        pass2_write(lds, 2, std::true_type{});
    }
    __syncthreads();
    if (unit == 0) {
        TC tw[10];
        load_tw(trs, S::T_P3 + (2 * TB + tau) * 10, tw);
#pragma unroll
        for (int n = 0; n < 16; ++n) x[n] = lds[tau + S::P2S * n];
        dit16<true, true>(x, tw);
        // 5. x[q] = 8 M y_m, m = tau + TB q (q < 8): r_{2m} = Re, r_{2m+1} = Im
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

template <int M, class IO, bool REV>
static hipError_t launch_dit(const void* v, const void* g, void* r, int64_t nch, int L, int head,
                             bool pair, const float2* tab, hipStream_t stream)
{
    constexpr int FT = fdit::Shape<M>::FT;
    if (!grid_ok(nch, FT)) return hipErrorInvalidValue;
    // the next generation's inputs touched into the L2 of the XCD that will run it
    static int64_t resident[16];
    const int64_t pf =
        resident_workgroups((const void*)fused_dit_kernel<M, IO, REV>, FT, resident) / 8 * 8;
    hipLaunchKernelGGL((fused_dit_kernel<M, IO, REV>), dim3((unsigned)nch), dim3(FT), 0, stream,
                       (const typename IO::T*)v, (const typename IO::T*)g, (typename IO::T*)r, L,
                       head, pair ? 1 : 0, tab, pf);
    return hipGetLastError();
}

hipError_t launch_fused_dit(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                            int M, int head, bool pair_store, bool rev, const float2* tab,
                            hipStream_t stream)
{
    if (L <= M / 2 || L > M || head > HEAD_MAX) return hipErrorInvalidValue;
#define SC_CALL(m)                                                                             \
    st == Store::F32                                                                           \
        ? (rev ? launch_dit<m, f32_io, true>(v, g, r, nch, L, head, pair_store, tab, stream)    \
               : launch_dit<m, f32_io, false>(v, g, r, nch, L, head, pair_store, tab, stream))  \
        : (rev ? launch_dit<m, bf16_io, true>(v, g, r, nch, L, head, pair_store, tab, stream)   \
               : launch_dit<m, bf16_io, false>(v, g, r, nch, L, head, pair_store, tab, stream))
    switch (M) {
    case 1024: return SC_CALL(1024);
    case 2048: return SC_CALL(2048);
    default: return hipErrorInvalidValue;
    }
#undef SC_CALL
}

}  // namespace sc
