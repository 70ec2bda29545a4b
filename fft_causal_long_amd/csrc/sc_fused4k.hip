// Fused in-LDS causal convolution for 2048 < L <= 4096 (transform length M = 4096), gfx950.
//
// The same method and data flow as the general fused kernel (sc_fused.hip): z = v + i g, the
// two branches u^b_n = z_n W_N^{b n} (N = 2M) transformed side by side by 256 threads each,
// the unpack of V G into the half-length real-output inverse spectrum Y, one length-M
// inverse transform, the first `head` outputs by direct summation ("Caracal: Causal
// Architecture via Spectral Mixing", key designs 1-2 and the real-FFT improvement its
// limitations name).  What differs is how each transform is organised for this chip:
//
//  * Radix-16 Stockham passes in decimation in time.  An item's 16 inputs carry twiddles
//    A^{n2} (input 0 none), so each 4-point sub-transform of the 4 x 4 split has input
//    twiddles (1, T, T^2, T^3) and every twiddle multiply can be merged into the butterfly
//    adds: with T = c (1 + i t) (t = tan of T's angle), T y = c (y + i t y), and
//    a +- T y = a +- c (y + i t y) costs 6 fused multiply-adds instead of 4 for the product
//    and 4 for the sums (Linzer and Feig's scaled-twiddle FFT).  A 16-point butterfly with
//    all its twiddles is 192 instructions instead of 160 + 60, from 10 (c, t) pairs per item
//    in a table (5 16-byte loads instead of 15 8-byte loads).  Where c is 0 (T = +-i) the
//    table holds c = 2^-40, t = +-2^40, which keeps c (y + i t y) accurate to fp32 round-off.
//  * Pass 1 takes each thread's loaded elements x[tau + 256 n2] as they are, so the loads
//    feed it directly.  Branch 1's rotation W_N^n = W_N^tau W_32^{n2} becomes the constant
//    twiddle base W_32 of pass 1, its per-item factor W_N^tau being carried into the
//    twiddle bases of passes 2 and 3 (W_512^{1+2j} and W_8192^{1+2j} instead of W_256^j and
//    W_4096^j): no separate multiply of the inputs.
//  * LDS layout pos(a) = (a + 16 (a >> 8)) XOR ((a >> 5) & 15) (float2 units).  An 8-byte LDS
//    access serves 32 lanes per cycle on gfx950; with this layout the passes' writes (runs of
//    consecutive elements) and reads (strides 16 and 256) hit 32 different bank pairs.  (The
//    general kernel's one-pad-per-16 layout, made for 16-lane groups, conflicts here.)
//  * The unpack works from registers: bins k and M + k of branch b sit in one thread, bins
//    N - k and M - k in its mirror thread (256 - tau - b) mod 256, which hands over 8 values
//    through LDS; each thread then forms 4 of its 8 pairs (its mirror forms the other 4).
//    Y is stored even bins first (Y_{2i} at i, Y_{2i+1} at 2064 + i), which keeps both its
//    writes and the inverse's reads free of bank conflicts.
//  * The inverse's last pass computes only the 8 outputs of each item that are kept.  Unit 1
//    computes the direct head meanwhile and then, for bf16 storage, touches the inputs of
//    the workgroup that will take this one's place (see touch_line), so that it starts
//    from L2 instead of HBM.

#include "sc_device.h"
#include "sc_fft_lds.h"
#include "sc_internal.h"
#include "sc_dit.h"

namespace sc {

namespace f4k {

constexpr int M = 4096, TB = 256, FT = 512;
constexpr int REGION = 4336;          // one branch unit's transform layout (pos < 4336)
constexpr int XCH = 4112;             // mirror exchange: [unit][8][256] after the Y buffer

__device__ __forceinline__ int fpos(int a) { return (a + ((a >> 8) << 4)) ^ ((a >> 5) & 15); }
// LDS float2 at a byte offset from base (the XORs below act on byte offsets directly)
__device__ __forceinline__ float2& at_byte(float2* base, int byte)
{
    return *(float2*)((char*)base + byte);
}
__device__ __forceinline__ int ypos(int k) { return (k >> 1) + (k & 1) * (M / 2 + 16); }

// operand types of the matrix-core first pass
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

using namespace dit;

}  // namespace f4k

template <class IO, bool REV, bool MF>
__global__ __launch_bounds__(512) void fused4k_kernel(const typename IO::T* __restrict__ v,
                                                      const typename IO::T* __restrict__ g,
                                                      typename IO::T* __restrict__ r, int L,
                                                      int head, int pair_store,
                                                      const float2* __restrict__ tab, int64_t pf)
{
    using namespace f4k;
    __shared__ float2 lds[2 * REGION];
    __shared__ float hbuf[2 * HEAD_MAX];

    const auto trs = __builtin_amdgcn_make_buffer_rsrc((void*)tab, (short)0, DIT4K_TABLE_FLOAT2 * 8,
                                                       0x00020000);
    const int tid = threadIdx.x, tau = tid & (TB - 1);
    const int unit = __builtin_amdgcn_readfirstlane(tid >> 8);   // uniform per wave
    const int64_t ch = blockIdx.x;
    const Span vs = make_span(v, ch * L, L);
    const Span gs = make_span(g, ch * L, L);

    // LDS positions fpos(a) of the access patterns, as per-thread bases plus constants:
    //  runs tau + 256 k2:        wb ^ (8 (k2 & 1)) + 272 k2
    //  pass 2 reads 256 j + k + 16 n2 (j = tau / 16, k = tau % 16):  r2 ^ (n2 / 2) + 16 n2
    //  pass 3 reads 16 tau + n2:  r3 ^ n2
    // (the unit's region offset is a multiple of 16, so it passes through the XORs, which
    // only touch the low 4 bits; indexing lds directly lets the XOR act on byte addresses)
    const int ro = unit * REGION;
    const int wb = ro + (tau & ~15) + ((tau & 15) ^ (tau >> 5));
    const int r2 = ro + 272 * (tau >> 4) + ((tau & 15) ^ (8 * ((tau >> 4) & 1)));
    const int r3 = ro + 16 * (tau + (tau >> 4)) + ((tau >> 1) & 15);
    const int wbb = wb << 3, r2b = r2 << 3, r3b = r3 << 3;   // byte offsets
    auto run_at = [&](int k2) -> float2& { return at_byte(lds, (wbb ^ (64 * (k2 & 1))) + 2176 * k2); };
    auto p2_at = [&](int n2) -> float2& { return at_byte(lds, (r2b ^ (8 * (n2 >> 1))) + 128 * n2); };
    auto p3_at = [&](int n2) -> float2& { return at_byte(lds, r3b ^ (8 * n2)); };

    float2 x[16];
    if constexpr (MF) {
        // 1-2. Pass 1 of branch `unit` on the matrix cores (bf16 storage).  Per item it is a
        //    fixed 32 x 32 real matrix (the 16-point DFT; on branch 1 times the rotation
        //    W_32^q of input q) applied to the item's 16 complex inputs as 32 reals.  The
        //    inputs are bf16 and the matrix is held as three bf16 parts (24 significant
        //    bits), so every product is exact and the fp32 sums give the pass to fp32
        //    round-off.  32 x 32 x 16 bf16 products: a wave's 64 items are two 32-column
        //    blocks, K = 32 reals in two halves h; lane l holds column l % 32 and, of half
        //    h, the reals of inputs q = 8 h + 4 (l / 32) + e (e < 4) as (v, g) bit pairs.
        const int lane = tid & 63, col = lane & 31, half = lane >> 5;
        const int wbase = tau & ~63;   // the wave's first item
        uint4 af[3][2];
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                af[t][h] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(
                               trs, (DIT4K_MF + ((unit * 3 + t) * 2 + h) * 128 + 2 * lane) * 8,
                               0, 0));
        // the (v, g) bits of each input, all 32 loads issued before any is used; for L = M
        // every offset is a per-lane base plus a constant (reversed v: from element
        // L - 1 - n), past L the loads read 0
        uint32_t rv[2][2][4], rg[2][2][4];
        if (L == M) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int it = wbase + 32 * b + col, q0 = 8 * h + 4 * half;
                    const int vb = REV ? L - 1 - it - TB * (q0 + 3) : it + TB * q0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        rv[b][h][e] = __builtin_amdgcn_raw_buffer_load_b16(
                            vs.rs, vb * 2, TB * 2 * (REV ? 3 - e : e), 0);
                        rg[b][h][e] = __builtin_amdgcn_raw_buffer_load_b16(
                            gs.rs, (it + TB * q0) * 2, TB * 2 * e, 0);
                    }
                }
        } else {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int n = wbase + 32 * b + col + TB * (8 * h + 4 * half + e);
                        const bool in = n < L;
                        const int ev = in ? (REV ? L - 1 - n : n) : IO::OOB;
                        const int eg = in ? n : IO::OOB;
                        rv[b][h][e] = __builtin_amdgcn_raw_buffer_load_b16(
                            vs.rs, (int)((uint32_t)ev * 2u), 0, 0);
                        rg[b][h][e] = __builtin_amdgcn_raw_buffer_load_b16(
                            gs.rs, (int)((uint32_t)eg * 2u), 0, 0);
                    }
        }
        uint4 bfr[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                bfr[b][h] = make_uint4(rv[b][h][0] | (rg[b][h][0] << 16),
                                       rv[b][h][1] | (rg[b][h][1] << 16),
                                       rv[b][h][2] | (rg[b][h][2] << 16),
                                       rv[b][h][3] | (rg[b][h][3] << 16));
        // input q = 0 of items 0..63 (wave 0 of unit 0, lanes l < 32) for the direct head
        if (unit == 0 && wbase == 0 && half == 0) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int t = 32 * b + col;
                if (t < head) {
                    hbuf[t] = __uint_as_float(bfr[b][0].x << 16);
                    hbuf[HEAD_MAX + t] = __uint_as_float(bfr[b][0].x & 0xffff0000u);
                }
            }
        }
        f4k::f32x16 acc[2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
        // within each K half, the small parts first
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int t = 2; t >= 0; --t)
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(f4k::bf16x8, af[t][h]),
                        __builtin_bit_cast(f4k::bf16x8, bfr[b][h]), acc[b], 0, 0, 0);
        // accumulator r of column c is real row i = 8 (r / 4) + 4 (l / 32) + r % 4 = 2 k2 + re/im
        // of item wbase + 32 b + c: registers 2 s, 2 s + 1 are output k2 = 4 (s / 2) +
        // 2 (l / 32) + s % 2, written where pass 2 reads the run of that item
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int it = wbase + 32 * b + col;
            const int wbi = (ro + (it & ~15) + ((it & 15) ^ (it >> 5))) << 3;
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) {
                const int k2 = 4 * (s2 >> 1) + 2 * half + (s2 & 1);
                at_byte(lds, (wbi ^ (64 * (k2 & 1))) + 2176 * k2) =
                    make_float2(acc[b][2 * s2], acc[b][2 * s2 + 1]);
            }
        }
    } else {
        // 1. z_n = v_n + i g_n, n = tau + 256 q (0 past L): pass 1's inputs as loaded.  For
        //    L = M the per-element offsets are scalar constants (no vector address arithmetic);
        //    reversed v runs from element L - 1 - tau - 3840 upwards.
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

        // 2. forward transform of branch `unit`
        if (unit == 0) {
            dft<16, false>(x);
        } else {
            TC tw[10];
            load_tw(trs, DIT4K_P1B1, tw);
            dit16<false>(x, tw);
        }
    #pragma unroll
        for (int k2 = 0; k2 < 16; ++k2) run_at(k2) = x[k2];
    }
    __syncthreads();
    {
        const int j = tau >> 4;
        TC tw[10];
        load_tw(trs, DIT4K_P2 + (unit * 16 + j) * 10, tw);
#pragma unroll
        for (int n2 = 0; n2 < 16; ++n2) x[n2] = p2_at(n2);
        __syncthreads();
        dit16<false>(x, tw);
        // outputs 16 j + 256 k2 + k = tau + 256 k2: a run
#pragma unroll
        for (int k2 = 0; k2 < 16; ++k2) run_at(k2) = x[k2];
    }
    __syncthreads();
    {
        TC tw[10];
        load_tw(trs, DIT4K_P3 + (unit * TB + tau) * 10, tw);
#pragma unroll
        for (int n2 = 0; n2 < 16; ++n2) x[n2] = p3_at(n2);
        __syncthreads();
        dit16<false>(x, tw);   // x[q] = Z_{2 (tau + 256 q) + unit}
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
            float2, __builtin_amdgcn_raw_buffer_load_b64(trs, k * 8, DIT4K_UNP * 8, 0));
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
    // ypos(k) = yb + 256 q, ypos(M - k) = ym - 256 q for k = 2 (tau + 256 q) + unit
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
    // The inverse alternates between the two regions, unit 1's being free now (its forward
    // data and the exchange are read): pass 1 writes region 1 while Y in region 0 may still
    // be read, pass 2 reads region 1 and writes region 0, so neither needs a barrier between
    // its reads and its writes.
    constexpr int R1B = REGION * 8;   // region 1, in bytes from region 0
    if (unit == 0) {
#pragma unroll
        for (int n2 = 0; n2 < 16; ++n2) x[n2] = ybuf[ypos(tau + TB * n2)];
        dft<16, true>(x);
#pragma unroll
        for (int k2 = 0; k2 < 16; ++k2)
            at_byte(lds, ((wbb ^ (64 * (k2 & 1))) + 2176 * k2) + R1B) = x[k2];
    } else {
        direct_head<TB>(hbuf, 1, 1, L, head, tau, [&](int, int t, float a) { put(t, a); });
        // the inputs of the channel pf ahead, which will run in this workgroup's place (same
        // XCD for pf a multiple of 8): one 128-byte line of v and of g per thread
        if (pf > 0 && ch + pf < (int64_t)gridDim.x)
            touched = touch_line(v, g, (ch + pf) * L, (int64_t)L, tau);
    }
    __syncthreads();
    const int j = tau >> 4;
    if (unit == 0) {
#pragma unroll
        for (int n2 = 0; n2 < 16; ++n2)
            x[n2] = at_byte(lds, ((r2b ^ (8 * (n2 >> 1))) + 128 * n2) + R1B);
        TC tw[10];
        load_tw(trs, DIT4K_P2 + (2 * 16 + j) * 10, tw);
        dit16<true>(x, tw);
#pragma unroll
        for (int k2 = 0; k2 < 16; ++k2) run_at(k2) = x[k2];
    }
    __syncthreads();
    if (unit == 0) {
        TC tw[10];
        load_tw(trs, DIT4K_P3 + (2 * TB + tau) * 10, tw);
#pragma unroll
        for (int n2 = 0; n2 < 16; ++n2) x[n2] = p3_at(n2);
        dit16<true, true>(x, tw);
        // 5. x[q] = 8 M y_m, m = tau + 256 q (q < 8): r_{2m} = Re, r_{2m+1} = Im
        const float scale = 1.0f / (8.0f * (float)M);
        if (L == M && pair_store) {
            // every pair is inside the row; only q = 0 (t < 512) can meet the direct head
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int t = 2 * (tau + TB * q);
                if (q > 0 || t >= head) {
                    if (REV) IO::store2(rs, L - 2 - t, x[q].y * scale, x[q].x * scale);
                    else IO::store2(rs, t, x[q].x * scale, x[q].y * scale);
                }
            }
            return;
        }
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

template <class IO, bool REV, bool MF = false>
static hipError_t launch4k(const void* v, const void* g, void* r, int64_t nch, int L, int head,
                           bool pair, const float2* tab, hipStream_t stream)
{
    static_assert(!MF || sizeof(typename IO::T) == 2, "the matrix-core first pass takes bf16");
    if (!grid_ok(nch, f4k::FT)) return hipErrorInvalidValue;
    // the next generation's inputs: bf16 only (16 KB per channel).  With fp32 (32 KB) the
    // touched lines of the 64 workgroups ahead on an XCD (2 MB) crowd the 4 MB L2 that the
    // running ones use, and the call got 2% slower instead of 4% faster.
    static int64_t resident[16];
    const int64_t pf =
        sizeof(typename IO::T) == 2
            ? resident_workgroups((const void*)fused4k_kernel<IO, REV, MF>, f4k::FT, resident) / 8 * 8
            : 0;
    hipLaunchKernelGGL((fused4k_kernel<IO, REV, MF>), dim3((unsigned)nch), dim3(f4k::FT), 0, stream,
                       (const typename IO::T*)v, (const typename IO::T*)g, (typename IO::T*)r, L,
                       head, pair ? 1 : 0, tab, pf);
    return hipGetLastError();
}

hipError_t launch_fused4k(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                          int head, bool pair_store, bool rev, bool mf, const float2* tab,
                          hipStream_t stream)
{
    if (L <= 2048 || L > 4096 || head > HEAD_MAX) return hipErrorInvalidValue;
    if (mf) {
        if (st != Store::BF16) return hipErrorInvalidValue;
        return rev ? launch4k<bf16_io, true, true>(v, g, r, nch, L, head, pair_store, tab, stream)
                   : launch4k<bf16_io, false, true>(v, g, r, nch, L, head, pair_store, tab, stream);
    }
    if (st == Store::F32)
        return rev ? launch4k<f32_io, true>(v, g, r, nch, L, head, pair_store, tab, stream)
                   : launch4k<f32_io, false>(v, g, r, nch, L, head, pair_store, tab, stream);
    return rev ? launch4k<bf16_io, true>(v, g, r, nch, L, head, pair_store, tab, stream)
               : launch4k<bf16_io, false>(v, g, r, nch, L, head, pair_store, tab, stream);
}

}  // namespace sc
