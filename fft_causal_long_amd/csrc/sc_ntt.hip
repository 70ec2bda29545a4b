// Exact causal convolution through a number-theoretic transform (gfx950), L <= 4096.
//
// "Catastrophic Token Leakage in Convolutional Sequence Modeling and How to Mitigate It"
// (abstract): float FFT convolutions leak future tokens through round-off; an FFT done on
// integers only cannot.  Here the pad-to-2L recipe of "Caracal: Causal Architecture via
// Spectral Mixing" (key designs 1 and 2) runs in Z_p, p = 998244353 = 119*2^23 + 1, with
// omega_n = 3^((p-1)/n) in place of exp(-2 pi i / n).  Every step is an exact residue
// computation, so output t is a function of v_0..v_t and g_0..g_t alone.
//
// Per channel, with N = 2M and the upper half of the padded inputs zero, the first
// decimation-in-frequency stage is a twiddle only:  V_{2j+b} = NTT_M(v_n omega_N^{b n})_j,
// likewise G.  For b = 0, 1 ("branches") the workgroup computes NTT_M of v and of g, the
// product X = V G N^{-1} and e^b = INTT_M(X^b); for n < L
//     x_n = N^{-1} sum_k X_k omega_N^{-nk} = e^0_n + omega_N^{-n} e^1_n      (N^{-1} folded)
// and the residue is lifted to [-(p-1)/2, (p-1)/2].  The inverse uses
//     INTT_M(X)_n = NTT_M(X)_{(M - n) mod M}
// so one forward transform serves both directions.
//
// Arithmetic.  Residues are integers carried in float64 registers: sums and differences
// are exact while magnitudes stay below 2^53 (here below 2^36), so butterflies need no
// reduction.  A product a*w mod p (|a| < 2^36, 0 <= w < p) is exact in six full-rate fp64
// operations:
//     h = fl(a w);  l = fma(a, w, -h)            (the exact rounding error, an integer)
//     q = round(a w / p)                         (fma with w/p and the 1.5*2^52 shift)
//     r = fma(-q, p, h) + l = a w - q p          (exact: |h - q p| < 2^31)
// giving |r| <= 1.5 p.  LDS holds int32 values (|x| < 2^31) between passes.
//
// Layout as in the float kernel: max(64, M/8) threads, a length-M transform held by TB = M/16
// threads with 16 values each, Stockham radix-16 passes through LDS (a v and a g array per
// branch unit), 68 KB of LDS per workgroup at M = 4096.

#include "sc_device.h"
#include "sc_internal.h"

namespace sc {

namespace ntt {

constexpr double SHIFT = 6755399441055744.0;   // 1.5 * 2^52: x + SHIFT - SHIFT = round(x), |x| < 2^51

// The NTT primes: p - 1 is divisible by 2^21 (transform lengths up to 2^21 have roots of
// unity) and 3 is a primitive root.  PrimeA is the exact kind's modulus; the three together
// carry the exact real-valued path (residues combined by the Chinese remainder theorem).
struct PrimeA {
    static constexpr uint64_t p = 998244353ull;    // 119 * 2^23 + 1
};
struct PrimeB {
    static constexpr uint64_t p = 1004535809ull;   // 479 * 2^21 + 1
};
struct PrimeC {
    static constexpr uint64_t p = 469762049ull;    // 7 * 2^26 + 1
};
constexpr uint64_t ROOT = 3;

// a constant residue w with w / p rounded to double
struct W {
    double w, q;
};

template <class Pr>
constexpr uint64_t powmod_c(uint64_t b, uint64_t e)
{
    uint64_t r = 1;
    b %= Pr::p;
    while (e) {
        if (e & 1) r = r * b % Pr::p;
        b = b * b % Pr::p;
        e >>= 1;
    }
    return r;
}
// omega_n^k as a W constant (n | p - 1)
template <class Pr>
constexpr W root_c(uint64_t n, uint64_t k)
{
    const uint64_t w = powmod_c<Pr>(powmod_c<Pr>(ROOT, (Pr::p - 1) / n), k);
    return W{(double)w, (double)w / (double)Pr::p};
}

__device__ __forceinline__ double round_int(double x)
{
    return (x + SHIFT) - SHIFT;
}
// a * w mod p, |a| < 2^36, |result| <= 1.5 p
template <class Pr>
__device__ __forceinline__ double mulc(double a, W w)
{
    constexpr double P = (double)Pr::p;
    const double h = a * w.w;
    const double l = __builtin_fma(a, w.w, -h);
    const double q = __builtin_fma(a, w.q, SHIFT) - SHIFT;
    return __builtin_fma(-q, P, h) + l;
}
// a * b mod p for |a|, |b| <= p, |result| <= p
template <class Pr>
__device__ __forceinline__ double mulv(double a, double b)
{
    constexpr double P = (double)Pr::p, PINV = 1.0 / (double)Pr::p;
    const double h = a * b;
    const double l = __builtin_fma(a, b, -h);
    const double q = __builtin_fma(h, PINV, SHIFT) - SHIFT;
    return __builtin_fma(-q, P, h) + l;
}
// a mod p into [-p/2, p/2] (up to one p at the edges), |a| < 2^51
template <class Pr>
__device__ __forceinline__ double reduce(double a)
{
    constexpr double P = (double)Pr::p, PINV = 1.0 / (double)Pr::p;
    const double q = __builtin_fma(a, PINV, SHIFT) - SHIFT;
    return __builtin_fma(-q, P, a);
}
// the balanced representative in [-(p-1)/2, (p-1)/2] of a value with |a| <= 2 p
template <class Pr>
__device__ __forceinline__ double balance(double a)
{
    constexpr double P = (double)Pr::p, H = 0.5 * ((double)Pr::p - 1.0);
    a = a > H ? a - P : (a < -H ? a + P : a);
    return a > H ? a - P : (a < -H ? a + P : a);
}

// twiddle bank entry i as W (double2 {w, w/p})
struct Tw {
    __amdgpu_buffer_rsrc_t rs;
    __device__ __forceinline__ W at(int voff_elems, int soff_elems) const
    {
        const auto d = __builtin_amdgcn_raw_buffer_load_b128(rs, voff_elems * 16, soff_elems * 16, 0);
        return __builtin_bit_cast(W, d);
    }
};

// in-register DFT_R over Z_p (forward, omega_R), natural order in and out, inputs < 2^33.
// R = 16 = 4 x 4:  X[4 k1 + k2] = sum_{n1} w4^{n1 k1} w16^{n1 k2} sum_{n2} x[n1 + 4 n2] w4^{n2 k2}
template <int R, class Pr>
__device__ __forceinline__ void dft(double* a)
{
    if constexpr (R == 2) {
        const double x = a[0];
        a[0] = x + a[1];
        a[1] = x - a[1];
    } else if constexpr (R == 4) {
        constexpr W w4 = root_c<Pr>(4, 1);
        const double t0 = a[0] + a[2], t1 = a[0] - a[2];
        const double t2 = a[1] + a[3], t3 = mulc<Pr>(a[1] - a[3], w4);
        a[0] = t0 + t2;
        a[2] = t0 - t2;
        a[1] = t1 + t3;
        a[3] = t1 - t3;
    } else if constexpr (R == 8) {
        constexpr W w1 = root_c<Pr>(8, 1), w2 = root_c<Pr>(8, 2), w3 = root_c<Pr>(8, 3);
        double u[4], t[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            u[n] = a[n] + a[n + 4];
            t[n] = a[n] - a[n + 4];
        }
        t[1] = mulc<Pr>(t[1], w1);
        t[2] = mulc<Pr>(t[2], w2);
        t[3] = mulc<Pr>(t[3], w3);
        dft<4, Pr>(u);
        dft<4, Pr>(t);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a[2 * k] = u[k];
            a[2 * k + 1] = t[k];
        }
    } else {
        static_assert(R == 16, "radix 2, 4, 8 or 16");
        double c[4];
#pragma unroll
        for (int n1 = 0; n1 < 4; ++n1) {
            c[0] = a[n1]; c[1] = a[n1 + 4]; c[2] = a[n1 + 8]; c[3] = a[n1 + 12];
            dft<4, Pr>(c);
            a[n1] = c[0]; a[n1 + 4] = c[1]; a[n1 + 8] = c[2]; a[n1 + 12] = c[3];
        }
        // a[n1 + 4 k2] *= w16^{n1 k2}
        a[5] = mulc<Pr>(a[5], root_c<Pr>(16, 1));
        a[9] = mulc<Pr>(a[9], root_c<Pr>(16, 2));
        a[13] = mulc<Pr>(a[13], root_c<Pr>(16, 3));
        a[6] = mulc<Pr>(a[6], root_c<Pr>(16, 2));
        a[10] = mulc<Pr>(a[10], root_c<Pr>(16, 4));
        a[14] = mulc<Pr>(a[14], root_c<Pr>(16, 6));
        a[7] = mulc<Pr>(a[7], root_c<Pr>(16, 3));
        a[11] = mulc<Pr>(a[11], root_c<Pr>(16, 6));
        a[15] = mulc<Pr>(a[15], root_c<Pr>(16, 9));
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) dft<4, Pr>(a + 4 * k2);
        // a[4 k2 + k1] = X[4 k1 + k2]: transpose to natural order
        double t;
        t = a[1]; a[1] = a[4]; a[4] = t;
        t = a[2]; a[2] = a[8]; a[8] = t;
        t = a[3]; a[3] = a[12]; a[12] = t;
        t = a[6]; a[6] = a[9]; a[9] = t;
        t = a[7]; a[7] = a[13]; a[13] = t;
        t = a[11]; a[11] = a[14]; a[14] = t;
    }
}

__device__ __forceinline__ int lds_pad(int a) { return a + (a >> 4); }

template <int TB>
__device__ __forceinline__ int reg_off(int tau, int q)
{
    if constexpr (TB % 16 == 0) return tau + (tau >> 4) + q * (TB + TB / 16);
    else return lds_pad(tau + TB * q);
}

// One Stockham DIF pass (index scheme as in the float kernel) over NA arrays sharing the
// twiddles.  Passes with twiddles are radix 16 with one item per thread; their outputs are
// reduced below 2^31 (k2 > 0 by the twiddle product, k2 = 0 explicitly) and stored as int32.
template <int M, int R, int S, int NA, class Pr>
__device__ __forceinline__ void pass(double (&x)[NA][16], int32_t* __restrict__ buf0,
                                     int32_t* __restrict__ buf1, int tau, const Tw& tw)
{
    constexpr int NB = 16 / R, Q = M / S, QN = Q / R;
    if constexpr (QN > 1) {
        static_assert(R == 16, "passes with twiddles are radix 16");
        const int s = tau & (S - 1), n1 = tau / S;
        W w[16];
#pragma unroll
        for (int k2 = 1; k2 < 16; ++k2) w[k2] = tw.at(n1, NTT_PASS_BASE + (Q - 32) + k2 * (Q / 16));
        constexpr int STEP = S == 1 ? 1 : S + S / 16;
        const int base = S == 1 ? 17 * n1 : (s + (s >> 4)) + 16 * n1 * STEP;
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            dft<16, Pr>(x[a]);
            int32_t* buf = a == 0 ? buf0 : buf1;
            buf[base] = (int32_t)reduce<Pr>(x[a][0]);
#pragma unroll
            for (int k2 = 1; k2 < 16; ++k2)
                buf[base + k2 * STEP] = (int32_t)mulc<Pr>(x[a][k2], w[k2]);
        }
    } else {
#pragma unroll
        for (int a = 0; a < NA; ++a) {
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                double b[R];
#pragma unroll
                for (int n2 = 0; n2 < R; ++n2) b[n2] = x[a][q + NB * n2];
                dft<R, Pr>(b);
#pragma unroll
                for (int k2 = 0; k2 < R; ++k2) x[a][q + NB * k2] = b[k2];
            }
        }
    }
}

template <int M, int NA, class Pr, int S = 1>
__device__ __forceinline__ void passes(double (&x)[NA][16], int32_t* __restrict__ buf0,
                                       int32_t* __restrict__ buf1, int tau, const Tw& tw)
{
    constexpr int TB = M / 16, Q = M / S, R = Q >= 16 ? 16 : Q;
    if constexpr (Q / R > 1) {
        pass<M, R, S, NA, Pr>(x, buf0, buf1, tau, tw);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            x[0][q] = (double)buf0[reg_off<TB>(tau, q)];
            if constexpr (NA > 1) x[1][q] = (double)buf1[reg_off<TB>(tau, q)];
        }
        __syncthreads();
        passes<M, NA, Pr, S * R>(x, buf0, buf1, tau, tw);
    } else {
        pass<M, R, S, NA, Pr>(x, buf0, buf1, tau, tw);
    }
}

}  // namespace ntt

// REV (the gradient kernels): the first input is read reversed and the output is written
// reversed: rev(causal(rev(dr), b))_j = sum_{t>=j} dr_t b_{t-j}.
// FIX: float32 inputs encoded as integers round(v 2^fv), round(g 2^fg) (nearest, ties to
// even; sv = 2^fv, sg = 2^fg, |v sv|, |g sg| < 2^51) instead of int32 inputs.
// Threads of the workgroup for length-M transforms: one channel from M = 512 on, as many
// as fill one wave below (as the float kernel).
template <int M>
constexpr int ntt_threads() { return M / 8 > 64 ? M / 8 : 64; }

template <int M, bool REV, class Pr, bool FIX>
__global__ __launch_bounds__(ntt_threads<M>(), 4) void ntt_conv_kernel(const void* __restrict__ v,
                                                       const void* __restrict__ g,
                                                       int32_t* __restrict__ r, int64_t nch,
                                                       int L, const double* __restrict__ bank,
                                                       double ninv, double ninv_q, double sv,
                                                       double sg)
{
    using namespace ntt;
    static_assert(M >= 64 && M <= 4096, "fused NTT handles 64 <= M <= 4096");
    constexpr int N = 2 * M, TB = M / 16, UNITS = ntt_threads<M>() / TB, CPW = UNITS / 2;
    constexpr int REG = M + M / 16;
    __shared__ int32_t lds[UNITS * 2 * REG];

    const Tw tw{__builtin_amdgcn_make_buffer_rsrc((void*)bank, (short)0, NTT_BANK_ENTRIES * 16,
                                                  0x00020000)};
    const int tid = threadIdx.x;
    const int unit = tid / TB, tau = tid % TB;
    const int cl = unit >> 1, beta = unit & 1;
    const int64_t ch0 = (int64_t)blockIdx.x * CPW;
    const int nvalid = (int)((nch - ch0) < CPW ? (nch - ch0) : CPW);
    // both input kinds have 4-byte elements
    const Span vs = make_span((const int32_t*)v, ch0 * L, (int64_t)nvalid * L);
    const Span gs = make_span((const int32_t*)g, ch0 * L, (int64_t)nvalid * L);
    const Span rs = make_span(r, ch0 * L, (int64_t)nvalid * L);
    int32_t* bv = lds + unit * 2 * REG;
    int32_t* bg = bv + REG;
    const int cbase = cl * L;

    // 1. inputs as exact doubles (|x| < 2^31), times omega_N^n on branch 1.  Positions past
    //    L are read at byte offset 2^31, beyond the descriptor's range, so they read 0 (a
    //    select instead of a branch keeps all the loads in flight together).  All 32 element
    //    loads are issued first and branch 1's 16 twiddle loads right after them: converting
    //    and multiplying element by element under the branch made every element wait for
    //    its own loads, one memory latency per element.
    uint32_t wa[16], wb[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int n = tau + TB * q;
        const bool in = L == M || n < L;
        const uint32_t ob = in ? (uint32_t)(cbase + n) * 4u : 0x80000000u;
        const uint32_t oa = in ? (uint32_t)(cbase + (REV ? L - 1 - n : n)) * 4u : 0x80000000u;
        wa[q] = __builtin_amdgcn_raw_buffer_load_b32(vs.rs, (int)oa, 0, 0);
        wb[q] = __builtin_amdgcn_raw_buffer_load_b32(gs.rs, (int)ob, 0, 0);
    }
    auto to_residue = [&](uint32_t w, double scale) -> double {
        if constexpr (FIX)   // exact: a float times a power of two, rounded, reduced mod p
            return reduce<Pr>(round_int((double)__uint_as_float(w) * scale));
        else
            return (double)(int32_t)w;
    };
    double x[2][16];
    if (beta) {
        // the twiddles in two batches of 8, which bounds the registers held at once
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            W wq[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wq[i] = tw.at((tau + TB * (8 * h + i)) * (NTT_TW_N / N), 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = 8 * h + i;
                x[0][q] = mulc<Pr>(to_residue(wa[q], sv), wq[i]);
                x[1][q] = mulc<Pr>(to_residue(wb[q], sg), wq[i]);
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            x[0][q] = to_residue(wa[q], sv);
            x[1][q] = to_residue(wb[q], sg);
        }
    }

    // 2. V, G = NTT_M(.) in natural order (values below 2^36)
    passes<M, 2, Pr>(x, bv, bg, tau, tw);

    // 3. X = V * (G N^{-1})
    double y[1][16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
        y[0][q] = mulv<Pr>(reduce<Pr>(x[0][q]), reduce<Pr>(mulc<Pr>(x[1][q], W{ninv, ninv_q})));

    // 4. f = NTT_M(X): e^beta_n = f_{(M - n) mod M}
    passes<M, 1, Pr>(y, bv, bv, tau, tw);

    // 5. register q of thread tau holds e^beta at n = (M - tau - TB q) mod M.
    //    x_n = e^0_n + omega_N^{-n} e^1_n: branch 0 finishes q < 8, branch 1 q >= 8, each
    //    handing the other half to its partner through LDS (branch 0's v region).
    int32_t* xch = lds + (2 * cl) * 2 * REG;
    double own[16];
    if (beta) {
        // omega_N^{-n} = omega_N^{N - n}; the 16 twiddle loads issued together
        W wq[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int n = (M - tau - TB * q) & (M - 1);
            wq[q] = tw.at(((N - n) & (N - 1)) * (NTT_TW_N / N), 0);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) own[q] = mulc<Pr>(y[0][q], wq[q]);
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) own[q] = reduce<Pr>(y[0][q]);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q)
        if ((q < 8) == (beta == 1)) xch[reg_off<TB>(tau, q)] = (int32_t)own[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        if ((q < 8) != (beta == 0)) continue;
        const int n = (M - tau - TB * q) & (M - 1);
        if (n >= L) continue;
        const double s = balance<Pr>(reduce<Pr>(own[q] + (double)xch[reg_off<TB>(tau, q)]));
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(int32_t)s, rs.rs,
                                              (cbase + (REV ? L - 1 - n : n)) * 4, 0, 0);
    }
}

// ---------------------------------------------------------------- Chinese remainder decode

namespace ntt {

// constants of Garner's algorithm for the primes A, B, C (as residues with w/p)
template <class Pr>
constexpr W wconst(uint64_t w)
{
    return W{(double)(w % Pr::p), (double)(w % Pr::p) / (double)Pr::p};
}
constexpr uint64_t PA = PrimeA::p, PB = PrimeB::p, PC = PrimeC::p;
constexpr W INV_A_MOD_B = wconst<PrimeB>(powmod_c<PrimeB>(PA % PB, PB - 2));
constexpr W A_MOD_C = wconst<PrimeC>(PA % PC);
constexpr W INV_AB_MOD_C = wconst<PrimeC>(powmod_c<PrimeC>((PA % PC) * (PB % PC) % PC, PC - 2));

// A B as the sum of two doubles: the nearest double and the (small, exact) rest
constexpr uint64_t AB = PA * PB;
constexpr double AB_HI = (double)AB;
constexpr double AB_LO = (double)((int64_t)AB - (int64_t)(uint64_t)AB_HI);

// error-free transformations: s + e == a + b (Knuth's two-sum) and p + e == a b (with an FMA).
// No contraction here: a product fused into a later sum would no longer be the p whose
// error e describes, and the sums would lose their exactness.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e)
{
#pragma clang fp contract(off)
    s = a + b;
    const double bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}
__device__ __forceinline__ void two_prod(double a, double b, double& p, double& e)
{
#pragma clang fp contract(off)
    p = a * b;
    e = __builtin_fma(a, b, -p);
}

// The float32 nearest to R 2^-F (ties to even, subnormals included) for the integer
// R = a0 + a1 A + a2 A B with balanced digits (|R| < 2^89).  R is first written exactly as
// hi + lo + e3 (doubles, |lo + e3| below the gap between hi and its neighbour on that
// side), then rounded to 53 bits by rounding to odd (hi, or its neighbour towards the rest
// when hi's last bit is even and the rest is not zero); from 53 bits a single rounding to
// float32's 24 (or fewer, subnormal) bits is the correct rounding of R itself (rounding to
// odd with at least two spare bits; Boldo and Melquiond, "When double rounding is odd").
// The scaling by 2^-F is exact in float64, since 1 <= |R| and F <= 128.
__device__ __forceinline__ float crt_to_f32(double a0, double a1, double a2, int F)
{
#pragma clang fp contract(off)
    double p1, e1, q1, e2;
    two_prod(a2, AB_HI, p1, e1);                 // |p1| < 2^88, |e1| <= 2^34
    two_prod(a1, (double)PA, q1, e2);            // |q1| < 2^59, |e2| <= 2^6
    // integers below 2^36 in magnitude: every sum is exact
    const double s = ((e1 + a2 * AB_LO) + e2) + a0;
    double h, l, H, e, lo, e3, hi, lo2;
    two_sum(q1, s, h, l);
    two_sum(p1, h, H, e);
    two_sum(e, l, lo, e3);
    two_sum(H, lo, hi, lo2);                     // R = hi + lo2 + e3, hi = R rounded
    double d = hi;
    if (hi == 0.0) {
        d = e3;                                  // then R = e3 exactly
    } else {
        const double rest = lo2 != 0.0 ? lo2 : e3;
        const long long b = __double_as_longlong(hi);
        if (rest != 0.0 && (b & 1) == 0)
            d = __longlong_as_double(b + (((rest > 0.0) == (hi > 0.0)) ? 1 : -1));
    }
    return (float)ldexp(d, -F);
}

}  // namespace ntt

// r = round_f32(R 2^-F) where R is the integer with the balanced residues sa, sb, sc modulo
// the primes A, B, C and |R| <= (A B C - 1) / 2.
__global__ void crt_decode_kernel(const int32_t* __restrict__ sa, const int32_t* __restrict__ sb,
                                  const int32_t* __restrict__ sc, float* __restrict__ r,
                                  int64_t n, int F)
{
    using namespace ntt;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const double a0 = (double)sa[i];
        const double a1 = balance<PrimeB>(mulc<PrimeB>((double)sb[i] - a0, INV_A_MOD_B));
        const double t2 = (double)sc[i] - a0 - mulc<PrimeC>(a1, A_MOD_C);
        const double a2 = balance<PrimeC>(mulc<PrimeC>(t2, INV_AB_MOD_C));
        // R = a0 + a1 A + a2 A B, every digit balanced, so |R| <= (A B C - 1) / 2
        r[i] = crt_to_f32(a0, a1, a2, F);
    }
}

template <int M, bool REV, class Pr, bool FIX>
static hipError_t launch_ntt_m(const void* v, const void* g, int32_t* r, int64_t nch, int L,
                               const NttTables& tb, double sv, double sg, hipStream_t stream)
{
    constexpr int CPW = (ntt_threads<M>() / (M / 16)) / 2;
    const int64_t blocks = (nch + CPW - 1) / CPW;
    const int lg = __builtin_ctz((unsigned)(2 * M));
    if (!grid_ok(blocks, ntt_threads<M>())) return hipErrorInvalidValue;
    hipLaunchKernelGGL((ntt_conv_kernel<M, REV, Pr, FIX>), dim3((unsigned)blocks), dim3(ntt_threads<M>()), 0,
                       stream, v, g, r, nch, L, tb.bank, tb.ninv[lg], tb.ninv_q[lg], sv, sg);
    return hipGetLastError();
}

template <bool REV, class Pr, bool FIX>
static hipError_t launch_ntt_any(const void* v, const void* g, int32_t* r, int64_t nch, int L,
                                 int M, const NttTables& tb, double sv, double sg, hipStream_t s)
{
    switch (M) {
    case 64: return launch_ntt_m<64, REV, Pr, FIX>(v, g, r, nch, L, tb, sv, sg, s);
    case 128: return launch_ntt_m<128, REV, Pr, FIX>(v, g, r, nch, L, tb, sv, sg, s);
    case 256: return launch_ntt_m<256, REV, Pr, FIX>(v, g, r, nch, L, tb, sv, sg, s);
    case 512: return launch_ntt_m<512, REV, Pr, FIX>(v, g, r, nch, L, tb, sv, sg, s);
    case 1024: return launch_ntt_m<1024, REV, Pr, FIX>(v, g, r, nch, L, tb, sv, sg, s);
    case 2048: return launch_ntt_m<2048, REV, Pr, FIX>(v, g, r, nch, L, tb, sv, sg, s);
    case 4096: return launch_ntt_m<4096, REV, Pr, FIX>(v, g, r, nch, L, tb, sv, sg, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ntt(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch, int L, int M,
                      bool rev, const NttTables& tb, hipStream_t s)
{
    return rev ? launch_ntt_any<true, ntt::PrimeA, false>(v, g, r, nch, L, M, tb, 0.0, 0.0, s)
               : launch_ntt_any<false, ntt::PrimeA, false>(v, g, r, nch, L, M, tb, 0.0, 0.0, s);
}

hipError_t launch_fixed(const float* v, const float* g, float* r, int32_t* scratch, int64_t nch,
                        int L, int M, int fv, int fg, const NttTables* tb, hipStream_t s)
{
    const int64_t n = nch * (int64_t)L;
    const double sv = ldexp(1.0, fv), sg = ldexp(1.0, fg);
    hipError_t e = launch_ntt_any<false, ntt::PrimeA, true>(v, g, scratch, nch, L, M, tb[0], sv,
                                                           sg, s);
    if (e == hipSuccess)
        e = launch_ntt_any<false, ntt::PrimeB, true>(v, g, scratch + n, nch, L, M, tb[1], sv, sg,
                                                     s);
    if (e == hipSuccess)
        e = launch_ntt_any<false, ntt::PrimeC, true>(v, g, scratch + 2 * n, nch, L, M, tb[2], sv,
                                                     sg, s);
    if (e != hipSuccess) return e;
    const int threads = 256;
    int64_t blocks = (n + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(crt_decode_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, scratch,
                       scratch + n, scratch + 2 * n, r, n, fv + fg);
    return hipGetLastError();
}

}  // namespace sc
