// Exact modular arithmetic and the LDS transform passes shared by the number-theoretic
// transform kernels: the fused NTT kernel (sc_ntt.hip), the exact real-valued kernel
// (sc_fixed.hip) and the four-step NTT kernels (sc_ntt4.hip).  The method, the primes and
// the arithmetic are described at the top of sc_ntt.hip.
#pragma once

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
// the odd part of n
constexpr uint64_t odd_part(uint64_t n) { return n % 2 ? n : odd_part(n / 2); }

// a * w mod p, |a| < 2^36, |result| <= 1.5 p.  q = a w / p rounded, within one of the exact
// quotient.  p - 1 = c 2^k with c < 2^15, so q (p - 1) is exact in float64, and
// a w - q (p - 1), an integer below 2^38 in magnitude, comes exactly out of one fused
// multiply-add; less q it is a w - q p.  Five operations.
template <class Pr>
__device__ __forceinline__ double mulc(double a, W w)
{
    static_assert(odd_part(Pr::p - 1) < (1u << 15), "q (p - 1) must be exact");
    constexpr double PM1 = (double)(Pr::p - 1);
    const double q = __builtin_fma(a, w.q, SHIFT) - SHIFT;
    return __builtin_fma(a, w.w, -(q * PM1)) - q;
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
    int salt = 0;   // 0, but opaque to the compiler after reseed()
    __device__ __forceinline__ W at(int voff_elems, int soff_elems) const
    {
        const auto d = __builtin_amdgcn_raw_buffer_load_b128(rs, voff_elems * 16,
                                                             soff_elems * 16 + salt, 0);
        return __builtin_bit_cast(W, d);
    }
    // Loads issued after this are not merged with earlier identical ones, and cannot be
    // issued before `after` is computed: a pass loads its twiddles in groups, each after the
    // previous group's last product, instead of keeping all fifteen live at once
    __device__ __forceinline__ void reseed(double after)
    {
        int z = 0;
        asm volatile("" : "+s"(z) : "v"(after));
        salt = z;
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

// LDS layout of a unit's arrays.  From M = 1024 on (whole waves per unit) the layout is
// chosen by the pass that wrote the array, so that both its stores and the reads that follow
// hit 64 different 4-byte banks in every wave (no linear padding serves all three patterns):
//   S = 1 stores, logical 16 n1 + k2:             a + a/64
//   S = 16 stores, logical s + 16 k2 + 256 n1:    a + a/64 + 12 (a/256)
// reads of 64 consecutive positions are conflict-free in both.  Smaller M keeps one pad word
// per 16 (several units share a wave there).
template <int M, int S>
constexpr int lds_words()
{
    if constexpr (M < 1024) return M + M / 16;
    else return M + M / 64 + (S == 16 ? 12 * (M / 256) : 0);
}
template <int M>
constexpr int lds_region() { return lds_words<M, 16>(); }

// position of logical element tau + TB q (a per-thread base plus a constant per q)
template <int M, int S>
__device__ __forceinline__ int reg_off(int tau, int q)
{
    constexpr int TB = M / 16;
    if constexpr (M < 1024) {
        if constexpr (TB % 16 == 0) return tau + (tau >> 4) + q * (TB + TB / 16);
        else {
            const int a = tau + TB * q;
            return a + (a >> 4);
        }
    } else {
        // TB is a multiple of 64, so (tau + TB q) / 64 = tau / 64 + q TB / 64, and likewise
        // for / 256 (tau < 256 when TB < 256)
        const int b = tau + (tau >> 6) + (S == 16 ? 12 * (tau >> 8) : 0);
        return b + q * TB + (q * TB) / 64 + (S == 16 ? 12 * ((q * TB) / 256) : 0);
    }
}

// One Stockham DIF pass (index scheme as in the float kernel) over NA arrays sharing the
// twiddles.  Arrays are held as int32 (|x| < 2^31) between passes and widened to float64 one
// array at a time inside the butterfly, so the array not being worked on takes half the
// registers.  Passes with twiddles are radix 16 with one item per thread; their outputs are
// reduced below 2^31 (k2 > 0 by the twiddle product, k2 = 0 explicitly) and stored to LDS.
// The last pass (no twiddles, in registers) hands each output, below 2^36, to
// fin(a, q, value) for array a and register q, all of array 0 before array 1.
template <int M, int R, int S, int NA, class Pr, class Fin>
__device__ __forceinline__ void pass(int32_t (&x)[NA][16], int32_t* __restrict__ buf0,
                                     int32_t* __restrict__ buf1, int tau, const Tw& tw, Fin& fin)
{
    constexpr int NB = 16 / R, Q = M / S, QN = Q / R;
    if constexpr (QN > 1) {
        static_assert(R == 16, "passes with twiddles are radix 16");
        static_assert(S == 1 || S == 16, "twiddled passes are the first two");
        const int s = tau & (S - 1), n1 = tau / S;
        // store position of output k2 = base + off(k2) (see lds_words)
        int base;
        if constexpr (M < 1024) base = S == 1 ? 17 * n1 : (s + (s >> 4)) + 17 * S * n1;
        else base = S == 1 ? 16 * n1 + (n1 >> 2) : s + 272 * n1;
        auto off = [](int k2) {
            if constexpr (M < 1024) return S == 1 ? k2 : k2 * (S + S / 16);
            else return S == 1 ? k2 : 16 * k2 + (k2 >> 2);
        };
        // the fifteen twiddles (cached) are loaded per array in two groups, each group after
        // the previous one's last product, so that at most eight are live
        Tw t = tw;
        double last = 0.0;
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            double d[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) d[q] = (double)x[a][q];
            dft<16, Pr>(d);
            int32_t* buf = a == 0 ? buf0 : buf1;
            buf[base] = (int32_t)reduce<Pr>(d[0]);
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                if (a || g) t.reseed(last);
                const int lo = g ? 8 : 1, hi = g ? 16 : 8;
                W w[8];
#pragma unroll
                for (int k2 = lo; k2 < hi; ++k2)
                    w[k2 - lo] = t.at(n1, NTT_PASS_BASE + (Q - 32) + k2 * (Q / 16));
#pragma unroll
                for (int k2 = lo; k2 < hi; ++k2) {
                    last = mulc<Pr>(d[k2], w[k2 - lo]);
                    buf[base + off(k2)] = (int32_t)last;
                }
            }
        }
    } else {
#pragma unroll
        for (int a = 0; a < NA; ++a) {
#pragma unroll
            for (int qb = 0; qb < NB; ++qb) {
                double b[R];
#pragma unroll
                for (int n2 = 0; n2 < R; ++n2) b[n2] = (double)x[a][qb + NB * n2];
                dft<R, Pr>(b);
#pragma unroll
                for (int k2 = 0; k2 < R; ++k2) fin(a, qb + NB * k2, b[k2]);
            }
        }
    }
}

template <int M, int NA, class Pr, int S = 1, class Fin>
__device__ __forceinline__ void passes(int32_t (&x)[NA][16], int32_t* __restrict__ buf0,
                                       int32_t* __restrict__ buf1, int tau, const Tw& tw,
                                       Fin& fin)
{
    constexpr int Q = M / S, R = Q >= 16 ? 16 : Q;
    if constexpr (Q / R > 1) {
        pass<M, R, S, NA, Pr>(x, buf0, buf1, tau, tw, fin);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            x[0][q] = buf0[reg_off<M, S>(tau, q)];
            if constexpr (NA > 1) x[1][q] = buf1[reg_off<M, S>(tau, q)];
        }
        __syncthreads();
        passes<M, NA, Pr, S * R>(x, buf0, buf1, tau, tw, fin);
    } else {
        pass<M, R, S, NA, Pr>(x, buf0, buf1, tau, tw, fin);
    }
}

}  // namespace ntt

// Threads of the workgroup for length-M transforms: one channel from M = 512 on, as many
// as fill one wave below (as the float kernel).
template <int M>
constexpr int ntt_threads() { return M / 8 > 64 ? M / 8 : 64; }

namespace ntt {

// zero, produced after x is computed, and not known to the compiler to be zero
__device__ __forceinline__ int after(int32_t x)
{
    int z = 0;
    asm volatile("" : "+s"(z) : "v"(x));
    return z;
}

}  // namespace ntt

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

// Garner's recombination of balanced residues ra, rb, rc modulo A, B, C into
// R = a0 + a1 A + a2 A B (every digit balanced, so |R| <= (A B C - 1) / 2), rounded once:
// round_f32(R 2^-F)
__device__ __forceinline__ float garner_f32(int32_t ra, int32_t rb, int32_t rc, int F)
{
    const double a0 = (double)ra;
    const double a1 = balance<PrimeB>(mulc<PrimeB>((double)rb - a0, INV_A_MOD_B));
    const double t2 = (double)rc - a0 - mulc<PrimeC>(a1, A_MOD_C);
    const double a2 = balance<PrimeC>(mulc<PrimeC>(t2, INV_AB_MOD_C));
    return crt_to_f32(a0, a1, a2, F);
}

}  // namespace ntt

// REV (the gradient kernels): the first input is read reversed and the output is written
// reversed: rev(causal(rev(dr), b))_j = sum_{t>=j} dr_t b_{t-j}.
// FIX: float32 inputs encoded as integers round(v 2^fv), round(g 2^fg) (nearest, ties to
// even; sv = 2^fv, sg = 2^fg, |v sv|, |g sg| < 2^51) instead of int32 inputs.

namespace ntt {

// The balanced residues mod Pr of one channel's causal convolution at the eight positions
// this thread finishes: out[i] belongs to n = (M - tau - TB q) mod M, q = i + 8 beta (a result
// only where n < L).  bv, bg: the unit's two LDS arrays; xch: the channel's exchange array
// (branch 0's bv).  The call begins with a barrier before its first LDS write, so calls for
// several primes may follow one another in a kernel.  salt is zero, but opaque (see after()):
// added to tau in the global and twiddle offsets, it keeps a later call's loads from being
// merged with an earlier call's or hoisted above its end.
template <int M, bool REV, class Pr, bool FIX>
__device__ __forceinline__ void residues(const Span& vs, const Span& gs, int cbase, int L,
                                         int tau, int beta, int32_t* bv, int32_t* bg,
                                         int32_t* xch, const Tw& tw, double ninv,
                                         double ninv_q, double sv, double sg, int salt,
                                         int32_t (&out)[8])
{
    constexpr int N = 2 * M, TB = M / 16;
    // 1. inputs as residues below 2^31 in magnitude, times omega_N^n on branch 1.
    //    Positions past L are read at byte offset 2^31, beyond the descriptor's range, so they
    //    read 0 (a select instead of a branch keeps all the loads in flight together).  All
    //    32 element loads are issued first and branch 1's twiddle loads right after them:
    //    converting and multiplying element by element under the branch made every element
    //    wait for its own loads, one memory latency per element.
    // taus = tau, but opaque: the global and twiddle offsets of one call are not shared
    // with another's (kept live from the first call to the last, they had been spilled)
    const int taus = tau + salt;
    uint32_t wa[16], wb[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int n = taus + TB * q;
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
    // With ONE_PATH, branch 0 multiplies by omega^0 = 1 (table entry 0) instead of taking
    // another path: in the three-prime kernel, arrays assigned on two paths had become
    // vectors merged in one block of registers, and spilled.  Without it (one prime), the
    // branch saves branch 0 the products.  The twiddles come in two batches of 8, which
    // bounds the registers held at once.
    constexpr bool ONE_PATH = FIX;
    int32_t x[2][16];
    const int twstep = beta ? NTT_TW_N / N : 0;
    if (ONE_PATH || beta) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            W wq[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) wq[i] = tw.at((taus + TB * (8 * h + i)) * twstep, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = 8 * h + i;
                x[0][q] = (int32_t)mulc<Pr>(to_residue(wa[q], sv), wq[i]);
                x[1][q] = (int32_t)mulc<Pr>(to_residue(wb[q], sg), wq[i]);
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            x[0][q] = (int32_t)to_residue(wa[q], sv);
            x[1][q] = (int32_t)to_residue(wb[q], sg);
        }
    }

    // the previous call's exchange reads are done before this call's passes write the LDS
    __syncthreads();

    // 2, 3. V, G = NTT_M(.) in natural order; the last pass hands out V_k, then G_k (below
    //    2^36), and X_k = V_k (G_k N^{-1}) is formed as they arrive
    int32_t y[1][16];
    auto product = [&](int a, int q, double val) {
        if (a == 0)
            x[0][q] = (int32_t)reduce<Pr>(val);
        else
            y[0][q] = (int32_t)mulv<Pr>((double)x[0][q],
                                        reduce<Pr>(mulc<Pr>(val, W{ninv, ninv_q})));
    };
    passes<M, 2, Pr>(x, bv, bg, tau, tw, product);

    // 4. f = NTT_M(X): e^beta_n = f_{(M - n) mod M}, reduced as it leaves the last pass
    int32_t f[16];
    auto keep = [&](int, int q, double val) { f[q] = (int32_t)reduce<Pr>(val); };
    passes<M, 1, Pr>(y, bv, bv, tau, tw, keep);

    // 5. register q of thread tau holds e^beta at n = (M - tau - TB q) mod M.
    //    x_n = e^0_n + omega_N^{-n} e^1_n: branch 0 finishes q < 8, branch 1 q >= 8, each
    //    handing the other half to its partner through LDS.
    if (beta) {
        // omega_N^{-n} = omega_N^{N - n}, loaded in two groups of 8, the second after the
        // first group's products (one path here spills more than it saves)
        Tw t = tw;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (h) t.reseed((double)f[7]);
            W wq[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int n = (M - taus - TB * (8 * h + i)) & (M - 1);
                wq[i] = t.at(((N - n) & (N - 1)) * (NTT_TW_N / N), 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                f[8 * h + i] = (int32_t)mulc<Pr>((double)f[8 * h + i], wq[i]);
        }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q)
        if ((q < 8) == (beta == 1)) xch[reg_off<M, 1>(tau, q)] = f[q];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // a choice between two values (a conditional between the two array elements would
        // pick an address and force f into memory or an indexed register block)
        const int32_t lo = f[i], hi = f[8 + i];
        const int32_t mine = beta ? hi : lo;
        const int32_t other = xch[beta ? reg_off<M, 1>(tau, 8 + i) : reg_off<M, 1>(tau, i)];
        out[i] = (int32_t)balance<Pr>(reduce<Pr>((double)mine + (double)other));
    }
}

}  // namespace ntt

// Workgroup geometry shared by the two kernels: TB = M / 16 threads per branch unit, two units
// (branches 0 and 1) per channel, CPW channels per workgroup, two LDS arrays per unit.
#define SC_NTT_SETUP(VP, GP, RP)                                                              \
    constexpr int TB = M / 16, UNITS = ntt_threads<M>() / TB, CPW = UNITS / 2;                \
    constexpr int REG = lds_region<M>();                                                      \
    __shared__ int32_t lds[UNITS * 2 * REG];                                                  \
    const int tid = threadIdx.x;                                                              \
    const int unit = tid / TB, tau = tid % TB;                                                \
    const int cl = unit >> 1, beta = unit & 1;                                                \
    const int64_t ch0 = (int64_t)blockIdx.x * CPW;                                            \
    const int nvalid = (int)((nch - ch0) < CPW ? (nch - ch0) : CPW);                          \
    const Span vs = make_span((const int32_t*)(VP), ch0 * L, (int64_t)nvalid * L);            \
    const Span gs = make_span((const int32_t*)(GP), ch0 * L, (int64_t)nvalid * L);            \
    const Span rs = make_span((RP), ch0 * L, (int64_t)nvalid * L);                            \
    int32_t* bv = lds + unit * 2 * REG;                                                       \
    int32_t* bg = bv + REG;                                                                   \
    int32_t* xch = lds + (2 * cl) * 2 * REG;                                                  \
    const int cbase = cl * L

}  // namespace sc
