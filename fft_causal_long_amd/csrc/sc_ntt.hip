// Exact causal convolution through a number-theoretic transform (gfx950), L <= 4096.
//
// "Catastrophic Token Leakage in Convolutional Sequence Modeling and How to Mitigate It"
// (abstract): float FFT convolutions leak future tokens through round-off; an FFT done on
// integers only cannot.  Here the pad-to-2L recipe of "Caracal: Causal Architecture via
// Spectral Mixing" (key designs 1 and 2) runs in Z_p, p = 998244353 = 119*2^23 + 1, with
// omega_n = 3^((p-1)/n) in place of exp(-2 pi i / n).  Every operation is an exact
// residue operation, so output t is a function of v_0..v_t and g_0..g_t alone.
//
// Per channel, with N = 2M and the upper half of the padded inputs zero, the first
// decimation-in-frequency stage is a twiddle only:  V_{2j+b} = NTT_M(v_n omega_N^{b n})_j,
// likewise G.  For b = 0, 1 ("branches") the workgroup computes NTT_M of v and g, the
// product X = V G N^{-1}, and e^b = INTT_M(X^b).  Then for n < L
//     x_n = N^{-1} sum_k X_k omega_N^{-nk} = e^0_n + omega_N^{-n} e^1_n     (N^{-1} folded)
// and the residue is lifted to [-(p-1)/2, (p-1)/2].
//
// Layout as in the float kernel: 512 threads, a length-M transform held by TB = M/16
// threads with 16 residues each (element tau + TB*r in register r), Stockham radix-16
// passes through LDS (a v and a g array per branch unit), 68 KB of LDS per workgroup.
//
// Arithmetic: residues are kept fully reduced in [0, p) as uint32.  Multiplication by a
// known constant w uses Shoup's method with w' = floor(w 2^32 / p) from a table;
// the pointwise product of two variables uses Montgomery reduction with R = 2^32.

#include "sc_device.h"
#include "sc_internal.h"

namespace sc {

namespace ntt {

constexpr uint32_t P = 998244353u;

constexpr uint32_t inv_mod_2_32(uint32_t a)
{
    uint32_t x = a;                  // correct to 3 bits for odd a; each step doubles
    for (int i = 0; i < 5; ++i) x *= 2u - a * x;
    return x;
}
constexpr uint32_t PINV = inv_mod_2_32(P);   // p^{-1} mod 2^32
static_assert((uint32_t)(P * PINV) == 1u, "p^{-1} mod 2^32");

__device__ __forceinline__ uint32_t addm(uint32_t a, uint32_t b)
{
    const uint32_t s = a + b;          // < 2p < 2^31
    return min(s, s - P);
}
__device__ __forceinline__ uint32_t subm(uint32_t a, uint32_t b)
{
    const uint32_t d = a - b;          // wraps when a < b
    return min(d, d + P);
}
// a * w mod p for a < 2^32, w < p, wq = floor(w * 2^32 / p)  (Shoup)
__device__ __forceinline__ uint32_t mulc(uint32_t a, uint2 w)
{
    const uint32_t q = __umulhi(a, w.y);
    const uint32_t r = a * w.x - q * P;   // exact value in [0, 2p)
    return min(r, r - P);
}
// a * b * 2^-32 mod p for a, b < p  (Montgomery)
__device__ __forceinline__ uint32_t mont(uint32_t a, uint32_t b)
{
    const uint32_t lo = a * b, hi = __umulhi(a, b);
    const uint32_t m = lo * PINV;
    const uint32_t r = hi - __umulhi(m, P);  // in (-p, p)
    return min(r, r + P);
}

// omega_n^e (or omega_n^-e) with its Shoup companion, from the table of omega_8192^i
template <bool INV>
__device__ __forceinline__ uint2 tw(const uint2* __restrict__ t, int n, int e)
{
    int i = (e & (n - 1)) * (FUSED_TW_N / n);
    if (INV) i = (FUSED_TW_N - i) & (FUSED_TW_N - 1);
    return t[i];
}

// in-register DFT_R over Z_p, natural order in and out (decimation in frequency)
template <int R, bool INV>
__device__ __forceinline__ void dft(uint32_t* a, const uint2* __restrict__ t)
{
    if constexpr (R == 2) {
        const uint32_t x = a[0];
        a[0] = addm(x, a[1]);
        a[1] = subm(x, a[1]);
    } else if constexpr (R == 4) {
        const uint2 w4 = tw<INV>(t, 4, 1);
        const uint32_t t0 = addm(a[0], a[2]), t1 = subm(a[0], a[2]);
        const uint32_t t2 = addm(a[1], a[3]), t3 = mulc(subm(a[1], a[3]), w4);
        a[0] = addm(t0, t2);
        a[2] = subm(t0, t2);
        a[1] = addm(t1, t3);
        a[3] = subm(t1, t3);
    } else {
        constexpr int H = R / 2;
        uint32_t u[H], w[H];
#pragma unroll
        for (int n = 0; n < H; ++n) {
            u[n] = addm(a[n], a[n + H]);
            const uint32_t d = subm(a[n], a[n + H]);
            w[n] = n == 0 ? d : mulc(d, tw<INV>(t, R, n));
        }
        dft<H, INV>(u, t);
        dft<H, INV>(w, t);
#pragma unroll
        for (int k = 0; k < H; ++k) {
            a[2 * k] = u[k];
            a[2 * k + 1] = w[k];
        }
    }
}

__device__ __forceinline__ int lds_pad(int a) { return a + (a >> 4); }

// One Stockham DIF pass (index scheme as in the float kernel) over NA arrays that share
// the twiddles.
template <int M, int R, int S, bool INV, int NA>
__device__ __forceinline__ void pass(uint32_t (&x)[NA][16], uint32_t* __restrict__ buf0,
                                     uint32_t* __restrict__ buf1, int tau,
                                     const uint2* __restrict__ t)
{
    constexpr int TB = M / 16, NB = 16 / R, Q = M / S, QN = Q / R;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const int item = tau + TB * q;
        const int s = item & (S - 1);
        const int n1 = item / S;
        uint2 wt[R];
        if constexpr (QN > 1) {
#pragma unroll
            for (int k2 = 1; k2 < R; ++k2) wt[k2] = tw<INV>(t, Q, n1 * k2);
        }
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            uint32_t b[R];
#pragma unroll
            for (int n2 = 0; n2 < R; ++n2) b[n2] = x[a][q + NB * n2];
            dft<R, INV>(b, t);
            if constexpr (QN > 1) {
                uint32_t* buf = a == 0 ? buf0 : buf1;
#pragma unroll
                for (int k2 = 1; k2 < R; ++k2) b[k2] = mulc(b[k2], wt[k2]);
#pragma unroll
                for (int k2 = 0; k2 < R; ++k2) buf[lds_pad(s + S * (k2 + R * n1))] = b[k2];
            } else {
#pragma unroll
                for (int k2 = 0; k2 < R; ++k2) x[a][q + NB * k2] = b[k2];
            }
        }
    }
}

template <int M, bool INV, int NA, int S = 1>
__device__ __forceinline__ void passes(uint32_t (&x)[NA][16], uint32_t* __restrict__ buf0,
                                       uint32_t* __restrict__ buf1, int tau,
                                       const uint2* __restrict__ t)
{
    constexpr int TB = M / 16, Q = M / S, R = Q >= 16 ? 16 : Q;
    if constexpr (Q / R > 1) {
        pass<M, R, S, INV, NA>(x, buf0, buf1, tau, t);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            x[0][q] = buf0[lds_pad(tau + TB * q)];
            if constexpr (NA > 1) x[1][q] = buf1[lds_pad(tau + TB * q)];
        }
        __syncthreads();
        passes<M, INV, NA, S * R>(x, buf0, buf1, tau, t);
    } else {
        pass<M, R, S, INV, NA>(x, buf0, buf1, tau, t);
    }
}

// int32 -> residue in [0, p)
__device__ __forceinline__ uint32_t to_zp(int32_t x)
{
    int32_t r = x % (int32_t)P;
    return (uint32_t)(r < 0 ? r + (int32_t)P : r);
}

}  // namespace ntt

template <int M>
__global__ __launch_bounds__(512) void ntt_conv_kernel(const int32_t* __restrict__ v,
                                                       const int32_t* __restrict__ g,
                                                       int32_t* __restrict__ r, int64_t nch,
                                                       int L, const uint2* __restrict__ t,
                                                       uint2 ninv_r)
{
    using namespace ntt;
    static_assert(M >= 64 && M <= 4096, "fused NTT handles 64 <= M <= 4096");
    constexpr int N = 2 * M, TB = M / 16, UNITS = 512 / TB, CPW = UNITS / 2;
    constexpr int REG = M + M / 16;
    __shared__ uint32_t lds[UNITS * 2 * REG];

    const int tid = threadIdx.x;
    const int unit = tid / TB, tau = tid % TB;
    const int cl = unit >> 1, beta = unit & 1;
    const int64_t ch = (int64_t)blockIdx.x * CPW + cl;
    const bool valid = ch < nch;
    uint32_t* bv = lds + unit * 2 * REG;
    uint32_t* bg = bv + REG;
    const int64_t base = ch * (int64_t)L;

    // 1. residues of v and g, times omega_N^n on branch 1
    uint32_t x[2][16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int n = tau + TB * q;
        uint32_t a = 0, b = 0;
        if (valid && n < L) {
            a = to_zp(v[base + n]);
            b = to_zp(g[base + n]);
        }
        if (beta) {
            const uint2 w = tw<false>(t, N, n);
            a = mulc(a, w);
            b = mulc(b, w);
        }
        x[0][q] = a;
        x[1][q] = b;
    }

    // 2. V^beta, G^beta = NTT_M(.), natural order in registers
    passes<M, false, 2>(x, bv, bg, tau, t);

    // 3. X = V G N^{-1}:  mont(V, G * (N^{-1} 2^32 mod p)) = V G N^{-1}
    uint32_t y[1][16];
#pragma unroll
    for (int q = 0; q < 16; ++q) y[0][q] = mont(x[0][q], mulc(x[1][q], ninv_r));

    // 4. e^beta = INTT_M(X^beta)
    passes<M, true, 1>(y, bv, bv, tau, t);

    // 5. x_n = e^0_n + omega_N^{-n} e^1_n: branch 0 finishes q < 8, branch 1 q >= 8;
    //    each hands the other half to its partner through LDS (region of branch 0)
    uint32_t* xch = lds + (2 * cl) * 2 * REG;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int n = tau + TB * q;
        if (beta == 0 && q >= 8) xch[lds_pad(n)] = y[0][q];
        if (beta == 1 && q < 8) xch[lds_pad(n)] = mulc(y[0][q], tw<true>(t, N, n));
    }
    __syncthreads();
    if (valid) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int n = tau + TB * q;
            if ((q < 8) != (beta == 0) || n >= L) continue;
            const uint32_t own = beta ? mulc(y[0][q], tw<true>(t, N, n)) : y[0][q];
            const uint32_t s = addm(own, xch[lds_pad(n)]);
            r[base + n] = (int32_t)(s > (P - 1) / 2 ? (int64_t)s - (int64_t)P : (int64_t)s);
        }
    }
}

template <int M>
static hipError_t launch_ntt_m(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch,
                               int L, const NttTables& tb, hipStream_t stream)
{
    constexpr int CPW = (512 / (M / 16)) / 2;
    const int64_t blocks = (nch + CPW - 1) / CPW;
    // N^{-1} * 2^32 mod p and its Shoup companion, for N = 2M
    const uint2 c = tb.ninv_r[__builtin_ctz((unsigned)(2 * M))];
    hipLaunchKernelGGL((ntt_conv_kernel<M>), dim3((unsigned)blocks), dim3(512), 0, stream, v, g,
                       r, nch, L, tb.tw, c);
    return hipGetLastError();
}

hipError_t launch_ntt(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch, int L, int M,
                      const NttTables& tb, hipStream_t s)
{
    switch (M) {
    case 64: return launch_ntt_m<64>(v, g, r, nch, L, tb, s);
    case 128: return launch_ntt_m<128>(v, g, r, nch, L, tb, s);
    case 256: return launch_ntt_m<256>(v, g, r, nch, L, tb, s);
    case 512: return launch_ntt_m<512>(v, g, r, nch, L, tb, s);
    case 1024: return launch_ntt_m<1024>(v, g, r, nch, L, tb, s);
    case 2048: return launch_ntt_m<2048>(v, g, r, nch, L, tb, s);
    case 4096: return launch_ntt_m<4096>(v, g, r, nch, L, tb, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace sc
