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
// giving |r| <= 1.5 p.  Between passes values are int32 (|x| < 2^31), in LDS and in
// registers; an array is widened to float64 only inside its butterflies.
//
// Layout as in the float kernel: max(64, M/8) threads, a length-M transform held by TB = M/16
// threads with 16 values each, Stockham radix-16 passes through LDS (a v and a g array per
// branch unit), 68 KB of LDS per workgroup at M = 4096.
//
// The exact real-valued kind runs the same per-prime steps three times in one kernel
// (fixed_conv_kernel, sc_fixed.hip): the residues modulo A and B of a thread's eight outputs
// wait in registers while the next prime is computed, and Garner's recombination ends the
// kernel, so no residue goes through memory.  The four-step split beyond L = 4096 is in
// sc_ntt4.hip; the arithmetic and the passes the three files share are in sc_ntt_arith.h.
// This file is compiled with the memory-clause instruction schedule (the build script's
// per-file options; the exact workload's call 1.2% faster, bit-identical).

#include "sc_device.h"
#include "sc_internal.h"
#include "sc_ntt_arith.h"

namespace sc {

template <int M, bool REV>
__global__ __launch_bounds__(ntt_threads<M>(), 4) void ntt_conv_kernel(
    const int32_t* __restrict__ v, const int32_t* __restrict__ g, int32_t* __restrict__ r,
    int64_t nch, int L, const double* __restrict__ bank, double ninv, double ninv_q)
{
    using namespace ntt;
    static_assert(M >= 64 && M <= 4096, "fused NTT handles 64 <= M <= 4096");
    SC_NTT_SETUP(v, g, r);
    const Tw tw{__builtin_amdgcn_make_buffer_rsrc((void*)bank, (short)0, NTT_BANK_ENTRIES * 16,
                                                  0x00020000)};
    int32_t out[8];
    residues<M, REV, PrimeA, false>(vs, gs, cbase, L, tau, beta, bv, bg, xch, tw, ninv, ninv_q,
                                    0.0, 0.0, 0, out);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int n = (M - tau - TB * (i + 8 * beta)) & (M - 1);
        if (n < L)
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)out[i], rs.rs,
                                                  (cbase + (REV ? L - 1 - n : n)) * 4, 0, 0);
    }
}

template <int M, bool REV>
static hipError_t launch_ntt_m(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch,
                               int L, const NttTables& tb, hipStream_t stream)
{
    constexpr int CPW = (ntt_threads<M>() / (M / 16)) / 2;
    const int64_t blocks = (nch + CPW - 1) / CPW;
    const int lg = __builtin_ctz((unsigned)(2 * M));
    if (!grid_ok(blocks, ntt_threads<M>())) return hipErrorInvalidValue;
    hipLaunchKernelGGL((ntt_conv_kernel<M, REV>), dim3((unsigned)blocks), dim3(ntt_threads<M>()),
                       0, stream, v, g, r, nch, L, tb.bank, tb.ninv[lg], tb.ninv_q[lg]);
    return hipGetLastError();
}

// F(M) expands to the call for each supported M
#define SC_NTT_SWITCH(F)                                                                      \
    switch (M) {                                                                              \
    case 64: return F(64);                                                                    \
    case 128: return F(128);                                                                  \
    case 256: return F(256);                                                                  \
    case 512: return F(512);                                                                  \
    case 1024: return F(1024);                                                                \
    case 2048: return F(2048);                                                                \
    case 4096: return F(4096);                                                                \
    default: return hipErrorInvalidValue;                                                     \
    }

hipError_t launch_ntt(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch, int L, int M,
                      bool rev, const NttTables& tb, hipStream_t s)
{
#define SC_CALL(m) rev ? launch_ntt_m<m, true>(v, g, r, nch, L, tb, s) \
                       : launch_ntt_m<m, false>(v, g, r, nch, L, tb, s)
    SC_NTT_SWITCH(SC_CALL)
#undef SC_CALL
}

#undef SC_NTT_SWITCH
#undef SC_NTT_SETUP

}  // namespace sc
