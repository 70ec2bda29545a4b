// The exactly causal real-valued convolution for L <= 4096 ("Catastrophic Token Leakage in
// Convolutional Sequence Modeling and How to Mitigate It", abstract: an integer transform
// cannot leak): fixed-point encodings, the residues modulo three NTT primes in one kernel,
// Garner's recombination and one rounding to float32.  The per-prime steps and the
// arithmetic are those of sc_ntt.hip (shared through sc_ntt_arith.h); a file of its own so
// that it keeps the default instruction schedule (the build script's per-file options).

#include "sc_device.h"
#include "sc_internal.h"
#include "sc_ntt_arith.h"

namespace sc {

// The exact real-valued convolution of float32 data, fused: per channel the residues modulo
// A, B and C in turn (each call re-reads v and g, which the first call brought into the
// cache), the first two kept in registers, then Garner's recombination and the one rounding
// to float32 per output, r = round_f32(R 2^-F) with R the integer with those residues and
// |R| <= (A B C - 1) / 2.
struct FixedArgs {
    const double* bank[3];
    double ninv[3], ninv_q[3];
    double sv, sg;
    int F;
};

template <int M>
__global__ __launch_bounds__(ntt_threads<M>(), 4) void fixed_conv_kernel(
    const float* __restrict__ v, const float* __restrict__ g, float* __restrict__ r, int64_t nch,
    int L, FixedArgs fa)
{
    using namespace ntt;
    static_assert(M >= 64 && M <= 4096, "fused NTT handles 64 <= M <= 4096");
    SC_NTT_SETUP(v, g, r);
    auto bank = [&](int i) {
        return Tw{__builtin_amdgcn_make_buffer_rsrc((void*)fa.bank[i], (short)0,
                                                    NTT_BANK_ENTRIES * 16, 0x00020000)};
    };
    int32_t ra[8], rb[8], rc[8];
    residues<M, false, PrimeA, true>(vs, gs, cbase, L, tau, beta, bv, bg, xch, bank(0),
                                     fa.ninv[0], fa.ninv_q[0], fa.sv, fa.sg, 0, ra);
    residues<M, false, PrimeB, true>(vs, gs, cbase, L, tau, beta, bv, bg, xch, bank(1),
                                     fa.ninv[1], fa.ninv_q[1], fa.sv, fa.sg, after(ra[7]), rb);
    residues<M, false, PrimeC, true>(vs, gs, cbase, L, tau, beta, bv, bg, xch, bank(2),
                                     fa.ninv[2], fa.ninv_q[2], fa.sv, fa.sg, after(rb[7]), rc);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int n = (M - tau - TB * (i + 8 * beta)) & (M - 1);
        const float res = garner_f32(ra[i], rb[i], rc[i], fa.F);
        if (n < L)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res), rs.rs, (cbase + n) * 4,
                                                  0, 0);
    }
}
template <int M>
static hipError_t launch_fixed_m(const float* v, const float* g, float* r, int64_t nch, int L,
                                 const NttTables* tb, double sv, double sg, int F,
                                 hipStream_t stream)
{
    constexpr int CPW = (ntt_threads<M>() / (M / 16)) / 2;
    const int64_t blocks = (nch + CPW - 1) / CPW;
    const int lg = __builtin_ctz((unsigned)(2 * M));
    if (!grid_ok(blocks, ntt_threads<M>())) return hipErrorInvalidValue;
    FixedArgs fa;
    for (int i = 0; i < 3; ++i) {
        fa.bank[i] = tb[i].bank;
        fa.ninv[i] = tb[i].ninv[lg];
        fa.ninv_q[i] = tb[i].ninv_q[lg];
    }
    fa.sv = sv;
    fa.sg = sg;
    fa.F = F;
    hipLaunchKernelGGL((fixed_conv_kernel<M>), dim3((unsigned)blocks), dim3(ntt_threads<M>()), 0,
                       stream, v, g, r, nch, L, fa);
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

hipError_t launch_fixed(const float* v, const float* g, float* r, int64_t nch, int L, int M,
                        int fv, int fg, const NttTables* tb, hipStream_t s)
{
    const double sv = ldexp(1.0, fv), sg = ldexp(1.0, fg);
#define SC_CALL(m) launch_fixed_m<m>(v, g, r, nch, L, tb, sv, sg, fv + fg, s)
    SC_NTT_SWITCH(SC_CALL)
#undef SC_CALL
}
#undef SC_NTT_SWITCH
#undef SC_NTT_SETUP

}  // namespace sc
