// Exact causal convolution beyond L = 4096: the four-step split of the number-theoretic
// transform (method and arithmetic as in sc_ntt.hip, shared through sc_ntt_arith.h), in a
// file of its own so that it keeps the default instruction schedule when the fused
// kernels' file takes another (the build script's per-file options).

#include "sc_device.h"
#include "sc_internal.h"
#include "sc_ntt_arith.h"

namespace sc {

// ---------------------------------------------------------------- four-step NTT (L > 4096)
//
// For 4096 < L <= NTT4_MAX_L each length-M branch transform (M = M1 * M2, M2 = 4096,
// M1 = M / 4096 <= 16) is split as
//   U_{M1 k1 + k2} = sum_{n1 < M2} w_M2^{n1 k1} [ w_M^{n1 k2} sum_{n2 < M1} u_{n1 + M2 n2} w_M1^{n2 k2} ]
// and its inverse, for m = m1 + M2 m2, as
//   e_m = sum_{k2 < M1} w_M1^{-m2 k2} [ w_M^{-m1 k2} sum_{k1 < M2} X_{M1 k1 + k2} w_M2^{-m1 k1} ].
//  kernel A (columns): per (channel, column n1), for b = 0, 1 and v, g: u^b_n = a_n w_N^{b n},
//     the length-M1 transform over n2 in registers, times w_M^{n1 k2} -> T[b][array][k2][n1];
//  kernel B (rows): per (channel, branch, row k2), the length-M2 transforms of the v and g
//     rows in LDS (the passes of the fused kernel), X = V G N^{-1}, the inverse over k1 (the
//     forward transform read at (M2 - m1) mod M2), times w_M^{-m1 k2} -> S[b][k2][m1];
//  kernel C (columns): per (channel, column m1), both branches' length-M1 inverses over k2
//     give e^b at n = m1 + M2 m2; x_n = e^0_n + w_N^{-n} e^1_n, lifted and stored for n < L.
// Values between kernels are int32 residues (|x| <= 1.5 p).  The per-M table holds, as
// doubles, wtab[j] = w_N^j (j < N = 2M), then ta[b][k2][n1] = w_N^{n1 (2 k2 + b)}, then
// tr[k2][m1] = w_M^{-m1 k2}, each laid out so that consecutive lanes read consecutive words.
// HBM traffic per channel: read v, g; write and read T (16 M bytes) and S (8 M bytes); write r.
// The exact real-valued kind runs kernels A (encoding its float32 inputs) and B once per
// prime, T reused and S kept per prime (40 M bytes of scratch per channel), and one kernel C
// that forms the three residues of each output in turn and recombines them.

namespace ntt4 {
constexpr int M2 = 4096;
constexpr int CT = 256;   // threads of the column kernels (one column each)
}  // namespace ntt4

// w_N^j modulo Pr from a table of doubles, as the W pair that mulc takes (w / p computed: its
// rounding error keeps the quotient within one of the exact one, as for a stored w / p)
template <class Pr>
__device__ __forceinline__ ntt::W ntt4_w(__amdgpu_buffer_rsrc_t rs, int j)
{
    const double w = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(rs, j * 8, 0, 0));
    return ntt::W{w, w * (1.0 / (double)Pr::p)};
}

// Kernel A: thread (channel, column n1) transforms the v and the g column for both branches
// (the inputs read once; per branch, the two arrays share the twiddles).  Branch 1's input
// rotation w_N^n, n = n1 + M2 n2, is w_N^{n1} w_2M1^{n2}: the second factor is a constant
// per n2, and the first is merged into the output twiddle, which becomes
// w_N^{n1 (2 k2 + b)} (w_M^{n1 k2} for b = 0): one read per output from the table
// ta[b][k2][n1], consecutive across the lanes.  FIX: float32 inputs, encoded as
// round(v sv), round(g sg) (as in the fused kernel) and reduced modulo Pr.
template <int M1, bool REV, class Pr, bool FIX>
__global__ __launch_bounds__(256) void ntt4_columns_fwd(const void* __restrict__ v,
                                                        const void* __restrict__ g,
                                                        int32_t* __restrict__ T, int64_t c0,
                                                        int L, const double* __restrict__ ta,
                                                        double sv, double sg)
{
    using namespace ntt;
    constexpr int M2 = ntt4::M2, M = M1 * M2, BPC = M2 / ntt4::CT;
    static_assert(M1 == 2 || M1 == 4 || M1 == 8 || M1 == 16, "M1 is a power of two <= 16");
    const int blk = blockIdx.x % BPC, cl = blockIdx.x / BPC;
    const int n1 = blk * ntt4::CT + threadIdx.x;
    const auto wrs = __builtin_amdgcn_make_buffer_rsrc((void*)ta, (short)0, 2 * M * 8, 0x00020000);
    uint32_t raw[2][M1];
#pragma unroll
    for (int arr = 0; arr < 2; ++arr) {
        // the first input is read reversed for the gradient form (as in the fused kernel)
        const bool rev = REV && arr == 0;
        const Span as = make_span((const uint32_t*)(arr ? g : v), (c0 + cl) * L, (int64_t)L);
#pragma unroll
        for (int n2 = 0; n2 < M1; ++n2) {
            const int n = n1 + M2 * n2;
            const uint32_t off = n < L ? (uint32_t)(rev ? L - 1 - n : n) * 4u : 0x80000000u;
            raw[arr][n2] = __builtin_amdgcn_raw_buffer_load_b32(as.rs, (int)off, 0, 0);
        }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int arr = 0; arr < 2; ++arr) {
        const int job = 2 * cl + b;
        double x[M1];
#pragma unroll
        for (int n2 = 0; n2 < M1; ++n2) {
            if constexpr (FIX)   // exact: a float times a power of two, rounded, reduced
                x[n2] = reduce<Pr>(round_int((double)__uint_as_float(raw[arr][n2]) *
                                             (arr ? sg : sv)));
            else
                x[n2] = (double)(int32_t)raw[arr][n2];
            if (b && n2) x[n2] = mulc<Pr>(x[n2], root_c<Pr>(2 * M1, n2));
        }
        dft<M1, Pr>(x);
        const Span ts = make_span(T, (int64_t)(2 * job + arr) * M, (int64_t)M);
#pragma unroll
        for (int k2 = 0; k2 < M1; ++k2) {
            const double y = (b || k2) ? mulc<Pr>(x[k2], ntt4_w<Pr>(wrs, (b * M1 + k2) * M2 + n1))
                                       : reduce<Pr>(x[0]);
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(int32_t)y, ts.rs, (k2 * M2 + n1) * 4,
                                                  0, 0);
        }
    }
}

template <class Pr>
__global__ __launch_bounds__(256, 4) void ntt4_rows(const int32_t* __restrict__ T,
                                                    int32_t* __restrict__ S, int M1,
                                                    const double* __restrict__ bank,
                                                    const double* __restrict__ tr, double ninv,
                                                    double ninv_q)
{
    using namespace ntt;
    constexpr int M2 = ntt4::M2, TB = M2 / 16, REG = lds_region<M2>();
    __shared__ int32_t lds[2 * REG];
    const int M = M1 * M2;
    const int k2 = blockIdx.x % M1, job = blockIdx.x / M1;   // job = cl * 2 + b
    const int tau = threadIdx.x;
    const Tw tw{__builtin_amdgcn_make_buffer_rsrc((void*)bank, (short)0, NTT_BANK_ENTRIES * 16,
                                                  0x00020000)};
    const auto wrs = __builtin_amdgcn_make_buffer_rsrc((void*)tr, (short)0, M * 8, 0x00020000);
    // rows k2 of this job's v and g column outputs
    const Span vs = make_span(T, (int64_t)(2 * job) * M + (int64_t)k2 * M2, (int64_t)M2);
    const Span gs = make_span(T, (int64_t)(2 * job + 1) * M + (int64_t)k2 * M2, (int64_t)M2);
    int32_t x[2][16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        x[0][q] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(vs.rs, (tau + TB * q) * 4, 0, 0);
        x[1][q] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(gs.rs, (tau + TB * q) * 4, 0, 0);
    }
    int32_t* bv = lds;
    int32_t* bg = lds + REG;
    int32_t y[1][16];
    auto product = [&](int a, int q, double val) {
        if (a == 0)
            x[0][q] = (int32_t)reduce<Pr>(val);
        else
            y[0][q] = (int32_t)mulv<Pr>((double)x[0][q],
                                        reduce<Pr>(mulc<Pr>(val, W{ninv, ninv_q})));
    };
    passes<M2, 2, Pr>(x, bv, bg, tau, tw, product);
    int32_t f[16];
    auto keep = [&](int, int q, double val) { f[q] = (int32_t)reduce<Pr>(val); };
    passes<M2, 1, Pr>(y, bv, bv, tau, tw, keep);
    // f[q] = NTT(X)_j, j = tau + TB q: the inverse over k1 at m1 = (M2 - j) mod M2, times
    // w_M^{-m1 k2} = tr[k2][m1]
    const Span ss = make_span(S, (int64_t)job * M + (int64_t)k2 * M2, (int64_t)M2);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int m1 = (M2 - (tau + TB * q)) & (M2 - 1);
        const double s = mulc<Pr>((double)f[q], ntt4_w<Pr>(wrs, k2 * M2 + m1));
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(int32_t)s, ss.rs, m1 * 4, 0, 0);
    }
}

// Kernel C's work for one prime: the balanced residues x_n of channel cl's convolution at
// n = m1 + M2 m2 (m2 < M1), from both branches' S rows.
template <int M1, class Pr>
__device__ __forceinline__ void ntt4_inverse_column(const int32_t* __restrict__ S, int cl,
                                                    int m1, const double* __restrict__ wtab,
                                                    int32_t (&out)[M1])
{
    using namespace ntt;
    constexpr int M2 = ntt4::M2, M = M1 * M2, N = 2 * M;
    const auto wrs = __builtin_amdgcn_make_buffer_rsrc((void*)wtab, (short)0, N * 8, 0x00020000);
    // e^b reduced to int32 as the transforms end (half the registers of doubles)
    int32_t e[2][M1];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const Span ss = make_span(S, (int64_t)(2 * cl + b) * M, (int64_t)M);
        double s[M1];
#pragma unroll
        for (int k2 = 0; k2 < M1; ++k2)
            s[k2] = (double)(int32_t)__builtin_amdgcn_raw_buffer_load_b32(ss.rs, (k2 * M2 + m1) * 4,
                                                                          0, 0);
        dft<M1, Pr>(s);
        // the inverse over k2 at m2 is the forward transform at (M1 - m2) mod M1
#pragma unroll
        for (int m2 = 0; m2 < M1; ++m2) e[b][m2] = (int32_t)reduce<Pr>(s[(M1 - m2) & (M1 - 1)]);
    }
#pragma unroll
    for (int m2 = 0; m2 < M1; ++m2) {
        const int n = m1 + M2 * m2;
        const double xn =
            (double)e[0][m2] + mulc<Pr>((double)e[1][m2], ntt4_w<Pr>(wrs, (N - n) & (N - 1)));
        out[m2] = (int32_t)balance<Pr>(reduce<Pr>(xn));
    }
}

template <int M1, bool REV>
__global__ __launch_bounds__(256) void ntt4_columns_inv(const int32_t* __restrict__ S,
                                                        int32_t* __restrict__ r, int64_t c0,
                                                        int L, const double* __restrict__ wtab)
{
    using namespace ntt;
    constexpr int M2 = ntt4::M2, BPC = M2 / ntt4::CT;
    const int blk = blockIdx.x % BPC, cl = blockIdx.x / BPC;
    const int m1 = blk * ntt4::CT + threadIdx.x;
    int32_t x[M1];
    ntt4_inverse_column<M1, PrimeA>(S, cl, m1, wtab, x);
    const Span rs = make_span(r, (c0 + cl) * L, (int64_t)L);
#pragma unroll
    for (int m2 = 0; m2 < M1; ++m2) {
        const int n = m1 + M2 * m2;
        if (n < L)
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)x[m2], rs.rs,
                                                  (REV ? L - 1 - n : n) * 4, 0, 0);
    }
}

// The exact real-valued kind's kernel C: the residues modulo A, B and C (S arrays sp apart)
// in turn, then Garner's recombination and one rounding to float32 per output.
template <int M1>
__global__ __launch_bounds__(256) void ntt4_columns_inv_fixed(const int32_t* __restrict__ S,
                                                              float* __restrict__ r, int64_t c0,
                                                              int L, int64_t sp,
                                                              const double* __restrict__ wa,
                                                              const double* __restrict__ wb,
                                                              const double* __restrict__ wc,
                                                              int F)
{
    using namespace ntt;
    constexpr int M2 = ntt4::M2, BPC = M2 / ntt4::CT;
    const int blk = blockIdx.x % BPC, cl = blockIdx.x / BPC;
    const int m1 = blk * ntt4::CT + threadIdx.x;
    int32_t xa[M1], xb[M1], xc[M1];
    // the column index salted with an opaque zero made after all of the previous prime's
    // residues: each prime's loads then wait for the previous prime's work (issued early,
    // they had needed more registers than a wave has)
    ntt4_inverse_column<M1, PrimeA>(S, cl, m1, wa, xa);
    int za = 0, zb = 0;
#pragma unroll
    for (int i = 0; i < M1; ++i) za += after(xa[i]);
    ntt4_inverse_column<M1, PrimeB>(S + sp, cl, m1 + za, wb, xb);
#pragma unroll
    for (int i = 0; i < M1; ++i) zb += after(xb[i]);
    ntt4_inverse_column<M1, PrimeC>(S + 2 * sp, cl, m1 + zb, wc, xc);
    const Span rs = make_span(r, (c0 + cl) * L, (int64_t)L);
#pragma unroll
    for (int m2 = 0; m2 < M1; ++m2) {
        const int n = m1 + M2 * m2;
        const float res = garner_f32(xa[m2], xb[m2], xc[m2], F);
        if (n < L) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res), rs.rs, n * 4, 0, 0);
    }
}

size_t ntt4_bytes_per_channel(int M) { return (size_t)M * 24; }
size_t fixed4_bytes_per_channel(int M) { return (size_t)M * 40; }

// The channels of a four-step call in parts: part(c0, nc, scratch, s) enqueues the kernels of
// channels c0 .. c0 + nc - 1 on stream s with its scratch.  Without a second stream (side
// null) the parts are `chunk` channels, one after the other on `stream`, each reusing the
// start of ws.  With one, the parts are chunk/2 channels and alternate between `stream` (even
// parts) and `side` (odd parts), each stream with its own half of ws, so that one part's
// column kernels overlap the other's row kernel; `side` waits for `stream` at the start
// (fork) and `stream` for `side` at the end (join), so the call is ordered on `stream` as a
// whole.  A part whose scratch would end past ws_bytes is refused before its launch.
template <class Part>
static hipError_t run_parts(int64_t nch, int64_t chunk, size_t per_channel, void* ws,
                            size_t ws_bytes, hipStream_t stream, hipStream_t side,
                            hipEvent_t fork, hipEvent_t join, Part&& part)
{
    if (chunk <= 0 || (size_t)chunk * per_channel > ws_bytes) return hipErrorInvalidValue;
    const int64_t pc = side ? (chunk / 2 > 0 ? chunk / 2 : 1) : chunk;
    hipError_t e = hipSuccess;
    if (side) {
        e = hipEventRecord(fork, stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(side, fork, 0);
        if (e != hipSuccess) return e;
    }
    int64_t i = 0;
    for (int64_t c0 = 0; c0 < nch && e == hipSuccess; c0 += pc, ++i) {
        const int64_t nc = nch - c0 < pc ? nch - c0 : pc;
        const int half = side ? (int)(i & 1) : 0;
        const size_t off = (size_t)half * (size_t)pc * per_channel;
        if (off + (size_t)nc * per_channel > ws_bytes) {
            e = hipErrorInvalidValue;
            break;
        }
        e = part(c0, nc, (int32_t*)((char*)ws + off), half ? side : stream);
    }
    if (side) {
        // join even after a failed launch, so that nothing of this call is left unordered
        hipError_t ej = hipEventRecord(join, side);
        if (ej == hipSuccess) ej = hipStreamWaitEvent(stream, join, 0);
        if (e == hipSuccess) e = ej;
    }
    return e;
}

template <int M1, bool REV>
static hipError_t launch_ntt4_m(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch,
                                int L, const NttTables& tb, const double* wtab, void* ws,
                                size_t ws_bytes, int64_t chunk, hipStream_t stream,
                                hipStream_t side, hipEvent_t fork, hipEvent_t join)
{
    constexpr int M = M1 * ntt4::M2, BPC = ntt4::M2 / ntt4::CT;
    const int lg = __builtin_ctz((unsigned)(2 * M));
    auto part = [&](int64_t c0, int64_t nc, int32_t* T, hipStream_t s) -> hipError_t {
        int32_t* S = T + nc * 4 * (int64_t)M;
        if (!grid_ok(nc * BPC, ntt4::CT) || !grid_ok(nc * 2 * M1, 256))
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((ntt4_columns_fwd<M1, REV, ntt::PrimeA, false>),
                           dim3((unsigned)(nc * BPC)), dim3(ntt4::CT), 0, s, v, g, T, c0, L,
                           wtab + 2 * M, 1.0, 1.0);
        hipLaunchKernelGGL(ntt4_rows<ntt::PrimeA>, dim3((unsigned)(nc * 2 * M1)), dim3(256), 0, s,
                           T, S, M1, tb.bank, wtab + 4 * M, tb.ninv[lg], tb.ninv_q[lg]);
        hipLaunchKernelGGL((ntt4_columns_inv<M1, REV>), dim3((unsigned)(nc * BPC)), dim3(ntt4::CT),
                           0, s, S, r, c0, L, wtab);
        return hipGetLastError();
    };
    return run_parts(nch, chunk, ntt4_bytes_per_channel(M), ws, ws_bytes, stream, side, fork,
                     join, part);
}

// per part: for each prime, kernels A and B (T reused, S per prime), then the fixed kernel C
template <int M1>
static hipError_t launch_fixed4_m(const float* v, const float* g, float* r, int64_t nch, int L,
                                  const NttTables* tb, const double* const* wtab, double sv,
                                  double sg, int F, void* ws, size_t ws_bytes, int64_t chunk,
                                  hipStream_t stream, hipStream_t side, hipEvent_t fork,
                                  hipEvent_t join)
{
    constexpr int M = M1 * ntt4::M2, BPC = ntt4::M2 / ntt4::CT;
    const int lg = __builtin_ctz((unsigned)(2 * M));
    auto part = [&](int64_t c0, int64_t nc, int32_t* T, hipStream_t s) -> hipError_t {
        const int64_t sp = nc * 2 * (int64_t)M;   // one prime's S
        int32_t* S = T + nc * 4 * (int64_t)M;
        if (!grid_ok(nc * BPC, ntt4::CT) || !grid_ok(nc * 2 * M1, 256))
            return hipErrorInvalidValue;
#define SC_PRIME(i, Pr)                                                                        \
        hipLaunchKernelGGL((ntt4_columns_fwd<M1, false, ntt::Pr, true>),                       \
                           dim3((unsigned)(nc * BPC)), dim3(ntt4::CT), 0, s, v, g, T, c0, L,  \
                           wtab[i] + 2 * M, sv, sg);                                           \
        hipLaunchKernelGGL(ntt4_rows<ntt::Pr>, dim3((unsigned)(nc * 2 * M1)), dim3(256), 0, s, \
                           T, S + i * sp, M1, tb[i].bank, wtab[i] + 4 * M, tb[i].ninv[lg],     \
                           tb[i].ninv_q[lg]);
        SC_PRIME(0, PrimeA)
        SC_PRIME(1, PrimeB)
        SC_PRIME(2, PrimeC)
#undef SC_PRIME
        hipLaunchKernelGGL((ntt4_columns_inv_fixed<M1>), dim3((unsigned)(nc * BPC)),
                           dim3(ntt4::CT), 0, s, S, r, c0, L, sp, wtab[0], wtab[1], wtab[2], F);
        return hipGetLastError();
    };
    return run_parts(nch, chunk, fixed4_bytes_per_channel(M), ws, ws_bytes, stream, side, fork,
                     join, part);
}

#define SC_NTT4_SWITCH(F)                                                                     \
    switch (M / ntt4::M2) {                                                                   \
    case 2: return F(2);                                                                      \
    case 4: return F(4);                                                                      \
    case 8: return F(8);                                                                      \
    case 16: return F(16);                                                                    \
    default: return hipErrorInvalidValue;                                                     \
    }

hipError_t launch_ntt4(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch, int L, int M,
                       bool rev, const NttTables& tb, const double* wtab, void* ws,
                       size_t ws_bytes, int64_t chunk, hipStream_t s, hipStream_t side,
                       hipEvent_t fork, hipEvent_t join)
{
#define SC_CALL(m1)                                                                            \
    rev ? launch_ntt4_m<m1, true>(v, g, r, nch, L, tb, wtab, ws, ws_bytes, chunk, s, side, fork, \
                                  join)                                                        \
        : launch_ntt4_m<m1, false>(v, g, r, nch, L, tb, wtab, ws, ws_bytes, chunk, s, side,     \
                                   fork, join)
    SC_NTT4_SWITCH(SC_CALL)
#undef SC_CALL
}

hipError_t launch_fixed4(const float* v, const float* g, float* r, int64_t nch, int L, int M,
                         int fv, int fg, const NttTables* tb, const double* const* wtab,
                         void* ws, size_t ws_bytes, int64_t chunk, hipStream_t s,
                         hipStream_t side, hipEvent_t fork, hipEvent_t join)
{
    const double sv = ldexp(1.0, fv), sg = ldexp(1.0, fg);
#define SC_CALL(m1) launch_fixed4_m<m1>(v, g, r, nch, L, tb, wtab, sv, sg, fv + fg, ws, ws_bytes, \
                                        chunk, s, side, fork, join)
    SC_NTT4_SWITCH(SC_CALL)
#undef SC_CALL
}
#undef SC_NTT4_SWITCH

}  // namespace sc
