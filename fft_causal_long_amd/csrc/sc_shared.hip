// Causal convolution with a filter shared by the whole batch (gfx950), L <= 4096.
//
//     r[b][c][t] = sum_{j<=t} v[b][c][j] * k[c][t-j]
//
// The Caracal notes contrast their data-dependent gate with filters that do not depend on
// the input ("Caracal: Causal Architecture via Spectral Mixing", related work: Hyena's
// position-based filter, FlashButterfly's static global kernel).  With such a filter the
// pad-to-2L recipe (key designs 1 and 2) needs the filter's spectrum only once per channel,
// and two batch rows share one complex transform: k is real, so for z = v_b + i v_{b+1}
//     IDFT_N(K Z) = (v_b * k) + i (v_{b+1} * k)      (* = circular convolution of length N)
// and the first L values of the real and imaginary parts are r_b and r_{b+1}.
//
// Spectrum kernel (once per filter): for channel pairs (c, c+1), Z = DFT_N(k_c + i k_{c+1}),
// K_c = (Z_k + conj Z_{N-k}) / 2, K_{c+1} = (Z_k - conj Z_{N-k}) / (2i), stored divided by N.
// Apply kernel: per job (channel c, rows 2p and 2p+1) the branch-b unit (b = 0, 1) computes
// U = DFT_M(z_n W_N^{b n}) = Z_{2j+b} (the zero half prunes the first stage), multiplies by
// K_{2j+b} and inverts in place: e^b = IDFT_M(K Z)_n restricted to parity b; then
//     y_n = e^0_n + W_N^{-n} e^1_n = IDFT_N(K Z)_n   (n < M).
// Every thread works in every phase (two length-M transforms per output row instead of the
// three of the per-row-gate kernel).  Outputs t < head use direct fp32 summation, as there.
//
// Spectrum layout per channel c (SPEC_STRIDE float2): [b][j] = K_{2j+b} / N for b < 2,
// j < M, then the filter's first HEAD_MAX values (float32, two per float2).

#include "sc_device.h"
#include "sc_fft_lds.h"
#include "sc_internal.h"

namespace sc {

namespace {

constexpr int SH_THREADS = 512;
// threads of the spectrum and apply workgroups for length-M transforms: one unit pair (a
// filter pair, or a job) per workgroup from M = 512 on, as many as fill one wave below
// (as the per-row-gate kernel: small workgroups share a CU at different phases)
template <int M>
constexpr int sh_threads() { return M / 8 > 64 ? M / 8 : 64; }
// threads of the gradient workgroups: one channel per workgroup from M = 1024 on (their
// head work goes to the threads past the transforms, which must be whole waves), 512 below
template <int M>
constexpr int sh_grad_threads() { return M >= 1024 ? M / 8 : SH_THREADS; }
constexpr int SH_HEAD_MAX = 64;
constexpr int SH_LDS_EXTRA = 24;

template <int M>
__host__ __device__ constexpr int spec_stride()
{
    return 2 * M + SH_HEAD_MAX / 2;
}

}  // namespace

int64_t shared_spec_stride(int M)
{
    return 2 * (int64_t)M + SH_HEAD_MAX / 2;
}

// ---------------------------------------------------------------- filter spectrum

template <int M, class IO>
__global__ __launch_bounds__(sh_threads<M>()) void shared_spectrum_kernel(
    const typename IO::T* __restrict__ k, float2* __restrict__ spec, int C, int L,
    const float2* __restrict__ tw)
{
    constexpr int N = 2 * M, TB = M / 16, UNITS = sh_threads<M>() / TB, PPW = UNITS / 2;
    constexpr int REG = M + M / 16 + (M >= 256 ? SH_LDS_EXTRA : 0);
    constexpr int SS = spec_stride<M>();
    __shared__ float2 lds[UNITS * REG];

    const Bank bank = make_bank(tw);
    const int tid = threadIdx.x;
    const int unit = tid / TB, tau = tid % TB;
    const int pl = unit >> 1, beta = unit & 1;
    const int c0 = 2 * (blockIdx.x * PPW + pl), c1 = c0 + 1;
    const bool v0 = c0 < C, v1 = c1 < C;
    const Span ks = make_span(k, 0, (int64_t)C * L);
    float2* ubuf = lds + unit * REG;

    float2 x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int n = tau + TB * q;
        const int e0 = (v0 && n < L) ? c0 * L + n : IO::OOB;
        const int e1 = (v1 && n < L) ? c1 * L + n : IO::OOB;
        x[q] = make_float2(IO::load(ks, e0), IO::load(ks, e1));
    }
    if (!beta) {
        // the filters' first values for the direct head: k_c[n] in float, n < SH_HEAD_MAX
#pragma unroll
        for (int q = 0; q < (TB >= SH_HEAD_MAX ? 1 : SH_HEAD_MAX / TB); ++q) {
            const int n = tau + TB * q;
            if (n < SH_HEAD_MAX) {
                float* h0 = (float*)(spec + (int64_t)c0 * SS + 2 * M);
                float* h1 = (float*)(spec + (int64_t)c1 * SS + 2 * M);
                if (v0) h0[n] = x[q].x;
                if (v1) h1[n] = x[q].y;
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) x[q] = cmul(x[q], tw_get<false>(bank, N, tau + TB * q));
    }
    fft_passes<M, false>(x, ubuf, tau, bank, true);
#pragma unroll
    for (int q = 0; q < 16; ++q) ubuf[reg_off<TB>(tau, q)] = x[q];
    __syncthreads();
    // x[q] = Z_k with k = 2 j + beta, j = tau + TB q; its mirror Z_{N-k} is Z_{2 (M - j - beta) + beta}
    const float inv = 1.0f / (float)N;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int j = tau + TB * q;
        const float2 z = x[q];
        const float2 w = conjf2(ubuf[lds_pad((M - j - beta) & (M - 1))]);
        const float2 s = cadd(z, w), d = csub(z, w);
        // K_c = s / 2, K_{c+1} = d / (2i) = (d.y - i d.x) / 2
        if (v0) spec[(int64_t)c0 * SS + beta * M + j] = make_float2(0.5f * inv * s.x, 0.5f * inv * s.y);
        if (v1) spec[(int64_t)c1 * SS + beta * M + j] = make_float2(0.5f * inv * d.y, -0.5f * inv * d.x);
    }
}

// ---------------------------------------------------------------- apply

// REV (the gradient dv): v is read reversed and r written reversed, so with v = dr the
// kernel gives dv[b][c][j] = sum_{t>=j} dr[b][c][t] k[c][t-j].
template <int M, class IO, bool REV>
__global__ __launch_bounds__(sh_threads<M>(), (M >= 512 ? 4 : 1)) void shared_apply_kernel(
    const typename IO::T* __restrict__ v, const float2* __restrict__ spec,
    typename IO::T* __restrict__ r, int B, int C, int L, int head,
    const float2* __restrict__ tw)
{
    constexpr int N = 2 * M, TB = M / 16, UNITS = sh_threads<M>() / TB, JPW = UNITS / 2;
    constexpr int REG = M + M / 16 + (M >= 256 ? SH_LDS_EXTRA : 0);
    constexpr int SS = spec_stride<M>();
    __shared__ float2 lds[UNITS * REG];
    // per job: v of row 2p, v of row 2p+1, k (first SH_HEAD_MAX values each)
    __shared__ float hbuf[JPW * 3 * SH_HEAD_MAX];

    const Bank bank = make_bank(tw);
    const int tid = threadIdx.x;
    const int unit = tid / TB, tau = tid % TB;
    const int jl = unit >> 1, beta = unit & 1;
    const int P = (B + 1) / 2;
    // Workgroups are dealt to the 8 XCDs round-robin; renumber them so that the workgroups
    // of one XCD take consecutive jobs, i.e. the pairs of one channel share that XCD's L2
    // and its filter spectrum is fetched from memory about once.
    const int g8 = gridDim.x >> 3;                       // the grid is a multiple of 8
    const int w = (blockIdx.x & 7) * g8 + (blockIdx.x >> 3);
    const int J = w * JPW + jl;                          // job: channel c, rows 2p, 2p+1
    const bool jv = J < C * P;
    const int c = jv ? J / P : 0, p = jv ? J - c * P : 0;
    const bool has1 = 2 * p + 1 < B;
    const int row0 = (2 * p * C + c) * L, row1 = ((2 * p + 1) * C + c) * L;
    const Span vs = make_span(v, 0, (int64_t)B * C * L);
    const Span rs = make_span(r, 0, (int64_t)B * C * L);
    float2* ubuf = lds + unit * REG;
    float* hb = hbuf + jl * 3 * SH_HEAD_MAX;
    const float2* sp = spec + (int64_t)c * SS;

    // 1. z_n = v[2p][c][n] + i v[2p+1][c][n] (zero past L and for a missing second row)
    float2 x[16];
    if (L == M) {
        // unconditional loads from rows that exist (their offsets fold into the
        // instructions), masked afterwards
        const bool m0 = jv, m1 = jv && has1;
        const int a0 = m0 ? row0 : 0, a1 = m1 ? row1 : a0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int n = tau + TB * q;
            const int nn = REV ? L - 1 - n : n;
            const float f0 = IO::load(vs, a0 + nn), f1 = IO::load(vs, a1 + nn);
            x[q] = make_float2(m0 ? f0 : 0.f, m1 ? f1 : 0.f);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int n = tau + TB * q;
            const int nn = REV ? L - 1 - n : n;
            const int e0 = (jv && n < L) ? row0 + nn : IO::OOB;
            const int e1 = (jv && has1 && n < L) ? row1 + nn : IO::OOB;
            x[q] = make_float2(IO::load(vs, e0), IO::load(vs, e1));
        }
    }
    if (!beta) {
#pragma unroll
        for (int q = 0; q < (TB >= SH_HEAD_MAX ? 1 : SH_HEAD_MAX / TB); ++q) {
            const int n = tau + TB * q;
            if (n < head) {
                hb[n] = x[q].x;
                hb[SH_HEAD_MAX + n] = x[q].y;
                hb[2 * SH_HEAD_MAX + n] = ((const float*)(sp + 2 * M))[n];
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) x[q] = cmul(x[q], tw_get<false>(bank, N, tau + TB * q));
    }

    // 2. U = DFT_M(.) = Z_{2j+beta}, times K_{2j+beta} / N
    fft_passes<M, false>(x, ubuf, tau, bank, true);
    // From here on an opaque copy of tau addresses the spectrum and the inverse's twiddles,
    // so those loads are neither hoisted above the forward transform nor merged with its
    // identical twiddle loads, which would hold them in registers in between.
    int tk = tau;
    asm volatile("" : "+v"(tk));
#pragma unroll
    for (int q = 0; q < 16; ++q) x[q] = cmul(x[q], sp[beta * M + tk + TB * q]);

    // 3. e^beta = IDFT_M(K Z restricted to parity beta), natural order.  (The forward's last
    //    pass runs in registers after a barrier that follows its last read of ubuf, so the
    //    inverse may write ubuf at once.)
    fft_passes<M, true>(x, ubuf, tk, bank, true);

    // 4. y_n = e^0_n + W_N^{-n} e^1_n: branch 1 hands W_N^{-n} e^1_n to branch 0 through LDS
    float2* xch = lds + (2 * jl + 1) * REG;
    if (beta) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int n = tk + TB * q;   // (W_N^n was also read for the pre-twiddle: keep apart)
            xch[lds_pad(n)] = cmulc(x[q], tw_get<false>(bank, N, n));
        }
    }
    __syncthreads();
    if (!beta) {
        if (jv) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int n = tau + TB * q;
                if (n < head || n >= L) continue;
                const float2 y = cadd(x[q], xch[lds_pad(n)]);
                const int nn = REV ? L - 1 - n : n;
                IO::store(rs, row0 + nn, y.x);
                if (has1) IO::store(rs, row1 + nn, y.y);
            }
        }
    } else if (jv) {
        // direct head of both rows: r_t = sum_{j<=t} v_j k_{t-j}, fp32, t < head, each sum
        // split over S lanes of this unit and reduced with lane shuffles
        const int nout = 2 * head;
        int S = 1;
        while (S < 8 && 2 * S * nout <= TB) S *= 2;
        if (TB >= 64) {
            for (int base = 0; base < nout * S; base += TB) {
                const int idx = base + tau, o = idx / S, s = idx - o * S;
                const int row = o >= head ? 1 : 0, t = o - row * head;
                float acc = 0.f;
                if (o < nout) {
                    const float* hv = hb + row * SH_HEAD_MAX;
                    const float* hk = hb + 2 * SH_HEAD_MAX;
                    for (int j = s; j <= t; j += S) acc = __builtin_fmaf(hv[j], hk[t - j], acc);
                }
                for (int d = 1; d < S; d <<= 1) acc += __shfl_xor(acc, d);
                if (o < nout && s == 0 && t < L && (row == 0 || has1))
                    IO::store(rs, (row ? row1 : row0) + (REV ? L - 1 - t : t), acc);
            }
        } else {
            // units narrower than a wave: one lane per output
            for (int o = tau; o < nout; o += TB) {
                const int row = o >= head ? 1 : 0, t = o - row * head;
                if (t >= L || (row && !has1)) continue;
                const float* hv = hb + row * SH_HEAD_MAX;
                const float* hk = hb + 2 * SH_HEAD_MAX;
                float acc = 0.f;
                for (int j = 0; j <= t; ++j) acc = __builtin_fmaf(hv[j], hk[t - j], acc);
                IO::store(rs, (row ? row1 : row0) + (REV ? L - 1 - t : t), acc);
            }
        }
    }
}

// ---------------------------------------------------------------- filter gradient (row loop)

// dk[c][j] = sum_b sum_{t>=j} dr[b][c][t] v[b][c][t-j] = sum_b rev(causal(rev(dr_b), v_b))_j.
// Per channel and batch row the transform of z = rev(dr_b) + i v_b carries both spectra;
// the unpacked inverse input Y_k of the real-output inverse is linear in X = DR' V, so it is
// summed over the rows in registers and inverted once.  The direct head (t < head) is
// summed over the rows in LDS.  A workgroup serves sh_grad_threads/(M/8) channels (one from
// M = 1024 on), looping over the B rows.
template <int M, class IO>
__global__ __launch_bounds__(sh_grad_threads<M>()) void shared_dk_kernel(
    const typename IO::T* __restrict__ dr, const typename IO::T* __restrict__ v,
    typename IO::T* __restrict__ dk, int B, int C, int L, int head, int pair_store,
    const float2* __restrict__ tw)
{
    constexpr int N = 2 * M, TB = M / 16, UNITS = sh_grad_threads<M>() / TB, CPW = UNITS / 2;
    constexpr int CT = CPW * TB;
    constexpr int REG = M + M / 16 + (M >= 256 ? SH_LDS_EXTRA : 0);
    __shared__ float2 lds[UNITS * REG];
    __shared__ float hbuf[CPW * 2 * SH_HEAD_MAX];    // rev(dr_b) then v_b, first values
    __shared__ float hsum[CPW * SH_HEAD_MAX];        // the head, summed over the rows

    const Bank bank = make_bank(tw);
    const int tid = threadIdx.x;
    const int unit = tid / TB, tau = tid % TB;
    const int cl = unit >> 1, beta = unit & 1;
    const int c0 = blockIdx.x * CPW;
    const int nvalid = (C - c0) < CPW ? (C - c0) : CPW;
    float2* ubuf = lds + unit * REG;
    float2* u0 = lds + (2 * cl) * REG;
    const float2* u1 = u0 + REG;
    const int lt = tid - cl * 2 * TB;
    const int cbase = cl * L;
    // head work of the upper half: output o (of CPW * head) split over S lanes
    const int nout = CPW * head;
    int S = 1;
    while (S < 8 && 2 * S * nout <= sh_grad_threads<M>() - CT) S *= 2;
    for (int i = tid; i < CPW * SH_HEAD_MAX; i += sh_grad_threads<M>()) hsum[i] = 0.f;

    float2 yacc[4], ymacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) yacc[i] = ymacc[i] = make_float2(0.f, 0.f);

    for (int b = 0; b < B; ++b) {
        const int64_t row = ((int64_t)b * C + c0) * L;
        const Span ds_ = make_span(dr, row, (int64_t)nvalid * L);
        const Span vs_ = make_span(v, row, (int64_t)nvalid * L);
        // Opaque copies of the thread's indices: the twiddle and LDS addresses below are the
        // same in every row, and without these the compiler hoists the twiddle loads out of
        // the row loop and holds them all in registers (175 VGPRs, serialised loads).
        int tau_r = tau, lt_r = lt;
        asm volatile("" : "+v"(tau_r), "+v"(lt_r));
        float2 x[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int n = tau_r + TB * q;
            const int e = n < L ? cbase + n : IO::OOB;
            const int er = n < L ? cbase + L - 1 - n : IO::OOB;
            x[q] = make_float2(IO::load(ds_, er), IO::load(vs_, e));
        }
        if (!beta) {
#pragma unroll
            for (int q = 0; q < (TB >= SH_HEAD_MAX ? 1 : SH_HEAD_MAX / TB); ++q) {
                const int n = tau_r + TB * q;
                if (n < head) {
                    hbuf[cl * 2 * SH_HEAD_MAX + n] = x[q].x;
                    hbuf[cl * 2 * SH_HEAD_MAX + SH_HEAD_MAX + n] = x[q].y;
                }
            }
        } else {
            float2 w[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) w[q] = tw_get<false>(bank, N, tau_r + TB * q);
#pragma unroll
            for (int q = 0; q < 16; ++q) x[q] = cmul(x[q], w[q]);
        }
        fft_passes<M, false>(x, ubuf, tau_r, bank, true);
#pragma unroll
        for (int q = 0; q < 16; ++q) ubuf[reg_off<TB>(tau_r, q)] = x[q];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = lt_r + 2 * TB * i;
            float2 yk, ymk;
            unpack_pair<M>(k, u0, u1, bank, yk, ymk);
            if (k == 0) {
                float2 unused;
                unpack_pair<M>(M / 2, u0, u1, bank, ymk, unused);
            }
            yacc[i] = cadd(yacc[i], yk);
            ymacc[i] = cadd(ymacc[i], ymk);
        }
        if (tid >= CT) {
            // this row's head terms, added to hsum by the group's first lane
            for (int base = 0; base < nout * S; base += sh_grad_threads<M>() - CT) {
                const int idx = base + tid - CT, o = idx / S, sl = idx - o * S;
                const int c2 = o / (head > 0 ? head : 1), t = o - c2 * head;
                float acc = 0.f;
                if (o < nout) {
                    const float* hv = hbuf + c2 * 2 * SH_HEAD_MAX;
                    const float* hg = hv + SH_HEAD_MAX;
                    for (int j = sl; j <= t; j += S) acc = __builtin_fmaf(hv[j], hg[t - j], acc);
                }
                for (int d = 1; d < S; d <<= 1) acc += __shfl_xor(acc, d);
                if (o < nout && sl == 0) hsum[c2 * SH_HEAD_MAX + t] += acc;
            }
        }
        __syncthreads();   // ubuf and hbuf are rewritten for the next row
    }

    // the summed Y into branch 0's region, then one inverse (as the per-row-gate kernel)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = lt + 2 * TB * i;
        u0[lds_pad(k)] = yacc[i];
        u0[lds_pad(k == 0 ? M / 2 : M - k)] = ymacc[i];
    }
    __syncthreads();
    const Span ks = make_span(dk, (int64_t)c0 * L, (int64_t)nvalid * L);
    const bool iact = tid < CT;
    const int icl = iact ? tid / TB : 0, itau = tid % TB;
    float2* ybuf = lds + (2 * icl) * REG;
    float2 x[16];
    if (iact) {
#pragma unroll
        for (int q = 0; q < 16; ++q) x[q] = ybuf[reg_off<TB>(itau, q)];
    }
    __syncthreads();
    if (!iact) {
        // the head, reversed like the rest: dk_{L-1-t} for t < head
        for (int o = tid - CT; o < nout; o += sh_grad_threads<M>() - CT) {
            const int c2 = o / head, t = o - c2 * head;
            if (c2 < nvalid && t < L) IO::store(ks, c2 * L + L - 1 - t, hsum[c2 * SH_HEAD_MAX + t]);
        }
    }
    fft_passes<M, true>(x, ybuf, itau, bank, iact);
    if (iact && icl < nvalid) {
        const float scale = 1.0f / (8.0f * (float)M);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int t = 2 * (itau + TB * q);
            if (t < head || t >= L) continue;
            const float a = x[q].x * scale, bb = x[q].y * scale;
            if (t + 1 < L) {
                if (pair_store) {
                    IO::store2(ks, icl * L + L - 2 - t, bb, a);
                } else {
                    IO::store(ks, icl * L + L - 1 - t, a);
                    IO::store(ks, icl * L + L - 2 - t, bb);
                }
            } else {
                IO::store(ks, icl * L + L - 1 - t, a);
            }
        }
    }
}

// ---------------------------------------------------------------- both gradients, one kernel

// From the branch spectra of z = rev(dr_b) + i v_b (u0[j] = Z_{2j}, u1[j] = Z_{2j+1}) form, at
// bins k and M - k, the real-output inverse inputs of both gradients:
//   dk: Y of X = DR' V (scaled by 8, as unpack_pair), summed over the rows by the caller;
//   dv: Y of X' = DR' K with K from the filter spectrum (stored / N), scaled by 1/(2N)
//       relative to the dk scaling, so dv takes the output scale 1/2 where dk takes 1/(8M).
// DR'_k = (Z_k + conj Z_{N-k}) / 2 and V_k = (Z_k - conj Z_{N-k}) / (2i).
template <int M>
__device__ __forceinline__ void y_of(float2 x1, float2 x2, float2 w, float2& yk, float2& ymk)
{
    // S = X_k + X_{k+M}, D = X_k - X_{k+M} with X_{k+M} = conj X_{M-k}
    const float2 sm = make_float2(x1.x + x2.x, x1.y - x2.y);
    const float2 df = make_float2(x1.x - x2.x, x1.y + x2.y);
    const float2 t = cmulc(df, w);                                 // W_N^{-k} D
    yk = make_float2(sm.x - t.y, sm.y + t.x);
    ymk = make_float2(sm.x + t.y, t.x - sm.y);
}

template <int M>
__device__ __forceinline__ void unpack_grads(int k, const float2* __restrict__ u0,
                                             const float2* __restrict__ u1,
                                             const float2* __restrict__ sp, const Bank& bank,
                                             float2& yk, float2& ymk, float2& zk, float2& zmk)
{
    constexpr int N = 2 * M;
    const int b = k & 1, j = k >> 1, jm = (M / 2 - j - b) & (M - 1);
    const float2* u = b ? u1 : u0;
    const float2 p1 = u[lds_pad(j)];
    const float2 q1 = conjf2(u[lds_pad((M - j - b) & (M - 1))]);
    const float2 p2 = u[lds_pad(jm)];
    const float2 q2 = conjf2(u[lds_pad(M / 2 + j)]);
    const float2 s1 = cadd(p1, q1), d1 = csub(p1, q1);
    const float2 s2 = cadd(p2, q2), d2 = csub(p2, q2);
    const float2 w = tw_get<false>(bank, N, k);
    // dk: 4 X = -i (P + Q)(P - Q) at k and M - k
    const float2 x1 = make_float2(__builtin_fmaf(s1.x, d1.y, s1.y * d1.x),
                                  __builtin_fmaf(s1.y, d1.y, -s1.x * d1.x));
    const float2 x2 = make_float2(__builtin_fmaf(s2.x, d2.y, s2.y * d2.x),
                                  __builtin_fmaf(s2.y, d2.y, -s2.x * d2.x));
    y_of<M>(x1, x2, w, yk, ymk);
    // dv: (P + Q) K / N = 2 DR' K / N at k and M - k
    y_of<M>(cmul(s1, sp[b * M + j]), cmul(s2, sp[b * M + jm]), w, zk, zmk);
}

// Gradients for a filter shared by the batch, one kernel:
//   dv[b][c][j] = sum_{t>=j} dr[b][c][t] k[c][t-j] = rev(causal(rev(dr_b), k))_j
//   dk[c][j]    = sum_b sum_{t>=j} dr[b][c][t] v[b][c][t-j] = sum_b rev(causal(rev(dr_b), v_b))_j
// A workgroup serves sh_grad_threads/(M/8) channels (one from M = 1024 on) and loops over the
// B rows.
// Per row, one transform of z = rev(dr_b) + i v_b carries the spectra of rev(dr_b) and v_b;
// the unpack gives the inverse input of dv_b (times the filter's spectrum), which is inverted
// and stored at once, and that of dk (times V), which is linear in the product and summed
// over the rows in registers and inverted once at the end.  Direct heads (t < head): dv_b's
// per row, dk's summed over the rows in LDS, both by the half of the workgroup that is idle
// during an inverse.  Outputs are written reversed.
template <int M, class IO>
__global__ __launch_bounds__(sh_grad_threads<M>(), (M >= 512 ? 4 : 1)) void shared_bwd_kernel(
    const typename IO::T* __restrict__ dr, const typename IO::T* __restrict__ v,
    const float2* __restrict__ spec, typename IO::T* __restrict__ dv,
    typename IO::T* __restrict__ dk, int B, int C, int L, int head, int pair_store,
    const float2* __restrict__ tw)
{
    constexpr int N = 2 * M, TB = M / 16, UNITS = sh_grad_threads<M>() / TB, CPW = UNITS / 2;
    constexpr int CT = CPW * TB;
    constexpr int REG = M + M / 16 + (M >= 256 ? SH_LDS_EXTRA : 0);
    constexpr int SS = spec_stride<M>();
    __shared__ float2 lds[UNITS * REG];
    __shared__ float hbuf[CPW * 3 * SH_HEAD_MAX];    // rev(dr_b), v_b, k: first values
    __shared__ float hsum[CPW * SH_HEAD_MAX];        // dk's head, summed over the rows

    const Bank bank = make_bank(tw);
    const int tid = threadIdx.x;
    const int unit = tid / TB, tau = tid % TB;
    const int cl = unit >> 1, beta = unit & 1;
    const int c0 = blockIdx.x * CPW;
    const int nvalid = (C - c0) < CPW ? (C - c0) : CPW;
    float2* ubuf = lds + unit * REG;
    float2* u0 = lds + (2 * cl) * REG;
    const float2* u1 = u0 + REG;
    const int lt = tid - cl * 2 * TB;
    const int cbase = cl * L;
    const float2* sp = spec + (int64_t)(c0 + (cl < nvalid ? cl : 0)) * SS;
    // inverse: the first CT threads, one channel per TB of them; heads: the others
    const bool iact = tid < CT;
    const int icl = iact ? tid / TB : 0, itau = tid % TB;
    float2* ybuf = lds + (2 * icl) * REG;
    const int nout = CPW * head;
    int S = 1;
    while (S < 8 && 2 * S * nout <= sh_grad_threads<M>() - CT) S *= 2;
    for (int i = tid; i < CPW * SH_HEAD_MAX; i += sh_grad_threads<M>()) {
        hsum[i] = 0.f;
        const int c2 = i / SH_HEAD_MAX, n = i - c2 * SH_HEAD_MAX;
        hbuf[c2 * 3 * SH_HEAD_MAX + 2 * SH_HEAD_MAX + n] =
            c2 < nvalid ? ((const float*)(spec + (int64_t)(c0 + c2) * SS + 2 * M))[n] : 0.f;
    }

    float2 yacc[4], ymacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) yacc[i] = ymacc[i] = make_float2(0.f, 0.f);

    for (int b = 0; b < B; ++b) {
        const int64_t row = ((int64_t)b * C + c0) * L;
        const Span ds_ = make_span(dr, row, (int64_t)nvalid * L);
        const Span vs_ = make_span(v, row, (int64_t)nvalid * L);
        const Span os_ = make_span(dv, row, (int64_t)nvalid * L);
        // Opaque copies of the thread's indices: the twiddle, spectrum and LDS addresses
        // below are the same in every row, and the compiler would otherwise hoist their loads
        // out of the row loop and hold them all in registers.
        int tau_r = tau, lt_r = lt, itau_r = itau;
        asm volatile("" : "+v"(tau_r), "+v"(lt_r), "+v"(itau_r));
        float2 x[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int n = tau_r + TB * q;
            const int e = n < L ? cbase + n : IO::OOB;
            const int er = n < L ? cbase + L - 1 - n : IO::OOB;
            x[q] = make_float2(IO::load(ds_, er), IO::load(vs_, e));
        }
        if (!beta) {
#pragma unroll
            for (int q = 0; q < (TB >= SH_HEAD_MAX ? 1 : SH_HEAD_MAX / TB); ++q) {
                const int n = tau_r + TB * q;
                if (n < head) {
                    hbuf[cl * 3 * SH_HEAD_MAX + n] = x[q].x;
                    hbuf[cl * 3 * SH_HEAD_MAX + SH_HEAD_MAX + n] = x[q].y;
                }
            }
        } else {
            float2 w[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) w[q] = tw_get<false>(bank, N, tau_r + TB * q);
#pragma unroll
            for (int q = 0; q < 16; ++q) x[q] = cmul(x[q], w[q]);
        }
        fft_passes<M, false>(x, ubuf, tau_r, bank, true);
#pragma unroll
        for (int q = 0; q < 16; ++q) ubuf[reg_off<TB>(tau_r, q)] = x[q];
        __syncthreads();

        // unpack: dk's Y summed, dv's Y kept
        float2 zk[4], zmk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = lt_r + 2 * TB * i;
            float2 yk, ymk;
            unpack_grads<M>(k, u0, u1, sp, bank, yk, ymk, zk[i], zmk[i]);
            if (k == 0) {
                // Y_{M/2} in place of the absent Y_M
                float2 u_, v_;
                unpack_grads<M>(M / 2, u0, u1, sp, bank, ymk, u_, zmk[i], v_);
            }
            yacc[i] = cadd(yacc[i], yk);
            ymacc[i] = cadd(ymacc[i], ymk);
        }
        __syncthreads();   // every unpack has read Z
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = lt_r + 2 * TB * i;
            u0[lds_pad(k)] = zk[i];
            u0[lds_pad(k == 0 ? M / 2 : M - k)] = zmk[i];
        }
        __syncthreads();
        if (iact) {
#pragma unroll
            for (int q = 0; q < 16; ++q) x[q] = ybuf[reg_off<TB>(itau_r, q)];
        }
        __syncthreads();
        if (!iact) {
            // this row's heads: dv_{L-1-t} = sum_{j<=t} rev(dr)_j k_{t-j} (stored), and the
            // row's share of dk's head sum_{j<=t} rev(dr)_j v_{t-j} (added to hsum by the
            // group's first lane); each sum split over S lanes
            for (int base = 0; base < 2 * nout * S; base += sh_grad_threads<M>() - CT) {
                const int idx = base + tid - CT, o2 = idx / S, sl = idx - o2 * S;
                const int which = o2 >= nout ? 1 : 0, o = o2 - which * nout;
                const int c2 = o / (head > 0 ? head : 1), t = o - c2 * head;
                float acc = 0.f;
                if (o2 < 2 * nout) {
                    const float* hd = hbuf + c2 * 3 * SH_HEAD_MAX;
                    const float* hg = hd + (which ? SH_HEAD_MAX : 2 * SH_HEAD_MAX);
                    for (int j = sl; j <= t; j += S) acc = __builtin_fmaf(hd[j], hg[t - j], acc);
                }
                for (int d = 1; d < S; d <<= 1) acc += __shfl_xor(acc, d);
                if (o2 < 2 * nout && sl == 0) {
                    if (which) hsum[c2 * SH_HEAD_MAX + t] += acc;
                    else if (c2 < nvalid && t < L) IO::store(os_, c2 * L + L - 1 - t, acc);
                }
            }
        }
        fft_passes<M, true>(x, ybuf, itau_r, bank, iact);
        if (iact && icl < nvalid) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int t = 2 * (itau_r + TB * q);
                if (t < head || t >= L) continue;
                const float a = x[q].x * 0.5f, bb = x[q].y * 0.5f;
                if (t + 1 < L) {
                    if (pair_store) {
                        IO::store2(os_, icl * L + L - 2 - t, bb, a);
                    } else {
                        IO::store(os_, icl * L + L - 1 - t, a);
                        IO::store(os_, icl * L + L - 2 - t, bb);
                    }
                } else {
                    IO::store(os_, icl * L + L - 1 - t, a);
                }
            }
        }
    }

    // dk: the summed Y into branch 0's region, one inverse
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = lt + 2 * TB * i;
        u0[lds_pad(k)] = yacc[i];
        u0[lds_pad(k == 0 ? M / 2 : M - k)] = ymacc[i];
    }
    __syncthreads();
    const Span ks = make_span(dk, (int64_t)c0 * L, (int64_t)nvalid * L);
    float2 x[16];
    if (iact) {
#pragma unroll
        for (int q = 0; q < 16; ++q) x[q] = ybuf[reg_off<TB>(itau, q)];
    }
    __syncthreads();
    if (!iact) {
        for (int o = tid - CT; o < nout; o += sh_grad_threads<M>() - CT) {
            const int c2 = o / head, t = o - c2 * head;
            if (c2 < nvalid && t < L) IO::store(ks, c2 * L + L - 1 - t, hsum[c2 * SH_HEAD_MAX + t]);
        }
    }
    fft_passes<M, true>(x, ybuf, itau, bank, iact);
    if (iact && icl < nvalid) {
        const float scale = 1.0f / (8.0f * (float)M);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int t = 2 * (itau + TB * q);
            if (t < head || t >= L) continue;
            const float a = x[q].x * scale, bb = x[q].y * scale;
            if (t + 1 < L) {
                if (pair_store) {
                    IO::store2(ks, icl * L + L - 2 - t, bb, a);
                } else {
                    IO::store(ks, icl * L + L - 1 - t, a);
                    IO::store(ks, icl * L + L - 2 - t, bb);
                }
            } else {
                IO::store(ks, icl * L + L - 1 - t, a);
            }
        }
    }
}

// ---------------------------------------------------------------- launch

namespace {

template <int M, class IO>
hipError_t spectrum_m(const void* k, float2* spec, int C, int L, const float2* tw, hipStream_t s)
{
    constexpr int PPW = (sh_threads<M>() / (M / 16)) / 2;
    const int64_t pairs = ((int64_t)C + 1) / 2;
    const int64_t blocks = (pairs + PPW - 1) / PPW;
    if (!grid_ok(blocks, sh_threads<M>())) return hipErrorInvalidValue;
    hipLaunchKernelGGL((shared_spectrum_kernel<M, IO>), dim3((unsigned)blocks), dim3(sh_threads<M>()),
                       0, s, (const typename IO::T*)k, spec, C, L, tw);
    return hipGetLastError();
}

template <int M, class IO, bool REV>
hipError_t apply_m(const void* v, const float2* spec, void* r, int B, int C, int L, int head,
                   const float2* tw, hipStream_t s)
{
    constexpr int JPW = (sh_threads<M>() / (M / 16)) / 2;
    const int64_t jobs = (int64_t)C * ((B + 1) / 2);
    const int64_t blocks = ((jobs + JPW - 1) / JPW + 7) / 8 * 8;   // a multiple of 8
    if (!grid_ok(blocks, sh_threads<M>())) return hipErrorInvalidValue;
    hipLaunchKernelGGL((shared_apply_kernel<M, IO, REV>), dim3((unsigned)blocks), dim3(sh_threads<M>()), 0,
                       s, (const typename IO::T*)v, spec, (typename IO::T*)r, B, C, L, head, tw);
    return hipGetLastError();
}

template <int M, class IO>
hipError_t dk_m(const void* dr, const void* v, void* dk, int B, int C, int L, int head, bool pair,
                const float2* tw, hipStream_t s)
{
    constexpr int CPW = (sh_grad_threads<M>() / (M / 16)) / 2;
    const int64_t blocks = ((int64_t)C + CPW - 1) / CPW;
    if (!grid_ok(blocks, sh_grad_threads<M>())) return hipErrorInvalidValue;
    hipLaunchKernelGGL((shared_dk_kernel<M, IO>), dim3((unsigned)blocks), dim3(sh_grad_threads<M>()), 0, s,
                       (const typename IO::T*)dr, (const typename IO::T*)v, (typename IO::T*)dk, B,
                       C, L, head, pair ? 1 : 0, tw);
    return hipGetLastError();
}

template <class IO>
hipError_t dk_io(const void* dr, const void* v, void* dk, int B, int C, int L, int M, int head,
                 bool pair, const float2* tw, hipStream_t s)
{
    switch (M) {
    case 64: return dk_m<64, IO>(dr, v, dk, B, C, L, head, pair, tw, s);
    case 128: return dk_m<128, IO>(dr, v, dk, B, C, L, head, pair, tw, s);
    case 256: return dk_m<256, IO>(dr, v, dk, B, C, L, head, pair, tw, s);
    case 512: return dk_m<512, IO>(dr, v, dk, B, C, L, head, pair, tw, s);
    case 1024: return dk_m<1024, IO>(dr, v, dk, B, C, L, head, pair, tw, s);
    case 2048: return dk_m<2048, IO>(dr, v, dk, B, C, L, head, pair, tw, s);
    case 4096: return dk_m<4096, IO>(dr, v, dk, B, C, L, head, pair, tw, s);
    default: return hipErrorInvalidValue;
    }
}

template <int M, class IO>
hipError_t bwd_m(const void* dr, const void* v, const float2* spec, void* dv, void* dk, int B,
                 int C, int L, int head, bool pair, const float2* tw, hipStream_t s)
{
    constexpr int CPW = (sh_grad_threads<M>() / (M / 16)) / 2;
    const int64_t blocks = ((int64_t)C + CPW - 1) / CPW;
    if (!grid_ok(blocks, sh_grad_threads<M>())) return hipErrorInvalidValue;
    hipLaunchKernelGGL((shared_bwd_kernel<M, IO>), dim3((unsigned)blocks), dim3(sh_grad_threads<M>()), 0,
                       s, (const typename IO::T*)dr, (const typename IO::T*)v, spec,
                       (typename IO::T*)dv, (typename IO::T*)dk, B, C, L, head, pair ? 1 : 0,
                       tw);
    return hipGetLastError();
}

template <class IO>
hipError_t bwd_io(const void* dr, const void* v, const float2* spec, void* dv, void* dk, int B,
                  int C, int L, int M, int head, bool pair, const float2* tw, hipStream_t s)
{
    switch (M) {
    case 64: return bwd_m<64, IO>(dr, v, spec, dv, dk, B, C, L, head, pair, tw, s);
    case 128: return bwd_m<128, IO>(dr, v, spec, dv, dk, B, C, L, head, pair, tw, s);
    case 256: return bwd_m<256, IO>(dr, v, spec, dv, dk, B, C, L, head, pair, tw, s);
    case 512: return bwd_m<512, IO>(dr, v, spec, dv, dk, B, C, L, head, pair, tw, s);
    case 1024: return bwd_m<1024, IO>(dr, v, spec, dv, dk, B, C, L, head, pair, tw, s);
    case 2048: return bwd_m<2048, IO>(dr, v, spec, dv, dk, B, C, L, head, pair, tw, s);
    case 4096: return bwd_m<4096, IO>(dr, v, spec, dv, dk, B, C, L, head, pair, tw, s);
    default: return hipErrorInvalidValue;
    }
}

template <class IO>
hipError_t spectrum_io(const void* k, float2* spec, int C, int L, int M, const float2* tw,
                       hipStream_t s)
{
    switch (M) {
    case 64: return spectrum_m<64, IO>(k, spec, C, L, tw, s);
    case 128: return spectrum_m<128, IO>(k, spec, C, L, tw, s);
    case 256: return spectrum_m<256, IO>(k, spec, C, L, tw, s);
    case 512: return spectrum_m<512, IO>(k, spec, C, L, tw, s);
    case 1024: return spectrum_m<1024, IO>(k, spec, C, L, tw, s);
    case 2048: return spectrum_m<2048, IO>(k, spec, C, L, tw, s);
    case 4096: return spectrum_m<4096, IO>(k, spec, C, L, tw, s);
    default: return hipErrorInvalidValue;
    }
}

template <class IO, bool REV>
hipError_t apply_io(const void* v, const float2* spec, void* r, int B, int C, int L, int M,
                    int head, const float2* tw, hipStream_t s)
{
    switch (M) {
    case 64: return apply_m<64, IO, REV>(v, spec, r, B, C, L, head, tw, s);
    case 128: return apply_m<128, IO, REV>(v, spec, r, B, C, L, head, tw, s);
    case 256: return apply_m<256, IO, REV>(v, spec, r, B, C, L, head, tw, s);
    case 512: return apply_m<512, IO, REV>(v, spec, r, B, C, L, head, tw, s);
    case 1024: return apply_m<1024, IO, REV>(v, spec, r, B, C, L, head, tw, s);
    case 2048: return apply_m<2048, IO, REV>(v, spec, r, B, C, L, head, tw, s);
    case 4096: return apply_m<4096, IO, REV>(v, spec, r, B, C, L, head, tw, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_shared_spectrum(Store st, const void* k, float2* spec, int C, int L, int M,
                                  const float2* tw, hipStream_t s)
{
    return st == Store::F32 ? spectrum_io<f32_io>(k, spec, C, L, M, tw, s)
                            : spectrum_io<bf16_io>(k, spec, C, L, M, tw, s);
}

hipError_t launch_shared_apply(Store st, const void* v, const float2* spec, void* r, int B, int C,
                               int L, int M, int head, bool rev, const float2* tw, hipStream_t s)
{
    if (st == Store::F32)
        return rev ? apply_io<f32_io, true>(v, spec, r, B, C, L, M, head, tw, s)
                   : apply_io<f32_io, false>(v, spec, r, B, C, L, M, head, tw, s);
    return rev ? apply_io<bf16_io, true>(v, spec, r, B, C, L, M, head, tw, s)
               : apply_io<bf16_io, false>(v, spec, r, B, C, L, M, head, tw, s);
}

hipError_t launch_shared_dk(Store st, const void* dr, const void* v, void* dk, int B, int C, int L,
                            int M, int head, bool pair_store, const float2* tw, hipStream_t s)
{
    return st == Store::F32 ? dk_io<f32_io>(dr, v, dk, B, C, L, M, head, pair_store, tw, s)
                            : dk_io<bf16_io>(dr, v, dk, B, C, L, M, head, pair_store, tw, s);
}

int64_t shared_bwd_blocks(int64_t C, int M)
{
    const int64_t cpw = ((M >= 1024 ? M / 8 : SH_THREADS) / (M / 16)) / 2;   // sh_grad_threads
    return (C + cpw - 1) / cpw;
}

hipError_t launch_shared_bwd(Store st, const void* dr, const void* v, const float2* spec, void* dv,
                             void* dk, int B, int C, int L, int M, int head, bool pair_store,
                             const float2* tw, hipStream_t s)
{
    return st == Store::F32
               ? bwd_io<f32_io>(dr, v, spec, dv, dk, B, C, L, M, head, pair_store, tw, s)
               : bwd_io<bf16_io>(dr, v, spec, dv, dk, B, C, L, M, head, pair_store, tw, s);
}

__global__ void zero16_kernel(uint16_t* __restrict__ p, int64_t n)
{
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) p[i] = 0;
}

hipError_t launch_zero16(void* p, int64_t n16, hipStream_t stream)
{
    if (n16 <= 0) return hipSuccess;
    constexpr int threads = 256;
    const int64_t want = (n16 + threads - 1) / threads;
    const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(zero16_kernel, dim3(blocks), dim3(threads), 0, stream, (uint16_t*)p, n16);
    return hipGetLastError();
}

}  // namespace sc
