// Fused in-LDS causal long convolution for L <= 4096 (gfx950).
//
// Method ("Caracal: Causal Architecture via Spectral Mixing", key designs 1 and 2):
// zero-pad v and g on the right to N = 2M (M = next power of two >= L), FFT, multiply the
// spectra bin by bin, inverse FFT, keep the first L values.  That equals the causal
// convolution r_t = sum_{j<=t} v_j g_{t-j}.  The improvement direction the notes list
// under limitations (a real FFT to halve the work) is taken here in three places:
//
//  1. v and g are real, so one complex transform of z = v + i g carries both spectra:
//     V_k = (Z_k + conj Z_{N-k}) / 2,  G_k = (Z_k - conj Z_{N-k}) / (2i).
//  2. The upper half of z is the zero padding, so the first decimation-in-frequency stage
//     of the length-N transform is only a twiddle: with u^b_n = z_n W_N^{b n} (n < M),
//     Z_{2j+b} = DFT_M(u^b)_j for b = 0, 1.  The two length-M transforms ("branches")
//     run side by side in one workgroup.
//  3. The result x = IDFT_N(V G) is real, so it is obtained from one length-M complex
//     inverse transform:  Y_k = [(X_k + X_{k+M}) + i W_N^{-k} (X_k - X_{k+M})] / 2,
//     y = IDFT_M(Y) / M gives y_m = x_{2m} + i x_{2m+1}.  With X_{k+M} = conj X_{M-k},
//     the four bins {k, N-k, M-k, M+k} of Z give Y_k and Y_{M-k} together.
//
// The first `head` outputs (default 32) are recomputed by direct fp32 summation: their
// error scale sum_j |v_j||g_{t-j}| holds only t+1 products, far below the global round-off
// of any float FFT.
//
// A length-M transform is held by TB = M/16 threads with 16 values each (element
// tau + TB*r sits in register r of thread tau, at the input and the output of every
// transform); between radix passes the values go through LDS.  A workgroup of
// max(64, M/8) threads serves CPW channels (two branch units of TB threads per channel):
// one channel from M = 512 on, as many as fill one wave below.  It uses
// 2*CPW*(M + M/16 + 24) complex values of LDS (35 KB at M = 2048).  Small workgroups let
// workgroups at different phases share a CU: at M = 1024 one channel per workgroup took
// 44 -> 39 us against four channels per 512-thread workgroup, at M = 256 (64 channels)
// 11 -> 7 us, bit for bit the same.  The library sends M = 4096 (2048 < L <= 4096) to the
// kernel of sc_fused4k.hip; this one serves it only as the reference form.
// HBM traffic is read v, read g, write r: nothing else leaves the chip.

#include "sc_device.h"
#include "sc_fft_lds.h"
#include "sc_internal.h"

namespace sc {

// threads of the workgroup for length-M transforms
template <int M>
constexpr int fused_threads() { return M / 8 > 64 ? M / 8 : 64; }
#ifndef SC_LDS_EXTRA
#define SC_LDS_EXTRA 24
#endif
// extra float2 between the LDS regions of the two branches of a channel: with it the
// unpack's alternating reads of u0[j] and u1[j] land in different banks
constexpr int LDS_EXTRA = SC_LDS_EXTRA;

// pf > 0 (M >= 1024): the threads idle during the inverse touch the cache lines of v and g of
// the channels pf workgroups ahead -- the workgroup that will take this one's place when
// pf = the workgroups resident at once, on the same XCD (pf a multiple of 8), whose L2 then
// holds its inputs: without it every generation of workgroups began by waiting on HBM.
template <int M, class IO, bool REV>
__global__ __launch_bounds__(fused_threads<M>()) void fused_conv_kernel(
    const typename IO::T* __restrict__ v, const typename IO::T* __restrict__ g,
    typename IO::T* __restrict__ r, int64_t nch, int L, int head, int pair_store,
    const float2* __restrict__ tw, int64_t pf)
{
    static_assert(M >= 64 && M <= 4096, "fused path handles 64 <= M <= 4096");
    constexpr int FT = fused_threads<M>();
    constexpr int N = 2 * M, TB = M / 16, UNITS = FT / TB, CPW = UNITS / 2;
    static_assert(CPW >= 1 && FT % 64 == 0, "whole waves, two branch units per channel");
    constexpr int REG = M + M / 16 + (M >= 256 ? LDS_EXTRA : 0);
    __shared__ float2 lds[UNITS * REG];
    // first HEAD_MAX inputs of each local channel (v then g) for the direct head
    __shared__ float hbuf[CPW * 2 * HEAD_MAX];

    const Bank bank = make_bank(tw);
    const int tid = threadIdx.x;
    const int unit = tid / TB, tau = tid % TB;
    const int cl = unit >> 1, beta = unit & 1;
    const int64_t ch0 = (int64_t)blockIdx.x * CPW;
    const int nvalid = (int)((nch - ch0) < CPW ? (nch - ch0) : CPW);
    // descriptors over this workgroup's channels: loads past them read 0, stores are dropped
    const Span vs = make_span(v, ch0 * L, (int64_t)nvalid * L);
    const Span gs = make_span(g, ch0 * L, (int64_t)nvalid * L);
    float2* ubuf = lds + unit * REG;

    // 1. u^beta_n = z_n W_N^{beta n},  z_n = v_n + i g_n for n < L, 0 otherwise
    float2 x[16];
    {
        const int cbase = cl * L;
        if (L == M) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int n = tau + TB * q;
                x[q] = make_float2(IO::load(vs, cbase + (REV ? L - 1 - n : n)),
                                   IO::load(gs, cbase + n));
            }
        } else {
            // elements past L are read at IO::OOB, beyond the descriptor's range, so they read
            // 0; a select instead of a branch keeps all 32 loads in flight together
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int n = tau + TB * q;
                const int e = n < L ? cbase + n : IO::OOB;
                const int ev = n < L ? cbase + (REV ? L - 1 - n : n) : IO::OOB;
                x[q] = make_float2(IO::load(vs, ev), IO::load(gs, e));
            }
        }
        if (!beta) {
#pragma unroll
            for (int q = 0; q < (TB >= HEAD_MAX ? 1 : HEAD_MAX / TB); ++q) {
                const int n = tau + TB * q;
                if (n < head) {
                    hbuf[cl * 2 * HEAD_MAX + n] = x[q].x;
                    hbuf[cl * 2 * HEAD_MAX + HEAD_MAX + n] = x[q].y;
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) x[q] = cmul(x[q], tw_get<false>(bank, N, tau + TB * q));
        }
    }

    // 2. U^beta = DFT_M(u^beta); x[q] = U^beta_{tau + TB q}
    fft_passes<M, false>(x, ubuf, tau, bank, true);
#pragma unroll
    for (int q = 0; q < 16; ++q) ubuf[reg_off<TB>(tau, q)] = x[q];
    __syncthreads();

    // 3. unpack + spectral product: channel-local thread lt takes k = lt + 2TB i, i < 4,
    //    covering k in [0, M/2); k = 0 also yields Y_{M/2} in place of the absent Y_M.
    const int lt = tid - cl * 2 * TB;
    float2* u0 = lds + (2 * cl) * REG;
    const float2* u1 = u0 + REG;
    float2 yk[4], ymk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = lt + 2 * TB * i;
        unpack_pair<M>(k, u0, u1, bank, yk[i], ymk[i]);
        if (k == 0) {
            float2 unused;
            unpack_pair<M>(M / 2, u0, u1, bank, ymk[i], unused);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = lt + 2 * TB * i;
        u0[lds_pad(k)] = yk[i];
        u0[lds_pad(k == 0 ? M / 2 : M - k)] = ymk[i];
    }
    __syncthreads();

    // output t of local channel c at flat index c L + t (at L-1-t when REV; pairs need L
    // even, which the host ensures)
    const Span rs = make_span(r, ch0 * L, (int64_t)nvalid * L);
    auto put = [&](int c, int t, float a) { IO::store(rs, c * L + (REV ? L - 1 - t : t), a); };
    auto put2 = [&](int c, int t, float a, float b) {
        if (REV) IO::store2(rs, c * L + L - 2 - t, b, a);
        else IO::store2(rs, c * L + t, a, b);
    };

    if constexpr (M <= 512) {
        // 4. y = IDFT_M(Y) with 8 values per thread: threads [c*TBI, (c+1)*TBI) serve local
        //    channel c, every thread of the workgroup busy (radix-8 passes).  For short
        //    transforms this beats the split below (M = 64: 86 -> 62 us per 64K channels;
        //    M = 512: 3%), from M = 1024 on it is slower (one more pass and exchange).
        constexpr int TBI = M / 8;
        const int icl = tid / TBI, itau = tid % TBI;
        float2* ybuf = lds + (2 * icl) * REG;
        float2 y[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] = ybuf[reg_off<TBI>(itau, q)];
        __syncthreads();
        fft_passes<M, true, 1, 8>(y, ybuf, itau, bank, true);

        // 5. store: y[q] = 8 M y_m with m = itau + TBI q (q < 4 covers m < M/2)
        const float scale = 1.0f / (8.0f * (float)M);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = 2 * (itau + TBI * q);
            if (t >= head && t < L) {
                const float a = y[q].x * scale, b = y[q].y * scale;
                if (t + 1 < L) {
                    if (pair_store) {
                        put2(icl, t, a, b);
                    } else {
                        put(icl, t, a);
                        put(icl, t + 1, b);
                    }
                } else {
                    put(icl, t, a);
                }
            }
        }
        // 6. the direct head, by all threads: r_t = sum_{j<=t} v_j g_{t-j}, fp32, t < head
        direct_head<FT>(hbuf, CPW, nvalid, L, head, tid, put);
    } else {
        // 4. y = IDFT_M(Y): threads [c*TB, (c+1)*TB) serve local channel c.  The other half of
        //    the workgroup computes the direct head meanwhile, from the inputs staged at load
        //    time: r_t = sum_{j<=t} v_j g_{t-j} in fp32 for t < head.
        const bool iact = tid < CPW * TB;
        const int icl = iact ? tid / TB : 0, itau = tid % TB;
        float2* ybuf = lds + (2 * icl) * REG;
        if (iact) {
#pragma unroll
            for (int q = 0; q < 16; ++q) x[q] = ybuf[reg_off<TB>(itau, q)];
        }
        __syncthreads();
        // between this barrier and the first one of the inverse, where the active threads run
        // their first radix-16 pass
        uint2 touched = make_uint2(0u, 0u);
        if (!iact) {
            direct_head<FT - CPW * TB>(hbuf, CPW, nvalid, L, head, tid - CPW * TB, put);
            // one line of v and one of g per idle thread covers the CPW channels ahead
            static_assert(CPW * M * sizeof(typename IO::T) <= 128 * (FT - CPW * TB),
                          "the idle threads cover the next workgroup's lines");
            if (pf > 0 && (int64_t)blockIdx.x + pf < (nch + CPW - 1) / CPW)
                touched = touch_line(v, g, (ch0 + pf * CPW) * L, (int64_t)CPW * L, tid - CPW * TB);
        }
        fft_passes<M, true>(x, ybuf, itau, bank, iact);
        if (!iact) keep_touched(touched, pf, rs);

        // 5. store: x[q] = 8 M y_m with m = itau + TB q; r_{2m} = Re y_m, r_{2m+1} = Im y_m
        if (iact) {
            const float scale = 1.0f / (8.0f * (float)M);
            if (L == M && pair_store) {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int t = 2 * (itau + TB * q);
                    if (2 * TB * q >= HEAD_MAX || t >= head)
                        put2(icl, t, x[q].x * scale, x[q].y * scale);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int t = 2 * (itau + TB * q);
                    if (t >= head && t < L) {
                        const float a = x[q].x * scale, b = x[q].y * scale;
                        if (t + 1 < L) {
                            if (pair_store) {
                                put2(icl, t, a, b);
                            } else {
                                put(icl, t, a);
                                put(icl, t + 1, b);
                            }
                        } else {
                            put(icl, t, a);
                        }
                    }
                }
            }
        }
    }
}

template <class IO, bool REV>
__global__ void direct_conv_kernel(const typename IO::T* __restrict__ v,
                                   const typename IO::T* __restrict__ g,
                                   typename IO::T* __restrict__ r, int64_t nch, int L)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nch * (int64_t)L) return;
    const int64_t c = idx / L;
    const int t = (int)(idx - c * L);
    const int64_t base = c * (int64_t)L;
    float acc = 0.f;
    for (int j = 0; j <= t; ++j)
        acc = __builtin_fmaf(IO::load(v, base + (REV ? L - 1 - j : j)), IO::load(g, base + t - j),
                             acc);
    IO::store(r, base + (REV ? L - 1 - t : t), acc);
}

template <int M, class IO, bool REV>
static hipError_t launch_fused_m(const void* v, const void* g, void* r, int64_t nch, int L,
                                 int head, bool pair, const float2* tw, hipStream_t stream)
{
    constexpr int CPW = (fused_threads<M>() / (M / 16)) / 2;
    const int64_t blocks = (nch + CPW - 1) / CPW;
    if (!grid_ok(blocks, fused_threads<M>())) return hipErrorInvalidValue;
    static int64_t resident[16];
    const int64_t pf = M >= 1024 ? resident_workgroups((const void*)fused_conv_kernel<M, IO, REV>,
                                                        fused_threads<M>(), resident) / 8 * 8
                                 : 0;
    hipLaunchKernelGGL((fused_conv_kernel<M, IO, REV>), dim3((unsigned)blocks), dim3(fused_threads<M>()), 0,
                       stream, (const typename IO::T*)v, (const typename IO::T*)g,
                       (typename IO::T*)r, nch, L, head, pair ? 1 : 0, tw, pf);
    return hipGetLastError();
}

template <class IO, bool REV>
static hipError_t launch_fused_io(const void* v, const void* g, void* r, int64_t nch, int L, int M,
                                  int head, bool pair, const float2* tw, hipStream_t s)
{
    switch (M) {
    case 64: return launch_fused_m<64, IO, REV>(v, g, r, nch, L, head, pair, tw, s);
    case 128: return launch_fused_m<128, IO, REV>(v, g, r, nch, L, head, pair, tw, s);
    case 256: return launch_fused_m<256, IO, REV>(v, g, r, nch, L, head, pair, tw, s);
    case 512: return launch_fused_m<512, IO, REV>(v, g, r, nch, L, head, pair, tw, s);
    case 1024: return launch_fused_m<1024, IO, REV>(v, g, r, nch, L, head, pair, tw, s);
    case 2048: return launch_fused_m<2048, IO, REV>(v, g, r, nch, L, head, pair, tw, s);
    case 4096: return launch_fused_m<4096, IO, REV>(v, g, r, nch, L, head, pair, tw, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fused(Store st, const void* v, const void* g, void* r, int64_t nch, int L, int M,
                        int head, bool pair_store, bool rev, const float2* tw, hipStream_t stream)
{
    if (st == Store::F32)
        return rev ? launch_fused_io<f32_io, true>(v, g, r, nch, L, M, head, pair_store, tw, stream)
                   : launch_fused_io<f32_io, false>(v, g, r, nch, L, M, head, pair_store, tw, stream);
    return rev ? launch_fused_io<bf16_io, true>(v, g, r, nch, L, M, head, pair_store, tw, stream)
               : launch_fused_io<bf16_io, false>(v, g, r, nch, L, M, head, pair_store, tw, stream);
}

template <bool REV>
static hipError_t launch_direct_rev(Store st, const void* v, const void* g, void* r, int64_t nch,
                                    int L, hipStream_t stream)
{
    const int64_t total = nch * (int64_t)L;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    if (!grid_ok(blocks, threads)) return hipErrorInvalidValue;
    if (st == Store::F32)
        hipLaunchKernelGGL((direct_conv_kernel<f32_io, REV>), dim3((unsigned)blocks), dim3(threads),
                           0, stream, (const float*)v, (const float*)g, (float*)r, nch, L);
    else
        hipLaunchKernelGGL((direct_conv_kernel<bf16_io, REV>), dim3((unsigned)blocks), dim3(threads),
                           0, stream, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)r, nch, L);
    return hipGetLastError();
}

hipError_t launch_direct(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                         bool rev, hipStream_t stream)
{
    return rev ? launch_direct_rev<true>(st, v, g, r, nch, L, stream)
               : launch_direct_rev<false>(st, v, g, r, nch, L, stream);
}

}  // namespace sc
