// Four-step (HBM-staged) causal long convolution for 4096 < L (gfx950).
//
// Same method as the fused kernel ("Caracal: Causal Architecture via Spectral Mixing", key
// designs 1 and 2: pad to N = 2M, FFT, multiply, inverse FFT, truncate), with the same
// reductions: z = v + i g packed into one complex sequence, the zero upper half turned
// into two length-M branch transforms U^b = DFT_M(z_n W_N^{b n}), the spectral product
// and the real-output inverse formed from bin quadruples.  When 2M complex values no
// longer fit the LDS of one CU, each length-M transform is split as M = M1 * M2:
//
//   U_{M1 k1 + k2} = sum_{n1<M2} W_M2^{n1 k1} [ W_M^{n1 k2} sum_{n2<M1} u_{n1 + M2 n2} W_M1^{n2 k2} ]
//
//  kernel A (columns): for every column n1 the length-M1 DFT over n2, times W_M^{n1 k2},
//     stored as T^b[k2][n1] (both branches, z read once).
//  kernel B (rows): the length-M2 DFT of rows k2 and of the mirror row M1 - k2 - b, which
//     hold every bin of the quadruples {j, M-j-b, M/2-j-b, M/2+j}; the product and the
//     real-output inverse spectrum Y^b_i = Y_{2i+b} (i = M1 i1 + i2, row i2 of length
//     M2/2); the length-M2/2 inverse DFT of each Y row and the twiddle W_{M/2}^{-m1 i2},
//     stored as S^b[i2][m1].
//  kernel C (columns): the length-M1 inverse DFT over i2 gives e (b = 0) and o (b = 1) at
//     m = m1 + (M2/2) m2; y_m = (e_m + W_M^{-m} o_m) / (8M) = x_{2m} + i x_{2m+1}.
//  A small kernel recomputes the first `head` outputs by direct fp32 summation.
//
// HBM traffic per channel: read v, g; write and read T (2M complex) and S (M complex);
// write r.  Channels are processed in chunks so T and S can stay in the last-level cache;
// the chunks can alternate between two streams, so that the memory-bound column kernels of
// one overlap the row kernel of the other.
// Every twiddle comes from a per-M table (see FsTw in sc_internal.h) laid out so that the
// lanes of a wave read consecutive entries.

#include "sc_device.h"
#include "sc_fft_lds.h"
#include "sc_internal.h"

namespace sc {


// ---------------------------------------------------------------- kernel A: columns, forward

// REV (the gradient kernels): v is read reversed here and the output is written reversed by
// kernel C and the head kernel: rev(causal(rev(dr), b))_j = sum_{t>=j} dr_t b_{t-j}.
template <int M1, class IO, bool REV>
__global__ __launch_bounds__(512) void fs_columns_fwd(const typename IO::T* __restrict__ v,
                                                      const typename IO::T* __restrict__ g,
                                                      float2* __restrict__ T, int64_t ch_begin,
                                                      int L, int M2, const float2* __restrict__ bankp,
                                                      FsTw tw)
{
    constexpr int TQ = M1 / 16, NCOL = 256 / TQ, CREG = M1 + M1 / 16 + 1;
    __shared__ float2 lds[2 * NCOL * CREG];
    const Bank bank = make_bank(bankp);
    const int tid = threadIdx.x, beta = tid >> 8, t = tid & 255;
    const int c = t % NCOL, tau = t / NCOL;
    const int tiles = M2 / NCOL;
    const int chl = blockIdx.x / tiles;
    const int n1 = (blockIdx.x - chl * tiles) * NCOL + c;
    // this channel's inputs; positions n >= L (the padding inside M) read as 0
    const Span vs = make_span(v, (ch_begin + chl) * (int64_t)L, L);
    const Span gs = make_span(g, (ch_begin + chl) * (int64_t)L, L);

    // all 32 input loads first, then (branch 1) the 16 twiddles W_N^n together: a multiply
    // under the branch inside the load loop made each element wait for its own loads
    float2 x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int n = n1 + M2 * (tau + TQ * q);
        const int nv = REV ? (n < L ? L - 1 - n : IO::OOB) : n;
        x[q] = make_float2(IO::load(vs, nv), IO::load(gs, n));
    }
    if (beta) {
        float2 w[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) w[q] = tw.tn[n1 + M2 * (tau + TQ * q)];
#pragma unroll
        for (int q = 0; q < 16; ++q) x[q] = cmul(x[q], w[q]);
    }
    fft_passes<M1, false>(x, lds + (beta * NCOL + c) * CREG, tau, bank, true);
    // x[q] = column output k2 = tau + TQ q; times W_M^{n1 k2}
    float2* out = T + (int64_t)(chl * 2 + beta) * M1 * M2;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int k2 = tau + TQ * q;
        out[(int64_t)k2 * M2 + n1] = cmul(x[q], tw.ta[(int64_t)k2 * M2 + n1]);
    }
}

// ---------------------------------------------------------------- kernel B: rows

// Bins of the quadruple of item (row rho, column k1): U[row][col] through `at`.
// Returns Y_j and Y_{partner}, both scaled by 8 like the fused kernel.
template <class At>
__device__ __forceinline__ void fs_unpack(int rho, int k1, int beta, int M1, int M2, int M,
                                          const At& at, const FsTw& tw, float2& yj, float2& yp)
{
    const bool zero = rho + beta == 0;
    const int prow = zero ? 0 : M1 - rho - beta;
    const float2 p1 = at(rho, k1);
    const float2 q1 = conjf2(at(prow, zero ? (M2 - k1) & (M2 - 1) : M2 - 1 - k1));
    const float2 p2 = at(prow, zero ? M2 / 2 - k1 : M2 / 2 - 1 - k1);
    const float2 q2 = conjf2(at(rho, M2 / 2 + k1));
    const float2 s1 = cadd(p1, q1), d1 = csub(p1, q1);
    const float2 s2 = cadd(p2, q2), d2 = csub(p2, q2);
    const float2 x1 = make_float2(__builtin_fmaf(s1.x, d1.y, s1.y * d1.x),
                                  __builtin_fmaf(s1.y, d1.y, -s1.x * d1.x));
    const float2 x2 = make_float2(__builtin_fmaf(s2.x, d2.y, s2.y * d2.x),
                                  __builtin_fmaf(s2.y, d2.y, -s2.x * d2.x));
    const float2 sm = make_float2(x1.x + x2.x, x1.y - x2.y);
    const float2 df = make_float2(x1.x - x2.x, x1.y + x2.y);
    // W_N^{-k} D with k = 2 (M1 k1 + rho) + b
    const float2 t = cmulc(df, tw.tu[(int64_t)(2 * rho + beta) * (M2 / 4 + 1) + k1]);
    yj = make_float2(sm.x - t.y, sm.y + t.x);
    yp = make_float2(sm.x + t.y, t.x - sm.y);
    (void)M;
}

template <int M2>
__global__ __launch_bounds__(512) void fs_rows(const float2* __restrict__ T, float2* __restrict__ S,
                                               int M1, const float2* __restrict__ bankp, FsTw tw)
{
    constexpr int TR = M2 / 16, PAIRS = (2048 / M2) > 1 ? 2048 / M2 : 1;
    constexpr int RREG = M2 + M2 / 16 + 1, H = M2 / 2;
    __shared__ float2 lds[PAIRS * 2 * RREG];
    const Bank bank = make_bank(bankp);
    const int M = M1 * M2;
    const int groups = (M1 / 2) / PAIRS;                 // slot groups per branch
    const int chl = blockIdx.x / (2 * groups);
    const int rem = blockIdx.x - chl * 2 * groups;
    const int beta = rem / groups;
    const int tid = threadIdx.x;
    const int pl = tid / (2 * TR), side = (tid / TR) & 1, tau = tid % TR;
    const int slot = (rem - beta * groups) * PAIRS + pl;
    const int ra = slot, rb = (beta == 0 && slot == 0) ? M1 / 2 : M1 - slot - beta;
    const int row = side ? rb : ra;
    float2* bufa = lds + (pl * 2) * RREG;
    float2* bufb = bufa + RREG;
    float2* mybuf = side ? bufb : bufa;

    // row DFT of length M2: x[q] = U_{M1 k1 + row}, k1 = tau + TR q
    const float2* in = T + ((int64_t)(chl * 2 + beta) * M1 + row) * M2;
    float2 x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) x[q] = in[tau + TR * q];
    fft_passes<M2, false>(x, mybuf, tau, bank, true);
#pragma unroll
    for (int q = 0; q < 16; ++q) mybuf[reg_off<TR>(tau, q)] = x[q];
    __syncthreads();

    // quadruple unpack: items (row, k1 < M2/4) of both rows of the slot, 4 per thread
    auto at = [&](int r_, int c_) { return (r_ == ra ? bufa : bufb)[lds_pad(c_)]; };
    const int lt = tid - pl * 2 * TR;
    float2 yj[4], yp[4];
    int rowj[4], colj[4], rowp[4], colp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int item = lt + 2 * TR * i;
        const int rsel = item / (M2 / 4), k1 = item - rsel * (M2 / 4);
        const int rho = rsel ? rb : ra;
        fs_unpack(rho, k1, beta, M1, M2, M, at, tw, yj[i], yp[i]);
        rowj[i] = rho;
        colj[i] = k1;
        if (rho + beta == 0) {
            rowp[i] = 0;
            colp[i] = H - k1;
            if (k1 == 0) {            // Y_M is absent: take Y_{M/2} (j = M/4, row 0)
                float2 unused;
                fs_unpack(0, M2 / 4, 0, M1, M2, M, at, tw, yp[i], unused);
                colp[i] = H / 2;
            }
        } else {
            rowp[i] = M1 - rho - beta;
            colp[i] = H - 1 - k1;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        (rowj[i] == ra ? bufa : bufb)[lds_pad(colj[i])] = yj[i];
        (rowp[i] == ra ? bufa : bufb)[lds_pad(colp[i])] = yp[i];
    }
    __syncthreads();

    // row inverse DFT of length H, 8 values per thread (H/8 = TR threads per row)
    float2 y8[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) y8[q] = mybuf[reg_off<TR>(tau, q)];
    __syncthreads();
    fft_passes<H, true, 1, 8>(y8, mybuf, tau, bank, true);
    float2* out = S + ((int64_t)(chl * 2 + beta) * M1 + row) * H;
    const float2* twr = tw.tb + (int64_t)row * H;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int m1 = tau + TR * q;
        out[m1] = cmulc(y8[q], twr[m1]);             // W_{M/2}^{-m1 row}
    }
}

// ---------------------------------------------------------------- kernel C: columns, inverse

template <int M1, class IO, bool REV>
__global__ __launch_bounds__(512) void fs_columns_inv(const float2* __restrict__ S,
                                                      typename IO::T* __restrict__ r,
                                                      int64_t ch_begin, int L, int M2, int head,
                                                      int pair_store,
                                                      const float2* __restrict__ bankp, FsTw tw)
{
    constexpr int TQ = M1 / 16, NCOL = 256 / TQ, CREG = M1 + M1 / 16 + 1;
    __shared__ float2 lds[2 * NCOL * CREG];
    const Bank bank = make_bank(bankp);
    const int H = M2 / 2, M = M1 * M2;
    const int tid = threadIdx.x, beta = tid >> 8, t = tid & 255;
    const int c = t % NCOL, tau = t / NCOL;
    const int tiles = (H + NCOL - 1) / NCOL;
    const int chl = blockIdx.x / tiles;
    const int m1 = (blockIdx.x - chl * tiles) * NCOL + c;
    const bool col_ok = m1 < H;
    const float2* in = S + (int64_t)(chl * 2 + beta) * M1 * H;

    float2 x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
        x[q] = col_ok ? in[(int64_t)(tau + TQ * q) * H + m1] : make_float2(0.f, 0.f);
    float2* mybuf = lds + (beta * NCOL + c) * CREG;
    fft_passes<M1, true>(x, mybuf, tau, bank, true);
    // x[q] = e (beta 0) or o (beta 1) at m = m1 + H m2, m2 = tau + TQ q
    if (beta) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int m = m1 + H * (tau + TQ * q);
            mybuf[reg_off<TQ>(tau, q)] = cmulc(x[q], tw.tn[2 * m]);   // W_M^{-m} o_m
        }
    }
    __syncthreads();
    if (!beta && col_ok) {
        const float2* obuf = lds + (NCOL + c) * CREG;
        const float scale = 1.0f / (8.0f * (float)M);
        const Span rs = make_span(r, (ch_begin + chl) * (int64_t)L, L);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int m = m1 + H * (tau + TQ * q);
            const int tt = 2 * m;
            if (tt < head || tt >= L) continue;
            const float2 o = obuf[reg_off<TQ>(tau, q)];
            const float a = (x[q].x + o.x) * scale, b = (x[q].y + o.y) * scale;
            // outputs tt, tt+1 (at L-1-tt, L-2-tt when REV; pairs need L even)
            if (tt + 1 < L) {
                if (pair_store) {
                    if (REV) IO::store2(rs, L - 2 - tt, b, a);
                    else IO::store2(rs, tt, a, b);
                } else {
                    IO::store(rs, REV ? L - 1 - tt : tt, a);
                    IO::store(rs, REV ? L - 2 - tt : tt + 1, b);
                }
            } else {
                IO::store(rs, REV ? L - 1 - tt : tt, a);
            }
        }
    }
}

// ---------------------------------------------------------------- direct head

template <class IO, bool REV>
__global__ void head_kernel(const typename IO::T* __restrict__ v, const typename IO::T* __restrict__ g,
                            typename IO::T* __restrict__ r, int64_t nch, int L, int head)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t c = idx / head;
    const int t = (int)(idx - c * head);
    if (c >= nch || t >= L) return;
    const int64_t base = c * (int64_t)L;
    float acc = 0.f;
    for (int j = 0; j <= t; ++j)
        acc = __builtin_fmaf(IO::load(v, base + (REV ? L - 1 - j : j)), IO::load(g, base + t - j),
                             acc);
    IO::store(r, base + (REV ? L - 1 - t : t), acc);
}

// ---------------------------------------------------------------- launch

template <class IO, bool REV, int M1>
static hipError_t launch_cols(bool fwd, const void* v, const void* g, void* r, float2* T,
                              const float2* S, int64_t c0, int nc, int L, int M2, int head,
                              bool pair, const float2* bank, const FsTw& tw, hipStream_t s)
{
    constexpr int NCOL = 256 / (M1 / 16);
    if (fwd) {
        const int64_t blocks = (int64_t)nc * (M2 / NCOL);
        if (!grid_ok(blocks, 512)) return hipErrorInvalidValue;
        hipLaunchKernelGGL((fs_columns_fwd<M1, IO, REV>), dim3((unsigned)blocks), dim3(512), 0, s,
                           (const typename IO::T*)v, (const typename IO::T*)g, T, c0, L, M2, bank,
                           tw);
    } else {
        const int H = M2 / 2;
        const int64_t blocks = (int64_t)nc * ((H + NCOL - 1) / NCOL);
        if (!grid_ok(blocks, 512)) return hipErrorInvalidValue;
        hipLaunchKernelGGL((fs_columns_inv<M1, IO, REV>), dim3((unsigned)blocks), dim3(512), 0, s, S,
                           (typename IO::T*)r, c0, L, M2, head, pair ? 1 : 0, bank, tw);
    }
    return hipGetLastError();
}

template <class IO, bool REV>
static hipError_t dispatch_cols(bool fwd, int M1, const void* v, const void* g, void* r, float2* T,
                                const float2* S, int64_t c0, int nc, int L, int M2, int head,
                                bool pair, const float2* bank, const FsTw& tw, hipStream_t s)
{
    switch (M1) {
    case 64: return launch_cols<IO, REV, 64>(fwd, v, g, r, T, S, c0, nc, L, M2, head, pair, bank, tw, s);
    case 128: return launch_cols<IO, REV, 128>(fwd, v, g, r, T, S, c0, nc, L, M2, head, pair, bank, tw, s);
    case 256: return launch_cols<IO, REV, 256>(fwd, v, g, r, T, S, c0, nc, L, M2, head, pair, bank, tw, s);
    case 512: return launch_cols<IO, REV, 512>(fwd, v, g, r, T, S, c0, nc, L, M2, head, pair, bank, tw, s);
    case 1024: return launch_cols<IO, REV, 1024>(fwd, v, g, r, T, S, c0, nc, L, M2, head, pair, bank, tw, s);
    default: return hipErrorInvalidValue;
    }
}

template <int M2>
static hipError_t launch_rows(const float2* T, float2* S, int nc, int M1, const float2* bank,
                              const FsTw& tw, hipStream_t s)
{
    constexpr int TR = M2 / 16, PAIRS = (2048 / M2) > 1 ? 2048 / M2 : 1;
    const int64_t blocks = (int64_t)nc * 2 * ((M1 / 2) / PAIRS);
    if (!grid_ok(blocks, PAIRS * 2 * TR)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fs_rows<M2>), dim3((unsigned)blocks), dim3(PAIRS * 2 * TR), 0, s, T, S, M1,
                       bank, tw);
    return hipGetLastError();
}

static hipError_t dispatch_rows(int M2, const float2* T, float2* S, int nc, int M1,
                                const float2* bank, const FsTw& tw, hipStream_t s)
{
    switch (M2) {
    case 64: return launch_rows<64>(T, S, nc, M1, bank, tw, s);
    case 128: return launch_rows<128>(T, S, nc, M1, bank, tw, s);
    case 256: return launch_rows<256>(T, S, nc, M1, bank, tw, s);
    case 512: return launch_rows<512>(T, S, nc, M1, bank, tw, s);
    case 1024: return launch_rows<1024>(T, S, nc, M1, bank, tw, s);
    case 2048: return launch_rows<2048>(T, S, nc, M1, bank, tw, s);
    case 4096: return launch_rows<4096>(T, S, nc, M1, bank, tw, s);
    default: return hipErrorInvalidValue;
    }
}

void fourstep_split(int M, int* M1, int* M2)
{
    int m1 = M / FOURSTEP_MAX_ROW;
    if (m1 < 64) m1 = 64;
    *M1 = m1;
    *M2 = M / m1;
}

size_t fourstep_bytes_per_channel(int M)
{
    // T: 2 branches x M complex; S: 2 branches x M/2 complex
    return (size_t)3 * (size_t)M * sizeof(float2);
}

template <bool REV>
static hipError_t launch_fourstep_rev(Store st, const void* v, const void* g, void* r, int64_t nch,
                                      int L, int M, int head, bool pair_store, const float2* bank,
                                      const FsTw& tw, void* ws, size_t ws_bytes, int64_t chunk,
                                      hipStream_t stream, hipStream_t side, hipEvent_t fork,
                                      hipEvent_t join)
{
    int M1, M2;
    fourstep_split(M, &M1, &M2);
    const int64_t part = side ? (chunk / 2 > 0 ? chunk / 2 : 1) : chunk;
    hipError_t e = hipSuccess;
    if (side) {
        e = hipEventRecord(fork, stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(side, fork, 0);
        if (e != hipSuccess) return e;
    }
    // part i on stream (i even) or side (i odd), with its own scratch: T (2 branches x M
    // complex per channel), then S (2 branches x M/2)
    int64_t i = 0;
    for (int64_t c0 = 0; c0 < nch && e == hipSuccess; c0 += part, ++i) {
        const int nc = (int)((nch - c0) < part ? (nch - c0) : part);
        // one stream: every part on `stream`, all in the first `chunk` channels of scratch
        const int half = side ? (int)(i & 1) : 0;
        const hipStream_t s = half ? side : stream;
        float2* T = (float2*)ws + (size_t)half * (size_t)part * 3 * M;
        float2* S = T + (size_t)part * 2 * M;
        if ((size_t)(half + 1) * (size_t)part * fourstep_bytes_per_channel(M) > ws_bytes) {
            e = hipErrorInvalidValue;
            break;
        }
        if (st == Store::F32)
            e = dispatch_cols<f32_io, REV>(true, M1, v, g, r, T, S, c0, nc, L, M2, head, pair_store,
                                           bank, tw, s);
        else
            e = dispatch_cols<bf16_io, REV>(true, M1, v, g, r, T, S, c0, nc, L, M2, head,
                                            pair_store, bank, tw, s);
        if (e != hipSuccess) break;
        e = dispatch_rows(M2, T, S, nc, M1, bank, tw, s);
        if (e != hipSuccess) break;
        if (st == Store::F32)
            e = dispatch_cols<f32_io, REV>(false, M1, v, g, r, T, S, c0, nc, L, M2, head,
                                           pair_store, bank, tw, s);
        else
            e = dispatch_cols<bf16_io, REV>(false, M1, v, g, r, T, S, c0, nc, L, M2, head,
                                            pair_store, bank, tw, s);
    }
    if (side) {
        // join even after a failed launch, so that nothing of this call is left unordered
        hipError_t ej = hipEventRecord(join, side);
        if (ej == hipSuccess) ej = hipStreamWaitEvent(stream, join, 0);
        if (e == hipSuccess) e = ej;
    }
    if (e != hipSuccess) return e;
    if (head > 0) {
        const int64_t total = nch * (int64_t)head;
        const int threads = 256;
        const int64_t blocks = (total + threads - 1) / threads;
        if (!grid_ok(blocks, threads)) return hipErrorInvalidValue;
        if (st == Store::F32)
            hipLaunchKernelGGL((head_kernel<f32_io, REV>), dim3((unsigned)blocks), dim3(threads), 0,
                               stream, (const float*)v, (const float*)g, (float*)r, nch, L, head);
        else
            hipLaunchKernelGGL((head_kernel<bf16_io, REV>), dim3((unsigned)blocks), dim3(threads), 0,
                               stream, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)r, nch, L,
                               head);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_fourstep(Store st, const void* v, const void* g, void* r, int64_t nch, int L,
                           int M, int head, bool pair_store, bool rev, const float2* bank,
                           const FsTw& tw, void* ws, size_t ws_bytes, int64_t chunk,
                           hipStream_t stream, hipStream_t side, hipEvent_t fork, hipEvent_t join)
{
    return rev ? launch_fourstep_rev<true>(st, v, g, r, nch, L, M, head, pair_store, bank, tw, ws,
                                           ws_bytes, chunk, stream, side, fork, join)
               : launch_fourstep_rev<false>(st, v, g, r, nch, L, M, head, pair_store, bank, tw, ws,
                                            ws_bytes, chunk, stream, side, fork, join);
}

}  // namespace sc
