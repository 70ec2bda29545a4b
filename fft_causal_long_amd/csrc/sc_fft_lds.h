// Length-Q DFTs held in registers and LDS by the threads of a workgroup (gfx950).
//
// A transform is held by TB = Q/P threads with P = 16 (or 8) values each: thread tau holds
// element tau + TB*r in register r (r < P) at the input and the output of the transform.
// Between radix-P passes (Stockham, decimation in frequency) the values go through a padded
// LDS region of Q + Q/16 complex values.  Twiddles come from the float twiddle bank (see
// sc_internal.h) through a raw buffer descriptor, so a load costs no vector ALU work for
// its address, and every twiddle load of a pass is one contiguous wave access.
#pragma once

#include "sc_device.h"
#include "sc_internal.h"

namespace sc {

// one float2 of padding after every 16 keeps stride-16 LDS accesses conflict free
__device__ __forceinline__ int lds_pad(int a) { return a + (a >> 4); }

// Float twiddle bank (device constant table built by the host):
//   [0, 8192)                              W_8192^i
//   [PASS16_TW_BASE + (Q - 32) + k*(Q/16) + n]   W_Q^{n k}, Q = 32 .. 4096, k < 16, n < Q/16
//   [PASS8_TW_BASE  + (Q - 16) + k*(Q/8)  + n]   W_Q^{n k}, Q = 16 .. 4096, k < 8,  n < Q/8
constexpr int PASS16_TW_BASE = FUSED_TW_N;
constexpr int PASS8_TW_BASE = FUSED_TW_N + (2 * 4096 - 32);

struct Bank {
    __amdgpu_buffer_rsrc_t rs;   // raw buffer over the whole bank, bounds-checked
    int salt = 0;                // 0, but opaque to the compiler after reseed()
    __device__ __forceinline__ float2 at(int voff_elems, int soff_elems) const
    {
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(rs, voff_elems * 8,
                                                            soff_elems * 8 + salt, 0);
        return __builtin_bit_cast(float2, w);
    }
    // Loads issued after this cannot be merged with, or hoisted above, earlier identical
    // loads: a loop that repeats a transform reloads its twiddles instead of keeping every
    // twiddle of every pass live in registers across iterations.
    __device__ __forceinline__ void reseed()
    {
        int z = 0;
        asm volatile("" : "+s"(z));
        salt = z;
    }
};

__device__ __forceinline__ Bank make_bank(const float2* tw)
{
    return Bank{__builtin_amdgcn_make_buffer_rsrc((void*)tw, (short)0, FUSED_BANK_FLOAT2 * 8,
                                                0x00020000), 0};
}

// W_n^e for a power of two n dividing 8192 (conj when INV)
template <bool INV>
__device__ __forceinline__ float2 tw_get(const Bank& b, int n, int e)
{
    const float2 w = b.at((e & (n - 1)) * (FUSED_TW_N / n), 0);
    return INV ? conjf2(w) : w;
}

// LDS offset of flat element tau + TB*q (register q of thread tau)
template <int TB>
__device__ __forceinline__ int reg_off(int tau, int q)
{
    if constexpr (TB % 16 == 0) return tau + (tau >> 4) + q * (TB + TB / 16);
    else return lds_pad(tau + TB * q);
}

// One Stockham decimation-in-frequency pass of radix R over a length-Q transform held by
// TB = Q/P threads.  Stage data: S sub-transforms of length Qs = Q/S, element (s, n) of
// sub-transform s at flat index s + S*n; thread tau holds flat index tau + TB*r in x[r].
// Butterfly "item" (s, n1), n1 < Qs/R, combines elements (s, n1 + (Qs/R) n2), n2 < R:
//   out[s + S*k2, n1] = W_Qs^{n1 k2} * sum_{n2} in[s, n1 + (Qs/R) n2] W_R^{n2 k2}
// which is written to flat index s + S*(k2 + R*n1).  Radix P is used while Qs > P, so a
// pass with twiddles has one item per thread (item = tau).  The last pass (Qs == R) leaves
// the result in registers: x[r] = X[tau + TB*r], natural order.
template <int Q, int R, int S, bool INV, int P>
__device__ __forceinline__ void stockham_pass(float2 (&x)[P], float2* __restrict__ buf, int tau,
                                              const Bank& bank)
{
    constexpr int NB = P / R, Qs = Q / S, QN = Qs / R;
    if constexpr (QN > 1) {
        static_assert(R == P, "passes with twiddles use the full radix");
        const int s = tau & (S - 1), n1 = tau / S;
        constexpr int TBASE = P == 16 ? PASS16_TW_BASE + (Qs - 32) : PASS8_TW_BASE + (Qs - 16);
        float2 w[P];
#pragma unroll
        for (int k2 = 1; k2 < P; ++k2) w[k2] = bank.at(n1, TBASE + k2 * (Qs / P));
        dft<P, INV>(x);
#pragma unroll
        for (int k2 = 1; k2 < P; ++k2) x[k2] = cmul_dir<INV>(x[k2], w[k2]);
        // padded flat index s + S*(k2 + P*n1) = base + off(k2)
        if constexpr (S == 1) {
            // (k2 + P n1) >> 4 == (P n1) >> 4 because k2 < P <= 16 and P n1 is a multiple of P
            const int base = P * n1 + ((P * n1) >> 4);
#pragma unroll
            for (int k2 = 0; k2 < P; ++k2) buf[base + k2] = x[k2];
        } else if constexpr (S % 16 == 0) {
            constexpr int STEP = S + S / 16;
            const int base = (s + (s >> 4)) + P * n1 * STEP;
#pragma unroll
            for (int k2 = 0; k2 < P; ++k2) buf[base + k2 * STEP] = x[k2];
        } else {
            static_assert(S == 8 && P == 8, "S = 8 occurs only for radix 8");
            // s < 8: (s + 8 k2 + 64 n1) >> 4 == (k2 >> 1) + 4 n1
            const int base = s + 68 * n1;
#pragma unroll
            for (int k2 = 0; k2 < P; ++k2) buf[base + 8 * k2 + (k2 >> 1)] = x[k2];
        }
    } else {
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            float2 b[R];
#pragma unroll
            for (int n2 = 0; n2 < R; ++n2) b[n2] = x[q + NB * n2];
            dft<R, INV>(b);
#pragma unroll
            for (int k2 = 0; k2 < R; ++k2) x[q + NB * k2] = b[k2];
        }
    }
}

// All passes of a length-Q DFT held with P values per thread (radix P while possible,
// then the remainder).  Inactive threads only join the barriers.  On return every thread
// has passed a barrier that follows its last read of buf.
template <int Q, bool INV, int S = 1, int P = 16>
__device__ __forceinline__ void fft_passes(float2 (&x)[P], float2* __restrict__ buf, int tau,
                                           const Bank& bank, bool active)
{
    constexpr int TB = Q / P, Qs = Q / S, R = Qs >= P ? P : Qs;
    if constexpr (Qs / R > 1) {
        if (active) stockham_pass<Q, R, S, INV, P>(x, buf, tau, bank);
        __syncthreads();
        if (active) {
#pragma unroll
            for (int q = 0; q < P; ++q) x[q] = buf[reg_off<TB>(tau, q)];
        }
        __syncthreads();
        fft_passes<Q, INV, S * R, P>(x, buf, tau, bank, active);
    } else {
        if (active) stockham_pass<Q, R, S, INV, P>(x, buf, tau, bank);
    }
}

// From the branch spectra u0[j] = Z_{2j}, u1[j] = Z_{2j+1} (natural order, padded) form
// Y_k and Y_{M-k} of the real-output inverse, both scaled by 8 (constants folded later).
template <int M>
__device__ __forceinline__ void unpack_pair(int k, const float2* __restrict__ u0,
                                            const float2* __restrict__ u1, const Bank& bank,
                                            float2& yk, float2& ymk)
{
    constexpr int N = 2 * M;
    const int b = k & 1, j = k >> 1;
    const float2* u = b ? u1 : u0;
    // bins k, N-k, M-k, M+k of Z
    const float2 p1 = u[lds_pad(j)];
    const float2 q1 = conjf2(u[lds_pad((M - j - b) & (M - 1))]);
    const float2 p2 = u[lds_pad((M / 2 - j - b) & (M - 1))];
    const float2 q2 = conjf2(u[lds_pad(M / 2 + j)]);
    // 4 X = 4 V G = -i (P + Q)(P - Q)
    const float2 s1 = cadd(p1, q1), d1 = csub(p1, q1);
    const float2 s2 = cadd(p2, q2), d2 = csub(p2, q2);
    const float2 x1 = make_float2(__builtin_fmaf(s1.x, d1.y, s1.y * d1.x),
                                  __builtin_fmaf(s1.y, d1.y, -s1.x * d1.x));   // 4 X_k
    const float2 x2 = make_float2(__builtin_fmaf(s2.x, d2.y, s2.y * d2.x),
                                  __builtin_fmaf(s2.y, d2.y, -s2.x * d2.x));   // 4 X_{M-k}
    // S = X_k + X_{k+M}, D = X_k - X_{k+M} with X_{k+M} = conj X_{M-k}
    const float2 sm = make_float2(x1.x + x2.x, x1.y - x2.y);
    const float2 df = make_float2(x1.x - x2.x, x1.y + x2.y);
    const float2 t = cmulc(df, tw_get<false>(bank, N, k));        // W_N^{-k} D
    // Y_k = S + i T,  Y_{M-k} = conj(S - i T)
    yk = make_float2(sm.x - t.y, sm.y + t.x);
    ymk = make_float2(sm.x + t.y, t.x - sm.y);
}

constexpr int HEAD_MAX = 64;   // largest direct head (the host clamps to this)

// Direct fp32 head r_t = sum_{j<=t} v_j g_{t-j}, t < head, of ncl channels whose first
// HEAD_MAX inputs are staged in hb (v then g per channel), by NT threads lt = 0..NT-1 made
// of whole waves.  Each output's sum is split over S consecutive lanes (terms j = s, s + S,
// ...; S <= 8, as many as the threads allow) and reduced with lane shuffles, so the head
// costs a few dependent steps instead of up to HEAD_MAX.
template <int NT, class Put>
__device__ __forceinline__ void direct_head(const float* __restrict__ hb, int ncl, int nvalid,
                                            int L, int head, int lt, const Put& put)
{
    const int nout = ncl * head;
    int S = 1;
    while (S < 8 && 2 * S * nout <= NT) S *= 2;
    for (int base = 0; base < nout * S; base += NT) {
        const int idx = base + lt, o = idx / S, s = idx - o * S;
        const int c2 = o / head, t = o - c2 * head;
        float acc = 0.f;
        if (o < nout) {
            const float* hv = hb + c2 * 2 * HEAD_MAX;
            const float* hg = hv + HEAD_MAX;
            for (int j = s; j <= t; j += S) acc = __builtin_fmaf(hv[j], hg[t - j], acc);
        }
        for (int d = 1; d < S; d <<= 1) acc += __shfl_xor(acc, d);
        if (o < nout && s == 0 && c2 < nvalid && t < L) put(c2, t, acc);
    }
}

// REV (the gradient kernels): the first input is read reversed and the output is written
// reversed, which turns the causal convolution into the correlation of the backward pass:
// rev(causal(rev(dr), b))_j = sum_{t>=j} dr_t b_{t-j}.

// Bring element range [first, first + count) of v and of g into the cache: thread i touches
// the 128-byte line i of each (lines past the range read nothing; the caller covers the range
// with its threads).  The two words come back unused: hand them to keep_touched() after the
// thread's last barrier and load wait, since using them waits for the loads and vector-memory
// waits are in order.
template <class T>
__device__ __forceinline__ uint2 touch_line(const T* v, const T* g, int64_t first, int64_t count,
                                            int i)
{
    const Span sv = make_span(v, first, count), sg = make_span(g, first, count);
    return make_uint2(__builtin_amdgcn_raw_buffer_load_b32(sv.rs, i * 128, 0, 0),
                      __builtin_amdgcn_raw_buffer_load_b32(sg.rs, i * 128, 0, 0));
}
// Keeps the touched words alive behind a condition that is false for every pf >= 0 the host
// passes, so the compiler neither removes the loads nor waits for them earlier.
__device__ __forceinline__ void keep_touched(uint2 w, int64_t pf, const Span& dst)
{
    if (pf < 0) __builtin_amdgcn_raw_buffer_store_b32(w.x ^ w.y, dst.rs, 0, 0, 0);
}

}  // namespace sc
