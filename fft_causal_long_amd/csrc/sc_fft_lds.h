// Length-Q DFTs held in registers and LDS by Q/16 threads of a workgroup (gfx950).
//
// Thread tau of a transform holds element tau + (Q/16)*r in register r (r < 16) at the
// input and the output of the transform.  Between radix-16 passes (Stockham, decimation in
// frequency) the values go through a padded LDS region of Q + Q/16 complex values.
// Twiddles come from the float twiddle bank (see sc_internal.h) through a raw buffer
// descriptor, so a load costs no vector ALU work for its address.
#pragma once

#include "sc_device.h"
#include "sc_internal.h"

namespace sc {

// one float2 of padding after every 16 keeps stride-16 LDS accesses conflict free
__device__ __forceinline__ int lds_pad(int a) { return a + (a >> 4); }

// Float twiddle bank (device constant table built by the host):
//   [0, 8192)                        W_8192^i
//   [8192 + (Q - 32) + k*(Q/16) + n] W_Q^{n k}, for each pass length Q = 32 .. 4096,
//                                    k < 16, n < Q/16  (row k contiguous in n)
// The pass tables make every twiddle load of a radix-16 pass a contiguous wave access.
constexpr int PASS_TW_BASE = FUSED_TW_N;

struct Bank {
    __amdgpu_buffer_rsrc_t rs;   // raw buffer over the whole bank, bounds-checked
    __device__ __forceinline__ float2 at(int voff_elems, int soff_elems) const
    {
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(rs, voff_elems * 8, soff_elems * 8, 0);
        return __builtin_bit_cast(float2, w);
    }
};

__device__ __forceinline__ Bank make_bank(const float2* tw)
{
    return Bank{__builtin_amdgcn_make_buffer_rsrc((void*)tw, (short)0, FUSED_BANK_FLOAT2 * 8,
                                                0x00020000)};
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

// One Stockham decimation-in-frequency pass of radix R over a length-M transform held by
// TB = M/16 threads.  Stage data: S sub-transforms of length Q = M/S, element (s, n) of
// sub-transform s at flat index s + S*n; thread tau holds flat index tau + TB*r in x[r].
// Butterfly "item" (s, n1), n1 < Q/R, combines elements (s, n1 + (Q/R) n2), n2 < R:
//   out[s + S*k2, n1] = W_Q^{n1 k2} * sum_{n2} in[s, n1 + (Q/R) n2] W_R^{n2 k2}
// which is written to flat index s + S*(k2 + R*n1).  Radix 16 is used while Q > 16, so a
// pass with twiddles has one item per thread (item = tau).  The last pass (Q == R) leaves
// the result in registers: x[r] = X[tau + TB*r], natural order.
template <int M, int R, int S, bool INV>
__device__ __forceinline__ void stockham_pass(float2 (&x)[16], float2* __restrict__ buf, int tau,
                                              const Bank& bank)
{
    constexpr int NB = 16 / R, Q = M / S, QN = Q / R;
    if constexpr (QN > 1) {
        static_assert(R == 16, "passes with twiddles are radix 16");
        const int s = tau & (S - 1), n1 = tau / S;
        float2 w[16];
#pragma unroll
        for (int k2 = 1; k2 < 16; ++k2) w[k2] = bank.at(n1, PASS_TW_BASE + (Q - 32) + k2 * (Q / 16));
        dft<16, INV>(x);
#pragma unroll
        for (int k2 = 1; k2 < 16; ++k2) x[k2] = cmul_dir<INV>(x[k2], w[k2]);
        // flat s + S*(k2 + 16 n1), padded: base + k2*STEP
        constexpr int STEP = S == 1 ? 1 : S + S / 16;
        const int base = S == 1 ? 17 * n1 : (s + (s >> 4)) + 16 * n1 * STEP;
#pragma unroll
        for (int k2 = 0; k2 < 16; ++k2) buf[base + k2 * STEP] = x[k2];
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

// All passes of a length-M DFT (radix 16 while possible, then the remainder).  Inactive
// threads only join the barriers.  On return every thread has passed a barrier that
// follows its last read of buf.
template <int M, bool INV, int S = 1>
__device__ __forceinline__ void fft_passes(float2 (&x)[16], float2* __restrict__ buf, int tau,
                                           const Bank& bank, bool active)
{
    constexpr int TB = M / 16, Q = M / S, R = Q >= 16 ? 16 : Q;
    if constexpr (Q / R > 1) {
        if (active) stockham_pass<M, R, S, INV>(x, buf, tau, bank);
        __syncthreads();
        if (active) {
#pragma unroll
            for (int q = 0; q < 16; ++q) x[q] = buf[reg_off<TB>(tau, q)];
        }
        __syncthreads();
        fft_passes<M, INV, S * R>(x, buf, tau, bank, active);
    } else {
        if (active) stockham_pass<M, R, S, INV>(x, buf, tau, bank);
    }
}

}  // namespace sc
