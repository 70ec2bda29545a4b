// Exact causal convolution through a number-theoretic transform whose stages are integer
// matrix products on the int8 matrix cores (gfx950), L <= 4096.
//
// "Catastrophic Token Leakage in Convolutional Sequence Modeling and How to Mitigate It"
// (abstract) proposes an FFT on 32-bit integers built from standard integer matrix
// multiplications; this kernel is that formulation on MI355X, for the same operation and
// the same result bits as the butterfly kernel (sc_ntt.hip): the pad-to-2L recipe of
// "Caracal: Causal Architecture via Spectral Mixing" (key designs 1 and 2) in Z_p,
// p = 998244353, omega_n = 3^((p-1)/n).
//
// Per channel (N = 2M, M = 64 * M2, the upper half of the padded inputs zero) the two
// "branches" b = 0, 1 are u^b_n = a_n omega_N^{b n}; V^b = NTT_M(u^b(v)), G^b likewise;
// X^b = V^b G^b N^{-1}; e^b = INTT_M(X^b) (unnormalised); x_n = e^0_n + omega_N^{-n} e^1_n,
// lifted to the balanced residue.  Each length-M transform is a four-step split held as a
// 64 x M2 matrix (element n = M2 n1 + n2 at row n1, column n2):
//   stage 1:  B[k1][n2] = sum_{n1} F64[k1][n1] a[n1][n2]        (left product, K = n1)
//   twiddle:  B[k1][n2] *= omega_M^{n2 k1}
//   stage 2:  A[k1][k2] = sum_{n2} B[k1][n2] F_M2[n2][k2]      (right product, K = n2)
// which leaves A_k at row k1, column k2 for k = k1 + 64 k2; the inverse takes that layout
// back to natural order with the conjugate matrices (right product by F_M2^{-1}, twiddle
// omega_M^{-m2 k1}, left product by F64^{-1}).  F_M2 is zero-padded to 64 x 64.
//
// Integer products.  The matrix-core operation is int8 x int8 with int32 sums, so both
// operands are split into bytes:
//  * data: a residue x in [0, p) is an unsigned 32-bit word; its bytes XOR 0x80 are signed
//    digits s_b = u_b - 128 with x = sum_b s_b 256^b + K0, K0 = 128 * 0x01010101;
//  * matrices: F^(b) = 256^b F mod p (precomputed) in balanced signed base-256 digits
//    F^(b) = sum_a f^(b)_a 256^a, |f| <= 128.
// Then sum_n F[k][n] x_n = sum_a 256^a P_a + K0 R_k (mod p) with the 4 accumulators
// P_a = sum_b sum_n f^(b)_a[k][n] s_{n,b} (|P_a| < 2^22, 16 matrix products per 16 x 16
// tile) and R_k the row sum of F (64 or M2 at k = 0, else 0).  sum_a 256^a P_a < 2^47 is
// formed exactly in float64 and reduced mod p with the exact fp64 remainder of the
// butterfly kernel.
//
// Workgroup: 4 waves, one channel.  Wave w owns block w (16 rows or columns) in every stage
// and holds that block of the stage's matrix digits in registers (16 x 16 bytes per lane)
// while it loops over the other dimension's blocks.  Two 64 x 65-word LDS matrices (a row
// padded by one word) hold the data between stages.

#include "sc_device.h"
#include "sc_internal.h"

namespace sc {

namespace nttm {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr double P = 998244353.0;
constexpr double PINV = 1.0 / 998244353.0;
constexpr double SHIFT = 6755399441055744.0;   // 1.5 * 2^52: x + SHIFT - SHIFT = round(x)
constexpr int ROW = 65;                        // LDS row stride in words
constexpr uint32_t FLIP = 0x80808080u;
// K0 = 128 * (1 + 2^8 + 2^16 + 2^24) mod p
constexpr double K0P = (double)((128ull * 0x01010101ull) % 998244353ull);

// a mod p into [-p/2, p/2] (up to one p at the edges), |a| < 2^51
__device__ __forceinline__ double reduce(double a)
{
    const double q = __builtin_fma(a, PINV, SHIFT) - SHIFT;
    return __builtin_fma(-q, P, a);
}
// [-p, p) -> [0, p)
__device__ __forceinline__ double nonneg(double a) { return a < 0.0 ? a + P : a; }
// a * w mod p with {w, w/p}, |a| < 2^36: exact, |result| <= 1.5 p (as the butterfly kernel)
__device__ __forceinline__ double mulc(double a, double w, double wq)
{
    const double h = a * w;
    const double l = __builtin_fma(a, w, -h);
    const double q = __builtin_fma(a, wq, SHIFT) - SHIFT;
    return __builtin_fma(-q, P, h) + l;
}
// a * b mod p for |a|, |b| <= p, |result| <= p
__device__ __forceinline__ double mulv(double a, double b)
{
    const double h = a * b;
    const double l = __builtin_fma(a, b, -h);
    const double q = __builtin_fma(h, PINV, SHIFT) - SHIFT;
    return __builtin_fma(-q, P, h) + l;
}
// the balanced representative in [-(p-1)/2, (p-1)/2] of a value with |a| <= 2 p
__device__ __forceinline__ double balance(double a)
{
    constexpr double H = 0.5 * (P - 1.0);
    a = a > H ? a - P : (a < -H ? a + P : a);
    return a > H ? a - P : (a < -H ? a + P : a);
}
// residue in [0, p) as the unsigned word the next stage splits
__device__ __forceinline__ uint32_t word(double a) { return (uint32_t)nonneg(reduce(a)); }

// The 16 words x[0..15] of one lane (consecutive K) -> the operand digits: op[b] holds digit
// b of the 16 words, byte j of op[b][i] from x[4 i + j].  Digits are the bytes XOR 0x80.
__device__ __forceinline__ void split(const uint32_t (&x)[16], v4i (&op)[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w0 = x[4 * i] ^ FLIP, w1 = x[4 * i + 1] ^ FLIP;
        const uint32_t w2 = x[4 * i + 2] ^ FLIP, w3 = x[4 * i + 3] ^ FLIP;
        // 4 x 4 byte transpose: word b of the result holds byte b of w0..w3
        const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
        const uint32_t t1 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
        const uint32_t t2 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
        const uint32_t t3 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
        op[0][i] = (int)__builtin_amdgcn_perm(t2, t0, 0x05040100u);
        op[1][i] = (int)__builtin_amdgcn_perm(t2, t0, 0x07060302u);
        op[2][i] = (int)__builtin_amdgcn_perm(t3, t1, 0x05040100u);
        op[3][i] = (int)__builtin_amdgcn_perm(t3, t1, 0x07060302u);
    }
}

// Matrix digits of block w: F[4 a + b] = lane's 16 bytes of f^(b)_a for rows 16 w + lane%16,
// K = 16 (lane/16) + j (the table is laid out [w][4 a + b][lane][16 bytes]).
// The offset is made opaque to the compiler, so that the loads of each stage stay in that
// stage (hoisted out of the branch loop, the four matrices' digits would all be live).
__device__ __forceinline__ void load_digits(const v4i* __restrict__ t, int w, int lane,
                                            v4i (&F)[16])
{
    int z = 0;
    asm volatile("" : "+v"(z));
#pragma unroll
    for (int c = 0; c < 16; ++c) F[c] = t[(w * 16 + c) * 64 + lane + z];
}

// acc[a] = sum_b (F digits a, b) x (data digits b): the matrix on the left (LEFT) or on the
// right of the data
template <bool LEFT>
__device__ __forceinline__ void product(const v4i (&F)[16], const v4i (&op)[4], v4i (&acc)[4])
{
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        v4i c = {0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < 4; ++b)
            c = LEFT ? __builtin_amdgcn_mfma_i32_16x16x64_i8(F[4 * a + b], op[b], c, 0, 0, 0)
                     : __builtin_amdgcn_mfma_i32_16x16x64_i8(op[b], F[4 * a + b], c, 0, 0, 0);
        acc[a] = c;
    }
}

// sum_a 256^a acc[a][i] + corr, exact in float64 (< 2^47), reduced mod p
__device__ __forceinline__ double combine(const v4i (&acc)[4], int i, double corr)
{
    double t = __builtin_fma((double)acc[3][i], 256.0, (double)acc[2][i]);
    t = __builtin_fma(t, 256.0, (double)acc[1][i]);
    t = __builtin_fma(t, 256.0, (double)acc[0][i]);
    return reduce(t + corr);
}

// lane's 16 K-consecutive words of a column block (left products: K runs down the rows)
__device__ __forceinline__ void read_col(const uint32_t* __restrict__ m, int col, int g16,
                                         uint32_t (&x)[16])
{
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = m[(16 * g16 + j) * ROW + col];
}
// ... of a row block (right products: K runs along the row)
__device__ __forceinline__ void read_row(const uint32_t* __restrict__ m, int row, int g16,
                                         uint32_t (&x)[16])
{
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = m[row * ROW + 16 * g16 + j];
}

}  // namespace nttm

template <bool REV>
__global__ __launch_bounds__(256) void ntt_mfma_kernel(
    const int32_t* __restrict__ v, const int32_t* __restrict__ g, int32_t* __restrict__ r,
    int L, int M2, const nttm::v4i* __restrict__ f64, const nttm::v4i* __restrict__ fm2,
    const nttm::v4i* __restrict__ i64, const nttm::v4i* __restrict__ im2,
    const double2* __restrict__ twf, const double2* __restrict__ twi,
    const double2* __restrict__ tn, double ninv, double ninv_q)
{
    using namespace nttm;
    __shared__ uint32_t lp[64 * ROW];
    __shared__ uint32_t lq[64 * ROW];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int g16 = lane >> 4, c16 = lane & 15;
    const int M = 64 * M2, nb = (M2 + 15) >> 4;   // column blocks holding data
    const int64_t ch = blockIdx.x;
    const Span vs = make_span(v, ch * L, L);
    const Span gs = make_span(g, ch * L, L);
    const Span rs = make_span(r, ch * L, L);
    const double c64 = (double)((uint64_t)K0P * 64ull % 998244353ull);
    const double cm2 = (double)((uint64_t)K0P * (uint64_t)M2 % 998244353ull);

    v4i F[16], op[4], acc[4];
    uint32_t x[16];
    uint32_t e0[4][4];      // e^0 of this lane's outputs, kept for branch 1
    uint32_t vk[4][4];      // V^b of this lane's stage-2 outputs, kept for the product

#pragma unroll 1
    for (int b = 0; b < 2; ++b) {
#pragma unroll 1
        for (int s = 0; s < 2; ++s) {
            // 1. u^b_n = a_n omega_N^{b n} for n < M (0 past L) into lp at row n / M2, column
            //    n % M2, as residues in [0, p)
            const Span& src = s == 0 ? vs : gs;
            for (int n = tid; n < M; n += 256) {
                const bool in = n < L;
                const int e = (s == 0 && REV) ? L - 1 - n : n;
                const uint32_t off = in ? (uint32_t)e * 4u : 0x80000000u;
                double a = (double)(int32_t)__builtin_amdgcn_raw_buffer_load_b32(src.rs, (int)off,
                                                                               0, 0);
                a = reduce(a);
                if (b) {
                    const double2 t = tn[n];
                    a = mulc(a, t.x, t.y);
                }
                lp[(n / M2) * ROW + n % M2] = word(a);
            }
            __syncthreads();

            // 2. stage 1: rows 16 w .. of B = F64 a, times omega_M^{n2 k1}, into lq
            load_digits(f64, w, lane, F);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c >= nb) break;
                read_col(lp, 16 * c + c16, g16, x);
                split(x, op);
                product<true>(F, op, acc);
                const int n2 = 16 * c + c16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k1 = 16 * w + 4 * g16 + i;
                    if (n2 < M2) {
                        const double2 t = twf[k1 * M2 + n2];
                        const double y = combine(acc, i, k1 == 0 ? c64 : 0.0);
                        lq[k1 * ROW + n2] = word(mulc(y, t.x, t.y));
                    }
                }
            }
            __syncthreads();

            // 3. stage 2: columns 16 w .. of A = B F_M2 (k = k1 + 64 k2); V kept in registers,
            //    G turned into X = V G N^{-1} and written to lp (row k1, column k2)
            if (16 * w < M2) {
                load_digits(fm2, w, lane, F);
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    read_row(lq, 16 * rb + c16, g16, x);
                    split(x, op);
                    product<false>(F, op, acc);
                    const int k2 = 16 * w + c16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const double y = combine(acc, i, k2 == 0 ? cm2 : 0.0);
                        if (s == 0) {
                            vk[rb][i] = word(y);
                        } else if (k2 < M2) {
                            const int k1 = 16 * rb + 4 * g16 + i;
                            const double xv = mulv((double)vk[rb][i], y);
                            lp[k1 * ROW + k2] = word(mulc(xv, ninv, ninv_q));
                        }
                    }
                }
            }
            __syncthreads();
        }

        // 4. inverse stage A: columns 16 w .. of Z = X F_M2^{-1}, times omega_M^{-m2 k1}, into lq
        if (16 * w < M2) {
            load_digits(im2, w, lane, F);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                read_row(lp, 16 * rb + c16, g16, x);
                split(x, op);
                product<false>(F, op, acc);
                const int m2 = 16 * w + c16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k1 = 16 * rb + 4 * g16 + i;
                    if (m2 < M2) {
                        const double2 t = twi[k1 * M2 + m2];
                        const double y = combine(acc, i, m2 == 0 ? cm2 : 0.0);
                        lq[k1 * ROW + m2] = word(mulc(y, t.x, t.y));
                    }
                }
            }
        }
        __syncthreads();

        // 5. inverse stage B: rows 16 w .. of e^b = F64^{-1} Z at n = M2 m1 + m2; branch 0
        //    keeps e^0, branch 1 forms x_n = e^0_n + omega_N^{-n} e^1_n, lifts and stores it
        load_digits(i64, w, lane, F);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (c >= nb) break;
            read_col(lq, 16 * c + c16, g16, x);
            split(x, op);
            product<true>(F, op, acc);
            const int m2 = 16 * c + c16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m1 = 16 * w + 4 * g16 + i;
                const double y = combine(acc, i, m1 == 0 ? c64 : 0.0);
                if (b == 0) {
                    e0[c][i] = word(y);
                } else {
                    const int n = M2 * m1 + m2;
                    if (m2 < M2 && n < L) {
                        const double2 t = tn[(2 * M - n) & (2 * M - 1)];
                        const double s = balance(reduce(mulc(y, t.x, t.y) + (double)e0[c][i]));
                        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(int32_t)s, rs.rs,
                                                              (REV ? L - 1 - n : n) * 4, 0, 0);
                    }
                }
            }
        }
        __syncthreads();
    }
}

hipError_t launch_ntt_mfma(const int32_t* v, const int32_t* g, int32_t* r, int64_t nch, int L,
                           int M, bool rev, const NttMfmaTables& t, hipStream_t stream)
{
    const int M2 = M / 64;
    if (M2 < 1 || M2 > 64 || 64 * M2 != M) return hipErrorInvalidValue;
    int lg = 0;
    while ((1 << lg) < M2) ++lg;
    if (!grid_ok(nch, 256)) return hipErrorInvalidValue;
    const nttm::v4i* f64 = (const nttm::v4i*)t.digits[0][6];
    const nttm::v4i* i64 = (const nttm::v4i*)t.digits[1][6];
    const nttm::v4i* fm2 = (const nttm::v4i*)t.digits[0][lg];
    const nttm::v4i* im2 = (const nttm::v4i*)t.digits[1][lg];
    const double2* twf = t.twiddle[0][lg];
    const double2* twi = t.twiddle[1][lg];
    const double2* tn = t.roots[lg];
    if (rev)
        hipLaunchKernelGGL((ntt_mfma_kernel<true>), dim3((unsigned)nch), dim3(256), 0, stream, v, g,
                           r, L, M2, f64, fm2, i64, im2, twf, twi, tn, t.ninv[lg], t.ninv_q[lg]);
    else
        hipLaunchKernelGGL((ntt_mfma_kernel<false>), dim3((unsigned)nch), dim3(256), 0, stream, v,
                           g, r, L, M2, f64, fm2, i64, im2, twf, twi, tn, t.ninv[lg],
                           t.ninv_q[lg]);
    return hipGetLastError();
}

}  // namespace sc
